/*
 * pda.h -- C ABI of the MI355X (gfx950) paged-decode attention library.
 *
 * One query token per sequence attends over a BF16 paged KV cache laid out
 * [num_blocks, block_size, num_kv_heads, head_dim], reached through
 * per-sequence block tables, with grouped-query (GQA) head sharing: q head h
 * reads KV head h / (num_q_heads / num_kv_heads).  The KV length of each
 * sequence is cut into num_splits chunks; each chunk leaves an FP32
 * (o[head_dim], m, l) partial in a caller-owned workspace and a merge pass
 * writes o / l as BF16, or 0 where l == 0.
 *
 * Sources: the "Module attn_splitk" page (rustdoc of the kernels crate's
 * split-K launch-geometry module) for the split count, the workspace and the
 * packed-kernel gate; the "metrale_storage/tiled_attention.rs" source page
 * for the tiled begin_step / step_tile / finalize state API and the two K/V
 * stride sets.  Those pages describe kernels for other GPUs; only their
 * interfaces and formulas are followed here.
 *
 * Conventions for every call
 * --------------------------
 * - Return codes: PDA_OK (0) on success; PDA_NOT_APPLICABLE (1) when a call
 *   asked explicitly for the packed kernel and the launch is not one it
 *   serves (nothing is launched; the caller runs the unpacked path); a
 *   negative code on error: PDA_EINVAL (bad argument), PDA_ENOMEM, or
 *   PDA_EHIP_BASE - hipError_t for a failing HIP call.  pda_last_error()
 *   then holds a message.  Nothing aborts and nothing throws across the ABI.
 * - Device pointers are plain `void*` / `T*` into device memory; the caller
 *   owns every buffer except the tiled state, which the handle owns.
 * - `stream` is a hipStream_t passed as void*; NULL is the null stream.
 *   Every launch is asynchronous on that stream; no call synchronises the
 *   host, and pda_paged_decode, pda_tiled_begin_step, pda_tiled_step_tile
 *   and pda_tiled_finalize allocate nothing.
 * - Arguments are checked on the host before any launch.  Values that live
 *   in device memory (block ids, sequence lengths, tile counts) cannot be
 *   checked there; the kernels clamp them so that no access leaves the
 *   buffers described by the arguments: a block id outside [0, num_blocks)
 *   drops its tokens, a length past the block table is cut to the table.
 *   Such inputs give unspecified (but memory-safe) results.
 * - BF16 is stored as 16-bit patterns; results are rounded to nearest even.
 */
#ifndef PDA_H
#define PDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PDA_OK 0
#define PDA_NOT_APPLICABLE 1
#define PDA_EINVAL (-22)
#define PDA_ENOMEM (-12)
#define PDA_EHIP_BASE (-1000)

/* Split-count policies (attn_splitk page, enum SplitkPolicy). */
#define PDA_SPLITK_LEGACY 0
#define PDA_SPLITK_AUTO 1
#define PDA_SPLITK_PINNED 2

/* pda_paged_decode flags. */
#define PDA_DECODE_UNPACKED 0u /* split-K kernel + merge (any shape)      */
#define PDA_DECODE_PACKED 1u   /* GQA-packed MFMA kernel, or NOT_APPLICABLE */
#define PDA_DECODE_DEFAULT 2u  /* packed iff pda_gqa_pack_enabled() and it
                                  applies, else unpacked; never NOT_APPLICABLE */

/* ------------------------------------------------------------------------
 * Constants.
 * ------------------------------------------------------------------------ */

/* Ceiling on the split count under Auto and Pinned, and so on the workspace
 * (attn_splitk page, MAX_DECODE_SPLITS; value not printed there: 16 here). */
uint32_t pda_max_decode_splits(void);
/* Waves of workgroups Auto aims for with one sequence in flight
 * (attn_splitk page, SPLITK_TARGET_WAVES; 2, as its examples imply). */
uint32_t pda_splitk_target_waves(void);
/* Query heads one packed workgroup carries (attn_splitk page,
 * DECODE_GQA_PACK_WIDTH; 8 here). */
uint32_t pda_gqa_pack_width(void);
/* Head dim of the packed kernel (attn_splitk page, DECODE_GQA_PACK_HEAD_DIM: 256). */
uint32_t pda_gqa_pack_head_dim(void);
/* Floor on a split's token count, from the sequence's own length
 * (attn_splitk page, module description on short contexts; 64 here). */
uint32_t pda_min_kv_per_split(void);
/* Largest head_dim the tiled state accepts (tiled_attention.rs, validate: 256). */
uint32_t pda_max_head_dim(void);

/* ------------------------------------------------------------------------
 * Launch geometry: pure host functions, no HIP calls, bit-exact integers.
 * 0 is returned for inputs with no defined result (a zero divisor).
 * ------------------------------------------------------------------------ */

/* clamp(ceil(WAVES * cu_count / num_q_heads), 1, MAX_DECODE_SPLITS)
 * (attn_splitk page, auto_splits).  0 if num_q_heads == 0. */
uint32_t pda_auto_splits(uint32_t cu_count, uint32_t num_q_heads);
/* max(max_decode_seqs, num_seqs) (attn_splitk page, legacy_splits). */
uint32_t pda_split_ref_seqs(uint32_t num_seqs, uint32_t max_decode_seqs);
/* Legacy rule: current = num_q_heads * ref_seqs; 1 if current >= cu_count,
 * else cu_count / current (integer).  Not clamped.  0 if current == 0
 * (attn_splitk page, module description and legacy_splits). */
uint32_t pda_legacy_splits(uint32_t cu_count, uint32_t num_q_heads, uint32_t ref_seqs);
/* clamp(pin, 1, MAX_DECODE_SPLITS) (attn_splitk page, MAX_DECODE_SPLITS, parse). */
uint32_t pda_pinned_splits(uint32_t pin);
/* The split count for a launch under `policy` (PDA_SPLITK_*); only Legacy
 * reads num_seqs / max_decode_seqs (attn_splitk page, num_splits and the
 * module invariants).  0 for an unknown policy or a zero divisor. */
uint32_t pda_num_splits(int policy, uint32_t pin, uint32_t cu_count, uint32_t num_q_heads,
                        uint32_t num_seqs, uint32_t max_decode_seqs);
/* FP32 values of the split-K workspace: rows * num_q_heads * num_splits *
 * (head_dim + 2) (attn_splitk page, MAX_DECODE_SPLITS and workspace_slots).
 * Layout: [rows][num_q_heads][num_splits][head_dim + 2], each slot holding
 * o[0..head_dim) (unnormalised), then m (natural-log units), then l. */
uint64_t pda_workspace_slots(uint64_t rows, uint32_t num_q_heads, uint32_t num_splits,
                             uint32_t head_dim);
/* 1 iff num_kv_heads > 0, head_dim == 256 and num_q_heads == num_kv_heads * 8
 * (attn_splitk page, module invariants and gqa_pack_shape_ok). */
int pda_gqa_pack_shape_ok(uint32_t num_q_heads, uint32_t num_kv_heads, uint32_t head_dim);
/* Workgroups of a packed launch in the page's shape, one per (sequence, KV
 * head): num_kv_heads * num_seqs (attn_splitk page, gqa_pack_ctas).  This
 * library's non-split packed launch (pda_paged_decode with
 * PDA_DECODE_PACKED and num_splits == 1) may split each (sequence, KV head)
 * of 33 blocks or more over up to 2 workgroups that combine in-kernel, so
 * it dispatches up to twice this count; the packed split-K form dispatches
 * this count times num_splits. */
uint64_t pda_gqa_pack_ctas(uint32_t num_kv_heads, uint32_t num_seqs);
/* Tokens per split of one sequence: ceil(seq_len / num_splits) floored at
 * pda_min_kv_per_split(), rounded up to whole blocks.  Split i covers
 * [i * chunk, min((i + 1) * chunk, seq_len)); a split starting at or past
 * seq_len is empty.  0 if num_splits or block_size is 0. */
uint32_t pda_split_chunk(uint32_t seq_len, uint32_t num_splits, uint32_t block_size);

/* ------------------------------------------------------------------------
 * One-shot paged decode over an FP8 KV cache (attn_splitk page: the FP8
 * paged-decode launches it names; the format and scaling are this
 * library's reading, as the page prints neither).
 *
 * Same as pda_paged_decode except:
 *   k_cache, v_cache  uint8 [num_blocks, block_size, num_kv_heads, head_dim],
 *                     OCP FP8 E4M3 codes (bias 7, 3 mantissa bits,
 *                     subnormals, S.1111.111 = NaN, largest finite 448)
 *   k_scale, v_scale  per-tensor FP32 scales: K = decode(k) * k_scale,
 *                     V = decode(v) * v_scale (scores are
 *                     scale * q . K; the workspace partials hold o of the
 *                     scaled V)
 *   flags             as for pda_paged_decode: the GQA-packed MFMA kernel
 *                     has an FP8 form (the page names a BF16 and an FP8
 *                     packed source), with the same gate, and
 *                     PDA_DECODE_DEFAULT arms it on non-split launches when
 *                     pda_gqa_pack_enabled() says so
 * q stays BF16 and out is BF16; the caches are checked for the same
 * alignment as pda_paged_decode's.
 * ------------------------------------------------------------------------ */
int pda_paged_decode_fp8(const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* block_tables, const int32_t* seq_lens, void* out,
                         float* workspace, uint64_t workspace_floats, uint32_t num_seqs,
                         uint32_t num_q_heads, uint32_t num_kv_heads, uint32_t head_dim,
                         uint32_t block_size, uint32_t max_blocks_per_seq, uint32_t num_blocks,
                         float scale, float k_scale, float v_scale, uint32_t num_splits,
                         uint32_t flags, void* stream);

/* pda_paged_decode_fp8 without the merge (num_splits >= 2): leaves the
 * partials in the workspace; pda_splitk_merge finishes them.  flags as for
 * pda_splitk_partials. */
int pda_splitk_partials_fp8(const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* block_tables, const int32_t* seq_lens,
                            float* workspace, uint64_t workspace_floats, uint32_t num_seqs,
                            uint32_t num_q_heads, uint32_t num_kv_heads, uint32_t head_dim,
                            uint32_t block_size, uint32_t max_blocks_per_seq,
                            uint32_t num_blocks, float scale, float k_scale, float v_scale,
                            uint32_t num_splits, uint32_t flags, void* stream);

/* ------------------------------------------------------------------------
 * Causal paged prefill (prefill page "prefill_attn_fa128.rs": `applies` and
 * the `paged` launcher; head dim 256, 128 query rows per workgroup).
 * ------------------------------------------------------------------------ */

/* Whether the prefill kernel serves a launch: head_dim == 256, causal,
 * sliding_window == 0, num_kv_heads > 0 and num_q_heads % num_kv_heads == 0. */
int pda_prefill_applies(uint32_t num_q_heads, uint32_t num_kv_heads, uint32_t head_dim,
                        int causal, uint32_t sliding_window);

/* Causal attention of one sequence's q_len new rows over its paged cache.
 *
 *   q            bf16 [q_len, num_q_heads, head_dim]; row i is the token at
 *                position q_offset + i
 *   k_cache      bf16 [num_blocks, block_size, num_kv_heads, head_dim]
 *   v_cache      bf16, same layout
 *   out          bf16 [q_len, num_q_heads, head_dim]
 *   block_table  int32 [max_blocks]: the sequence's pool blocks in token
 *                order (entry j holds tokens [j*block_size, (j+1)*block_size))
 *   kv_len       tokens of the sequence in the cache (<= max_blocks*block_size)
 *   scale        multiplies q.k (the page's inv_sqrt_d)
 * Row i attends the keys at positions j <= q_offset + i with j < kv_len;
 * q head h reads KV head h / (num_q_heads / num_kv_heads); a row with no key
 * is 0.  Returns PDA_NOT_APPLICABLE, launching nothing, when q_len == 0 or
 * pda_prefill_applies(num_q_heads, num_kv_heads, head_dim, 1, sliding_window)
 * is 0 (the caller runs another kernel); PDA_EINVAL for a bad argument.
 * Requirements: block_size > 0, num_blocks > 0, q_offset + q_len and kv_len
 * below 2^31, q / caches / out 16-byte aligned.  Block ids outside
 * [0, num_blocks) give unspecified but in-bounds results.  Allocates nothing;
 * asynchronous on `stream`. */
int pda_paged_prefill(const void* q, const void* k_cache, const void* v_cache, void* out,
                      const int32_t* block_table, uint32_t q_len, uint32_t kv_len,
                      uint32_t q_offset, uint32_t num_q_heads, uint32_t num_kv_heads,
                      uint32_t head_dim, uint32_t block_size, uint32_t max_blocks,
                      uint32_t num_blocks, uint32_t sliding_window, float scale, void* stream);

/* ------------------------------------------------------------------------
 * Policy resolution (attn_splitk page: parse, parse_gqa_pack,
 * resolve_policy, policy_from_env, resolve_gqa_pack, gqa_pack_enabled,
 * DECODE_GQA_PACK_DECLARED).  Host-only; no HIP calls.  Text is trimmed of
 * ASCII whitespace and compared without regard to ASCII case.
 * ------------------------------------------------------------------------ */

/* A split-count policy: PDA_SPLITK_* and, for Pinned, the split count. */
typedef struct {
    int32_t policy;
    uint32_t pin;
} pda_splitk_policy;

/* "legacy" -> Legacy; "auto" -> Auto; "0" / "off" / "false" / "no" -> Pinned
 * 1 (split-K off); a decimal count (ASCII digits) -> Pinned, clamped to
 * 1..pda_max_decode_splits() (too large a number saturates first).
 * Returns 1 and fills *out when `s` parses, else 0 (also for NULL). */
int pda_parse_splitk_policy(const char* s, pda_splitk_policy* out);

/* "1" / "on" / "true" / "yes" -> 1; "0" / "off" / "false" / "no" -> 0.
 * Returns 1 and fills *on when `s` parses, else 0 (also for NULL). */
int pda_parse_gqa_pack(const char* s, int* on);

/* The split-count declaration this library carries for MI355X: "auto". */
const char* pda_splitk_declared(void);

/* `declared`, overridden by `env_value` when that parses; a declaration
 * that does not parse is Legacy.  env_value NULL means unset.  Pure. */
void pda_resolve_policy(const char* declared, const char* env_value, pda_splitk_policy* out);

/* pda_resolve_policy(pda_splitk_declared(),
 * getenv("METRALE_ATTN_DECODE_SPLITK")); reads the environment each call. */
void pda_policy_from_env(pda_splitk_policy* out);

/* DECODE_GQA_PACK_DECLARED: the packed kernel is declared off (0). */
int pda_decode_gqa_pack_declared(void);

/* `declared` (0 / 1), overridden by `env_value` when that parses.  Pure. */
int pda_resolve_gqa_pack(int declared, const char* env_value);

/* Whether the packed kernel is armed in this process:
 * pda_resolve_gqa_pack(pda_decode_gqa_pack_declared(),
 * getenv("METRALE_ATTN_DECODE_GQA_PACK")), resolved on the first call and
 * fixed for the life of the process (so captured launches stay consistent
 * with later ones).  Thread-safe. */
int pda_gqa_pack_enabled(void);

/* Compute units of HIP device `device` (the cu_count the policies take). */
int pda_device_cu_count(int device, uint32_t* cu_count);

/* ------------------------------------------------------------------------
 * One-shot paged decode.
 *
 * The operation is the problem statement this library answers: one query
 * per sequence attends softmax(scale * q.K^T).V over its paged cache; the
 * split-K form follows the "Module attn_splitk" page: its module
 * description (the KV length of each sequence is cut into num_splits
 * chunks whose partial states are merged, and because that merge is not
 * associative the split count must not follow the batch), MAX_DECODE_SPLITS
 * and workspace_slots (the [o, m, l] partials of every (row, head, split));
 * the running state (m, l, o unnormalised) and the o / l finalize with 0
 * where l == 0 follow the "metrale_storage/tiled_attention.rs" page
 * (module comment, begin_step, finalize).
 *
 *   q            bf16 [num_seqs, num_q_heads, head_dim]        (device)
 *   k_cache      bf16 [num_blocks, block_size, num_kv_heads, head_dim]
 *   v_cache      bf16, same layout as k_cache
 *   block_tables int32 [num_seqs, max_blocks_per_seq]; entry j of row s is
 *                the pool block holding tokens [j*block_size, (j+1)*block_size)
 *                of sequence s
 *   seq_lens     int32 [num_seqs]; 0 is allowed (output 0)
 *   out          bf16 [num_seqs, num_q_heads, head_dim]; out = o / l, 0 if l == 0
 *   workspace    f32, at least pda_workspace_slots(num_seqs, num_q_heads,
 *                num_splits, head_dim) values; may be NULL iff num_splits == 1.
 *                On return (stream-ordered) it holds every split's partial.
 *   scale        multiplies q.k before the softmax (e.g. 1/sqrt(head_dim))
 *   num_splits   1..pda_max_decode_splits(); pick it with pda_num_splits.
 *                A sequence's output bytes depend on its own data, scale,
 *                num_splits and the shape only, never on the other rows of
 *                the batch.
 *   flags        PDA_DECODE_UNPACKED; PDA_DECODE_PACKED to run the
 *                GQA-packed MFMA kernel, which serves only
 *                pda_gqa_pack_shape_ok shapes (else PDA_NOT_APPLICABLE,
 *                nothing launched), with num_splits == 1 (bf16 out
 *                directly) or, as this library's extension of the pages'
 *                non-split packed kernels, num_splits > 1 (the same
 *                workspace partials and merge as the unpacked path); or
 *                PDA_DECODE_DEFAULT: the packed kernel when
 *                pda_gqa_pack_enabled(), the shape qualifies and
 *                num_splits == 1, the unpacked path otherwise.
 *
 * Requirements: num_kv_heads > 0, num_q_heads % num_kv_heads == 0,
 * head_dim in {64, 128, 256}, block_size a positive multiple of 16, q /
 * caches / out 16-byte aligned, workspace 8-byte aligned.  num_seqs == 0
 * launches nothing.
 *
 * Launches with fewer than 128 (KV head, split) pairs per sequence split
 * each split of 129 blocks or more (a long single sequence) over several
 * workgroups, and non-split launches of the packed kernel split each
 * sequence of 33 blocks or more over two; the workgroups hand partial
 * results to each other through device arrays the library owns (per GPU:
 * 16 MiB of records and 64 Ki counters for each of the two kernels; no
 * allocation; batches beyond them run as several launches).  The number of
 * workgroups a sequence uses depends only on the shape, the split count and
 * its own length, so its bytes still do not depend on the batch.  Such
 * calls (this one, pda_splitk_partials and their FP8 forms) must not
 * overlap on one GPU: issue them on one stream, or order the streams.
 * ------------------------------------------------------------------------ */
int pda_paged_decode(const void* q, const void* k_cache, const void* v_cache,
                     const int32_t* block_tables, const int32_t* seq_lens, void* out,
                     float* workspace, uint64_t workspace_floats, uint32_t num_seqs,
                     uint32_t num_q_heads, uint32_t num_kv_heads, uint32_t head_dim,
                     uint32_t block_size, uint32_t max_blocks_per_seq, uint32_t num_blocks,
                     float scale, uint32_t num_splits, uint32_t flags, void* stream);

/* pda_paged_decode for callers that cannot allocate device memory or pass a
 * workspace (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the same arguments without workspace /
 * workspace_floats, the same kernels and the same output bytes.  The split-K
 * partials go to a scratch array the library holds in device memory, one per
 * GPU, 16 MiB (4 Mi FP32 values), for the life of the process.
 *
 *   Limit: pda_workspace_slots(num_seqs, num_q_heads, num_splits, head_dim)
 *   must not exceed 4194304 (the batch decode shape of 32 sequences, 32 q
 *   heads, head dim 128 at 16 splits needs 2129920); larger calls return
 *   PDA_EINVAL before anything is launched.  num_splits == 1 uses no
 *   scratch.  Nothing in the scratch has to start at any value: every slot
 *   the merge reads is written earlier in the same call.
 *
 * Every call on one GPU shares that GPU's scratch, so calls that overlap on
 * one GPU (different streams, or several threads) race and give undefined
 * results: issue them on one stream, or order the streams.  The same holds
 * with pda_paged_decode calls that split items into parts (see above).
 * Calls no hipMalloc, hipFree or allocating routine; the first call on a
 * device looks the scratch address up (hipGetSymbolAddress). */
int pda_paged_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                             const int32_t* block_tables, const int32_t* seq_lens, void* out,
                             uint32_t num_seqs, uint32_t num_q_heads, uint32_t num_kv_heads,
                             uint32_t head_dim, uint32_t block_size,
                             uint32_t max_blocks_per_seq, uint32_t num_blocks, float scale,
                             uint32_t num_splits, uint32_t flags, void* stream);

/* The merge pass alone ("Module attn_splitk", module description: the
 * split partial states of one (row, head) are combined into one output;
 * workspace_slots for their layout): reads the workspace written by a
 * split-K launch of the same shape and writes out (bf16 [num_seqs,
 * num_q_heads, head_dim]): per (row, head), over the splits in index order,
 * M = max m_i, w_i = exp(m_i - M), out = sum w_i o_i / sum w_i l_i, or 0 when
 * every split has l == 0.
 * Splits with l == 0 are skipped; their o is never read.  Exposed so the
 * partials can be checked and timed on their own; pda_paged_decode already
 * runs it. */
int pda_splitk_merge(const float* workspace, uint64_t workspace_floats, void* out,
                     uint32_t num_seqs, uint32_t num_q_heads, uint32_t head_dim,
                     uint32_t num_splits, void* stream);

/* pda_paged_decode without the merge ("Module attn_splitk": the split
 * partials of workspace_slots, one [o, m, l] slot per (row, head, split)):
 * leaves the partials in the workspace (num_splits >= 2); o is unnormalised,
 * m in natural-log units, and an empty split holds m = -inf, l = 0.  flags: PDA_DECODE_UNPACKED or PDA_DECODE_DEFAULT (the
 * split-K fold kernel), or PDA_DECODE_PACKED (the packed MFMA kernel's
 * split-K form; PDA_NOT_APPLICABLE unless pda_gqa_pack_shape_ok). */
int pda_splitk_partials(const void* q, const void* k_cache, const void* v_cache,
                        const int32_t* block_tables, const int32_t* seq_lens,
                        float* workspace, uint64_t workspace_floats, uint32_t num_seqs,
                        uint32_t num_q_heads, uint32_t num_kv_heads, uint32_t head_dim,
                        uint32_t block_size, uint32_t max_blocks_per_seq, uint32_t num_blocks,
                        float scale, uint32_t num_splits, uint32_t flags, void* stream);

/* ------------------------------------------------------------------------
 * Tiled state API (tiled_attention.rs page: TiledAttention).
 *
 * A decode step is pda_tiled_begin_step (m, l, o := -inf, 0, 0 for the
 * first num_seqs sequences), one pda_tiled_step_tile per tile of KV blocks
 * (folding the tile into the FP32 running state), and pda_tiled_finalize
 * (out = o / l as BF16, 0 where l == 0).  The state is allocated once, for
 * max_seqs sequences, by pda_tiled_create and reused by every step.
 * State layout: m, l f32 [max_seqs * num_q_heads]; o f32 [max_seqs *
 * num_q_heads * head_dim]; index (s * num_q_heads + h).  m is in natural-log
 * units; the scores are q.k / sqrt(head_dim) (the step takes no scale).
 * ------------------------------------------------------------------------ */
typedef struct pda_tiled_dims {
    uint32_t max_seqs;
    uint32_t num_q_heads;
    uint32_t num_kv_heads;
    uint32_t head_dim;
    uint32_t block_size;
    uint32_t tile_capacity; /* blocks per sequence per step_tile */
} pda_tiled_dims;

typedef struct pda_tiled pda_tiled;

/* PDA_OK if the dims are usable: num_kv_heads > 0, num_q_heads a multiple of
 * num_kv_heads, head_dim <= 256 (tiled_attention.rs, validate), and for the
 * kernels head_dim in {64, 128, 256}, block_size a positive multiple of 16,
 * max_seqs, num_q_heads and tile_capacity > 0. */
int pda_tiled_validate(const pda_tiled_dims* dims);
/* Validates, then allocates the state on the current HIP device.  *out is
 * set only on success; release it with pda_tiled_destroy. */
int pda_tiled_create(const pda_tiled_dims* dims, pda_tiled** out);
void pda_tiled_destroy(pda_tiled* t);
int pda_tiled_get_dims(const pda_tiled* t, pda_tiled_dims* dims);
/* Device pointers of the running state (owned by the handle). */
int pda_tiled_state(const pda_tiled* t, float** m, float** l, float** o);
/* (blk, tok, kvh) strides in bf16 elements of the paged layout
 * [num_blocks, block_size, num_kv_heads, head_dim]: (bs*nkv*D, nkv*D, D)
 * (tiled_attention.rs, paged_strides). */
void pda_tiled_paged_strides(const pda_tiled_dims* dims, int64_t out[3]);
/* (blk, tok, kvh) strides in bf16 elements of the scratch-pool slot layout
 * [slot, K|V, kv_head, block_size, head_dim]: (2*nkv*bs*D, D, bs*D)
 * (tiled_attention.rs, scratch_pool_strides).  With that layout the V pool
 * pointer is the K pool pointer plus nkv*bs*D elements. */
void pda_tiled_scratch_pool_strides(const pda_tiled_dims* dims, int64_t out[3]);
/* m, l, o := -inf, 0, 0 for the first num_seqs sequences; PDA_EINVAL if
 * num_seqs > max_seqs (tiled_attention.rs, begin_step).  Uses a fill kernel,
 * so it is safe to record in a HIP graph. */
int pda_tiled_begin_step(pda_tiled* t, uint32_t num_seqs, void* stream);
/* Fold one tile into the state.
 *   q                  bf16 [num_seqs, num_q_heads, head_dim]
 *   k_pool, v_pool     bf16 pools addressed as base + blk*blk_stride +
 *                      slot*tok_stride + kvh*kvh_stride + d (elements)
 *   pool_blocks        blocks the pools hold (ids outside are dropped)
 *   tile_blocks        int32 [num_seqs, tile_capacity]: the tile's block ids
 *   tile_block_counts  int32 [num_seqs]: blocks in this tile per sequence
 *                      (0 leaves that sequence's state untouched)
 *   last_block_valid_slots  valid token slots (1..block_size) of the last
 *                      block (index count-1) of every sequence in the call;
 *                      its other blocks are full.
 * Strides must be multiples of 8 and the pool pointers 16-byte aligned. */
int pda_tiled_step_tile(pda_tiled* t, const void* q, const void* k_pool, const void* v_pool,
                        uint64_t pool_blocks, const int32_t* tile_blocks,
                        const int32_t* tile_block_counts, uint32_t num_seqs,
                        int64_t blk_stride, int64_t tok_stride, int64_t kvh_stride,
                        int32_t last_block_valid_slots, void* stream);
/* out bf16 [num_seqs, num_q_heads, head_dim] = o / l, 0 where l == 0
 * (tiled_attention.rs, finalize). */
int pda_tiled_finalize(pda_tiled* t, void* out, uint32_t num_seqs, void* stream);

/* Message of the last failing call on this thread ("" if none). */
const char* pda_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PDA_H */
