// Split-K paged-decode attention kernels for gfx950 (CDNA4, wave64).
//
// One workgroup folds a token range of one (sequence, KV head, head group)
// into an online-softmax state: the range is one split of the sequence
// (one-shot decode) or one tile of blocks (tiled step).  The running state
// (m, l, o) with o unnormalised, the -inf/0/0 start and the o / l finalize
// rule (0 where l is 0) follow the "metrale_storage/tiled_attention.rs"
// page (module comment, begin_step, finalize); the split-K workspace of
// [o[head_dim], m, l] FP32 slots follows the "Module attn_splitk" page
// (MAX_DECODE_SPLITS, workspace_slots).
//
// Work layout of a wave (the hot loop runs on VALU, so every step is laid
// out to spend as few vector instructions per K/V byte as possible):
//   * A K/V row of one token and one KV head is head_dim BF16 values; LPT =
//     head_dim / 8 lanes share it, each holding one 16-byte piece, so one
//     wave-wide buffer load fetches ROWS = 64 / LPT token rows.  A group is
//     U such loads (TG = ROWS * U tokens, inside one block: one scalar
//     block-table read per group).
//   * Every lane keeps the q pieces of all GC query heads of its KV head, so
//     each K/V byte is read from HBM once and serves all GC heads from
//     registers.  q.k is a v_dot2_f32_bf16 chain over the piece: GC * U
//     partial dots per lane.
//   * The partial dots are transposed through LDS so that each lane owns
//     whole (head, token) scores: one lane per score, so one exponential per
//     score instead of one per score and lane, and no cross-lane butterfly.
//     The U scores of a head sit in adjacent lanes; their max and sum are
//     two DPP steps.  The probabilities and the per-head rescale factors go
//     back through LDS to the lanes that hold V, which accumulate P.V in
//     FP32.  LDS traffic never leaves the wave, so no barrier is needed.
//   * The unnormalised o is rescaled only when some running max grew (the
//     factor is exactly 1 otherwise, so skipping it changes no bit).
//   * Each token row keeps its own state; at the end every (wave, row)
//     state goes to LDS and one fixed-order pass merges them, so the result
//     depends only on the sequence's own data and the launch shape, never
//     on the rest of the batch.
//   * Parts: a long item (a split of a long sequence when a launch gives
//     each sequence few items, or a long tile of a tiled step) is split
//     over several workgroups, each folding a contiguous run of its blocks
//     into an FP32 record; the last to take a ticket combines the records
//     in part order.  How many parts an item uses depends only on its own
//     block count, so the bytes still depend only on the sequence's data.
// Exponentials are v_exp_f32 (base 2): scores are scaled by scale * log2(e)
// and m is converted back to natural-log units when it is stored.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
#include <utility>
#include <vector>

#include "pda_geometry.h"
#include "pda_kernels.h"

namespace pda {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c, false);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    bf16x2_t v;
    v[0] = (__bf16)a;
    v[1] = (__bf16)b;
    return __builtin_bit_cast(uint32_t, v);
}

// Two E4M3 codes (bytes 0, 1 of w, or bytes 2, 3 with HI) as a BF16 pair,
// first code in the low half.  Exact: 3 mantissa bits, and every E4M3
// exponent is in BF16's range; the scale operand 1.0 leaves values as they
// are (the conversion uses only its exponent).
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.f, HI));
}
__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Part records are written and read at device scope (stores that write
// through to the level every XCD shares, loads that do not hit a stale
// copy), so handing them over needs no L2 writeback or invalidate: a writer
// waits for its record stores to complete before its workgroup takes a
// ticket, and the combining workgroup loads the records only after taking
// the last ticket.  This relies on the hardware's ordering of those
// operations rather than on a release / acquire pair (PDA_PARTS_ORDER in
// pda_kernels.h states the argument and the measured cost of the formal
// forms).
__device__ __forceinline__ void put_dev(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float get_dev(const float* p) {
    return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __int_as_float(
        __builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Max / sum over the N adjacent lanes (N = 2 or 4, aligned) holding the
// scores of one head; every lane of the set gets identical bits.
template <int N>
__device__ __forceinline__ float nmax(float x) {
    x = fmaxf(x, dpp<0xB1>(x));                      // quad_perm [1,0,3,2]
    if constexpr (N == 4) x = fmaxf(x, dpp<0x4E>(x));  // quad_perm [2,3,0,1]
    return x;
}
template <int N>
__device__ __forceinline__ float nsum(float x) {
    x += dpp<0xB1>(x);
    if constexpr (N == 4) x += dpp<0x4E>(x);
    return x;
}

// Values of the two lanes 16 apart (rows 2i and 2i + 1 of 16 lanes) and of
// the two lanes 32 apart (the wave's halves), identical on both partners.
__device__ __forceinline__ void swap16(float x, float& a, float& b) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
}
__device__ __forceinline__ void swap32(float x, float& a, float& b) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
}

// Max / sum over the 64 / LPT token rows of a wave (lanes LPT apart), in a
// fixed butterfly order; every lane gets identical bits.
template <int LPT>
__device__ __forceinline__ float rows_max(float x) {
    float a, b;
    if constexpr (LPT <= 8) x = fmaxf(x, dpp<0x128>(x));   // row_ror:8, lanes 8 apart
    if constexpr (LPT <= 16) {
        swap16(x, a, b);
        x = fmaxf(a, b);
    }
    swap32(x, a, b);
    return fmaxf(a, b);
}
template <int LPT>
__device__ __forceinline__ float rows_sum(float x) {
    float a, b;
    if constexpr (LPT <= 8) x = x + dpp<0x128>(x);
    if constexpr (LPT <= 16) {
        swap16(x, a, b);
        x = a + b;
    }
    swap32(x, a, b);
    return a + b;
}

// Orders this wave's LDS accesses: the writes before it are complete, and
// visible to every lane of the wave, before the reads after it.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Buffer descriptor over `bytes` bytes from `base` (raw, unswizzled; reads
// past the range return 0).
// The base and size are wave-uniform; readfirstlane makes that explicit so
// the descriptor always lives in scalar registers (a descriptor the compiler
// cannot prove uniform costs a loop over lanes around every load).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    void* ub = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(ub, (short)0,
                                             (int)__builtin_amdgcn_readfirstlane(bytes),
                                             0x00020000);
}

// Sequences are folded longest first: blockIdx.y is a rank in descending
// order of length (ties by index), so the hardware dispatcher, which hands
// out workgroups in id order, schedules the longest work first and the grid
// drains with short work items (longest-processing-time-first).  Only the
// schedule changes; each item's arithmetic is the same in any order.
//
// Every wave ranks the lengths itself: one wave-wide load of up to 64
// lengths, then one compare per sequence against a value read from another
// lane (v_readlane), so the cost is one memory round trip, not one per
// sequence.  The sort key packs the length (saturated at 2^23 - 1, which
// only coarsens the schedule of longer sequences) above the inverted index,
// so keys are distinct and a larger key ranks first.  Batches of more than
// kRankMax sequences keep their given order.
constexpr int kRankMax = 64;

__device__ __forceinline__ int clamp_len(int x, int cap) {
    return x < 0 ? 0 : (x > cap ? cap : x);
}

#ifndef PDA_FOLD_LPT
#define PDA_FOLD_LPT 1
#endif
// The sequence this workgroup works on and its length clamped to [0, cap].
__device__ __forceinline__ void seq_of_rank(const int32_t* __restrict__ lens, int S, int r,
                                            int cap, int& seq, int& len) {
    if (!PDA_FOLD_LPT || S > kRankMax) {
        seq = r;
        len = clamp_len(lens[r], cap);
        return;
    }
    const int lane = (int)__lane_id();
    const int Li = lane < S ? clamp_len(lens[lane], cap) : -1;
    const int key = lane < S ? (min(Li, (1 << 23) - 1) << 8) | (255 - lane) : -1;
    int cnt = 0;
    for (int j = 0; j < S; ++j) cnt += __builtin_amdgcn_readlane(key, j) > key;
    const uint64_t mask = __builtin_amdgcn_ballot_w64(lane < S && cnt == r);
    const int src = mask ? __builtin_ctzll(mask) : 0;
    seq = src;
    len = __builtin_amdgcn_readlane(Li, src);
}

// Cache policy of the K/V loads: non-temporal (each K/V byte is read once;
// measured ~9 % faster than the default policy on the batch decode step).
#ifndef PDA_FOLD_AUX
#define PDA_FOLD_AUX 2
#endif

// P.V with P rounded to BF16 on token pairs (v_dot2, the default) or, with
// 1, in FP32 FMAs (kept measurable: measured slower, with a smaller error).
#ifndef PDA_FOLD_PV_FP32
#define PDA_FOLD_PV_FP32 0
#endif

// Workgroups of at least this many waves merge each wave's token rows in
// registers before the LDS merge (see the epilogue).
constexpr int kRowMergeWaves = 4;

// The library's own part records and arrival tickets, for launches that
// split an item over several workgroups without a handle of their own.
// Tickets start at 0 (zero-initialised) and the combining workgroup puts
// its ticket back to 0, so every launch finds them at 0.
__device__ __align__(256) float g_part_sub[kPartSubFloats];
__device__ __align__(256) uint32_t g_part_tick[kPartTickets];

// Lane layout of the fold for head_dim D and GC heads per workgroup.
template <int D, int GC>
struct FoldShape {
    static constexpr int LPT = D / 8;                 // lanes per token row
    static constexpr int ROWS = 64 / LPT;             // token rows per wave load
    static constexpr int U = ROWS == 8 ? 2 : 4;       // loads (tokens per lane) per group
    static constexpr int TG = ROWS * U;                // tokens per group
    static constexpr int NP = GC * U;                 // (head, token) scores per row
    static constexpr int NP4 = (NP + 3) / 4 * 4;
    static constexpr int PPL = (NP + LPT - 1) / LPT;  // scores a lane owns
    static constexpr int TS = NP4 + 4;                // LDS floats per lane of partials
    static constexpr int TROW = LPT * TS + 16;        // per token row (shifts the banks)
    static constexpr int XS = (NP + GC + 3) / 4 * 4 + 4;  // exchange record per row
    static constexpr int WAVE_FLOATS = ROWS * (TROW + XS);
    static_assert(kBlockQuantum % TG == 0, "a block holds whole groups");
    static_assert(LPT % U == 0, "a head's scores sit in aligned lane sets");
};

// Largest workgroup of the fold for GC heads: 12 waves up to 6 heads (3 waves
// per SIMD fit their registers), 8 beyond.
__host__ __device__ constexpr int fold_max_threads(int gc) { return gc <= 6 ? 768 : 512; }

// PARTS: the item may be split over p.parts workgroups (one-shot modes);
// without it the kernel has no part code at all.
template <int MODE, int D, int GC, bool KV8, bool PARTS>
__global__ __launch_bounds__(fold_max_threads(GC)) void fold_kernel(const FoldParams p) {
    using S = FoldShape<D, GC>;
    constexpr int LPT = S::LPT, ROWS = S::ROWS, U = S::U, TG = S::TG, NP = S::NP,
                  NP4 = S::NP4, PPL = S::PPL, TS = S::TS, TROW = S::TROW, XS = S::XS;
    extern __shared__ __align__(16) float lds[];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nw = blockDim.x >> 6;
    const int row = lane / LPT, sub = lane % LPT;
    int seq, slen;   // slen: tokens (one-shot) or tile blocks (tiled), clamped
    seq_of_rank(p.lens, (int)gridDim.y, (int)blockIdx.y,
                MODE == kModeTiled ? p.table_stride : p.table_stride * p.bs, seq, slen);
    const int per_seq = p.nkv * p.HG;
    const int PL = PARTS ? p.parts : 1;           // workgroups per item in the grid
    const int bx = (int)blockIdx.x / PL;          // the item's index in the row
    const int part = (int)blockIdx.x - bx * PL;
    const int kvhg = MODE == kModeTiled ? bx : bx % per_seq;
    const int split = MODE == kModeTiled ? 0 : bx / per_seq;
    const int kvh = kvhg / p.HG, hg = kvhg % p.HG;
    const int h0 = kvh * p.G + hg * GC;                 // first q head of the group
    const int gcount = min(GC, p.G - hg * GC);          // heads this group carries

    const int32_t* blocks = p.tables + (int64_t)seq * p.table_stride;
    int t_begin, t_end;
    if constexpr (MODE == kModeTiled) {
        const int cnt = slen;
        if (cnt == 0) return;  // an empty tile leaves the state bit-identical
        t_begin = 0;
        t_end = (cnt - 1) * p.bs + p.lbvs;
    } else {
        const int L = slen;
        const int chunk = (int)split_chunk((uint32_t)L, (uint32_t)p.nsplit, (uint32_t)p.bs);
        const int64_t b0 = (int64_t)split * chunk;
        t_begin = b0 < L ? (int)b0 : L;
        t_end = (int64_t)t_begin + chunk < L ? t_begin + chunk : L;
        if (t_begin >= t_end) {
            // nothing to fold: an empty split leaves m = -inf, l = 0 (its o is
            // never read); a single empty split is an all-zero output.  Every
            // part sees the same empty item, so none takes a ticket.
            if (part != 0) return;
            const int64_t row_q0 = (int64_t)seq * p.nq + h0;
            if constexpr (MODE == kModePartial) {
                if (tid < gcount) {
                    float* slot = p.ws + ((row_q0 + tid) * p.nsplit + split) * (int64_t)(D + 2);
                    slot[D] = kNegInf;
                    slot[D + 1] = 0.f;
                }
            } else {
                for (int i = tid; i < gcount * (D / 2); i += blockDim.x)
                    *reinterpret_cast<uint32_t*>(p.out + row_q0 * D + 2 * i) = 0u;
            }
            return;
        }
    }

    // q pieces of the group's heads (zeros for heads past gcount).  The
    // loads are unconditional (a head past gcount re-reads the last one) so
    // that they issue back to back with no branch between them.
    uint32_t q2[GC][4];
#pragma unroll
    for (int h = 0; h < GC; ++h) {
        const int hq = h < gcount ? h : gcount - 1;
        const u32x4 w = *reinterpret_cast<const u32x4*>(
            p.q + ((int64_t)seq * p.nq + h0 + hq) * D + sub * 8);
#pragma unroll
        for (int j = 0; j < 4; ++j) q2[h][j] = h < gcount ? w[j] : 0u;
    }

    // Row state: o for every head (this lane's 8 dims); m and l for the
    // heads of the scores this lane owns (pair j = sub + LPT * k is head
    // j / U, token j % U of the row).
    float o[GC][8];
#pragma unroll
    for (int h = 0; h < GC; ++h)
#pragma unroll
        for (int d = 0; d < 8; ++d) o[h][d] = 0.f;
    float m[PPL], l[PPL];
#pragma unroll
    for (int k = 0; k < PPL; ++k) {
        m[k] = kNegInf;
        l[k] = 0.f;
    }

    float* tw = lds + wave * S::WAVE_FLOATS;         // this wave's scratch
    float* trow = tw + row * TROW;                   // partials of this row
    float* xrow = tw + ROWS * TROW + row * XS;       // exchange record of this row

    // element bytes: 2 (BF16 cache) or 1 (FP8 E4M3 cache); a lane's 8 dims
    // are one 16- or 8-byte load
    constexpr int EB = KV8 ? 1 : 2;
    const int tok_b = (int)p.tok_s * EB;
    uint32_t voff[U];
#pragma unroll
    for (int u = 0; u < U; ++u) voff[u] = (uint32_t)((row + ROWS * u) * tok_b + sub * 8 * EB);
    const uint32_t voff0 = (uint32_t)(sub * 8 * EB);           // the group's first token
    const uint32_t rec = (uint32_t)((p.bs - 1) * tok_b + D * EB);  // bytes a block spans

    // This workgroup's run of the item: with parts, part i folds blocks
    // [i * per, (i + 1) * per) of the item (per = ceil(blocks / parts)),
    // possibly none.
    // The parts an item uses: at most PL, and no more than one per
    // p.part_min of its blocks (short items gain nothing from the
    // hand-over); a function of the sequence's own length, so its bytes do
    // not depend on the batch.  Parts past that count have nothing to do.
    int P = PL;
    if (PARTS) {
        const int nb_item = (t_end - t_begin + p.bs - 1) / p.bs;
        const int want = (nb_item + p.part_min - 1) / p.part_min;
        P = want < PL ? (want > 1 ? want : 1) : PL;
        if (part >= P) return;
    }
    if (P > 1) {
        const int nb_item = (t_end - t_begin + p.bs - 1) / p.bs;
        const int per = (nb_item + P - 1) / P;
        const int64_t fb = (int64_t)t_begin + (int64_t)part * per * p.bs;
        const int f_begin = fb < t_end ? (int)fb : t_end;
        t_end = (int64_t)f_begin + (int64_t)per * p.bs < t_end ? f_begin + per * p.bs : t_end;
        t_begin = f_begin;
    }

    // A tiled launch without parts joins the running state in its epilogue:
    // that state is requested here, so its loads overlap the fold instead of
    // following it (two memory round trips fewer per call; the calls that
    // fold one partial block per sequence are mostly such latency).  The
    // parts form keeps its registers for the fold loop.
    float pre_m = kNegInf, pre_l = 0.f;
    float2 pre_o[2] = {make_float2(0.f, 0.f), make_float2(0.f, 0.f)};
    if constexpr (MODE == kModeTiled && !PARTS) {
        {
            const int64_t rq = (int64_t)seq * p.nq + h0;
            if (tid < gcount) {
                pre_m = p.ws[rq + tid];
                pre_l = p.l_state[rq + tid];
            }
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int i = tid + j * (int)blockDim.x;
                if (i < gcount * (D / 2)) {
                    const int h = i / (D / 2);
                    const int d = (i - h * (D / 2)) * 2;
                    pre_o[j] = *reinterpret_cast<const float2*>(p.o_state + (rq + h) * D + d);
                }
            }
        }
    }

    // a live range starts on a block (hence group) boundary; an empty split
    // or part starts at the range end, which need not be aligned: it folds
    // nothing
    const int gpb = p.bs / TG;  // groups per block
    const int g_first = t_begin / TG;
    const int g_end = t_end > t_begin ? (t_end + TG - 1) / TG : g_first;
    const char* kh = reinterpret_cast<const char*>(p.k) + (int64_t)kvh * p.kvh_s * EB;
    const char* vh = reinterpret_cast<const char*>(p.v) + (int64_t)kvh * p.kvh_s * EB;

    // Block ids of the range in windows of 64: lane i holds the id of block
    // b_lo + wbase + i, and the next window is requested one window ahead,
    // so a group reads its block id from a register (v_readlane) instead of
    // waiting on a table load before its K/V loads can start.
    const int b_lo = g_first / gpb;
    const int nbk = g_end > g_first ? (g_end - 1) / gpb - b_lo + 1 : 0;  // blocks in range
    int wbase = 0;
    int bw = lane < nbk ? blocks[b_lo + lane] : -1;
    int bw_next = lane + 64 < nbk ? blocks[b_lo + 64 + lane] : -1;

    for (int g = g_first + wave; g < g_end; g += nw) {
        const int b = g / gpb;
        const int slot0 = (g - b * gpb) * TG;
        while (b - b_lo - wbase >= 64) {   // wave-uniform; at most once per 64 blocks
            wbase += 64;
            bw = bw_next;
            bw_next = lane + wbase + 64 < nbk ? blocks[b_lo + wbase + 64 + lane] : -1;
        }
        const int blk = __builtin_amdgcn_readlane(bw, b - b_lo - wbase);
        if ((uint32_t)blk >= p.num_blocks) continue;  // dropped: never dereferenced
        const int nvalid = min(TG, t_end - g * TG);
        const __amdgpu_buffer_rsrc_t krs = make_rsrc(kh + (int64_t)blk * p.blk_s * EB, rec);
        const __amdgpu_buffer_rsrc_t vrs = make_rsrc(vh + (int64_t)blk * p.blk_s * EB, rec);
        const int soff = slot0 * tok_b;

        // kr: K as BF16 pairs (dims 2j, 2j + 1 in word j); vr: V as loaded
        // (BF16 pairs, or 4 E4M3 codes per word in words 0 and 1)
        uint32_t kr[U][4], vr[U][4];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            // a masked token re-reads the group's first row (always valid),
            // so canary memory past the end never enters the arithmetic
            const uint32_t off = row + ROWS * u < nvalid ? voff[u] : voff0;
            if constexpr (KV8) {
                const u32x2 x = __builtin_amdgcn_raw_buffer_load_b64(krs, off, soff, PDA_FOLD_AUX);
                const u32x2 y = __builtin_amdgcn_raw_buffer_load_b64(vrs, off, soff, PDA_FOLD_AUX);
                // E4M3 -> FP32 -> BF16 is exact (3 mantissa bits, exponents in range)
#pragma unroll
                for (int w = 0; w < 2; ++w) {
                    kr[u][2 * w] = fp8x2_to_bf16x2<false>(x[w]);
                    kr[u][2 * w + 1] = fp8x2_to_bf16x2<true>(x[w]);
                    vr[u][w] = y[w];
                }
                vr[u][2] = vr[u][3] = 0u;
            } else {
                const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(krs, off, soff, PDA_FOLD_AUX);
                const u32x4 y = __builtin_amdgcn_raw_buffer_load_b128(vrs, off, soff, PDA_FOLD_AUX);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    kr[u][j] = x[j];
                    vr[u][j] = y[j];
                }
            }
        }

        // partial dots of this lane's piece -> LDS, [row][lane][pair]
        float part[NP4];
#pragma unroll
        for (int h = 0; h < GC; ++h)
#pragma unroll
            for (int u = 0; u < U; ++u) {
                float a = 0.f;
#pragma unroll
                for (int j = 0; j < 4; ++j) a = dot2(q2[h][j], kr[u][j], a);
                part[h * U + u] = a;
            }
#pragma unroll
        for (int j = NP; j < NP4; ++j) part[j] = 0.f;
#pragma unroll
        for (int c = 0; c < NP4 / 4; ++c) {
            const f32x4 w = {part[4 * c], part[4 * c + 1], part[4 * c + 2], part[4 * c + 3]};
            *reinterpret_cast<f32x4*>(trow + sub * TS + 4 * c) = w;
        }
        wave_lds_sync();

        // owned scores: sum the row's LPT partials in lane order
        float sc[PPL];
#pragma unroll
        for (int k = 0; k < PPL; ++k) {
            const int j = sub + LPT * k;
            float a = 0.f;
            if (j < NP) {
#pragma unroll
                for (int jj = 0; jj < LPT; ++jj) a += trow[jj * TS + j];
            }
            const bool live = j < NP && row + ROWS * (j % U) < nvalid;
            sc[k] = live ? a * p.c : kNegInf;
        }

        // per head: max over its U scores, new running max, p, l
        float alpha[PPL];
        bool grow = false;
#pragma unroll
        for (int k = 0; k < PPL; ++k) {
            const float bm = nmax<U>(sc[k]);
            const float mn = fmaxf(m[k], bm);
            const float ms = mn == kNegInf ? 0.f : mn;
            alpha[k] = fexp2(m[k] - ms);
            grow |= mn != m[k];
            m[k] = mn;
            const float pk = fexp2(sc[k] - ms);
            l[k] = l[k] * alpha[k] + nsum<U>(pk);
            sc[k] = pk;
        }

        // probabilities and rescale factors back to every lane of the row
#pragma unroll
        for (int k = 0; k < PPL; ++k) {
            const int j = sub + LPT * k;
            if (j < NP) {
                xrow[j] = sc[k];
                if (j % U == 0) xrow[NP + j / U] = alpha[k];
            }
        }
        wave_lds_sync();
        float pa[NP + GC];
#pragma unroll
        for (int c = 0; c < (NP + GC + 3) / 4; ++c) {
            const f32x4 w = *reinterpret_cast<const f32x4*>(xrow + 4 * c);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (4 * c + e < NP + GC) pa[4 * c + e] = w[e];
        }

        if (__builtin_amdgcn_ballot_w64(grow) != 0) {
#pragma unroll
            for (int h = 0; h < GC; ++h) {
                const float a = pa[NP + h];
#pragma unroll
                for (int d = 0; d < 8; ++d) o[h][d] *= a;
            }
        }

        if constexpr (PDA_FOLD_PV_FP32) {
            // P.V in FP32 (P not rounded): each token's V piece widened to
            // FP32 (a BF16 pair is two shifts; E4M3 codes decode to BF16
            // pairs first), one FMA per (head, dim, token)
#pragma unroll
            for (int u = 0; u < U; ++u) {
                uint32_t vw[4];
                if constexpr (KV8) {
#pragma unroll
                    for (int w = 0; w < 2; ++w) {
                        vw[2 * w] = fp8x2_to_bf16x2<false>(vr[u][w]);
                        vw[2 * w + 1] = fp8x2_to_bf16x2<true>(vr[u][w]);
                    }
                } else {
#pragma unroll
                    for (int j = 0; j < 4; ++j) vw[j] = vr[u][j];
                }
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float v0 = __uint_as_float(vw[j] << 16);
                    const float v1 = __uint_as_float(vw[j] & 0xFFFF0000u);
#pragma unroll
                    for (int h = 0; h < GC; ++h) {
                        o[h][2 * j] = fmaf(pa[h * U + u], v0, o[h][2 * j]);
                        o[h][2 * j + 1] = fmaf(pa[h * U + u], v1, o[h][2 * j + 1]);
                    }
                }
            }
        } else if constexpr (KV8) {
            // P.V on token pairs: the two tokens' codes of one dim are
            // interleaved (v_perm) and decoded to a BF16 pair, then v_dot2
            // with (p_u, p_u+1) rounded to BF16, accumulated in FP32 (fewer
            // instructions per byte, which this half-size stream needs)
#pragma unroll
            for (int u = 0; u < U; u += 2) {
                uint32_t vp[8];
#pragma unroll
                for (int w = 0; w < 2; ++w) {
                    const uint32_t x0 = __builtin_amdgcn_perm(vr[u + 1][w], vr[u][w], 0x05010400u);
                    const uint32_t x1 = __builtin_amdgcn_perm(vr[u + 1][w], vr[u][w], 0x07030602u);
                    vp[4 * w] = fp8x2_to_bf16x2<false>(x0);
                    vp[4 * w + 1] = fp8x2_to_bf16x2<true>(x0);
                    vp[4 * w + 2] = fp8x2_to_bf16x2<false>(x1);
                    vp[4 * w + 3] = fp8x2_to_bf16x2<true>(x1);
                }
#pragma unroll
                for (int h = 0; h < GC; ++h) {
                    const uint32_t pp = pack_bf16x2(pa[h * U + u], pa[h * U + u + 1]);
#pragma unroll
                    for (int d = 0; d < 8; ++d) o[h][d] = dot2(pp, vp[d], o[h][d]);
                }
            }
        } else {
            // P.V on token pairs: (p_u, p_u+1) rounded to BF16 (as the MFMA
            // kernels do) against the two tokens' values of one dim, v_dot2,
            // accumulated in FP32: half the instructions of FP32 FMAs
#pragma unroll
            for (int u = 0; u < U; u += 2) {
                uint32_t vlo[4], vhi[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    vlo[j] = __builtin_amdgcn_perm(vr[u + 1][j], vr[u][j], 0x05040100u);
                    vhi[j] = __builtin_amdgcn_perm(vr[u + 1][j], vr[u][j], 0x07060302u);
                }
#pragma unroll
                for (int h = 0; h < GC; ++h) {
                    const uint32_t pp = pack_bf16x2(pa[h * U + u], pa[h * U + u + 1]);
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        o[h][2 * j] = dot2(pp, vlo[j], o[h][2 * j]);
                        o[h][2 * j + 1] = dot2(pp, vhi[j], o[h][2 * j + 1]);
                    }
                }
            }
        }
        wave_lds_sync();  // the next group's partials overwrite this scratch
    }

    if constexpr (KV8) {   // V = decode(v8) * v_scale: scale o once
#pragma unroll
        for (int h = 0; h < GC; ++h)
#pragma unroll
            for (int d = 0; d < 8; ++d) o[h][d] *= p.v_scale;
    }

    // Wave epilogue, then every contributor's state goes to LDS and one
    // fixed-order pass merges them.  Layout (aliasing the loop scratch):
    // o [NC][GC][D], m [NC][GC], l [NC][GC], weights [max(NC, kMaxParts) +
    // 1][GC], L [GC], ticket.
    //  * nw < kRowMergeWaves: each (wave, row) state is a contributor,
    //    NC = nw * ROWS (cheapest for few waves).
    //  * otherwise the wave's ROWS row states merge first, with cross-lane
    //    reductions over the rows (a fixed butterfly, so every lane ends
    //    with the same bits): per head, the row's m and l are broadcast to
    //    the row's lanes, M = max over rows, w = exp(m - M), and l and o are
    //    summed with weight w; NC = nw, which keeps the LDS small enough for
    //    wide workgroups.
    const bool row_merge = nw >= kRowMergeWaves;
    const int NC = row_merge ? nw : nw * ROWS;
    float* eo = lds;
    float* em = eo + NC * GC * D;
    float* el = em + NC * GC;
    float* ew = el + NC * GC;
    float* eL = ew + ((NC > kMaxParts ? NC : kMaxParts) + 1) * GC;
    if (row_merge) {
        float wM[GC], wL[GC];   // per head, identical in every lane of the wave
#pragma unroll
        for (int h = 0; h < GC; ++h) {
            const int j = h * U;                        // the head's first score pair
            const int src = (row * LPT + j % LPT) * 4;  // its owner in this row (bytes)
            const float mr =
                __int_as_float(__builtin_amdgcn_ds_bpermute(src, __float_as_int(m[j / LPT])));
            const float lr =
                __int_as_float(__builtin_amdgcn_ds_bpermute(src, __float_as_int(l[j / LPT])));
            const float M = rows_max<LPT>(mr);
            const float w = fexp2(mr - (M == kNegInf ? 0.f : M));
            wM[h] = M;
            wL[h] = rows_sum<LPT>(w * lr);
#pragma unroll
            for (int d = 0; d < 8; ++d) o[h][d] = rows_sum<LPT>(w * o[h][d]);
        }
        __syncthreads();
        if (row == 0) {
#pragma unroll
            for (int h = 0; h < GC; ++h) {
                float* dst = eo + (wave * GC + h) * D + sub * 8;
                *reinterpret_cast<f32x4*>(dst) = f32x4{o[h][0], o[h][1], o[h][2], o[h][3]};
                *reinterpret_cast<f32x4*>(dst + 4) = f32x4{o[h][4], o[h][5], o[h][6], o[h][7]};
            }
        }
#pragma unroll
        for (int h = 0; h < GC; ++h) {
            if (lane == h) {
                em[wave * GC + h] = wM[h];
                el[wave * GC + h] = wL[h];
            }
        }
    } else {
        const int ci = wave * ROWS + row;
        __syncthreads();
#pragma unroll
        for (int h = 0; h < GC; ++h) {
            float* dst = eo + (ci * GC + h) * D + sub * 8;
            *reinterpret_cast<f32x4*>(dst) = f32x4{o[h][0], o[h][1], o[h][2], o[h][3]};
            *reinterpret_cast<f32x4*>(dst + 4) = f32x4{o[h][4], o[h][5], o[h][6], o[h][7]};
        }
#pragma unroll
        for (int k = 0; k < PPL; ++k) {
            const int j = sub + LPT * k;
            if (j < NP && j % U == 0) {
                em[ci * GC + j / U] = m[k];
                el[ci * GC + j / U] = l[k];
            }
        }
    }
    __syncthreads();

    // Per head: the workgroup max, every contributor's weight, and l, and
    // the running state of a tiled launch (when the item is split into
    // parts, the state joins when they are combined).
    const bool with_old = MODE == kModeTiled && P == 1;
    const int64_t row_q = (int64_t)seq * p.nq + h0;  // first q slot of the group
    // this part's record: o [GC][D], m [GC] (log2 units), l [GC]
    const int64_t item = (int64_t)blockIdx.y * (gridDim.x / PL) + bx;
    constexpr int REC = (int)part_rec_floats(GC, D);
    float* const psub = p.sub ? p.sub : g_part_sub;
    float* const prec = psub + (item * PL + part) * REC;
    if (tid < gcount) {
        const int h = tid;
        float M = kNegInf, m_old = kNegInf, m2_old = kNegInf, l_old = 0.f;
        if (with_old) {
            m_old = PARTS ? p.ws[row_q + h] : pre_m;
            l_old = PARTS ? p.l_state[row_q + h] : pre_l;
            m2_old = m_old * kLog2e;
            M = m2_old;
        }
        for (int c = 0; c < NC; ++c) M = fmaxf(M, em[c * GC + h]);
        const float Ms = M == kNegInf ? 0.f : M;
        float L = 0.f;
        if (with_old) {
            const float wo = fexp2(m2_old - Ms);
            ew[NC * GC + h] = wo;
            L = wo * l_old;
        }
        // chunks of 8 contributors: all reads of a chunk are issued before
        // its writes (the compiler cannot tell ew from em / el, so a write
        // between reads would make every read wait for it)
        for (int c0 = 0; c0 < NC; c0 += 8) {
            float mv[8], lv[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int c = c0 + j < NC ? c0 + j : NC - 1;
                mv[j] = em[c * GC + h];
                lv[j] = el[c * GC + h];
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                if (c0 + j < NC) {
                    const float wt = fexp2(mv[j] - Ms);
                    ew[(c0 + j) * GC + h] = wt;
                    L += wt * lv[j];
                }
            }
        }
        eL[h] = L;
        if (P > 1) {
            put_dev(prec + GC * D + h, M);
            put_dev(prec + GC * D + GC + h, L);
        } else {
            const float m_nat = M * kLn2;
            if constexpr (MODE == kModePartial) {
                float* slot = p.ws + ((row_q + h) * p.nsplit + split) * (int64_t)(D + 2);
                slot[D] = m_nat;
                slot[D + 1] = L;
            } else if constexpr (MODE == kModeTiled) {
                // keep the stored max bit-identical when this tile did not raise it
                p.ws[row_q + h] = M == m2_old ? m_old : m_nat;
                p.l_state[row_q + h] = L;
            }
        }
    }
    __syncthreads();

    // Per (head, pair of dims): o of every contributor, in a fixed order.
    const int nitems = gcount * (D / 2);
    for (int i = tid, j = 0; i < nitems; i += blockDim.x, ++j) {
        const int h = i / (D / 2);
        const int d = (i - h * (D / 2)) * 2;
        float o0 = 0.f, o1 = 0.f;
        const int64_t qs = row_q + h;
        if (with_old) {
            const float2 prev =
                !PARTS && j == 0   ? pre_o[0]
                : !PARTS && j == 1 ? pre_o[1]
                                   : *reinterpret_cast<const float2*>(p.o_state + qs * D + d);
            const float wo = ew[NC * GC + h];
            o0 = wo * prev.x;
            o1 = wo * prev.y;
        }
        for (int c = 0; c < NC; ++c) {
            const float wt = ew[c * GC + h];
            const float2 x = *reinterpret_cast<const float2*>(eo + (c * GC + h) * D + d);
            o0 += wt * x.x;
            o1 += wt * x.y;
        }
        const float L = eL[h];
        if (P > 1) {
            put_dev(prec + h * D + d, o0);
            put_dev(prec + h * D + d + 1, o1);
        } else if constexpr (MODE == kModePartial) {
            if (L > 0.f) {
                float* slot = p.ws + (qs * p.nsplit + split) * (int64_t)(D + 2);
                *reinterpret_cast<float2*>(slot + d) = make_float2(o0, o1);
            }
        } else if constexpr (MODE == kModeFinal) {
            const uint32_t v = L > 0.f ? pack_bf16x2(o0 / L, o1 / L) : 0u;
            *reinterpret_cast<uint32_t*>(p.out + qs * D + d) = v;
        } else {
            *reinterpret_cast<float2*>(p.o_state + qs * D + d) = make_float2(o0, o1);
        }
    }
    if (P == 1) return;

    // Parts: publish this record, take a ticket; the last part to arrive
    // combines every part's record, in part order, with the same weighting
    // (after the running state, for a tiled launch), so the result depends
    // on the item's data and the part count only, never on arrival order.
    if constexpr (PARTS) {
        uint32_t* const tick = (p.tick ? p.tick : g_part_tick) + item;
        uint32_t* const eT = reinterpret_cast<uint32_t*>(eL + GC);
        __builtin_amdgcn_s_waitcnt(0);   // this thread's record stores are complete
        __syncthreads();
        if (tid == 0)
            *eT = PDA_PARTS_ORDER == 1
                      ? __hip_atomic_fetch_add(tick, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT)
                      : __hip_atomic_fetch_add(tick, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        if (*eT != (uint32_t)(P - 1)) return;
        // the records are read only after this point
        if (PDA_PARTS_ORDER >= 1) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        if (tid == 0) __hip_atomic_store(tick, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const float* const recs = psub + item * PL * REC;
        // weights: ew[i * GC + h] for part i, ew[P * GC + h] for the state
        if (tid < gcount) {
            const int h = tid;
            float M = kNegInf, m_old = kNegInf, m2_old = kNegInf, l_old = 0.f;
            if constexpr (MODE == kModeTiled) {
                m_old = p.ws[row_q + h];
                l_old = p.l_state[row_q + h];
                m2_old = m_old * kLog2e;
                M = m2_old;
            }
            float mv[kMaxParts], lv[kMaxParts];
#pragma unroll
            for (int i = 0; i < kMaxParts; ++i) {
                const int ii = i < P ? i : P - 1;
                mv[i] = get_dev(recs + ii * REC + GC * D + h);
                lv[i] = get_dev(recs + ii * REC + GC * D + GC + h);
            }
#pragma unroll
            for (int i = 0; i < kMaxParts; ++i)
                if (i < P && lv[i] > 0.f) M = fmaxf(M, mv[i]);
            const float Ms = M == kNegInf ? 0.f : M;
            float L = 0.f;
            if constexpr (MODE == kModeTiled) {
                const float wo = fexp2(m2_old - Ms);
                ew[P * GC + h] = wo;
                L = wo * l_old;
            }
#pragma unroll
            for (int i = 0; i < kMaxParts; ++i) {
                if (i < P) {
                    // a part that folded nothing has l = 0 and takes no weight
                    const float wt = lv[i] > 0.f ? fexp2(mv[i] - Ms) : 0.f;
                    ew[i * GC + h] = wt;
                    L += wt * lv[i];
                }
            }
            eL[h] = L;
            if constexpr (MODE == kModePartial) {
                float* slot = p.ws + ((row_q + h) * p.nsplit + split) * (int64_t)(D + 2);
                slot[D] = M * kLn2;
                slot[D + 1] = L;
            } else if constexpr (MODE == kModeTiled) {
                // keep the stored max bit-identical when this tile did not raise it
                p.ws[row_q + h] = M == m2_old ? m_old : M * kLn2;
                p.l_state[row_q + h] = L;
            }
        }
        __syncthreads();
        for (int i = tid; i < nitems; i += blockDim.x) {
            const int h = i / (D / 2);
            const int d = (i - h * (D / 2)) * 2;
            float o0 = 0.f, o1 = 0.f;
            const int64_t qs = row_q + h;
            if constexpr (MODE == kModeTiled) {
                const float2 prev = *reinterpret_cast<const float2*>(p.o_state + qs * D + d);
                const float wo = ew[P * GC + h];
                o0 = wo * prev.x;
                o1 = wo * prev.y;
            }
            for (int c = 0; c < P; ++c) {
                const float wt = ew[c * GC + h];
                if (wt != 0.f) {   // an empty part's o is never read
                    const float* x = recs + c * REC + h * D + d;
                    o0 += wt * get_dev(x);
                    o1 += wt * get_dev(x + 1);
                }
            }
            const float L = eL[h];
            if constexpr (MODE == kModePartial) {
                if (L > 0.f) {
                    float* slot = p.ws + (qs * p.nsplit + split) * (int64_t)(D + 2);
                    *reinterpret_cast<float2*>(slot + d) = make_float2(o0, o1);
                }
            } else if constexpr (MODE == kModeFinal) {
                const uint32_t v = L > 0.f ? pack_bf16x2(o0 / L, o1 / L) : 0u;
                *reinterpret_cast<uint32_t*>(p.out + qs * D + d) = v;
            } else {
                *reinterpret_cast<float2*>(p.o_state + qs * D + d) = make_float2(o0, o1);
            }
        }
    }
}

// Split-K merge: for each (sequence, q head), over splits in index order,
// skipping splits with l == 0 (their o is never used):
//   M = max m_i,  w_i = exp(m_i - M),  L = sum w_i l_i,  O = sum w_i o_i,
//   out = bf16(O / L), or 0 when every split is empty.
// One wave per (sequence, head); lane j owns D/64 consecutive dims.  Every
// split's (m, l) and o slice is requested before any is used, so the
// wave waits for memory once, not once per split.
template <int D>
__global__ __launch_bounds__(256) void merge_kernel(const float* __restrict__ ws,
                                                    uint16_t* __restrict__ out, int nq,
                                                    int nsplit) {
    constexpr int DPL = D / 64;
    constexpr int NMAX = kMaxDecodeSplits;
    const int lane = threadIdx.x & 63;
    const int h = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (h >= nq) return;
    const int64_t qs = (int64_t)blockIdx.y * nq + h;
    const float* base = ws + qs * nsplit * (int64_t)(D + 2);
    float mi[NMAX], li[NMAX], oi[NMAX][DPL];
#pragma unroll
    for (int i = 0; i < NMAX; ++i) {
        const int ii = i < nsplit ? i : nsplit - 1;   // re-read a valid slot
        const float* slot = base + ii * (D + 2);
        mi[i] = slot[D];
        li[i] = slot[D + 1];
#pragma unroll
        for (int d = 0; d < DPL; ++d) oi[i][d] = slot[lane * DPL + d];
    }
    float M = kNegInf;
#pragma unroll
    for (int i = 0; i < NMAX; ++i)
        if (i < nsplit && li[i] > 0.f) M = fmaxf(M, mi[i]);
    // selects rather than branches: every load above stays unconditional
    // (so none is deferred into a branch), and a skipped split's o, which
    // may be stale, never meets a multiply
    float L = 0.f, O[DPL];
#pragma unroll
    for (int d = 0; d < DPL; ++d) O[d] = 0.f;
#pragma unroll
    for (int i = 0; i < NMAX; ++i) {
        const bool use = i < nsplit && li[i] > 0.f;
        const float w = fexp2((mi[i] - M) * kLog2e);
        L = use ? fmaf(w, li[i], L) : L;
#pragma unroll
        for (int d = 0; d < DPL; ++d) O[d] = use ? fmaf(w, oi[i][d], O[d]) : O[d];
    }
    uint16_t* dst = out + qs * D + lane * DPL;
    if constexpr (DPL == 1) {
        const float r = L > 0.f ? O[0] / L : 0.f;
        const __bf16 b = (__bf16)r;
        *dst = __builtin_bit_cast(uint16_t, b);
    } else {
#pragma unroll
        for (int d = 0; d < DPL; d += 2) {
            const uint32_t v = L > 0.f ? pack_bf16x2(O[d] / L, O[d + 1] / L) : 0u;
            *reinterpret_cast<uint32_t*>(dst + d) = v;
        }
    }
}

__global__ __launch_bounds__(256) void tiled_begin_kernel(float* __restrict__ m,
                                                          float* __restrict__ l,
                                                          float* __restrict__ o, uint64_t n_q,
                                                          int D) {
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    const uint64_t n_o = n_q * (uint64_t)D;
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_o; i += stride) {
        o[i] = 0.f;
        if (i < n_q) {
            m[i] = kNegInf;
            l[i] = 0.f;
        }
    }
}

__global__ __launch_bounds__(256) void tiled_finalize_kernel(const float* __restrict__ l,
                                                             const float* __restrict__ o,
                                                             uint16_t* __restrict__ out,
                                                             uint64_t n_q, int D) {
    const uint64_t half = (uint64_t)(D / 2);
    const uint64_t n = n_q * half;
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
        const uint64_t qs = i / half;
        const uint64_t d = (i - qs * half) * 2;
        const float L = l[qs];
        const float2 x = *reinterpret_cast<const float2*>(o + qs * D + d);
        const uint32_t v = L > 0.f ? pack_bf16x2(x.x / L, x.y / L) : 0u;
        *reinterpret_cast<uint32_t*>(out + qs * D + d) = v;
    }
}

using FoldFn = void (*)(FoldParams);

template <int MODE, int D, bool KV8, bool PARTS>
FoldFn pick_gc(int gc) {
    switch (gc) {
        case 1: return fold_kernel<MODE, D, 1, KV8, PARTS>;
        case 2: return fold_kernel<MODE, D, 2, KV8, PARTS>;
        case 3: return fold_kernel<MODE, D, 3, KV8, PARTS>;
        case 4: return fold_kernel<MODE, D, 4, KV8, PARTS>;
        case 5: return fold_kernel<MODE, D, 5, KV8, PARTS>;
        case 6: return fold_kernel<MODE, D, 6, KV8, PARTS>;
        case 7: return fold_kernel<MODE, D, 7, KV8, PARTS>;
        case 8: return fold_kernel<MODE, D, 8, KV8, PARTS>;
        default: return nullptr;
    }
}

template <int MODE, bool KV8, bool PARTS = false>
FoldFn pick_d(int D, int gc) {
    switch (D) {
        case 64: return pick_gc<MODE, 64, KV8, PARTS>(gc);
        case 128: return pick_gc<MODE, 128, KV8, PARTS>(gc);
        case 256: return pick_gc<MODE, 256, KV8, PARTS>(gc);
        default: return nullptr;
    }
}

// One-shot modes, with or without parts.
template <int MODE>
FoldFn pick_oneshot(int D, int gc, bool kv8, bool parts) {
    if (parts) return kv8 ? pick_d<MODE, true, true>(D, gc) : pick_d<MODE, false, true>(D, gc);
    return kv8 ? pick_d<MODE, true>(D, gc) : pick_d<MODE, false>(D, gc);
}

template <int D, int GC>
size_t fold_lds_floats(int waves) {
    using S = FoldShape<D, GC>;
    const size_t nc = (size_t)(waves >= kRowMergeWaves ? waves : waves * S::ROWS);
    // o, m, l per contributor; weights for max(contributors, parts) + 1;
    // L per head; the ticket word
    const size_t nw8 = nc > (size_t)kMaxParts ? nc : (size_t)kMaxParts;
    const size_t epi = nc * GC * D + 2 * nc * GC + (nw8 + 1) * GC + GC + 1;
    const size_t loop = (size_t)waves * S::WAVE_FLOATS;
    return epi > loop ? epi : loop;
}

template <int D>
size_t lds_floats_d(int gc, int waves) {
    switch (gc) {
        case 1: return fold_lds_floats<D, 1>(waves);
        case 2: return fold_lds_floats<D, 2>(waves);
        case 3: return fold_lds_floats<D, 3>(waves);
        case 4: return fold_lds_floats<D, 4>(waves);
        case 5: return fold_lds_floats<D, 5>(waves);
        case 6: return fold_lds_floats<D, 6>(waves);
        case 7: return fold_lds_floats<D, 7>(waves);
        case 8: return fold_lds_floats<D, 8>(waves);
        default: return 0;
    }
}

}  // namespace

size_t fold_lds_bytes(int head_dim, int gc, int waves) {
    size_t f = 0;
    switch (head_dim) {
        case 64: f = lds_floats_d<64>(gc, waves); break;
        case 128: f = lds_floats_d<128>(gc, waves); break;
        case 256: f = lds_floats_d<256>(gc, waves); break;
        default: break;
    }
    return f * sizeof(float);
}

hipError_t launch_fold(int mode, int head_dim, int gc, const FoldParams& p, uint32_t grid_x,
                       uint32_t grid_y, int waves, hipStream_t stream, bool kv8) {
    FoldFn fn = nullptr;
    const bool parts = p.parts > 1;
    switch (mode) {
        case kModePartial: fn = pick_oneshot<kModePartial>(head_dim, gc, kv8, parts); break;
        case kModeFinal: fn = pick_oneshot<kModeFinal>(head_dim, gc, kv8, parts); break;
        case kModeTiled:
            fn = kv8 ? nullptr
                     : (parts ? pick_d<kModeTiled, false, true>(head_dim, gc)
                              : pick_d<kModeTiled, false>(head_dim, gc));
            break;
        default: break;
    }
    if (!fn || waves < 1 || 64 * waves > fold_max_threads(gc)) return hipErrorInvalidValue;
    if (p.parts < 1 || p.parts > kMaxParts || grid_x % (uint32_t)p.parts != 0 ||
        (p.parts > 1 && p.part_min < 1))
        return hipErrorInvalidValue;
    const size_t lds = fold_lds_bytes(head_dim, gc, waves);
    if (lds > 64 * 1024) {
        // dynamic LDS past 64 KiB is requested per kernel, once
        static std::mutex mu;
        static std::vector<std::pair<FoldFn, size_t>> granted;
        std::lock_guard<std::mutex> g(mu);
        bool have = false;
        for (const auto& e : granted) have |= e.first == fn && e.second >= lds;
        if (!have) {
            hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(fn),
                                               hipFuncAttributeMaxDynamicSharedMemorySize,
                                               (int)lds);
            if (e != hipSuccess) return e;
            granted.emplace_back(fn, lds);
        }
    }
    hipLaunchKernelGGL(fn, dim3(grid_x, grid_y), dim3(64 * waves), lds, stream, p);
    return hipGetLastError();
}

int fold_max_waves(int gc) { return fold_max_threads(gc) / 64; }

hipError_t launch_merge(const float* ws, uint16_t* out, uint32_t num_seqs, int nq, int head_dim,
                        int nsplit, hipStream_t stream) {
    const dim3 grid((nq + 3) / 4, num_seqs);
    switch (head_dim) {
        case 64: hipLaunchKernelGGL(merge_kernel<64>, grid, dim3(256), 0, stream, ws, out, nq, nsplit); break;
        case 128: hipLaunchKernelGGL(merge_kernel<128>, grid, dim3(256), 0, stream, ws, out, nq, nsplit); break;
        case 256: hipLaunchKernelGGL(merge_kernel<256>, grid, dim3(256), 0, stream, ws, out, nq, nsplit); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_tiled_begin(float* m, float* l, float* o, uint64_t n_q, int head_dim,
                              hipStream_t stream) {
    const uint64_t n = n_q * (uint64_t)head_dim;
    uint64_t blocks = (n + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL(tiled_begin_kernel, dim3((uint32_t)blocks), dim3(256), 0, stream, m, l,
                       o, n_q, head_dim);
    return hipGetLastError();
}

hipError_t launch_tiled_finalize(const float* l, const float* o, uint16_t* out, uint64_t n_q,
                                 int head_dim, hipStream_t stream) {
    const uint64_t n = n_q * (uint64_t)(head_dim / 2);
    uint64_t blocks = (n + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL(tiled_finalize_kernel, dim3((uint32_t)blocks), dim3(256), 0, stream, l,
                       o, out, n_q, head_dim);
    return hipGetLastError();
}

}  // namespace pda
