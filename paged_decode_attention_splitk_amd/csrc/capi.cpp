// C-ABI entry points: argument checks, kernel choice and launches.
//
// The one-shot call takes the problem statement's arguments (q, caches, block
// tables, sequence lengths, scale, split count); the tiled handle follows the
// "metrale_storage/tiled_attention.rs" page (TiledAttention: new / validate,
// begin_step, step_tile, finalize, the public state buffers); "not
// applicable" for the packed kernel mirrors that page set's convention of a
// launcher that launches nothing and lets the caller run the other path.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include <mutex>
#include <utility>
#include <vector>

#include "pda.h"
#include "pda_geometry.h"
#include "pda_kernels.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}

int ok() {
    g_last_error.clear();
    return PDA_OK;
}

int hip_fail(hipError_t e, const char* what) {
    return fail(PDA_EHIP_BASE - (int)e, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

bool head_dim_supported(uint32_t d) { return d == 64 || d == 128 || d == 256; }

constexpr float kLog2e = 1.4426950408889634f;

// Head groups of one KV head: G q heads in groups of at most 8, as even as
// possible.  Returns the group width; *hg receives the group count.
// Head groups per KV head (at most kMaxHeadsPerGroup heads each, so every
// K/V byte serves as many heads as one workgroup holds) and heads per group.
int head_groups(uint32_t G, int* hg) {
    const int groups = (int)((G + pda::kMaxHeadsPerGroup - 1) / pda::kMaxHeadsPerGroup);
    *hg = groups;
    return (int)((G + groups - 1) / groups);
}

// Waves per fold workgroup of a one-shot launch.  A pure function of the
// shape and the split count (never of the batch), so a sequence's
// reduction order, and its output bytes, do not depend on what it is
// batched with.  Launches that give a single sequence few workgroups get
// wider workgroups; LDS caps the width.
//
// With many workgroups: 2 waves per workgroup for a BF16 cache, 1 for an FP8
// cache (half the bytes per token: one wave per item keeps all items of the
// batch decode shape resident at once; measured 39.4 -> 37.0 us, while BF16
// is fastest with 2).
#ifndef PDA_ONESHOT_WAVES_WIDE
#define PDA_ONESHOT_WAVES_WIDE 2
#endif
#ifndef PDA_ONESHOT_WAVES_WIDE_FP8
#define PDA_ONESHOT_WAVES_WIDE_FP8 1
#endif

// LDS bytes one workgroup may use on the current device (64 KiB if the
// runtime does not say), cached per device.
size_t lds_per_block() {
    static std::mutex mu;
    static std::vector<std::pair<int, size_t>> cache;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 64 * 1024;
    std::lock_guard<std::mutex> g(mu);
    for (const auto& c : cache)
        if (c.first == dev) return c.second;
    int v = 0;
    size_t bytes = 64 * 1024;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) == hipSuccess &&
        v > 0)
        bytes = (size_t)v;
    cache.emplace_back(dev, bytes);
    return bytes;
}

// Whether a one-shot launch gives each sequence few workgroups (fewer than
// 128 (KV head, split) items): such launches may split a long item over
// several workgroups (oneshot_parts, grid_parts), and use workgroups of
// PDA_FEW_WAVES waves for a BF16 cache (8:
// measured on the 131072-token sequence with 4 parts, fold 53.5 us against
// 58.4 us at 12 waves and 59.0 at 6) and PDA_FEW_WAVES_FP8 for an FP8 one,
// within the kernel's limit and the device's LDS per workgroup.
bool few_items(uint32_t nkv, uint32_t nsplit) { return (uint64_t)nkv * nsplit < 128; }

// 0: the widest the kernel allows (the FP8 form, half the bytes per token,
// measured fastest at 12 waves: long-sequence fold 44.8 us vs 47.6 at 8)
#ifndef PDA_FEW_WAVES
#define PDA_FEW_WAVES 8
#endif
#ifndef PDA_FEW_WAVES_FP8
#define PDA_FEW_WAVES_FP8 0
#endif
int oneshot_waves(uint32_t nkv, uint32_t nsplit, uint32_t head_dim, int gc, bool fp8) {
    const int few = fp8 ? PDA_FEW_WAVES_FP8 : PDA_FEW_WAVES;
    int w = few_items(nkv, nsplit)
                ? (few > 0 && few < pda::fold_max_waves(gc) ? few : pda::fold_max_waves(gc))
                : (fp8 ? PDA_ONESHOT_WAVES_WIDE_FP8 : PDA_ONESHOT_WAVES_WIDE);
    const size_t cap = lds_per_block();
    while (w > 1 && pda::fold_lds_bytes((int)head_dim, gc, w) > cap) --w;
    return w;
}

struct DecodeShape {
    uint32_t num_seqs, nq, nkv, D, bs, max_blocks, num_blocks;
};

// Parts per item of a one-shot launch (workgroups that share one split of
// one sequence and head group, the last to finish combining them).  Like the
// wave count, a pure function of the shape and the split count: launches
// that give a sequence few (KV head, split) items split each item so that a
// single sequence still offers about PDA_PART_TARGET workgroups (the CU count
// of an MI355X), within kMaxParts and the library's part arrays.
// (Measured on the 131072-token sequence: targets 256, 384 and 512 give the
// same fold, 53.1-53.8 us at 8 waves per workgroup; 58-59 us at 6.)
#ifndef PDA_PART_TARGET
#define PDA_PART_TARGET 256
#endif
int oneshot_parts(uint32_t nkv, uint32_t hg, uint32_t nsplit, int gc, uint32_t head_dim) {
    if (!few_items(nkv, nsplit)) return 1;
    const uint64_t items = (uint64_t)nkv * hg * nsplit;   // per sequence
    uint64_t parts = (PDA_PART_TARGET + items - 1) / items;
    if (parts > (uint64_t)pda::kMaxParts) parts = pda::kMaxParts;
    while (parts > 1 && (items * parts * pda::part_rec_floats(gc, (int)head_dim) >
                             pda::kPartSubFloats ||
                         items > pda::kPartTickets))
        --parts;
    return (int)parts;
}

// Sequences per launch that the library's part arrays hold at `parts`.
uint32_t part_rows(uint64_t items_per_row, int parts, int gc, uint32_t head_dim) {
    const uint64_t by_tick = pda::kPartTickets / items_per_row;
    const uint64_t by_sub =
        pda::kPartSubFloats / (items_per_row * parts * pda::part_rec_floats(gc, (int)head_dim));
    const uint64_t r = by_tick < by_sub ? by_tick : by_sub;
    return r > 0xFFFFFFFFull ? 0xFFFFFFFFu : (uint32_t)r;
}

// Blocks per part at least, for one-shot launches.  Measured: the
// 131072-token sequence is as fast at 128 as at 32 (58.2 vs 59.8 us), while
// 64 sequences at 4 splits (head dim 256, 8 heads per KV head), which need
// no parts, took 447 / 350 / 276 us at 32 / 64 / 128 (271 without parts).
#ifndef PDA_PART_MIN
#define PDA_PART_MIN 128
#endif

// Part workgroups the grid needs per item: an item of n blocks uses
// min(cap, ceil(n / part_min)) of them, and no item of this launch has more
// blocks than the largest split a table row of max_blocks blocks allows, so
// the grid carries no part slot that no item can use (such slots are not
// free: 64 sequences at head dim 256 and 16 splits, where every item uses
// one part, took 1196 us with 4 slots per item against 357 us with one).
// The parts an item uses do not depend on this count, only on its length.
int grid_parts(int cap, uint32_t max_blocks, uint32_t nsplit, uint32_t bs, int part_min) {
    if (cap <= 1) return 1;
    const uint32_t most = pda::split_chunk(max_blocks * bs, nsplit, bs) / bs;  // blocks
    const uint32_t need = (most + part_min - 1) / part_min;
    return need < 2 ? 1 : (need < (uint32_t)cap ? (int)need : cap);
}

// Launches a one-shot fold over all sequences; with parts, in runs of
// sequences that fit the library's part arrays (each run is an ordinary
// launch over fewer rows: a sequence's arithmetic does not change).
hipError_t launch_oneshot(int mode, const DecodeShape& s, int gc, int hg, pda::FoldParams p,
                          uint32_t nsplit, int waves, hipStream_t stream, bool kv8) {
    const int cap = oneshot_parts(s.nkv, (uint32_t)hg, nsplit, gc, s.D);
    const int parts = grid_parts(cap, s.max_blocks, nsplit, s.bs, PDA_PART_MIN);
    const uint64_t items = (uint64_t)s.nkv * hg * nsplit;
    p.parts = parts;
    p.part_min = PDA_PART_MIN;
    p.sub = nullptr;
    p.tick = nullptr;
    const uint32_t gx = (uint32_t)(items * parts);
    const uint32_t chunk = parts > 1 ? part_rows(items, parts, gc, s.D) : s.num_seqs;
    if (chunk == 0) return hipErrorInvalidValue;   // oneshot_parts keeps one row in the arrays
    for (uint32_t r0 = 0; r0 < s.num_seqs; r0 += chunk) {
        const uint32_t rows = s.num_seqs - r0 < chunk ? s.num_seqs - r0 : chunk;
        pda::FoldParams c = p;
        c.q = p.q + (uint64_t)r0 * s.nq * s.D;
        c.tables = p.tables + (uint64_t)r0 * s.max_blocks;
        c.lens = p.lens + r0;
        if (p.ws) c.ws = p.ws + (uint64_t)r0 * s.nq * nsplit * (s.D + 2);
        if (p.out) c.out = p.out + (uint64_t)r0 * s.nq * s.D;
        hipError_t e = pda::launch_fold(mode, (int)s.D, gc, c, gx, rows, waves, stream, kv8);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

#ifndef PDA_TILED_WAVES
#define PDA_TILED_WAVES 8
#endif
// Parts per tile of a tiled launch: up to PDA_TILED_PARTS, one per
// kMinTilePartBlocks blocks of the sequence's own tile, so a full tile of the
// later calls of a step (which hold only the longer sequences) still spreads
// over the chip while a call that folds one partial last block per
// sequence runs one workgroup each, with no hand-over.  Measured on 128
// sequences of 0-16K tokens, 64-block tiles: 1 part 1134 us per step, 2
// parts 1103, 3 parts 1079, 4 parts 1100 (each part workgroup in the grid
// costs the partial-block calls dispatch time).  Again with the balanced
// tile plan and the partial-block calls at one part: 3 parts 1058 us, 4
// parts 1055, 2 parts 1099; 12 waves 1164; 4 parts of 6 waves 1134.
#ifndef PDA_TILED_PARTS
#define PDA_TILED_PARTS 3
#endif
int tiled_parts(const pda_tiled_dims& d) {
    uint32_t parts = (d.tile_capacity + pda::kMinTilePartBlocks - 1) / pda::kMinTilePartBlocks;
    if (parts > PDA_TILED_PARTS) parts = PDA_TILED_PARTS;
    return parts < 2 ? 1 : (int)parts;
}

// A call whose last block is partial (last_block_valid_slots < block_size)
// folds, under the library's tile plan, one partial block per sequence: it
// runs with one part (a tile of fewer than kMinTilePartBlocks blocks uses
// one part anyway, so its bytes are those of the parts grid) and
// PDA_TILED_TAIL_WAVES waves, instead of dispatching part workgroups that
// find nothing to fold.  Measured on 128 sequences of 0-16K tokens (31 such
// calls per step): 2 / 4 / 8 waves 1087 / 1068 / 1058 us per step; with the
// part slots of the full calls, 1080.
#ifndef PDA_TILED_TAIL_WAVES
#define PDA_TILED_TAIL_WAVES 8
#endif

int tiled_waves(uint32_t head_dim, int gc, int want = PDA_TILED_WAVES) {
    int w = want;
    while (w > 1 && pda::fold_lds_bytes((int)head_dim, gc, w) > 64 * 1024) --w;
    return w;
}

int check_decode(const DecodeShape& s, const void* q, const void* k, const void* v,
                 const int32_t* bt, const int32_t* lens, const void* out, bool need_out) {
    if (s.num_seqs == 0) return PDA_OK;
    if (!q || !k || !v || !bt || !lens || (need_out && !out))
        return fail(PDA_EINVAL, "null pointer argument");
    if (s.nkv == 0) return fail(PDA_EINVAL, "num_kv_heads is 0");
    if (s.nq == 0 || s.nq % s.nkv != 0)
        return fail(PDA_EINVAL, "num_q_heads (%u) is not a positive multiple of num_kv_heads (%u)",
                    s.nq, s.nkv);
    if (!head_dim_supported(s.D))
        return fail(PDA_EINVAL, "head_dim %u not supported (64, 128 or 256)", s.D);
    if (s.bs == 0 || s.bs % pda::kBlockQuantum != 0)
        return fail(PDA_EINVAL, "block_size %u is not a positive multiple of %u", s.bs,
                    pda::kBlockQuantum);
    if (s.max_blocks == 0) return fail(PDA_EINVAL, "max_blocks_per_seq is 0");
    if ((uint64_t)s.max_blocks * s.bs > 0x7FFFFFFFull)
        return fail(PDA_EINVAL, "max_blocks_per_seq * block_size exceeds 2^31 - 1");
    if (s.num_blocks == 0) return fail(PDA_EINVAL, "num_blocks is 0");
    if ((uint64_t)s.bs * s.nkv * s.D > 0x7FFFFFFFull)
        return fail(PDA_EINVAL, "one block exceeds 2^31 elements");
    const size_t va = s.D == 64 ? 8 : 16;
    if (!aligned(q, va) || !aligned(k, va) || !aligned(v, va) || (out && !aligned(out, 4)))
        return fail(PDA_EINVAL, "q / k_cache / v_cache must be %zu-byte aligned", va);
    if (!aligned(bt, 4) || !aligned(lens, 4))
        return fail(PDA_EINVAL, "block_tables / seq_lens must be 4-byte aligned");
    return PDA_OK;
}

pda::FoldParams fold_params(const DecodeShape& s, const void* q, const void* k, const void* v,
                            const int32_t* bt, const int32_t* lens, int hg, float scale,
                            uint32_t nsplit) {
    pda::FoldParams p{};
    p.q = static_cast<const uint16_t*>(q);
    p.k = static_cast<const uint16_t*>(k);
    p.v = static_cast<const uint16_t*>(v);
    p.tables = bt;
    p.lens = lens;
    p.blk_s = (int64_t)s.bs * s.nkv * s.D;
    p.tok_s = (int64_t)s.nkv * s.D;
    p.kvh_s = (int64_t)s.D;
    p.num_blocks = s.num_blocks;
    p.nq = (int)s.nq;
    p.nkv = (int)s.nkv;
    p.G = (int)(s.nq / s.nkv);
    p.HG = hg;
    p.bs = (int)s.bs;
    p.table_stride = (int)s.max_blocks;
    p.nsplit = (int)nsplit;
    p.c = scale * kLog2e;
    p.parts = 1;
    return p;
}

pda::PackedParams packed_params(const DecodeShape& s, const void* q, const void* k,
                                const void* v, const int32_t* bt, const int32_t* lens,
                                float scale, uint32_t nsplit) {
    pda::PackedParams p{};
    p.q = static_cast<const uint16_t*>(q);
    p.k = static_cast<const uint16_t*>(k);
    p.v = static_cast<const uint16_t*>(v);
    p.tables = bt;
    p.lens = lens;
    p.blk_s = (int64_t)s.bs * s.nkv * s.D;
    p.tok_s = (int64_t)s.nkv * s.D;
    p.kvh_s = s.D;
    p.num_blocks = s.num_blocks;
    p.nq = (int)s.nq;
    p.nkv = (int)s.nkv;
    p.bs = (int)s.bs;
    p.table_stride = (int)s.max_blocks;
    p.nsplit = (int)nsplit;
    p.c = scale * kLog2e;
    p.parts = 1;
    return p;
}

// The element type of the K/V caches: BF16, or OCP E4M3 bytes with
// per-tensor scales (K = decode(k) * k_scale, V = decode(v) * v_scale).
struct KvType {
    bool fp8;
    float k_scale, v_scale;
};
constexpr KvType kBf16Kv{false, 1.f, 1.f};

int run_partials(const DecodeShape& s, const void* q, const void* k, const void* v,
                 const int32_t* bt, const int32_t* lens, float* ws, uint64_t ws_floats,
                 float scale, uint32_t nsplit, bool packed, hipStream_t stream,
                 const KvType& kv) {
    const float sc = kv.fp8 ? scale * kv.k_scale : scale;   // k_scale joins the score factor
    if (!ws) return fail(PDA_EINVAL, "workspace is NULL with num_splits > 1");
    if (!aligned(ws, 8)) return fail(PDA_EINVAL, "workspace must be 8-byte aligned");
    const uint64_t need = pda_workspace_slots(s.num_seqs, s.nq, nsplit, s.D);
    if (ws_floats < need)
        return fail(PDA_EINVAL, "workspace holds %llu floats, needs %llu",
                    (unsigned long long)ws_floats, (unsigned long long)need);
    if (packed) {
        pda::PackedParams p = packed_params(s, q, k, v, bt, lens, sc, nsplit);
        p.ws = ws;
        p.v_scale = kv.v_scale;
        hipError_t e = pda::launch_packed(p, s.num_seqs, stream, kv.fp8);
        if (e != hipSuccess) return hip_fail(e, "packed split-K partial launch");
        return PDA_OK;
    }
    int hg = 0;
    const int gc = head_groups(s.nq / s.nkv, &hg);
    pda::FoldParams p = fold_params(s, q, k, v, bt, lens, hg, sc, nsplit);
    p.ws = ws;
    p.v_scale = kv.v_scale;
    const int waves = oneshot_waves(s.nkv, nsplit, s.D, gc, kv.fp8);
    hipError_t e =
        launch_oneshot(pda::kModePartial, s, gc, hg, p, nsplit, waves, stream, kv.fp8);
    if (e != hipSuccess) return hip_fail(e, "split-K partial launch");
    return PDA_OK;
}

bool scales_finite(float scale, const KvType& kv) {
    return std::isfinite(scale) && std::isfinite(kv.k_scale) && std::isfinite(kv.v_scale);
}

const char* const kPackNotApplicable =
    "packed kernel not applicable: needs num_q_heads == 8 * num_kv_heads and head_dim 256";

// pda_splitk_partials and its FP8 form.
int partials_impl(const DecodeShape& s, const void* q, const void* k, const void* v,
                  const int32_t* bt, const int32_t* lens, float* ws, uint64_t ws_floats,
                  float scale, uint32_t nsplit, uint32_t flags, hipStream_t stream,
                  const KvType& kv) {
    int rc = check_decode(s, q, k, v, bt, lens, nullptr, false);
    if (rc != PDA_OK) return rc;
    if (flags > PDA_DECODE_DEFAULT) return fail(PDA_EINVAL, "unknown flags 0x%x", flags);
    if (nsplit < 2 || nsplit > pda::kMaxDecodeSplits)
        return fail(PDA_EINVAL, "num_splits %u outside 2..%u for a partials launch", nsplit,
                    pda::kMaxDecodeSplits);
    if (!scales_finite(scale, kv)) return fail(PDA_EINVAL, "scale (or an FP8 scale) is not finite");
    const bool packed = flags == PDA_DECODE_PACKED;
    if (packed && !pda_gqa_pack_shape_ok(s.nq, s.nkv, s.D)) {
        g_last_error = kPackNotApplicable;
        return PDA_NOT_APPLICABLE;
    }
    if (s.num_seqs == 0) return ok();
    rc = run_partials(s, q, k, v, bt, lens, ws, ws_floats, scale, nsplit, packed, stream, kv);
    return rc == PDA_OK ? ok() : rc;
}

// Workgroups per (sequence, KV head) of the packed kernel's non-split
// launch (its parts form; 1 = one workgroup each, the pages' launch shape).
// Measured on 64 sequences of 1K-8K tokens (32 q / 4 kv heads, D 256):
// 1 part 253 us, 2 parts of 8 waves 213 us (all 512 workgroups resident at
// once, two per CU), 4 of 4 waves 221 us, 8 parts 280 us and more; again
// with the kernel's non-temporal K/V loads: 2 of 8 waves 204.7 us, 3 of 4
// 209.0, 3 of 8 210.9, 4 of 4 216.7, 2 of 4 242.6.
#ifndef PDA_PACKED_PARTS
#define PDA_PACKED_PARTS 2
#endif

// pda_paged_decode and its FP8 form.
int decode_impl(const DecodeShape& s, const void* q, const void* k, const void* v,
                const int32_t* bt, const int32_t* lens, void* out, float* ws,
                uint64_t ws_floats, float scale, uint32_t nsplit, uint32_t flags,
                hipStream_t st, const KvType& kv) {
    int rc = check_decode(s, q, k, v, bt, lens, out, true);
    if (rc != PDA_OK) return rc;
    if (flags > PDA_DECODE_DEFAULT) return fail(PDA_EINVAL, "unknown flags 0x%x", flags);
    if (nsplit < 1 || nsplit > pda::kMaxDecodeSplits)
        return fail(PDA_EINVAL, "num_splits %u outside 1..%u", nsplit, pda::kMaxDecodeSplits);
    if (!scales_finite(scale, kv)) return fail(PDA_EINVAL, "scale (or an FP8 scale) is not finite");

    const bool shape_packs = pda_gqa_pack_shape_ok(s.nq, s.nkv, s.D);
    // the default arms the packed kernel on non-split launches only, as the
    // pages do (for BF16 and FP8 caches alike); an explicit request also
    // takes it with split-K
    if (flags == PDA_DECODE_DEFAULT)
        flags = shape_packs && nsplit == 1 && pda_gqa_pack_enabled() ? PDA_DECODE_PACKED
                                                                     : PDA_DECODE_UNPACKED;
    const bool packed = flags == PDA_DECODE_PACKED;
    if (packed && !shape_packs) {
        g_last_error = kPackNotApplicable;
        return PDA_NOT_APPLICABLE;
    }
    if (s.num_seqs == 0) return ok();
    const float sc = kv.fp8 ? scale * kv.k_scale : scale;
    if (packed && nsplit == 1) {
        // PDA_PACKED_PARTS workgroups per (sequence, KV head), a constant,
        // so a sequence's bytes do not depend on its batch; batches beyond
        // the library's part records run as several launches
        pda::PackedParams p = packed_params(s, q, k, v, bt, lens, sc, 1);
        p.out = static_cast<uint16_t*>(out);
        p.v_scale = kv.v_scale;
        p.parts = grid_parts(PDA_PACKED_PARTS, s.max_blocks, 1, s.bs, pda::kMinPartBlocks);
        const uint32_t chunk = p.parts > 1 ? pda::packed_part_rows(s.nkv, p.parts) : s.num_seqs;
        if (chunk == 0) return fail(PDA_EINVAL, "num_kv_heads too large for the packed kernel");
        for (uint32_t r0 = 0; r0 < s.num_seqs; r0 += chunk) {
            const uint32_t rows = s.num_seqs - r0 < chunk ? s.num_seqs - r0 : chunk;
            pda::PackedParams c = p;
            c.q = p.q + (uint64_t)r0 * s.nq * s.D;
            c.tables = p.tables + (uint64_t)r0 * s.max_blocks;
            c.lens = p.lens + r0;
            c.out = p.out + (uint64_t)r0 * s.nq * s.D;
            hipError_t e = pda::launch_packed(c, rows, st, kv.fp8);
            if (e != hipSuccess) return hip_fail(e, "packed decode launch");
        }
        return ok();
    }
    if (nsplit == 1) {
        int hg = 0;
        const int gc = head_groups(s.nq / s.nkv, &hg);
        pda::FoldParams p = fold_params(s, q, k, v, bt, lens, hg, sc, 1);
        p.out = static_cast<uint16_t*>(out);
        p.v_scale = kv.v_scale;
        const int waves = oneshot_waves(s.nkv, 1, s.D, gc, kv.fp8);
        hipError_t e = launch_oneshot(pda::kModeFinal, s, gc, hg, p, 1, waves, st, kv.fp8);
        if (e != hipSuccess) return hip_fail(e, "single-split decode launch");
        return ok();
    }
    rc = run_partials(s, q, k, v, bt, lens, ws, ws_floats, scale, nsplit, packed, st, kv);
    if (rc != PDA_OK) return rc;
    hipError_t e = pda::launch_merge(ws, static_cast<uint16_t*>(out), s.num_seqs, (int)s.nq,
                                     (int)s.D, (int)nsplit, st);
    if (e != hipSuccess) return hip_fail(e, "split-K merge launch");
    return ok();
}

// Workspace of pda_paged_decode_noalloc: a device array of this library,
// one copy per GPU, which each GPU holds until the process ends.  Its host
// name is not a device address: host code uses only the address that
// hipGetSymbolAddress returns for the current device (noalloc_scratch).
constexpr uint64_t kNoAllocWorkspaceFloats = 1u << 22;   // 16 MiB
static __device__ __align__(256) float scratch[kNoAllocWorkspaceFloats];

// Address of `scratch` on the current device, looked up once per device
// with that device current; *err receives a failing HIP code.
float* noalloc_scratch(hipError_t* err) {
    static std::mutex mu;
    static std::vector<std::pair<int, float*>> cache;
    int dev = 0;
    *err = hipGetDevice(&dev);
    if (*err != hipSuccess) return nullptr;
    std::lock_guard<std::mutex> g(mu);
    for (const auto& c : cache)
        if (c.first == dev) return c.second;
    void* ptr = nullptr;
    *err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (*err != hipSuccess || !ptr) {
        if (*err == hipSuccess) *err = hipErrorInvalidSymbol;
        return nullptr;
    }
    cache.emplace_back(dev, static_cast<float*>(ptr));
    return static_cast<float*>(ptr);
}

}  // namespace

extern "C" {

const char* pda_last_error(void) { return g_last_error.c_str(); }

int pda_device_cu_count(int device, uint32_t* cu_count) {
    if (!cu_count) return fail(PDA_EINVAL, "cu_count is NULL");
    int n = 0;
    hipError_t e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, device);
    if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute");
    *cu_count = (uint32_t)n;
    return ok();
}

int pda_splitk_partials(const void* q, const void* k_cache, const void* v_cache,
                        const int32_t* block_tables, const int32_t* seq_lens, float* workspace,
                        uint64_t workspace_floats, uint32_t num_seqs, uint32_t num_q_heads,
                        uint32_t num_kv_heads, uint32_t head_dim, uint32_t block_size,
                        uint32_t max_blocks_per_seq, uint32_t num_blocks, float scale,
                        uint32_t num_splits, uint32_t flags, void* stream) {
    const DecodeShape s{num_seqs, num_q_heads, num_kv_heads, head_dim,
                        block_size, max_blocks_per_seq, num_blocks};
    return partials_impl(s, q, k_cache, v_cache, block_tables, seq_lens, workspace,
                         workspace_floats, scale, num_splits, flags, (hipStream_t)stream,
                         kBf16Kv);
}

int pda_paged_decode_fp8(const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* block_tables, const int32_t* seq_lens, void* out,
                         float* workspace, uint64_t workspace_floats, uint32_t num_seqs,
                         uint32_t num_q_heads, uint32_t num_kv_heads, uint32_t head_dim,
                         uint32_t block_size, uint32_t max_blocks_per_seq, uint32_t num_blocks,
                         float scale, float k_scale, float v_scale, uint32_t num_splits,
                         uint32_t flags, void* stream) {
    const DecodeShape s{num_seqs, num_q_heads, num_kv_heads, head_dim,
                        block_size, max_blocks_per_seq, num_blocks};
    return decode_impl(s, q, k_cache, v_cache, block_tables, seq_lens, out, workspace,
                       workspace_floats, scale, num_splits, flags, (hipStream_t)stream,
                       KvType{true, k_scale, v_scale});
}

int pda_splitk_partials_fp8(const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* block_tables, const int32_t* seq_lens,
                            float* workspace, uint64_t workspace_floats, uint32_t num_seqs,
                            uint32_t num_q_heads, uint32_t num_kv_heads, uint32_t head_dim,
                            uint32_t block_size, uint32_t max_blocks_per_seq,
                            uint32_t num_blocks, float scale, float k_scale, float v_scale,
                            uint32_t num_splits, uint32_t flags, void* stream) {
    const DecodeShape s{num_seqs, num_q_heads, num_kv_heads, head_dim,
                        block_size, max_blocks_per_seq, num_blocks};
    return partials_impl(s, q, k_cache, v_cache, block_tables, seq_lens, workspace,
                         workspace_floats, scale, num_splits, flags, (hipStream_t)stream,
                         KvType{true, k_scale, v_scale});
}

int pda_prefill_applies(uint32_t num_q_heads, uint32_t num_kv_heads, uint32_t head_dim,
                        int causal, uint32_t sliding_window) {
    return head_dim == pda::kPrefillHeadDim && causal && sliding_window == 0 &&
           num_kv_heads > 0 &&
           num_q_heads % num_kv_heads == 0;
}

int pda_paged_prefill(const void* q, const void* k_cache, const void* v_cache, void* out,
                      const int32_t* block_table, uint32_t q_len, uint32_t kv_len,
                      uint32_t q_offset, uint32_t num_q_heads, uint32_t num_kv_heads,
                      uint32_t head_dim, uint32_t block_size, uint32_t max_blocks,
                      uint32_t num_blocks, uint32_t sliding_window, float scale, void* stream) {
    if (q_len == 0 ||
        !pda_prefill_applies(num_q_heads, num_kv_heads, head_dim, 1, sliding_window)) {
        g_last_error = "prefill kernel not applicable: needs q_len > 0, head_dim 256, causal, "
                       "no sliding window and num_q_heads a multiple of num_kv_heads";
        return PDA_NOT_APPLICABLE;
    }
    if (!q || !k_cache || !v_cache || !out || !block_table)
        return fail(PDA_EINVAL, "null pointer argument");
    if (block_size == 0 || num_blocks == 0 || max_blocks == 0)
        return fail(PDA_EINVAL, "block_size, num_blocks and max_blocks must be positive");
    if ((uint64_t)q_offset + q_len >= (1ull << 31) || kv_len >= (1u << 31))
        return fail(PDA_EINVAL, "q_offset + q_len and kv_len must be below 2^31");
    if ((uint64_t)kv_len > (uint64_t)max_blocks * block_size)
        return fail(PDA_EINVAL, "kv_len %u exceeds the block table (%u blocks of %u)", kv_len,
                    max_blocks, block_size);
    if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 16))
        return fail(PDA_EINVAL, "q, caches and out must be 16-byte aligned");
    if (!std::isfinite(scale)) return fail(PDA_EINVAL, "scale is not finite");
    pda::PrefillParams p{};
    p.q = static_cast<const uint16_t*>(q);
    p.k = static_cast<const uint16_t*>(k_cache);
    p.v = static_cast<const uint16_t*>(v_cache);
    p.table = block_table;
    p.out = static_cast<uint16_t*>(out);
    p.blk_s = (int64_t)block_size * num_kv_heads * head_dim;
    p.tok_s = (int64_t)num_kv_heads * head_dim;
    p.num_blocks = num_blocks;
    p.nq = (int)num_q_heads;
    p.nkv = (int)num_kv_heads;
    p.bs = (int)block_size;
    p.q_len = (int)q_len;
    p.kv_len = (int)kv_len;
    p.q_offset = (int)q_offset;
    p.c = scale * kLog2e;
    hipError_t e = pda::launch_prefill(p, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "prefill launch");
    return ok();
}

int pda_splitk_merge(const float* workspace, uint64_t workspace_floats, void* out,
                     uint32_t num_seqs, uint32_t num_q_heads, uint32_t head_dim,
                     uint32_t num_splits, void* stream) {
    if (num_seqs == 0) return ok();
    if (!workspace || !out) return fail(PDA_EINVAL, "null pointer argument");
    if (!head_dim_supported(head_dim))
        return fail(PDA_EINVAL, "head_dim %u not supported (64, 128 or 256)", head_dim);
    if (num_q_heads == 0) return fail(PDA_EINVAL, "num_q_heads is 0");
    if (num_splits < 1 || num_splits > pda::kMaxDecodeSplits)
        return fail(PDA_EINVAL, "num_splits %u outside 1..%u", num_splits, pda::kMaxDecodeSplits);
    if (!aligned(workspace, 8) || !aligned(out, 4))
        return fail(PDA_EINVAL, "workspace must be 8-byte and out 4-byte aligned");
    const uint64_t need = pda_workspace_slots(num_seqs, num_q_heads, num_splits, head_dim);
    if (workspace_floats < need)
        return fail(PDA_EINVAL, "workspace holds %llu floats, needs %llu",
                    (unsigned long long)workspace_floats, (unsigned long long)need);
    hipError_t e = pda::launch_merge(workspace, static_cast<uint16_t*>(out), num_seqs,
                                     (int)num_q_heads, (int)head_dim, (int)num_splits,
                                     (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "split-K merge launch");
    return ok();
}

int pda_paged_decode(const void* q, const void* k_cache, const void* v_cache,
                     const int32_t* block_tables, const int32_t* seq_lens, void* out,
                     float* workspace, uint64_t workspace_floats, uint32_t num_seqs,
                     uint32_t num_q_heads, uint32_t num_kv_heads, uint32_t head_dim,
                     uint32_t block_size, uint32_t max_blocks_per_seq, uint32_t num_blocks,
                     float scale, uint32_t num_splits, uint32_t flags, void* stream) {
    const DecodeShape s{num_seqs, num_q_heads, num_kv_heads, head_dim,
                        block_size, max_blocks_per_seq, num_blocks};
    return decode_impl(s, q, k_cache, v_cache, block_tables, seq_lens, out, workspace,
                       workspace_floats, scale, num_splits, flags, (hipStream_t)stream,
                       kBf16Kv);
}

int pda_paged_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                             const int32_t* block_tables, const int32_t* seq_lens, void* out,
                             uint32_t num_seqs, uint32_t num_q_heads, uint32_t num_kv_heads,
                             uint32_t head_dim, uint32_t block_size,
                             uint32_t max_blocks_per_seq, uint32_t num_blocks, float scale,
                             uint32_t num_splits, uint32_t flags, void* stream) {
    const DecodeShape s{num_seqs, num_q_heads, num_kv_heads, head_dim,
                        block_size, max_blocks_per_seq, num_blocks};
    // every argument check runs before the scratch lookup (the first HIP call)
    int rc = check_decode(s, q, k_cache, v_cache, block_tables, seq_lens, out, true);
    if (rc != PDA_OK) return rc;
    if (num_splits < 1 || num_splits > pda::kMaxDecodeSplits)
        return fail(PDA_EINVAL, "num_splits %u outside 1..%u", num_splits, pda::kMaxDecodeSplits);
    const uint64_t need =
        num_splits > 1 ? pda_workspace_slots(num_seqs, num_q_heads, num_splits, head_dim) : 0;
    if (need > kNoAllocWorkspaceFloats)
        return fail(PDA_EINVAL,
                    "the split-K workspace needs %llu floats; pda_paged_decode_noalloc holds "
                    "%llu (pass a workspace to pda_paged_decode instead)",
                    (unsigned long long)need, (unsigned long long)kNoAllocWorkspaceFloats);
    float* ws = nullptr;
    if (need > 0 && num_seqs > 0) {
        hipError_t e = hipSuccess;
        ws = noalloc_scratch(&e);
        if (!ws) return hip_fail(e, "hipGetSymbolAddress (scratch workspace)");
    }
    return decode_impl(s, q, k_cache, v_cache, block_tables, seq_lens, out, ws, need, scale,
                       num_splits, flags, (hipStream_t)stream, kBf16Kv);
}

// ---------------------------------------------------------------------------
// Tiled state API
// ---------------------------------------------------------------------------

}  // extern "C"

struct pda_tiled {
    pda_tiled_dims dims;
    int device;
    float* m;
    float* l;
    float* o;
    int parts;        // workgroups per (sequence, head group) tile
    float* sub;       // part records (parts > 1)
    uint32_t* tick;   // arrival tickets, zeroed at creation (parts > 1)
};

extern "C" {

int pda_tiled_validate(const pda_tiled_dims* d) {
    if (!d) return fail(PDA_EINVAL, "dims is NULL");
    if (d->num_kv_heads == 0) return fail(PDA_EINVAL, "num_kv_heads is 0");
    if (d->num_q_heads % d->num_kv_heads != 0)
        return fail(PDA_EINVAL, "num_q_heads (%u) is not a multiple of num_kv_heads (%u)",
                    d->num_q_heads, d->num_kv_heads);
    if (d->head_dim > pda::kMaxHeadDim)
        return fail(PDA_EINVAL, "head_dim %u exceeds the maximum of %u", d->head_dim,
                    pda::kMaxHeadDim);
    if (!head_dim_supported(d->head_dim))
        return fail(PDA_EINVAL, "head_dim %u not supported (64, 128 or 256)", d->head_dim);
    if (d->num_q_heads == 0 || d->max_seqs == 0 || d->tile_capacity == 0)
        return fail(PDA_EINVAL, "max_seqs, num_q_heads and tile_capacity must be positive");
    if (d->block_size == 0 || d->block_size % pda::kBlockQuantum != 0)
        return fail(PDA_EINVAL, "block_size %u is not a positive multiple of %u", d->block_size,
                    pda::kBlockQuantum);
    if ((uint64_t)d->tile_capacity * d->block_size > 0x7FFFFFFFull)
        return fail(PDA_EINVAL, "tile_capacity * block_size exceeds 2^31 - 1");
    return ok();
}

int pda_tiled_create(const pda_tiled_dims* d, pda_tiled** out) {
    if (!out) return fail(PDA_EINVAL, "out is NULL");
    int rc = pda_tiled_validate(d);
    if (rc != PDA_OK) return rc;
    pda_tiled* t = new (std::nothrow) pda_tiled{};
    if (!t) return fail(PDA_ENOMEM, "handle allocation failed");
    t->dims = *d;
    hipError_t e = hipGetDevice(&t->device);
    if (e != hipSuccess) {
        delete t;
        return hip_fail(e, "hipGetDevice");
    }
    const uint64_t slots = (uint64_t)d->max_seqs * d->num_q_heads;
    e = hipMalloc((void**)&t->m, slots * sizeof(float));
    if (e == hipSuccess) e = hipMalloc((void**)&t->l, slots * sizeof(float));
    if (e == hipSuccess) e = hipMalloc((void**)&t->o, slots * d->head_dim * sizeof(float));
    t->parts = tiled_parts(*d);
    if (t->parts > 1 && e == hipSuccess) {
        int hg = 0;
        const int gc = head_groups(d->num_q_heads / d->num_kv_heads, &hg);
        const uint64_t items = (uint64_t)d->max_seqs * d->num_kv_heads * hg;
        e = hipMalloc((void**)&t->sub, items * t->parts *
                                           pda::part_rec_floats(gc, (int)d->head_dim) *
                                           sizeof(float));
        if (e == hipSuccess) e = hipMalloc((void**)&t->tick, items * sizeof(uint32_t));
        if (e == hipSuccess) e = hipMemset(t->tick, 0, items * sizeof(uint32_t));
    }
    if (e != hipSuccess) {
        pda_tiled_destroy(t);
        return e == hipErrorOutOfMemory ? fail(PDA_ENOMEM, "tiled state allocation failed")
                                        : hip_fail(e, "hipMalloc");
    }
    *out = t;
    return ok();
}

void pda_tiled_destroy(pda_tiled* t) {
    if (!t) return;
    if (t->m) (void)hipFree(t->m);
    if (t->l) (void)hipFree(t->l);
    if (t->o) (void)hipFree(t->o);
    if (t->sub) (void)hipFree(t->sub);
    if (t->tick) (void)hipFree(t->tick);
    delete t;
}

int pda_tiled_get_dims(const pda_tiled* t, pda_tiled_dims* dims) {
    if (!t || !dims) return fail(PDA_EINVAL, "null pointer argument");
    *dims = t->dims;
    return ok();
}

int pda_tiled_state(const pda_tiled* t, float** m, float** l, float** o) {
    if (!t) return fail(PDA_EINVAL, "handle is NULL");
    if (m) *m = t->m;
    if (l) *l = t->l;
    if (o) *o = t->o;
    return ok();
}

int pda_tiled_begin_step(pda_tiled* t, uint32_t num_seqs, void* stream) {
    if (!t) return fail(PDA_EINVAL, "handle is NULL");
    if (num_seqs > t->dims.max_seqs)
        return fail(PDA_EINVAL, "begin_step num_seqs %u > max_seqs %u", num_seqs,
                    t->dims.max_seqs);
    const uint64_t n_q = (uint64_t)num_seqs * t->dims.num_q_heads;
    hipError_t e = pda::launch_tiled_begin(t->m, t->l, t->o, n_q, (int)t->dims.head_dim,
                                           (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "begin_step launch");
    return ok();
}

int pda_tiled_step_tile(pda_tiled* t, const void* q, const void* k_pool, const void* v_pool,
                        uint64_t pool_blocks, const int32_t* tile_blocks,
                        const int32_t* tile_block_counts, uint32_t num_seqs, int64_t blk_stride,
                        int64_t tok_stride, int64_t kvh_stride, int32_t last_block_valid_slots,
                        void* stream) {
    if (!t) return fail(PDA_EINVAL, "handle is NULL");
    const pda_tiled_dims& d = t->dims;
    if (num_seqs > d.max_seqs)
        return fail(PDA_EINVAL, "step_tile num_seqs %u > max_seqs %u", num_seqs, d.max_seqs);
    if (num_seqs == 0) return ok();
    if (!q || !k_pool || !v_pool || !tile_blocks || !tile_block_counts)
        return fail(PDA_EINVAL, "null pointer argument");
    if (last_block_valid_slots < 1 || (uint32_t)last_block_valid_slots > d.block_size)
        return fail(PDA_EINVAL, "last_block_valid_slots %d outside 1..%u", last_block_valid_slots,
                    d.block_size);
    if (pool_blocks == 0 || pool_blocks > 0xFFFFFFFFull)
        return fail(PDA_EINVAL, "pool_blocks must be in 1..2^32-1");
    const size_t va = d.head_dim == 64 ? 8 : 16;
    const int64_t se = (int64_t)(va / 2);
    if (!aligned(q, va) || !aligned(k_pool, va) || !aligned(v_pool, va))
        return fail(PDA_EINVAL, "q / pools must be %zu-byte aligned", va);
    if (blk_stride < 0 || tok_stride < 0 || kvh_stride < 0 || blk_stride % se ||
        tok_stride % se || kvh_stride % se)
        return fail(PDA_EINVAL, "strides must be non-negative multiples of %lld elements",
                    (long long)se);
    if (tok_stride * (int64_t)d.block_size + d.head_dim > 0x7FFFFFFFll)
        return fail(PDA_EINVAL, "tok_stride * block_size exceeds 2^31 - 1");
    if (!aligned(tile_blocks, 4) || !aligned(tile_block_counts, 4))
        return fail(PDA_EINVAL, "tile arrays must be 4-byte aligned");
    int hg = 0;
    const int gc = head_groups(d.num_q_heads / d.num_kv_heads, &hg);
    pda::FoldParams p{};
    p.q = static_cast<const uint16_t*>(q);
    p.k = static_cast<const uint16_t*>(k_pool);
    p.v = static_cast<const uint16_t*>(v_pool);
    p.tables = tile_blocks;
    p.lens = tile_block_counts;
    p.ws = t->m;
    p.l_state = t->l;
    p.o_state = t->o;
    p.blk_s = blk_stride;
    p.tok_s = tok_stride;
    p.kvh_s = kvh_stride;
    p.num_blocks = (uint32_t)pool_blocks;
    p.nq = (int)d.num_q_heads;
    p.nkv = (int)d.num_kv_heads;
    p.G = (int)(d.num_q_heads / d.num_kv_heads);
    p.HG = hg;
    p.bs = (int)d.block_size;
    p.table_stride = (int)d.tile_capacity;
    p.nsplit = 1;
    p.lbvs = last_block_valid_slots;
    // the step takes no scale: 1 / sqrt(head_dim), rounded once to FP32
    p.c = (float)(1.0 / std::sqrt((double)d.head_dim)) * kLog2e;
    const bool tail = (uint32_t)last_block_valid_slots < d.block_size;
    p.parts = tail ? 1 : t->parts;
    p.part_min = pda::kMinTilePartBlocks;
    p.sub = t->sub;
    p.tick = t->tick;
    const int waves = tiled_waves(d.head_dim, gc, tail ? PDA_TILED_TAIL_WAVES : PDA_TILED_WAVES);
    hipError_t e = pda::launch_fold(pda::kModeTiled, (int)d.head_dim, gc, p,
                                    (uint32_t)(d.num_kv_heads * hg * p.parts), num_seqs, waves,
                                    (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "step_tile launch");
    return ok();
}

int pda_tiled_finalize(pda_tiled* t, void* out, uint32_t num_seqs, void* stream) {
    if (!t) return fail(PDA_EINVAL, "handle is NULL");
    if (num_seqs > t->dims.max_seqs)
        return fail(PDA_EINVAL, "finalize num_seqs %u > max_seqs %u", num_seqs, t->dims.max_seqs);
    if (num_seqs == 0) return ok();
    if (!out || !aligned(out, 4)) return fail(PDA_EINVAL, "out is NULL or not 4-byte aligned");
    const uint64_t n_q = (uint64_t)num_seqs * t->dims.num_q_heads;
    hipError_t e = pda::launch_tiled_finalize(t->l, t->o, static_cast<uint16_t*>(out), n_q,
                                              (int)t->dims.head_dim, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "finalize launch");
    return ok();
}

}  // extern "C"
