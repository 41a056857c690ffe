// GQA-packed paged decode on MFMA (gfx950): one workgroup per (sequence, KV
// head) carries that KV head's 8 query heads at head_dim 256 ("Module
// attn_splitk" page: gqa_pack_shape_ok, gqa_pack_ctas, DECODE_GQA_PACK_*),
// and is used only for single-split launches.  The 8 heads against a tile
// of 16 tokens are a dense 16 x 16 product (heads padded to 16), so q.k and
// P.V run on matrix cores:
//
//   S^T[16 tok][16 head] = K[16 tok][256] . Q^T[256][16 head]
//       8 x v_mfma_f32_16x16x32_bf16; K enters as the A operand straight from
//       its 16-byte row pieces (lane = token, 8 consecutive dims), q as B.
//   O[16 head][256]     += P[16 head][16 tok] . V[16 tok][256]
//       16 x v_mfma_f32_16x16x16_bf16, one per 16 output dims.  The S^T
//       accumulator already holds P in the A-operand layout (lane = head,
//       four consecutive tokens), so P never moves; V goes through LDS and
//       comes back transposed by ds_read_b64_tr_b16 (lane = dim, four
//       consecutive tokens), with an XOR swizzle on the 8-byte chunks that
//       keeps the transposed reads free of bank conflicts.
//
// The online softmax (FP32, base 2, m per head) runs on the S^T accumulator:
// each head's 16 scores sit in one column spread over the four 16-lane
// groups.  W waves take 16-token tiles round-robin; their states are merged
// through LDS in wave order at the end.
//
// The FP8 form (KV8 = true) reads OCP E4M3 caches (the page names a BF16
// and an FP8 packed source): codes are decoded exactly to BF16 in registers
// (K before the A operand, V before its LDS tile), so the matrix products
// are the BF16 ones; k_scale is part of the score factor c and v_scale
// multiplies o once at the end.  To read K in 16-byte pieces, the FP8 form
// orders the contraction differently (see kdim): q follows the same order.
//
// The split-K form (SPLIT = true) takes one split of the sequence per
// workgroup, with the split partition of the unpacked kernels, and leaves
// each head's FP32 (o unnormalised, m natural-log, l) in the split-K
// workspace slot that the merge kernel reads.  The pages arm the packed
// kernels only on non-split launches; the split-K form is this library's
// extension for long, uneven batches, where one workgroup per sequence and
// KV head leaves the device waiting on the longest sequence.
//
// The parts form (PARTS = true, non-split launches) answers the same
// imbalance without a workspace or a second launch: p.parts workgroups share
// one (sequence, KV head), each folding a contiguous run of its blocks into
// an FP32 record (o unnormalised, m in log2 units, l) of a device array the
// library owns; the last to take a ticket combines the records in part
// order and writes the BF16 output.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pda_geometry.h"
#include "pda_kernels.h"

namespace pda {
namespace {

constexpr float kNegInf = -__builtin_inff();
constexpr int kD = 256;            // packed head dim
constexpr int kG = 8;              // packed query heads per KV head
// The kernel is compiled for exactly the shape the host gate dispatches to
// it ("Module attn_splitk": DECODE_GQA_PACK_WIDTH, DECODE_GQA_PACK_HEAD_DIM,
// gqa_pack_shape_ok); a change to either side that breaks the match fails
// the build.
static_assert(kG == (int)kGqaPackWidth, "packed kernel width differs from the dispatch gate");
static_assert(kD == (int)kGqaPackHeadDim, "packed kernel head dim differs from the dispatch gate");
constexpr int kTile = 16;          // tokens per tile
constexpr int kWaves = 8;          // waves per workgroup, non-split form
constexpr int kVTileElems = kTile * kD;   // one wave's V tile in LDS (8 KiB)
#ifndef PDA_PACKED_PARTS_WAVES
#define PDA_PACKED_PARTS_WAVES 8   /* waves per workgroup of the parts form */
#endif

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    bf16x2_t v;
    v[0] = (__bf16)a;
    v[1] = (__bf16)b;
    return __builtin_bit_cast(uint32_t, v);
}

// Eight E4M3 codes (w0 bytes 0..3, then w1 bytes 0..3) as eight BF16 values
// in the same order; exact (3 mantissa bits, every exponent in range; the
// conversion's scale operand 1.0 leaves values as they are).
__device__ __forceinline__ u32x4_t fp8x8_to_bf16(uint32_t w0, uint32_t w1) {
    return u32x4_t{
        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.f, false)),
        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.f, true)),
        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.f, false)),
        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.f, true))};
}

// First of the 8 consecutive head dims that lanes of 16-lane group g hold
// in k-step kb of S^T = K . Q^T.  BF16: 32 kb + 8 g (one 16-byte K piece per
// step).  FP8: 64 (kb / 2) + 16 g + 8 (kb % 2), so one 16-byte load of 16
// codes feeds steps 2j and 2j + 1.  Any order is the same sum as long as K
// and q agree.
template <bool KV8>
__device__ __forceinline__ int kdim(int kb, int g) {
    return KV8 ? 64 * (kb >> 1) + 16 * g + 8 * (kb & 1) : 32 * kb + 8 * g;
}

// Values of the lower and upper 32-lane halves, and of the even and odd
// 16-lane rows of this lane's pair (identical bits on both partners).
__device__ __forceinline__ void halves(float x, float& a, float& b) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
}
__device__ __forceinline__ void rowpair(float x, float& a, float& b) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
}
// Max / sum over the four 16-lane groups (lanes c, c+16, c+32, c+48).
__device__ __forceinline__ float group_max(float x) {
    float a, b;
    rowpair(x, a, b);
    x = fmaxf(a, b);
    halves(x, a, b);
    return fmaxf(a, b);
}
__device__ __forceinline__ float group_sum(float x) {
    float a, b;
    rowpair(x, a, b);
    x = a + b;
    halves(x, a, b);
    return a + b;
}

__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Element offset of 8-byte chunk `chunk` (0..63) of token row `row` in a V
// tile: chunks are XOR-swizzled by 4 * (row & 7) so that the four rows a
// 16-lane group reads at once, in both 32-lane halves, hit distinct banks.
__device__ __forceinline__ int vchunk(int row, int chunk) {
    return row * kD + ((chunk ^ ((row & 7) << 2)) << 2);
}

__device__ __forceinline__ int clamp_len(int x, int cap) {
    return x < 0 ? 0 : (x > cap ? cap : x);
}

// Rank -> sequence, longest first (ties by index), and its clamped length;
// the same schedule rule as the split-K fold: one wave-wide load of the
// lengths, one compare per sequence against a value read from another lane.
// Batches of more than 64 sequences keep their order.  Only the order of
// work depends on it.
__device__ __forceinline__ void packed_seq_of_rank(const int32_t* __restrict__ lens, int S,
                                                   int r, int cap, int& seq, int& len) {
    if (S > 64) {
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

constexpr float kLn2 = 0.6931471805599453f;

// Part records (kPackedRec floats each: o [8][256], m [8], l [8], padded to
// whole 128-byte lines) and arrival tickets of the parts form.  Tickets
// start at 0 and the combining workgroup puts its ticket back to 0.
constexpr int kPackedRec = (int)part_rec_floats(kG, kD);
__device__ __align__(256) float g_packed_sub[kPartSubFloats];
__device__ __align__(256) uint32_t g_packed_tick[kPartTickets];

// Records are written and read at device scope (write-through stores, loads
// that do not hit a stale copy), so the hand-over needs no L2 writeback or
// invalidate: a writer waits for its stores to complete before its
// workgroup takes a ticket, and the combiner loads after the last ticket.
__device__ __forceinline__ void put_dev(float* a, float v) {
    __hip_atomic_store(a, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float get_dev(const float* a) {
    return __hip_atomic_load(const_cast<float*>(a), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// A 16-byte K / V load: non-temporal (streaming) with NT, which the
// non-split launch uses (each K/V byte is read once; measured on the packed
// workload 210.0-211.2 -> 205.8-206.1 us, FP8 127.7-128.0 -> 125.3-125.7);
// the split-K form keeps the default policy (1.7 % slower with it).
template <bool NT>
__device__ __forceinline__ u32x4_t load16(const char* a) {
    if constexpr (NT) return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(a));
    else return *reinterpret_cast<const u32x4_t*>(a);
}

template <bool SPLIT, int W, bool KV8, bool PARTS>
__global__ __launch_bounds__(64 * W, 2) void packed_kernel(const PackedParams p) {
    static_assert(!(SPLIT && PARTS), "parts serve non-split launches");
    constexpr int EB = KV8 ? 1 : 2;   // bytes per cache element
    extern __shared__ __align__(16) uint16_t smem[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, c = lane & 15;   // 16-lane group, lane in group
    const int PL = PARTS ? p.parts : 1;       // workgroups per (sequence, KV head) in the grid
    const int bx = (int)blockIdx.x / PL;
    const int part = (int)blockIdx.x - bx * PL;
    const int kvh = SPLIT ? bx % p.nkv : bx;
    const int sp = SPLIT ? bx / p.nkv : 0;
    const int cap = p.table_stride * p.bs;
    int seq, L;
    packed_seq_of_rank(p.lens, (int)gridDim.y, (int)blockIdx.y, cap, seq, L);
    const int64_t q_row = (int64_t)seq * p.nq + (int64_t)kvh * kG;   // first q slot

    // this workgroup's tokens: the whole sequence, or split sp of it
    int t_begin = 0, t_end = L;
    if constexpr (SPLIT) {
        const int chunk = (int)split_chunk((uint32_t)L, (uint32_t)p.nsplit, (uint32_t)p.bs);
        const int64_t b0 = (int64_t)sp * chunk;
        t_begin = b0 < L ? (int)b0 : L;
        t_end = (int64_t)t_begin + chunk < L ? t_begin + chunk : L;
        if (t_begin >= t_end) {
            // an empty split: m = -inf, l = 0 (its o is never read)
            if (tid < kG) {
                float* slot = p.ws + ((q_row + tid) * p.nsplit + sp) * (int64_t)(kD + 2);
                slot[kD] = kNegInf;
                slot[kD + 1] = 0.f;
            }
            return;
        }
    }
    // The parts this sequence uses: at most PL, no more than one per
    // kMinPartBlocks of its blocks (a function of its own length, so its
    // bytes do not depend on the batch); parts past that count exit.
    int P = 1;
    if constexpr (PARTS) {
        const int nb = (t_end - t_begin + p.bs - 1) / p.bs;
        const int want = (nb + kMinPartBlocks - 1) / kMinPartBlocks;
        P = want < PL ? (want > 1 ? want : 1) : PL;
        if (part >= P) return;
    }
    if (P > 1) {
        // part i: blocks [i * per, (i + 1) * per) of the sequence, per =
        // ceil(blocks / parts); possibly none
        const int nb = (t_end - t_begin + p.bs - 1) / p.bs;
        const int per = (nb + P - 1) / P;
        const int64_t fb = (int64_t)t_begin + (int64_t)part * per * p.bs;
        const int f_begin = fb < t_end ? (int)fb : t_end;
        t_end = (int64_t)f_begin + (int64_t)per * p.bs < t_end ? f_begin + per * p.bs : t_end;
        t_begin = f_begin;
    }

    // q as the B operand: lane = head c (zeros for the 8 padding heads),
    // 8 consecutive dims 32 * kb + 8 * g of k-step kb.  Unconditional loads
    // (padding lanes re-read head 0) so they issue with no branch between.
    bf16x8_t qb[8];
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) {
        const int hq = c < kG ? c : 0;
        const u32x4_t w =
            *reinterpret_cast<const u32x4_t*>(p.q + (q_row + hq) * kD + kdim<KV8>(kb, g));
        const u32x4_t z = {0u, 0u, 0u, 0u};
        qb[kb] = __builtin_bit_cast(bf16x8_t, c < kG ? w : z);
    }

    f32x4_t O[16];   // O[head 4g + r][dim 16 nb + c]
#pragma unroll
    for (int nb = 0; nb < 16; ++nb) O[nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float m = kNegInf, l = 0.f;   // of head c (same in all four groups)

    uint16_t* vt = smem + wave * kVTileElems;
    const int32_t* blocks = p.tables + (int64_t)seq * p.table_stride;
    const char* kbase = reinterpret_cast<const char*>(p.k) + (int64_t)kvh * p.kvh_s * EB;
    const char* vbase = reinterpret_cast<const char*>(p.v) + (int64_t)kvh * p.kvh_s * EB;
    const int64_t tok_b = p.tok_s * EB;
    // t_begin is a block boundary, and blocks hold whole tiles
    const int t_first = t_begin / kTile;
    const int t_last = (t_end + kTile - 1) / kTile;

    // Block ids of the range in windows of 64 (lane i: block b_lo + wbase +
    // i), the next window requested one window ahead, so a tile reads its
    // block id from a register instead of waiting on a table load.
    const int b_lo = t_begin / p.bs;
    const int nbk = t_end > t_begin ? (t_end - 1) / p.bs - b_lo + 1 : 0;   // blocks in range
    int wbase = 0;
    int bw = lane < nbk ? blocks[b_lo + lane] : -1;
    int bw_next = lane + 64 < nbk ? blocks[b_lo + 64 + lane] : -1;

    for (int t = t_first + wave; t < t_last; t += W) {
        const int tok0 = t * kTile;
        const int b = tok0 / p.bs;
        const int slot0 = tok0 - b * p.bs;
        while (b - b_lo - wbase >= 64) {   // wave-uniform; once per 64 blocks
            wbase += 64;
            bw = bw_next;
            bw_next = lane + wbase + 64 < nbk ? blocks[b_lo + wbase + 64 + lane] : -1;
        }
        const int blk = __builtin_amdgcn_readlane(bw, b - b_lo - wbase);
        if ((uint32_t)blk >= p.num_blocks) continue;  // dropped: never dereferenced
        const int nvalid = min(kTile, t_end - tok0);
        const char* kblk = kbase + ((int64_t)blk * p.blk_s + (int64_t)slot0 * p.tok_s) * EB;
        const char* vblk = vbase + ((int64_t)blk * p.blk_s + (int64_t)slot0 * p.tok_s) * EB;

        // K as the A operand (lane = token c); a masked token re-reads the
        // tile's first row, so canary memory never enters the arithmetic
        const int tk = c < nvalid ? c : 0;
        bf16x8_t ka[8];
        if constexpr (KV8) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const u32x4_t x = load16<!SPLIT>(kblk + tk * tok_b + 64 * j + 16 * g);
                ka[2 * j] = __builtin_bit_cast(bf16x8_t, fp8x8_to_bf16(x[0], x[1]));
                ka[2 * j + 1] = __builtin_bit_cast(bf16x8_t, fp8x8_to_bf16(x[2], x[3]));
            }
        } else {
#pragma unroll
            for (int kb = 0; kb < 8; ++kb)
                ka[kb] = __builtin_bit_cast(
                    bf16x8_t, load16<!SPLIT>(kblk + tk * tok_b + 2 * kdim<KV8>(kb, g)));
        }
        // V rows in natural order: BF16 load i covers tokens 2i and 2i + 1
        // (8 dims a lane), FP8 load i tokens 4i .. 4i + 3 (16 dims a lane)
        constexpr int NV = KV8 ? 4 : 8;
        u32x4_t vr[NV];
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int row = KV8 ? 4 * i + (lane >> 4) : 2 * i + (lane >> 5);
            const int tv = row < nvalid ? row : 0;
            const int col_b = KV8 ? (lane & 15) * 16 : (lane & 31) * 16;
            vr[i] = load16<!SPLIT>(vblk + tv * tok_b + col_b);
        }

        // S^T = K . Q^T ; acc[r] = score of token 4g + r for head c
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < 8; ++kb)
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[kb], qb[kb], acc, 0, 0, 0);

        float s[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) s[r] = 4 * g + r < nvalid ? acc[r] * p.c : kNegInf;
        const float tmax = group_max(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])));
        const float mn = fmaxf(m, tmax);
        const float ms = mn == kNegInf ? 0.f : mn;
        const float alpha = fexp2(m - ms);
        const bool grow = mn != m;
        m = mn;
        float pr[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) pr[r] = c < kG ? fexp2(s[r] - ms) : 0.f;
        l = l * alpha + group_sum((pr[0] + pr[1]) + (pr[2] + pr[3]));

        // P as the A operand: lane = head c, tokens 4g .. 4g + 3 (in place)
        const s16x4_t pa = __builtin_bit_cast(
            s16x4_t, uint64_t(pack_bf16x2(pr[0], pr[1])) | (uint64_t(pack_bf16x2(pr[2], pr[3])) << 32));

        // V tile -> LDS (swizzled rows), then rescale o while the writes land
        if constexpr (KV8) {
            // dims 16 q .. 16 q + 15 (q = lane & 15) are chunks 4q .. 4q + 3,
            // which the swizzle keeps contiguous (it flips chunk bits 2..4)
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                const int row = 4 * i + (lane >> 4);
                uint16_t* dst = vt + vchunk(row, 4 * (lane & 15));
                *reinterpret_cast<u32x4_t*>(dst) = fp8x8_to_bf16(vr[i][0], vr[i][1]);
                *reinterpret_cast<u32x4_t*>(dst + 8) = fp8x8_to_bf16(vr[i][2], vr[i][3]);
            }
        } else {
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                const int row = 2 * i + (lane >> 5);
                *reinterpret_cast<u32x4_t*>(vt + vchunk(row, 2 * (lane & 31))) = vr[i];
            }
        }
        if (__builtin_amdgcn_ballot_w64(grow) != 0) {
            // O rows are heads 4g + r; their factor lives in lane 4g + r
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float a = __int_as_float(
                    __builtin_amdgcn_ds_bpermute((4 * g + r) * 4, __float_as_int(alpha)));
#pragma unroll
                for (int nb = 0; nb < 16; ++nb) O[nb][r] *= a;
            }
        }
        wave_lds_sync();

        // O += P . V, 16 output dims at a time; V^T read transposed from LDS:
        // lane c of group g addresses row 4g + c/4, chunk 4 nb + c%4
        const int trow = 4 * g + (c >> 2);
#pragma unroll
        for (int nb = 0; nb < 16; ++nb) {
            typedef __attribute__((address_space(3))) s16x4_t* lds_s16x4_p;
            const uint16_t* src = vt + vchunk(trow, 4 * nb + (c & 3));
            const s16x4_t vb = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_s16x4_p)(__attribute__((address_space(3))) uint16_t*)src);
            O[nb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa, vb, O[nb], 0, 0, 0);
        }
        wave_lds_sync();  // the next tile overwrites this wave's V tile
    }

    if constexpr (KV8) {   // V = decode(v) * v_scale: scale o once
#pragma unroll
        for (int nb = 0; nb < 16; ++nb)
#pragma unroll
            for (int r = 0; r < 4; ++r) O[nb][r] *= p.v_scale;
    }

    // Merge the waves in order.  LDS (reusing the V tiles): per wave and
    // real head m and l, then o for one half of the dims at a time.
    __syncthreads();
    float* ml = reinterpret_cast<float*>(smem);                 // [W][8][2]
    float* ow = ml + W * kG * 2;                           // [W][8][128]
    if (g == 0 && c < kG) {
        ml[(wave * kG + c) * 2] = m;
        ml[(wave * kG + c) * 2 + 1] = l;
    }
    __syncthreads();
    // per head: max, weights, L (every thread computes the 8 heads' values
    // it needs; cheap at 8 waves)
    for (int half = 0; half < 2; ++half) {
        // waves write the real heads' o (groups 0 and 1 hold heads 0..7)
        if (g < 2) {
#pragma unroll
            for (int nb = 0; nb < 8; ++nb)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    ow[(wave * kG + 4 * g + r) * 128 + nb * 16 + c] = O[half * 8 + nb][r];
        }
        __syncthreads();
        for (int i = tid; i < kG * 64; i += 64 * W) {
            const int h = i / 64, d2 = (i % 64) * 2;     // two dims of this half
            float M = kNegInf;
            for (int w = 0; w < W; ++w) M = fmaxf(M, ml[(w * kG + h) * 2]);
            const float Ms = M == kNegInf ? 0.f : M;
            float Lsum = 0.f, o0 = 0.f, o1 = 0.f;
            for (int w = 0; w < W; ++w) {
                const float wt = fexp2(ml[(w * kG + h) * 2] - Ms);
                Lsum += wt * ml[(w * kG + h) * 2 + 1];
                o0 += wt * ow[(w * kG + h) * 128 + d2];
                o1 += wt * ow[(w * kG + h) * 128 + d2 + 1];
            }
            if constexpr (SPLIT) {
                float* slot = p.ws + ((q_row + h) * p.nsplit + sp) * (int64_t)(kD + 2);
                if (Lsum > 0.f)
                    *reinterpret_cast<float2*>(slot + half * 128 + d2) = make_float2(o0, o1);
                if (half == 0 && d2 == 0) {
                    slot[kD] = M * kLn2;
                    slot[kD + 1] = Lsum;
                }
            } else if (PARTS && P > 1) {
                float* rec = g_packed_sub +
                             ((int64_t)blockIdx.y * p.nkv * PL + blockIdx.x) * kPackedRec;
                put_dev(rec + h * kD + half * 128 + d2, o0);
                put_dev(rec + h * kD + half * 128 + d2 + 1, o1);
                if (half == 0 && d2 == 0) {
                    put_dev(rec + kG * kD + h, M);
                    put_dev(rec + kG * kD + kG + h, Lsum);
                }
            } else {
                const uint32_t v = Lsum > 0.f ? pack_bf16x2(o0 / Lsum, o1 / Lsum) : 0u;
                *reinterpret_cast<uint32_t*>(p.out + (q_row + h) * kD + half * 128 + d2) = v;
            }
        }
        __syncthreads();
    }

    if (PARTS && P > 1) {
        // take a ticket; the last part combines the records in part order
        // (max over parts with l > 0, weights exp2(m_i - M), weighted sums of
        // l and o), so the bytes do not depend on arrival order
        const int64_t item = (int64_t)blockIdx.y * p.nkv + kvh;
        uint32_t* const tick = g_packed_tick + item;
        uint32_t* const eT = reinterpret_cast<uint32_t*>(smem);
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
        const float* const recs = g_packed_sub + item * PL * kPackedRec;
        float* const cw = reinterpret_cast<float*>(smem) + 4;   // weights [part][head]
        float* const cL = cw + kMaxParts * kG;                   // L [head]
        if (tid < kG) {
            const int h = tid;
            float mv[kMaxParts], lv[kMaxParts];
#pragma unroll
            for (int i = 0; i < kMaxParts; ++i) {
                const int ii = i < P ? i : P - 1;
                mv[i] = get_dev(recs + ii * kPackedRec + kG * kD + h);
                lv[i] = get_dev(recs + ii * kPackedRec + kG * kD + kG + h);
            }
            float M = kNegInf;
#pragma unroll
            for (int i = 0; i < kMaxParts; ++i)
                if (i < P && lv[i] > 0.f) M = fmaxf(M, mv[i]);
            const float Ms = M == kNegInf ? 0.f : M;
            float Lsum = 0.f;
#pragma unroll
            for (int i = 0; i < kMaxParts; ++i) {
                if (i < P) {
                    const float wt = lv[i] > 0.f ? fexp2(mv[i] - Ms) : 0.f;
                    cw[i * kG + h] = wt;
                    Lsum += wt * lv[i];
                }
            }
            cL[h] = Lsum;
        }
        __syncthreads();
        for (int i = tid; i < kG * (kD / 2); i += 64 * W) {
            const int h = i / (kD / 2), d = (i % (kD / 2)) * 2;
            float o0 = 0.f, o1 = 0.f;
            for (int c2 = 0; c2 < P; ++c2) {
                const float wt = cw[c2 * kG + h];
                if (wt != 0.f) {   // a part that folded nothing is never read
                    const float* x = recs + c2 * kPackedRec + h * kD + d;
                    o0 += wt * get_dev(x);
                    o1 += wt * get_dev(x + 1);
                }
            }
            const float Lsum = cL[h];
            const uint32_t v = Lsum > 0.f ? pack_bf16x2(o0 / Lsum, o1 / Lsum) : 0u;
            *reinterpret_cast<uint32_t*>(p.out + (q_row + h) * kD + d) = v;
        }
    }
}

template <bool KV8>
hipError_t launch_packed_t(const PackedParams& p, uint32_t num_seqs, hipStream_t stream) {
    if (p.nsplit > 1) {
        // A split holds about 1/nsplit of a sequence: the more splits, the
        // fewer tiles each item has, and the fewer waves pay off (measured
        // on 64 sequences of 1K-8K tokens: 2 waves best at 16 splits, 4 at
        // 4-8, 8 at 2).  Results do not depend on the wave count choice
        // beyond the order of the final in-workgroup merge.
        const dim3 grid((uint32_t)(p.nkv * p.nsplit), num_seqs);
        const int w = p.nsplit >= 12 ? 2 : (p.nsplit >= 3 ? 4 : 8);
        const size_t lds = sizeof(uint16_t) * (size_t)w * kVTileElems;
        if (w == 2)
            hipLaunchKernelGGL((packed_kernel<true, 2, KV8, false>), grid, dim3(128), lds, stream, p);
        else if (w == 4)
            hipLaunchKernelGGL((packed_kernel<true, 4, KV8, false>), grid, dim3(256), lds, stream, p);
        else
            hipLaunchKernelGGL((packed_kernel<true, 8, KV8, false>), grid, dim3(512), lds, stream, p);
    } else if (p.parts > 1) {
        // PDA_PACKED_PARTS_WAVES waves per part workgroup
        if (p.parts > kMaxParts || (uint64_t)num_seqs * p.nkv > kPartTickets ||
            (uint64_t)num_seqs * p.nkv * p.parts * kPackedRec > kPartSubFloats)
            return hipErrorInvalidValue;
        constexpr int w = PDA_PACKED_PARTS_WAVES;
        const size_t lds = sizeof(uint16_t) * (size_t)w * kVTileElems;
        hipLaunchKernelGGL((packed_kernel<false, w, KV8, true>),
                           dim3((uint32_t)(p.nkv * p.parts), num_seqs), dim3(64 * w), lds, stream, p);
    } else {
        const size_t lds = sizeof(uint16_t) * (size_t)kWaves * kVTileElems;   // 64 KiB
        hipLaunchKernelGGL((packed_kernel<false, kWaves, KV8, false>), dim3((uint32_t)p.nkv, num_seqs),
                           dim3(64 * kWaves), lds, stream, p);
    }
    return hipGetLastError();
}

}  // namespace

uint32_t packed_part_rows(uint32_t nkv, int parts) {
    const uint64_t by_tick = kPartTickets / nkv;
    const uint64_t by_sub = kPartSubFloats / ((uint64_t)nkv * parts * kPackedRec);
    const uint64_t r = by_tick < by_sub ? by_tick : by_sub;
    return r > 0xFFFFFFFFull ? 0xFFFFFFFFu : (uint32_t)r;
}

hipError_t launch_packed(const PackedParams& p, uint32_t num_seqs, hipStream_t stream,
                         bool kv8) {
    return kv8 ? launch_packed_t<true>(p, num_seqs, stream)
               : launch_packed_t<false>(p, num_seqs, stream);
}

}  // namespace pda
