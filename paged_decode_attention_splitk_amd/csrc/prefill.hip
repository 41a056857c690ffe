// Causal paged prefill attention on MFMA (gfx950), head_dim 256.
//
// The launch shape follows the prefill page ("metrale_model_layers/layers/
// ops/prefill_attn_fa128.rs", the paged launcher and its constants): grid
// [num_q_heads, ceil(q_len / 128)], 128 query rows per workgroup, K and V
// tiles of 32 rows staged in LDS and read once per 128 rows, P kept in
// registers, every wave doing both q.k and P.V.  Here a workgroup is 8 waves
// of 16 query rows (wave64), and the arithmetic is laid out for CDNA4:
//
//   S^T[16 key][16 query] = K[16][256] . Q^T[256][16]
//       8 x v_mfma_f32_16x16x32_bf16; K (A operand: lane = key, 8 dims) comes
//       from the LDS tile, Q (B operand: lane = query) stays in registers.
//   online softmax (FP32, base 2) on the accumulator: each query's 16
//       scores sit in one column across the four 16-lane groups; the causal
//       mask and the end of the cache turn scores into -inf there.
//   O[16 query][256] += P[16][32] . V[32][256] per 32-key tile
//       16 x v_mfma_f32_16x16x32_bf16; the two S^T accumulators of the tile
//       are P in the A-operand layout (lane = query, k index 8g + t = key
//       4g + t of the first block or 4g + t - 4 of the second), and the B
//       operand takes V in the same k order from two ds_read_b64_tr_b16
//       transposed reads of the LDS tile.
//
// Query row i is the token at position q_offset + i and attends the keys at
// positions j <= q_offset + i with j < kv_len.  K / V rows past kv_len, or in
// a block whose id is outside the pool, are staged from key 0 instead (their
// scores are masked, so p = 0 meets a finite value), so canary memory never
// enters the arithmetic (a dropped block inside the cache gives unspecified
// but in-bounds results).  A row with no key writes 0.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pda_geometry.h"
#include "pda_kernels.h"

namespace pda {
namespace {

constexpr float kNegInf = -__builtin_inff();
constexpr int kD = 256;           // head dim
// compiled for the head dim the host gate (pda_prefill_applies) accepts
static_assert(kD == (int)kPrefillHeadDim, "prefill kernel head dim differs from its gate");
#ifndef PDA_PREFILL_WAVES
#define PDA_PREFILL_WAVES 8
#endif
constexpr int kWaves = PDA_PREFILL_WAVES;   // 16 query rows each
constexpr int kRows = 16 * kWaves;          // query rows per workgroup
constexpr int kKT = 32;           // keys per staged tile (two 16-key blocks)
#ifndef PDA_PREFILL_LAZY
#define PDA_PREFILL_LAZY 8
#endif
constexpr float kLazy = PDA_PREFILL_LAZY;   // running-max slack, log2 units (p <= 2^kLazy)
#ifndef PDA_PREFILL_XCD
#define PDA_PREFILL_XCD 1
#endif
constexpr int kThreads = 64 * kWaves;
constexpr int kTileElems = kKT * kD;          // one K (or V) tile: 16 KiB
constexpr int kChunksPerThread = kKT * (kD / 8) / kThreads;   // 16-byte pieces
static_assert(kChunksPerThread * kThreads == kKT * (kD / 8), "threads divide a tile's pieces");

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

// Max / sum over the four 16-lane groups (lanes c, c + 16, c + 32, c + 48);
// every lane of the set gets identical bits.
__device__ __forceinline__ float group_max(float x) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
    r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float group_sum(float x) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// K tile: row r's 16-byte piece j (dims 8j .. 8j + 7) sits at piece j ^ (r & 15),
// so the 16 rows one A-operand read touches land in 16 distinct bank groups.
__device__ __forceinline__ int kpiece(int row, int piece) {
    return row * kD + ((piece ^ (row & 15)) << 3);
}
// V tile (per 16-row key block): 8-byte chunks XOR-swizzled by 4 * (row & 7),
// so the transposed reads are free of bank conflicts.
__device__ __forceinline__ int vchunk(int row, int chunk) {
    return row * kD + ((chunk ^ ((row & 7) << 2)) << 2);
}

// UNIFORM: the block size is a multiple of 16 (see the staging below).
template <bool UNIFORM>
__global__ __launch_bounds__(kThreads, 1) void prefill_kernel(const PrefillParams p) {
    extern __shared__ __align__(16) uint16_t smem[];   // 2 x (K tile, V tile)
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, c = lane & 15;
    // Workgroup ids go to the 8 XCDs round-robin (id % 8).  When the head
    // count is a multiple of 8, XCD x takes the consecutive heads
    // x * nq/8 .. x * nq/8 + nq/8 - 1, which share KV heads, so each XCD's
    // L2 holds the K/V of one or two KV heads instead of all of them.  Only
    // the placement changes.
    const int h = PDA_PREFILL_XCD && p.nq % 8 == 0
                      ? ((int)blockIdx.x % 8) * (p.nq / 8) + (int)blockIdx.x / 8
                      : (int)blockIdx.x;
    const int kvh = h / (p.nq / p.nkv);
    // row tiles are taken last (longest causal range) first
    const int n_tiles_q = (p.q_len + kRows - 1) / kRows;
    const int r0 = (n_tiles_q - 1 - (int)blockIdx.y) * kRows;
    const int row_end = min(r0 + kRows, p.q_len);
    // keys this workgroup needs: up to its last row's position
    const int n_keys = min(p.kv_len, p.q_offset + row_end);
    const int n_tiles = (n_keys + kKT - 1) / kKT;

    const int wr0 = r0 + wave * 16;                 // this wave's first row
    const int qrow = min(wr0 + c, p.q_len - 1);     // the query row of lane c
    const int qpos = p.q_offset + wr0 + c;          // its position
    const int wave_last_pos = p.q_offset + wr0 + 15;
    const int wave_first_pos = p.q_offset + wr0;
    const int64_t row_s = (int64_t)p.nq * kD;       // elements between query rows

    // Q as the B operand: lane = query c, 8 dims 32 kb + 8 g of k-step kb
    bf16x8_t qb[8];
#pragma unroll
    for (int kb = 0; kb < 8; ++kb)
        qb[kb] = __builtin_bit_cast(
            bf16x8_t, *reinterpret_cast<const u32x4_t*>(p.q + qrow * row_s + (int64_t)h * kD +
                                                        kb * 32 + g * 8));

    f32x4_t O[16];   // O[query 4g + r][dim 16 nb + c]
#pragma unroll
    for (int nb = 0; nb < 16; ++nb) O[nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // m: the reference max of query c (the same in all four lane groups);
    // l: this lane's part of query c's sum, the groups' parts added at the end
    float m = kNegInf, l = 0.f;

    const uint16_t* kbase = p.k + (int64_t)kvh * kD;
    const uint16_t* vbase = p.v + (int64_t)kvh * kD;
    // the pool row of key j, or of key 0 for a key past the cache or in a
    // block outside the pool (its scores are masked); bj = table entry of
    // key j's block (read for key 0 past the cache), b0 = table entry 0
    auto key_row = [&](int j, int bj, int b0) -> int64_t {
        const bool ok = j < p.kv_len && (uint32_t)bj < p.num_blocks;
        const int blk = ok ? bj : ((uint32_t)b0 < p.num_blocks ? b0 : 0);   // (any in-pool block)
        return (int64_t)blk * p.blk_s + (int64_t)((ok ? j : 0) % p.bs) * p.tok_s;
    };
    // staging: thread t moves 16-byte pieces t + kThreads * i of the tile
    // (row = idx / 32, piece = idx % 32) for K and for V
    typedef u32x4_t Stage[2][kChunksPerThread];   // K, V pieces of one tile
    // Table entries.  With a block size that is a multiple of 16 (UNIFORM),
    // the 16 rows a thread's piece i lies in (rows 16 i .. 16 i + 15 of the
    // tile) sit in one block, since tiles start on a multiple of 32, so
    // those entries are the same for the whole workgroup: they are read one
    // tile ahead of the loads that use them (key kv_len - 1 stands in past
    // the cache), and a piece's address is a workgroup-uniform base plus the
    // thread's constant byte offset, so staging a tile costs no vector
    // arithmetic.  Other block sizes read each piece's entry with the tile's
    // loads, every table read of the tile first, with no branch between
    // them, so they are waited for once.
    static_assert(kThreads == 512 && kChunksPerThread == 2, "piece i covers rows 16 i .. 16 i + 15");
    auto tbl_half = [&](int tile, int i) {
        return UNIFORM ? p.table[min(tile * kKT + 16 * i, p.kv_len - 1) / p.bs] : 0;
    };
    const int b0 = p.table[0];
    // the thread's bytes inside its 16-row run: row tid / 32, piece tid % 32
    const uint32_t lane_b = (uint32_t)(((tid >> 5) * p.tok_s + (tid & 31) * 8) * 2);
    auto stage_load = [&](int tile, Stage& st, const int (&bt)[2]) {
        if constexpr (UNIFORM) {
#pragma unroll
            for (int i = 0; i < kChunksPerThread; ++i) {
                // a block outside the pool inside the cache (unspecified
                // result) reads rows of the first block instead
                const int j0 = tile * kKT + 16 * i;
                const bool ok = (uint32_t)bt[i] < p.num_blocks;
                const int blk = ok ? bt[i] : ((uint32_t)b0 < p.num_blocks ? b0 : 0);
                const int64_t ub =
                    ((int64_t)blk * p.blk_s + (int64_t)(ok ? j0 % p.bs : 0) * p.tok_s) * 2;
                st[0][i] = *reinterpret_cast<const u32x4_t*>(
                    reinterpret_cast<const char*>(kbase) + ub + lane_b);
                st[1][i] = *reinterpret_cast<const u32x4_t*>(
                    reinterpret_cast<const char*>(vbase) + ub + lane_b);
            }
            if (tile * kKT + kKT > p.kv_len) {
                // rows past the cache (read from inside the last block) are
                // zeroed: their scores are masked and p = 0 meets 0
#pragma unroll
                for (int i = 0; i < kChunksPerThread; ++i)
                    if (tile * kKT + 16 * i + (tid >> 5) >= p.kv_len)
                        st[0][i] = st[1][i] = u32x4_t{0u, 0u, 0u, 0u};
            }
        } else {
            int jr[kChunksPerThread], bj[kChunksPerThread];
#pragma unroll
            for (int i = 0; i < kChunksPerThread; ++i) {
                jr[i] = tile * kKT + ((tid + kThreads * i) >> 5);
                bj[i] = p.table[(jr[i] < p.kv_len ? jr[i] : 0) / p.bs];
            }
#pragma unroll
            for (int i = 0; i < kChunksPerThread; ++i) {
                const int64_t off = key_row(jr[i], bj[i], b0) + ((tid + kThreads * i) & 31) * 8;
                st[0][i] = *reinterpret_cast<const u32x4_t*>(kbase + off);
                st[1][i] = *reinterpret_cast<const u32x4_t*>(vbase + off);
            }
        }
    };
    auto stage_store = [&](int buf, const Stage& st) {
        uint16_t* kt = smem + buf * 2 * kTileElems;
        uint16_t* vt = kt + kTileElems;
#pragma unroll
        for (int i = 0; i < kChunksPerThread; ++i) {
            const int idx = tid + kThreads * i;
            const int row = idx >> 5, piece = idx & 31;
            *reinterpret_cast<u32x4_t*>(kt + kpiece(row, piece)) = st[0][i];
            *reinterpret_cast<u32x4_t*>(vt + (row >> 4) * 16 * kD + vchunk(row & 15, 2 * piece)) =
                st[1][i];
        }
    };
    Stage ra, rb;   // tile j's pieces live in (j even ? ra : rb) from load to store

    int tb[2] = {0, 0};   // table entries of the next tile to load
    if (n_tiles > 0) {
        const int t0[2] = {tbl_half(0, 0), tbl_half(0, 1)};
        stage_load(0, ra, t0);
        stage_store(0, ra);
        if (n_tiles > 1) {
            const int t1[2] = {tbl_half(1, 0), tbl_half(1, 1)};
            stage_load(1, rb, t1);
        }
        if (n_tiles > 2) {
            tb[0] = tbl_half(2, 0);
            tb[1] = tbl_half(2, 1);
        }
    }
    __syncthreads();

    // tile t: loads of tile t + 2 go out (into the registers tile t held),
    // tile t computes, tile t + 1 (loaded an iteration earlier) goes to LDS
    auto body = [&](int t, Stage& cur, Stage& nxt) {
        const int buf = t & 1;
        if (t + 2 < n_tiles) stage_load(t + 2, cur, tb);
        if (t + 3 < n_tiles) {
            tb[0] = tbl_half(t + 3, 0);
            tb[1] = tbl_half(t + 3, 1);
        }
        const uint16_t* kt = smem + buf * 2 * kTileElems;
        const uint16_t* vt = kt + kTileElems;
        const int key0 = t * kKT;
        // wave-uniform: the tile (or its second 16-key block) lies past every
        // row of this wave, or past the cache
        if (key0 <= wave_last_pos && key0 < p.kv_len) {
            const bool live1 = key0 + 16 <= wave_last_pos && key0 + 16 < p.kv_len;
            // S^T = K . Q^T over the 256 dims, both 16-key blocks interleaved.
            // Every K fragment of the tile is requested before the first
            // MFMA, each into registers of its own, so the LDS reads overlap
            // one another instead of each waiting for the MFMA before it.
            f32x4_t acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
            bf16x8_t ka0[8], ka1[8];
#pragma unroll
            for (int kb = 0; kb < 8; ++kb)
                ka0[kb] = __builtin_bit_cast(
                    bf16x8_t, *reinterpret_cast<const u32x4_t*>(kt + kpiece(c, 4 * kb + g)));
            if (live1) {
#pragma unroll
                for (int kb = 0; kb < 8; ++kb)
                    ka1[kb] = __builtin_bit_cast(
                        bf16x8_t,
                        *reinterpret_cast<const u32x4_t*>(kt + kpiece(16 + c, 4 * kb + g)));
#pragma unroll
                for (int kb = 0; kb < 8; ++kb) {
                    acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka0[kb], qb[kb], acc0, 0, 0, 0);
                    acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka1[kb], qb[kb], acc1, 0, 0, 0);
                }
            } else {
#pragma unroll
                for (int kb = 0; kb < 8; ++kb)
                    acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka0[kb], qb[kb], acc0, 0, 0, 0);
            }
            // V fragments of the first 8 dim blocks, requested now (they do
            // not depend on P), so their LDS reads overlap the softmax: the
            // transposed reads of the two 16-key blocks (lane c of group g
            // addresses row 4g + c/4, chunk 4 nb + c%4) give keys 4g .. 4g + 3
            // of each, in the k order of P below
            typedef __attribute__((address_space(3))) s16x4_t* lds_s16x4_p;
            const int trow = 4 * g + (c >> 2);
            auto vread = [&](int nb, int blk) {
                const uint16_t* src = vt + vchunk(trow, 4 * nb + (c & 3)) + blk * 16 * kD;
                return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_s16x4_p)(__attribute__((address_space(3))) uint16_t*)src);
            };
            s16x4_t vv0[8], vv1[8];
#pragma unroll
            for (int nb = 0; nb < 8; ++nb) {
                vv0[nb] = vread(nb, 0);
                vv1[nb] = vread(nb, 1);
            }
            // one softmax step over the tile's 32 keys; acc_b[r]: key
            // key0 + 16 b + 4g + r, query c
            float s[8];
            if (key0 + kKT - 1 <= wave_first_pos && key0 + kKT <= p.kv_len) {
                // every key of the tile is visible to every row of the wave
                // (so both 16-key blocks were computed)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    s[r] = acc0[r] * p.c;
                    s[4 + r] = acc1[r] * p.c;
                }
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int k0 = key0 + 4 * g + r, k1 = k0 + 16;
                    s[r] = k0 <= qpos && k0 < p.kv_len ? acc0[r] * p.c : kNegInf;
                    s[4 + r] = live1 && k1 <= qpos && k1 < p.kv_len ? acc1[r] * p.c : kNegInf;
                }
            }
            float lmax = s[0];
#pragma unroll
            for (int i = 1; i < 8; ++i) lmax = fmaxf(lmax, s[i]);
            // The reference max m moves only when a score passes it by more
            // than kLazy (log2 units), so p <= 2^kLazy and O is rescaled far
            // less often; O and l share the reference, so O / l is the same
            // up to rounding.  The max over the four lane groups is taken
            // only when some lane's own scores pass the slack.
            bool grow = false;   // m = -inf: any finite score grows it
            float alpha = 1.f;
            if (__builtin_amdgcn_ballot_w64(lmax > m + kLazy) != 0) {
                const float tmax = group_max(lmax);
                grow = tmax > m + kLazy;
                if (grow) {
                    alpha = m == kNegInf ? 0.f : fexp2(m - tmax);
                    m = tmax;
                }
            }
            const float ms = m == kNegInf ? 0.f : m;
            float pr[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) pr[i] = fexp2(s[i] - ms);
            // this lane's part of l (its own keys of the tile); the four
            // groups' parts are added once, after the last tile
            l = l * alpha + (((pr[0] + pr[1]) + (pr[2] + pr[3])) + ((pr[4] + pr[5]) + (pr[6] + pr[7])));
            // P as the A operand of a 32-key step: lane = query c, k index
            // 8g + t = key 4g + t of block 0 (t < 4) or of block 1 (t >= 4)
            const u32x4_t pw = {pack_bf16x2(pr[0], pr[1]), pack_bf16x2(pr[2], pr[3]),
                                pack_bf16x2(pr[4], pr[5]), pack_bf16x2(pr[6], pr[7])};
            const bf16x8_t pa = __builtin_bit_cast(bf16x8_t, pw);
            if (__builtin_amdgcn_ballot_w64(grow) != 0) {
                // O rows are queries 4g + r; their factor lives in lane 4g + r
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float a = __int_as_float(
                        __builtin_amdgcn_ds_bpermute((4 * g + r) * 4, __float_as_int(alpha)));
#pragma unroll
                    for (int nb = 0; nb < 16; ++nb) O[nb][r] *= a;
                }
            }
            // O += P . V with the same k order on the B side; the second 8
            // dim blocks' fragments are requested as the first 8 are used
#pragma unroll
            for (int nb = 0; nb < 8; ++nb) {
                const bf16x8_t vb = __builtin_bit_cast(
                    bf16x8_t, __builtin_shufflevector(vv0[nb], vv1[nb], 0, 1, 2, 3, 4, 5, 6, 7));
                O[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, vb, O[nb], 0, 0, 0);
                vv0[nb] = vread(nb + 8, 0);
                vv1[nb] = vread(nb + 8, 1);
            }
#pragma unroll
            for (int nb = 0; nb < 8; ++nb) {
                const bf16x8_t vb = __builtin_bit_cast(
                    bf16x8_t, __builtin_shufflevector(vv0[nb], vv1[nb], 0, 1, 2, 3, 4, 5, 6, 7));
                O[nb + 8] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, vb, O[nb + 8], 0, 0, 0);
            }
        }
        if (t + 1 < n_tiles) stage_store(buf ^ 1, nxt);
        __syncthreads();
    };
    for (int t = 0; t < n_tiles; t += 2) {
        body(t, ra, rb);
        if (t + 1 < n_tiles) body(t + 1, rb, ra);
    }

    // out = O / l (0 where l is 0), rows 4g + r of this wave
    l = group_sum(l);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const float L =
            __int_as_float(__builtin_amdgcn_ds_bpermute((4 * g + r) * 4, __float_as_int(l)));
        const int row = wr0 + 4 * g + r;
        if (row >= p.q_len) continue;
        const float inv = L > 0.f ? 1.f / L : 0.f;
        uint16_t* dst = p.out + row * row_s + (int64_t)h * kD + c;
#pragma unroll
        for (int nb = 0; nb < 16; ++nb) {
            const __bf16 b = (__bf16)(L > 0.f ? O[nb][r] * inv : 0.f);
            dst[nb * 16] = __builtin_bit_cast(uint16_t, b);
        }
    }
}

}  // namespace

hipError_t launch_prefill(const PrefillParams& p, hipStream_t stream) {
    const size_t lds = sizeof(uint16_t) * 4 * (size_t)kTileElems;   // 2 x (K, V) tiles
    static_assert(sizeof(uint16_t) * 4 * (size_t)kTileElems <= 64 * 1024,
                  "the staged tiles fit the default LDS limit of a workgroup");
    const dim3 grid((uint32_t)p.nq, (uint32_t)((p.q_len + kRows - 1) / kRows));
    if (p.bs % 16 == 0)
        hipLaunchKernelGGL(prefill_kernel<true>, grid, dim3(kThreads), lds, stream, p);
    else
        hipLaunchKernelGGL(prefill_kernel<false>, grid, dim3(kThreads), lds, stream, p);
    return hipGetLastError();
}

}  // namespace pda
