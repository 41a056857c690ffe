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
// Work layout inside a workgroup (W waves):
//   * A K/V row of one token and one KV head is head_dim BF16 values.  LPT
//     lanes share it (16 lanes for head_dim 64/128, 32 lanes for 256), each
//     holding DPL = head_dim / LPT consecutive values, so one wave-wide
//     vector load fetches ROWS = 64 / LPT token rows of 16-byte pieces.
//   * Every lane keeps the q slices of all GC query heads of its KV head, so
//     each K/V byte is read from HBM once and used by all GC heads straight
//     from registers; no LDS staging is needed on the hot loop.
//   * q.k is a chain of v_dot2_f32_bf16 over the lane's slice followed by a
//     fixed DPP butterfly (quad xor 1, quad xor 2, half-row mirror, row
//     mirror, and a permlane16 swap at 32 lanes), which leaves the same
//     bits in every lane of the token row.
//   * Each token row keeps its own (m, l, o) per head; tokens arrive in
//     groups of TG = ROWS * U (one scalar block-table load per group), and a
//     group updates the state once: new max, one rescale, U exponentials.
//   * Waves take groups round-robin; at the end the rows of a wave are
//     merged with permlane swaps and the waves through LDS, always in the
//     same order, so the result depends only on the sequence's own data and
//     the launch shape, never on the rest of the batch.
// Exponentials are v_exp_f32 (base 2): scores are scaled by scale * log2(e)
// and m is converted back to natural-log units when it is stored.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pda_geometry.h"
#include "pda_kernels.h"

namespace pda {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c, false);
}
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    bf16x2_t v;
    v[0] = (__bf16)a;
    v[1] = (__bf16)b;
    return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __int_as_float(
        __builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Values of the even and the odd 16-lane row of this lane's row pair.
__device__ __forceinline__ void rows16(float x, float& even, float& odd) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                              false);
    even = __uint_as_float(r[0]);
    odd = __uint_as_float(r[1]);
}
// Values of the lower and the upper 32-lane half of the wave.
__device__ __forceinline__ void rows32(float x, float& lo, float& hi) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                              false);
    lo = __uint_as_float(r[0]);
    hi = __uint_as_float(r[1]);
}

// Sum over the LPT lanes of a token row; every lane gets identical bits.
template <int LPT>
__device__ __forceinline__ float row_sum(float x) {
    static_assert(LPT == 8 || LPT == 16 || LPT == 32, "lanes per token row");
    x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]
    x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]
    x += dpp<0x141>(x);  // row_half_mirror
    if constexpr (LPT >= 16) x += dpp<0x140>(x);  // row_mirror
    if constexpr (LPT >= 32) {
        float e, o;
        rows16(x, e, o);
        x = e + o;
    }
    return x;
}

template <int N>
__device__ __forceinline__ void load_words(uint32_t (&d)[N], const uint16_t* p) {
    static_assert(N == 2 || N == 4, "16- or 8-byte pieces");
    if constexpr (N == 4) {
        const uint4 x = *reinterpret_cast<const uint4*>(p);
        d[0] = x.x; d[1] = x.y; d[2] = x.z; d[3] = x.w;
    } else {
        const uint2 x = *reinterpret_cast<const uint2*>(p);
        d[0] = x.x; d[1] = x.y;
    }
}

template <int D>
struct FoldShape {
    static constexpr int LPT = D == 256 ? 32 : 16;  // lanes per token row
    static constexpr int DPL = D / LPT;             // values per lane
    static constexpr int VEC = DPL / 2;             // 32-bit words per lane
    static constexpr int ROWS = 64 / LPT;           // token rows per wave load
    static constexpr int U = 4;                     // tokens per lane per group
    static constexpr int TG = ROWS * U;             // tokens per group
    static_assert(kBlockQuantum % TG == 0, "a block holds whole groups");
};

// Merge the states of this lane's row with the partner row (XOR 16 or 32).
template <int X, int GC, int DPL>
__device__ __forceinline__ void merge_rows(float (&m)[GC], float (&l)[GC], float (&o)[GC][DPL]) {
#pragma unroll
    for (int h = 0; h < GC; ++h) {
        float ma, mb, la, lb;
        if constexpr (X == 16) { rows16(m[h], ma, mb); rows16(l[h], la, lb); }
        else { rows32(m[h], ma, mb); rows32(l[h], la, lb); }
        const float M = fmaxf(ma, mb);
        const float Ms = M == kNegInf ? 0.f : M;
        const float wa = fexp2(ma - Ms), wb = fexp2(mb - Ms);
        m[h] = M;
        l[h] = wa * la + wb * lb;
#pragma unroll
        for (int d = 0; d < DPL; ++d) {
            float oa, ob;
            if constexpr (X == 16) rows16(o[h][d], oa, ob);
            else rows32(o[h][d], oa, ob);
            o[h][d] = wa * oa + wb * ob;
        }
    }
}

template <int MODE, int D, int GC>
__global__ __launch_bounds__(512) void fold_kernel(const FoldParams p) {
    using S = FoldShape<D>;
    constexpr int LPT = S::LPT, DPL = S::DPL, VEC = S::VEC, ROWS = S::ROWS, U = S::U,
                  TG = S::TG;
    extern __shared__ float lds[];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nw = blockDim.x >> 6;
    const int row = lane / LPT, sub = lane % LPT;
    const int seq = blockIdx.y;
    const int per_seq = p.nkv * p.HG;
    const int kvhg = MODE == kModeTiled ? (int)blockIdx.x : (int)blockIdx.x % per_seq;
    const int split = MODE == kModeTiled ? 0 : (int)blockIdx.x / per_seq;
    const int kvh = kvhg / p.HG, hg = kvhg % p.HG;
    const int h0 = kvh * p.G + hg * GC;                 // first q head of the group
    const int gcount = min(GC, p.G - hg * GC);          // heads this group carries

    const int32_t* blocks = p.tables + (int64_t)seq * p.table_stride;
    int t_begin, t_end;
    if constexpr (MODE == kModeTiled) {
        int cnt = p.lens[seq];
        cnt = cnt < 0 ? 0 : (cnt > p.table_stride ? p.table_stride : cnt);
        if (cnt == 0) return;  // an empty tile leaves the state bit-identical
        t_begin = 0;
        t_end = (cnt - 1) * p.bs + p.lbvs;
    } else {
        int L = p.lens[seq];
        const int cap = p.table_stride * p.bs;
        L = L < 0 ? 0 : (L > cap ? cap : L);
        const int chunk = (int)split_chunk((uint32_t)L, (uint32_t)p.nsplit, (uint32_t)p.bs);
        const int64_t b0 = (int64_t)split * chunk;
        t_begin = b0 < L ? (int)b0 : L;
        t_end = (int64_t)t_begin + chunk < L ? t_begin + chunk : L;
    }

    // q slices of the group's heads (zeros for heads past gcount).
    uint32_t q2[GC][VEC];
#pragma unroll
    for (int h = 0; h < GC; ++h) {
        if (h < gcount) {
            load_words(q2[h], p.q + ((int64_t)seq * p.nq + h0 + h) * D + sub * DPL);
        } else {
#pragma unroll
            for (int j = 0; j < VEC; ++j) q2[h][j] = 0u;
        }
    }

    float m[GC], l[GC], o[GC][DPL];
#pragma unroll
    for (int h = 0; h < GC; ++h) {
        m[h] = kNegInf;
        l[h] = 0.f;
#pragma unroll
        for (int d = 0; d < DPL; ++d) o[h][d] = 0.f;
    }

    const int gpb = p.bs / TG;  // groups per block
    // a live range starts on a block (hence group) boundary; an empty split
    // starts at the sequence end, which need not be aligned: it folds nothing
    const int g_first = t_begin / TG;
    const int g_end = t_end > t_begin ? (t_end + TG - 1) / TG : g_first;
    const int tok_s = (int)p.tok_s;
    const uint16_t* kh = p.k + (int64_t)kvh * p.kvh_s;
    const uint16_t* vh = p.v + (int64_t)kvh * p.kvh_s;

    for (int g = g_first + wave; g < g_end; g += nw) {
        const int b = g / gpb;
        const int slot0 = (g - b * gpb) * TG;
        const int blk = blocks[b];
        if ((uint32_t)blk >= p.num_blocks) continue;  // dropped: never dereferenced
        const int nvalid = min(TG, t_end - g * TG);
        const uint16_t* kb = kh + (int64_t)blk * p.blk_s;
        const uint16_t* vb = vh + (int64_t)blk * p.blk_s;

        uint32_t kr[U][VEC], vr[U][VEC];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int r = row + ROWS * u;
            // a masked token re-reads the group's first row (always valid),
            // so canary memory past the end never enters the arithmetic
            const int slot = slot0 + (r < nvalid ? r : 0);
            const uint32_t off = (uint32_t)(slot * tok_s + sub * DPL);
            load_words(kr[u], kb + off);
            load_words(vr[u], vb + off);
        }

        float s[U][GC];
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
            for (int h = 0; h < GC; ++h) {
                float a = 0.f;
#pragma unroll
                for (int j = 0; j < VEC; ++j) a = dot2(q2[h][j], kr[u][j], a);
                s[u][h] = a;
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const bool ok = row + ROWS * u < nvalid;
#pragma unroll
            for (int h = 0; h < GC; ++h) {
                const float a = row_sum<LPT>(s[u][h]);
                s[u][h] = ok ? a * p.c : kNegInf;
            }
        }

        float vf[U][DPL];
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
            for (int j = 0; j < VEC; ++j) {
                vf[u][2 * j] = bf_lo(vr[u][j]);
                vf[u][2 * j + 1] = bf_hi(vr[u][j]);
            }
        }

#pragma unroll
        for (int h = 0; h < GC; ++h) {
            float bm = s[0][h];
#pragma unroll
            for (int u = 1; u < U; ++u) bm = fmaxf(bm, s[u][h]);
            const float mn = fmaxf(m[h], bm);
            const float ms = mn == kNegInf ? 0.f : mn;
            const float alpha = fexp2(m[h] - ms);
            m[h] = mn;
            float pu[U];
            float lsum = alpha * l[h];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                pu[u] = fexp2(s[u][h] - ms);
                lsum += pu[u];
            }
            l[h] = lsum;
#pragma unroll
            for (int d = 0; d < DPL; ++d) {
                float acc = alpha * o[h][d];
#pragma unroll
                for (int u = 0; u < U; ++u) acc = fmaf(pu[u], vf[u][d], acc);
                o[h][d] = acc;
            }
        }
    }

    // Rows of the wave -> one state per wave (identical in every row).
    if constexpr (ROWS >= 4) merge_rows<16, GC, DPL>(m, l, o);
    if constexpr (ROWS >= 2) merge_rows<32, GC, DPL>(m, l, o);

    // Waves -> LDS.  Layout: o [W][GC][D], m [W][GC], l [W][GC],
    // weights [W + 1][GC], Lsum [GC].
    float* lo_ = lds;
    float* lm = lo_ + nw * GC * D;
    float* ll = lm + nw * GC;
    float* lw = ll + nw * GC;
    float* lL = lw + (nw + 1) * GC;
    if (row == 0) {
#pragma unroll
        for (int h = 0; h < GC; ++h)
#pragma unroll
            for (int d = 0; d < DPL; ++d) lo_[(wave * GC + h) * D + sub * DPL + d] = o[h][d];
    }
    if (lane == 0) {
#pragma unroll
        for (int h = 0; h < GC; ++h) {
            lm[wave * GC + h] = m[h];
            ll[wave * GC + h] = l[h];
        }
    }
    __syncthreads();

    // Per head: the workgroup max, every contributor's weight, and l.
    const int64_t row_q = (int64_t)seq * p.nq + h0;  // first q slot of the group
    if (tid < gcount) {
        const int h = tid;
        float M = kNegInf, m_old = kNegInf, m2_old = kNegInf, l_old = 0.f;
        if constexpr (MODE == kModeTiled) {
            m_old = p.ws[row_q + h];
            l_old = p.l_state[row_q + h];
            m2_old = m_old * kLog2e;
            M = m2_old;
        }
        for (int w = 0; w < nw; ++w) M = fmaxf(M, lm[w * GC + h]);
        const float Ms = M == kNegInf ? 0.f : M;
        float L = 0.f;
        if constexpr (MODE == kModeTiled) {
            const float wo = fexp2(m2_old - Ms);
            lw[nw * GC + h] = wo;
            L = wo * l_old;
        }
        for (int w = 0; w < nw; ++w) {
            const float wt = fexp2(lm[w * GC + h] - Ms);
            lw[w * GC + h] = wt;
            L += wt * ll[w * GC + h];
        }
        lL[h] = L;
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
    __syncthreads();

    // Per (head, pair of dims): o of every contributor, in a fixed order.
    const int nitems = gcount * (D / 2);
    for (int i = tid; i < nitems; i += blockDim.x) {
        const int h = i / (D / 2);
        const int d = (i - h * (D / 2)) * 2;
        float o0 = 0.f, o1 = 0.f;
        const int64_t qs = row_q + h;
        if constexpr (MODE == kModeTiled) {
            const float2 prev = *reinterpret_cast<const float2*>(p.o_state + qs * D + d);
            const float wo = lw[nw * GC + h];
            o0 = wo * prev.x;
            o1 = wo * prev.y;
        }
        for (int w = 0; w < nw; ++w) {
            const float wt = lw[w * GC + h];
            o0 += wt * lo_[(w * GC + h) * D + d];
            o1 += wt * lo_[(w * GC + h) * D + d + 1];
        }
        const float L = lL[h];
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

// Split-K merge: for each (sequence, q head), over splits in index order,
// skipping splits with l == 0 (their o is never read):
//   M = max m_i,  w_i = exp(m_i - M),  L = sum w_i l_i,  O = sum w_i o_i,
//   out = bf16(O / L), or 0 when every split is empty.
// One wave per (sequence, head); lane j owns D/64 consecutive dims.
template <int D>
__global__ __launch_bounds__(256) void merge_kernel(const float* __restrict__ ws,
                                                    uint16_t* __restrict__ out, int nq,
                                                    int nsplit) {
    constexpr int DPL = D / 64;
    const int lane = threadIdx.x & 63;
    const int h = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (h >= nq) return;
    const int64_t qs = (int64_t)blockIdx.y * nq + h;
    const float* base = ws + qs * nsplit * (int64_t)(D + 2);
    float M = kNegInf;
    for (int i = 0; i < nsplit; ++i) {
        const float li = base[i * (D + 2) + D + 1];
        if (li > 0.f) M = fmaxf(M, base[i * (D + 2) + D]);
    }
    float L = 0.f, O[DPL];
#pragma unroll
    for (int d = 0; d < DPL; ++d) O[d] = 0.f;
    for (int i = 0; i < nsplit; ++i) {
        const float* slot = base + i * (D + 2);
        const float li = slot[D + 1];
        if (!(li > 0.f)) continue;
        const float w = fexp2((slot[D] - M) * kLog2e);
        L += w * li;
        if constexpr (DPL == 1) {
            O[0] += w * slot[lane];
        } else {
#pragma unroll
            for (int d = 0; d < DPL; d += 2) {
                const float2 x = *reinterpret_cast<const float2*>(slot + lane * DPL + d);
                O[d] += w * x.x;
                O[d + 1] += w * x.y;
            }
        }
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

template <int MODE, int D>
FoldFn pick_gc(int gc) {
    switch (gc) {
        case 1: return fold_kernel<MODE, D, 1>;
        case 2: return fold_kernel<MODE, D, 2>;
        case 3: return fold_kernel<MODE, D, 3>;
        case 4: return fold_kernel<MODE, D, 4>;
        case 5: return fold_kernel<MODE, D, 5>;
        case 6: return fold_kernel<MODE, D, 6>;
        case 7: return fold_kernel<MODE, D, 7>;
        case 8: return fold_kernel<MODE, D, 8>;
        default: return nullptr;
    }
}

template <int MODE>
FoldFn pick_d(int D, int gc) {
    switch (D) {
        case 64: return pick_gc<MODE, 64>(gc);
        case 128: return pick_gc<MODE, 128>(gc);
        case 256: return pick_gc<MODE, 256>(gc);
        default: return nullptr;
    }
}

}  // namespace

size_t fold_lds_bytes(int head_dim, int gc, int waves) {
    return sizeof(float) * ((size_t)waves * gc * head_dim + 2 * (size_t)waves * gc +
                            (size_t)(waves + 1) * gc + (size_t)gc);
}

hipError_t launch_fold(int mode, int head_dim, int gc, const FoldParams& p, uint32_t grid_x,
                       uint32_t grid_y, int waves, hipStream_t stream) {
    FoldFn fn = nullptr;
    switch (mode) {
        case kModePartial: fn = pick_d<kModePartial>(head_dim, gc); break;
        case kModeFinal: fn = pick_d<kModeFinal>(head_dim, gc); break;
        case kModeTiled: fn = pick_d<kModeTiled>(head_dim, gc); break;
        default: break;
    }
    if (!fn) return hipErrorInvalidValue;
    const size_t lds = fold_lds_bytes(head_dim, gc, waves);
    hipLaunchKernelGGL(fn, dim3(grid_x, grid_y), dim3(64 * waves), lds, stream, p);
    return hipGetLastError();
}

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
