// Launch-geometry rules shared by the host library and the device kernels.
//
// The split-count rules follow the "Module attn_splitk" page (items
// auto_splits, legacy_splits, num_splits, MAX_DECODE_SPLITS,
// SPLITK_TARGET_WAVES, workspace_slots, gqa_pack_shape_ok, gqa_pack_ctas).
// Values that page does not print are readings: 2 target waves (what its
// worked asks of 264 and 13 imply), a ceiling of 16 splits, a pack width of
// 8 q heads, and a per-split floor of 64 tokens.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define PDA_HD __host__ __device__ inline
#else
#define PDA_HD inline
#endif

namespace pda {

constexpr uint32_t kSplitkTargetWaves = 2;
constexpr uint32_t kMaxDecodeSplits = 16;
constexpr uint32_t kGqaPackWidth = 8;
constexpr uint32_t kGqaPackHeadDim = 256;
constexpr uint32_t kMinKvPerSplit = 64;
constexpr uint32_t kMaxHeadDim = 256;
// Head dim of the causal prefill kernel (prefill page, applies: head_dim 256).
constexpr uint32_t kPrefillHeadDim = 256;
// Block sizes are multiples of this, so a split (which starts on a block)
// always starts on a token group of the fold loop.
constexpr uint32_t kBlockQuantum = 16;

// Tokens of one split of a sequence of `seq_len` tokens: ceil(L / n) floored
// at kMinKvPerSplit and rounded up to whole blocks, so every split starts on
// a block boundary.  0 when n or block_size is 0.
// Only 32-bit divisions (ceil written as quotient plus a remainder test),
// so a kernel that calls it keeps no 64-bit division constants live.
PDA_HD uint32_t split_chunk(uint32_t seq_len, uint32_t n, uint32_t block_size) {
    if (n == 0 || block_size == 0) return 0;
    uint32_t per = seq_len / n + (seq_len % n != 0u ? 1u : 0u);
    if (per < kMinKvPerSplit) per = kMinKvPerSplit;
    const uint64_t c = (uint64_t)((per - 1u) / block_size + 1u) * block_size;
    return c > 0xFFFFFFFFull ? 0xFFFFFFFFu : (uint32_t)c;
}

}  // namespace pda
