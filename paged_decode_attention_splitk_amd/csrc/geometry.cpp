// Pure launch-geometry functions of the C ABI (no HIP calls).
// Formulas: "Module attn_splitk" page, items auto_splits, legacy_splits,
// split_ref_seqs (inside legacy_splits), num_splits, workspace_slots,
// gqa_pack_shape_ok, gqa_pack_ctas; "metrale_storage/tiled_attention.rs"
// page for the two stride sets.
#include "pda.h"
#include "pda_geometry.h"

extern "C" {

uint32_t pda_max_decode_splits(void) { return pda::kMaxDecodeSplits; }
uint32_t pda_splitk_target_waves(void) { return pda::kSplitkTargetWaves; }
uint32_t pda_gqa_pack_width(void) { return pda::kGqaPackWidth; }
uint32_t pda_gqa_pack_head_dim(void) { return pda::kGqaPackHeadDim; }
uint32_t pda_min_kv_per_split(void) { return pda::kMinKvPerSplit; }
uint32_t pda_max_head_dim(void) { return pda::kMaxHeadDim; }

uint32_t pda_auto_splits(uint32_t cu_count, uint32_t num_q_heads) {
    if (num_q_heads == 0) return 0;
    const uint64_t want = (uint64_t)pda::kSplitkTargetWaves * cu_count;
    uint64_t n = (want + num_q_heads - 1) / num_q_heads;
    if (n < 1) n = 1;
    if (n > pda::kMaxDecodeSplits) n = pda::kMaxDecodeSplits;
    return (uint32_t)n;
}

uint32_t pda_split_ref_seqs(uint32_t num_seqs, uint32_t max_decode_seqs) {
    return num_seqs > max_decode_seqs ? num_seqs : max_decode_seqs;
}

uint32_t pda_legacy_splits(uint32_t cu_count, uint32_t num_q_heads, uint32_t ref_seqs) {
    const uint64_t ctas = (uint64_t)num_q_heads * ref_seqs;
    if (ctas == 0) return 0;
    if (ctas >= cu_count) return 1;
    return (uint32_t)(cu_count / ctas);
}

uint32_t pda_pinned_splits(uint32_t pin) {
    if (pin < 1) return 1;
    return pin > pda::kMaxDecodeSplits ? pda::kMaxDecodeSplits : pin;
}

uint32_t pda_num_splits(int policy, uint32_t pin, uint32_t cu_count, uint32_t num_q_heads,
                        uint32_t num_seqs, uint32_t max_decode_seqs) {
    switch (policy) {
        case PDA_SPLITK_LEGACY:
            return pda_legacy_splits(cu_count, num_q_heads,
                                     pda_split_ref_seqs(num_seqs, max_decode_seqs));
        case PDA_SPLITK_AUTO:
            return pda_auto_splits(cu_count, num_q_heads);
        case PDA_SPLITK_PINNED:
            return pda_pinned_splits(pin);
        default:
            return 0;
    }
}

uint64_t pda_workspace_slots(uint64_t rows, uint32_t num_q_heads, uint32_t num_splits,
                             uint32_t head_dim) {
    return rows * num_q_heads * num_splits * ((uint64_t)head_dim + 2);
}

int pda_gqa_pack_shape_ok(uint32_t num_q_heads, uint32_t num_kv_heads, uint32_t head_dim) {
    return num_kv_heads > 0 && head_dim == pda::kGqaPackHeadDim &&
           (uint64_t)num_q_heads == (uint64_t)num_kv_heads * pda::kGqaPackWidth;
}

uint64_t pda_gqa_pack_ctas(uint32_t num_kv_heads, uint32_t num_seqs) {
    return (uint64_t)num_kv_heads * num_seqs;
}

uint32_t pda_split_chunk(uint32_t seq_len, uint32_t num_splits, uint32_t block_size) {
    return pda::split_chunk(seq_len, num_splits, block_size);
}

void pda_tiled_paged_strides(const pda_tiled_dims* d, int64_t out[3]) {
    if (!d || !out) return;
    out[0] = (int64_t)d->block_size * d->num_kv_heads * d->head_dim;
    out[1] = (int64_t)d->num_kv_heads * d->head_dim;
    out[2] = (int64_t)d->head_dim;
}

void pda_tiled_scratch_pool_strides(const pda_tiled_dims* d, int64_t out[3]) {
    if (!d || !out) return;
    const int64_t kv_stripe = (int64_t)d->num_kv_heads * d->block_size * d->head_dim;
    out[0] = 2 * kv_stripe;
    out[1] = (int64_t)d->head_dim;
    out[2] = (int64_t)d->block_size * d->head_dim;
}

}  // extern "C"
