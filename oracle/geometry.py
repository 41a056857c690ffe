"""Launch-geometry formulas of paged-decode split-K, as plain Python integers.

Test infrastructure (see ``oracle/__init__.py``).  Written from the
"Module attn_splitk" page (the kernels crate's split-K launch-geometry
module) and the "metrale_storage/tiled_attention.rs" source page; no code
here is shared with the C++ geometry of the HIP library.

Values the pages do not print are readings, marked as such:
  * SPLITK_TARGET_WAVES = 2: the MAX_DECODE_SPLITS item explains its ceiling
    with an ask of twice the SM count over the q-head count (264 for one head
    on 132 SMs, 13 for 24 heads on 148 SMs), which fixes the wave count at 2.
  * MAX_DECODE_SPLITS = 16: must be >= 13 (that item's example is not
    clamped) and, for a 24-head model on 256 CUs, below the ask of 22.
  * DECODE_GQA_PACK_WIDTH = 8: not printed; 8 query heads per KV head.
  * PD_MIN_KV_PER_SPLIT = 64 tokens, and the partition rule of
    ``split_chunk`` (floor each split at 64 tokens of the sequence's own
    length, rounded up to whole blocks): parity unpinned.
"""
from __future__ import annotations

SPLITK_TARGET_WAVES = 2
MAX_DECODE_SPLITS = 16
DECODE_GQA_PACK_WIDTH = 8
DECODE_GQA_PACK_HEAD_DIM = 256          # printed: the packed sources are built for head dim 256
PD_MIN_KV_PER_SPLIT = 64
MAX_HEAD_DIM = 256                      # tiled_attention.rs, TiledAttentionDims::validate
NEG_INF_F32_BITS = 0xFF800000           # tiled_attention.rs, the -inf pattern begin_step writes

LEGACY, AUTO, PINNED = 0, 1, 2


def _ceil_div(a: int, b: int) -> int:
    return -((-a) // b)


def _clamp(x: int, lo: int, hi: int) -> int:
    return max(lo, min(hi, x))


def auto_splits_ask(sm_count: int, num_q_heads: int) -> int:
    """The unclamped Auto ask, ceil(WAVES * sm_count / num_q_heads)
    (attn_splitk page, items auto_splits and MAX_DECODE_SPLITS)."""
    return _ceil_div(SPLITK_TARGET_WAVES * sm_count, num_q_heads)


def auto_splits(sm_count: int, num_q_heads: int) -> int:
    """clamp(ceil(WAVES * sm_count / num_q_heads), 1, MAX_DECODE_SPLITS)
    (attn_splitk page, item auto_splits).  0 when num_q_heads is 0."""
    if num_q_heads == 0:
        return 0
    return _clamp(auto_splits_ask(sm_count, num_q_heads), 1, MAX_DECODE_SPLITS)


def split_ref_seqs(num_seqs: int, max_decode_seqs: int) -> int:
    """max(max_decode_seqs, num_seqs) (attn_splitk page, item legacy_splits)."""
    return max(max_decode_seqs, num_seqs)


def legacy_splits(sm_count: int, num_q_heads: int, ref_seqs: int) -> int:
    """The Legacy rule (attn_splitk page, module description and item
    legacy_splits): with current = num_q_heads * ref_seqs, one split when
    current reaches the SM count, else the integer quotient sm_count / current.
    Not clamped to MAX_DECODE_SPLITS.  0 when current is 0 (no quotient)."""
    current = num_q_heads * ref_seqs
    if current == 0:
        return 0
    return 1 if current >= sm_count else sm_count // current


def pinned_splits(pin: int) -> int:
    """A pinned count is clamped into 1..=MAX_DECODE_SPLITS (attn_splitk page,
    items MAX_DECODE_SPLITS and parse)."""
    return _clamp(pin, 1, MAX_DECODE_SPLITS)


def num_splits(policy: int, pin: int, sm_count: int, num_q_heads: int,
               num_seqs: int, max_decode_seqs: int) -> int:
    """The split count for a launch under a policy (attn_splitk page, enum
    SplitkPolicy and item num_splits).  Only Legacy reads the batch."""
    if policy == LEGACY:
        return legacy_splits(sm_count, num_q_heads, split_ref_seqs(num_seqs, max_decode_seqs))
    if policy == AUTO:
        return auto_splits(sm_count, num_q_heads)
    if policy == PINNED:
        return pinned_splits(pin)
    return 0


def workspace_slots(rows: int, num_q_heads: int, n_splits: int, head_dim: int) -> int:
    """FP32 values the split-K workspace holds: rows * heads * splits *
    (head_dim + 2), one [o[head_dim], m, l] slot per (row, head, split)
    (attn_splitk page, items MAX_DECODE_SPLITS and workspace_slots)."""
    return rows * num_q_heads * n_splits * (head_dim + 2)


def gqa_pack_shape_ok(num_q_heads: int, num_kv_heads: int, head_dim: int) -> bool:
    """num_q_heads == num_kv_heads * PACK_WIDTH at head_dim == 256 (attn_splitk
    page, module invariants and item gqa_pack_shape_ok); no KV heads never fits."""
    return (num_kv_heads > 0 and head_dim == DECODE_GQA_PACK_HEAD_DIM
            and num_q_heads == num_kv_heads * DECODE_GQA_PACK_WIDTH)


def gqa_pack_ctas(num_kv_heads: int, num_seqs: int) -> int:
    """Workgroups of a packed launch: num_kv_heads * num_seqs (attn_splitk
    page, item gqa_pack_ctas)."""
    return num_kv_heads * num_seqs


def split_chunk(seq_len: int, n_splits: int, block_size: int) -> int:
    """Tokens per split for one sequence: ceil(L / n) floored at
    PD_MIN_KV_PER_SPLIT, then rounded up to whole blocks (reading of the
    attn_splitk page's module description on short contexts)."""
    per = max(_ceil_div(seq_len, n_splits), PD_MIN_KV_PER_SPLIT)
    return _ceil_div(per, block_size) * block_size


def split_ranges(seq_len: int, n_splits: int, block_size: int):
    """[begin, end) token range of every split; an empty split has begin == end."""
    c = split_chunk(seq_len, n_splits, block_size)
    out = []
    for i in range(n_splits):
        b = min(i * c, seq_len)
        e = min((i + 1) * c, seq_len)
        out.append((b, e))
    return out


def paged_strides(block_size: int, num_kv_heads: int, head_dim: int):
    """(blk, tok, kvh) strides in elements of [num_blocks, block_size,
    num_kv_heads, head_dim] (tiled_attention.rs, paged_strides)."""
    return (block_size * num_kv_heads * head_dim, num_kv_heads * head_dim, head_dim)


def scratch_pool_strides(block_size: int, num_kv_heads: int, head_dim: int):
    """(blk, tok, kvh) strides in elements of the slot layout [slot, K|V,
    kv_head, block_size, head_dim] (tiled_attention.rs, scratch_pool_strides)."""
    kv_stripe = num_kv_heads * block_size * head_dim
    return (2 * kv_stripe, head_dim, block_size * head_dim)


def scratch_pool_v_offset(block_size: int, num_kv_heads: int, head_dim: int) -> int:
    """Elements from a slot's K half to its V half (reading: V follows K
    inside each slot, one kv_stripe later)."""
    return num_kv_heads * block_size * head_dim


def tiled_dims_error(max_seqs, num_q_heads, num_kv_heads, head_dim, block_size, tile_capacity):
    """None when the dims are acceptable, else a reason (tiled_attention.rs,
    TiledAttentionDims::validate: q heads a multiple of kv heads, head_dim
    at most 256; kv heads must be non-zero for the ratio to exist)."""
    if num_kv_heads == 0:
        return "num_kv_heads is 0"
    if num_q_heads % num_kv_heads != 0:
        return "num_q_heads is not a multiple of num_kv_heads"
    if head_dim > MAX_HEAD_DIM:
        return "head_dim exceeds 256"
    return None


def tiled_state_bytes(max_seqs: int, num_q_heads: int, head_dim: int):
    """(m, l, o, output) byte sizes of the tiled state (tiled_attention.rs,
    m_bytes / l_bytes / o_bytes / output_bytes): FP32 m and l per q slot,
    FP32 o and BF16 output of head_dim per q slot."""
    slots = max_seqs * num_q_heads
    return (slots * 4, slots * 4, slots * head_dim * 4, slots * head_dim * 2)
