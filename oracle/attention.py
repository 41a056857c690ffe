"""Paged-decode attention in FP64: the plain definition, written out.

Test infrastructure (see ``oracle/__init__.py``).

What is computed (north-star problem statement, and the "tiled_attention.rs"
page's module comment for the running state and the finalize rule):

  for sequence s, query head h, with G = num_q_heads / num_kv_heads and the
  KV head kvh = h // G serving h (reading: contiguous head groups):
    gather the sequence's L tokens through its block table
        k_t = K[table[t // bs], t % bs, kvh, :],   v_t likewise
    s_t = scale * <q, k_t>
    m   = max_t s_t
    l   = sum_t exp(s_t - m)
    o   = sum_t exp(s_t - m) * v_t          (unnormalised, as the tiled state)
    out = o / l, and 0 (with m = -inf, l = 0) when L = 0

Every BF16 value is widened exactly to FP64 before any arithmetic; ``scale``
is the FP32 argument widened exactly.  Nothing is blocked, fused or
reordered: one numpy reduction per sum.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

from . import geometry


def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """BF16 bit patterns -> FP64 (exact: a BF16 is the top half of an FP32)."""
    u32 = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u32.view(np.float32).astype(np.float64)


@dataclasses.dataclass
class HeadResult:
    out: np.ndarray      # [D] float64, o / l (0 when l == 0)
    m: float             # running max in natural units (-inf when empty)
    l: float             # sum of exp(s_t - m)
    o: np.ndarray        # [D] unnormalised


def gather_tokens(k_flat: np.ndarray, v_flat: np.ndarray, blocks: np.ndarray,
                  token_begin: int, token_end: int, kvh: int,
                  strides, block_size: int, head_dim: int):
    """K and V rows of tokens [token_begin, token_end) of one KV head, as
    [n, D] FP64, addressed through the block list with (blk, tok, kvh)
    element strides (tiled_attention.rs, paged_strides / scratch_pool_strides):
        offset(t) = blocks[t // bs] * blk + (t % bs) * tok + kvh * kvh_stride
    """
    blk_s, tok_s, kvh_s = strides
    t = np.arange(token_begin, token_end, dtype=np.int64)
    base = (blocks[t // block_size].astype(np.int64) * blk_s
            + (t % block_size) * tok_s + kvh * kvh_s)
    idx = base[:, None] + np.arange(head_dim, dtype=np.int64)[None, :]
    return decode_bf16(k_flat[idx]), decode_bf16(v_flat[idx])


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> HeadResult:
    """Softmax attention of one query over n gathered tokens, FP64."""
    D = q.shape[0]
    if K.shape[0] == 0:
        return HeadResult(np.zeros(D), -math.inf, 0.0, np.zeros(D))
    s = scale * (K @ q)
    m = float(s.max())
    p = np.exp(s - m)
    l = float(p.sum())
    o = p @ V
    return HeadResult(o / l, m, l, o)


def _fp32(x) -> float:
    return float(np.float32(x))


def paged_decode(q_bits, k_cache_bits, v_cache_bits, block_tables, seq_lens, scale,
                 heads=None):
    """One-shot paged decode over the layout [num_blocks, block_size,
    num_kv_heads, head_dim].

    Returns (out [S, nq, D], m [S, nq], l [S, nq]) in FP64; ``heads`` may
    restrict the work to a list of (s, h) pairs (the other entries are NaN).
    """
    S, nq, D = q_bits.shape
    nb, bs, nkv, D2 = k_cache_bits.shape
    assert D2 == D and v_cache_bits.shape == k_cache_bits.shape
    G = nq // nkv
    strides = geometry.paged_strides(bs, nkv, D)
    kf = k_cache_bits.reshape(-1)
    vf = v_cache_bits.reshape(-1)
    qd = decode_bf16(q_bits)
    scale = _fp32(scale)
    out = np.full((S, nq, D), np.nan)
    m = np.full((S, nq), np.nan)
    l = np.full((S, nq), np.nan)
    pairs = heads if heads is not None else [(s, h) for s in range(S) for h in range(nq)]
    cache = {}
    for s, h in pairs:
        kvh = h // G
        key = (s, kvh)
        if key not in cache:
            cache.clear()
            cache[key] = gather_tokens(kf, vf, np.asarray(block_tables[s]), 0, int(seq_lens[s]),
                                       kvh, strides, bs, D)
        K, V = cache[key]
        r = attend(qd[s, h], K, V, scale)
        out[s, h], m[s, h], l[s, h] = r.out, r.m, r.l
    return out, m, l


def split_partials(q_bits, k_cache_bits, v_cache_bits, block_tables, seq_lens, scale,
                   n_splits: int):
    """Per-split partial states of the split-K workspace: for each (s, h, i)
    the unnormalised o, m and l over split i's token range alone.  An empty
    split holds m = -inf, l = 0, o = 0.

    Returns (o [S, nq, n, D], m [S, nq, n], l [S, nq, n]) in FP64.
    """
    S, nq, D = q_bits.shape
    nb, bs, nkv, _ = k_cache_bits.shape
    G = nq // nkv
    strides = geometry.paged_strides(bs, nkv, D)
    kf = k_cache_bits.reshape(-1)
    vf = v_cache_bits.reshape(-1)
    qd = decode_bf16(q_bits)
    scale = _fp32(scale)
    o = np.zeros((S, nq, n_splits, D))
    m = np.full((S, nq, n_splits), -math.inf)
    l = np.zeros((S, nq, n_splits))
    for s in range(S):
        ranges = geometry.split_ranges(int(seq_lens[s]), n_splits, bs)
        for kvh in range(nkv):
            for i, (b, e) in enumerate(ranges):
                K, V = gather_tokens(kf, vf, np.asarray(block_tables[s]), b, e, kvh, strides, bs, D)
                for h in range(kvh * G, (kvh + 1) * G):
                    r = attend(qd[s, h], K, V, scale)
                    o[s, h, i], m[s, h, i], l[s, h, i] = r.o, r.m, r.l
    return o, m, l


def tiled_scale(head_dim: int) -> float:
    """The tiled step kernel takes no scale argument (tiled_attention.rs,
    step_tile_on_stream passes none); reading: 1/sqrt(head_dim) as FP32."""
    return _fp32(1.0 / math.sqrt(head_dim))


def tiled_state(q_bits, pool_bits, slot_tables, seq_lens, seqs=None):
    """Final (m, l, o) running state and the finalize output after every KV
    block of each sequence has been folded in, for the scratch-pool slot
    layout [slot, K|V, kv_head, block_size, head_dim] with V one kv_stripe
    after K inside each slot.

    Folding tiles of an online softmax in any grouping reaches, in exact
    arithmetic, the state of the whole sequence at once, so this is the
    one-pass definition over all L tokens.

    Returns (out [S, nq, D], m [S, nq], l [S, nq], o [S, nq, D]) in FP64;
    rows not listed in ``seqs`` are NaN.
    """
    S, nq, D = q_bits.shape
    nslots, two, nkv, bs, D2 = pool_bits.shape
    assert two == 2 and D2 == D
    G = nq // nkv
    strides = geometry.scratch_pool_strides(bs, nkv, D)
    flat = pool_bits.reshape(-1)
    voff = geometry.scratch_pool_v_offset(bs, nkv, D)
    kf = flat
    vf = flat[voff:]
    qd = decode_bf16(q_bits)
    scale = tiled_scale(D)
    out = np.full((S, nq, D), np.nan)
    o = np.full((S, nq, D), np.nan)
    m = np.full((S, nq), np.nan)
    l = np.full((S, nq), np.nan)
    for s in (range(S) if seqs is None else seqs):
        for kvh in range(nkv):
            K, V = gather_tokens(kf, vf, np.asarray(slot_tables[s]), 0, int(seq_lens[s]),
                                 kvh, strides, bs, D)
            for h in range(kvh * G, (kvh + 1) * G):
                r = attend(qd[s, h], K, V, scale)
                out[s, h], m[s, h], l[s, h], o[s, h] = r.out, r.m, r.l, r.o
    return out, m, l, o
