"""Causal paged prefill attention in FP64 (test infrastructure; see
``oracle/__init__.py``).

Written from the prefill page ("metrale_model_layers/layers/ops/
prefill_attn_fa128.rs": the module comment and the ``paged`` launcher): one
sequence's query rows attend, causally, over its BF16 paged KV cache
[num_blocks, block_size, num_kv_heads, head_dim] through its block table,
with grouped-query heads and the scale ``inv_sqrt_d``.

Readings (the page prints the launcher, not the kernel):
  * query row i is the token at position q_offset + i and attends the keys
    at positions j with j <= q_offset + i and j < kv_len (causal);
  * q and the output are [q_len, num_q_heads, head_dim];
  * q head h reads KV head h // (num_q_heads // num_kv_heads);
  * a row with no key (kv_len == 0) outputs 0, as the decode finalize does.

The definition is written out directly: for each head, scores
``S = scale * Q K^T`` over the gathered keys, masked, ``p = exp(S - max)``,
``out = (p V) / sum(p)``; numpy's matmul is the only library step.
"""
from __future__ import annotations

import numpy as np

from .attention import decode_bf16, gather_tokens


def paged_prefill(q_bits, k_cache_bits, v_cache_bits, block_table, kv_len: int,
                  q_offset: int, scale: float, rows=None):
    """FP64 causal prefill output, [len(rows), num_q_heads, head_dim]
    (``rows`` = query row indices, default all)."""
    q_len, nq, D = q_bits.shape
    nb, bs, nkv, _ = k_cache_bits.shape
    G = nq // nkv
    rows = np.arange(q_len) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.zeros((len(rows), nq, D), dtype=np.float64)
    if kv_len == 0 or len(rows) == 0:
        return out
    kf = k_cache_bits.reshape(-1)
    vf = v_cache_bits.reshape(-1)
    strides = (bs * nkv * D, nkv * D, D)
    pos = q_offset + rows                                     # query positions
    last = np.minimum(pos, kv_len - 1)                        # last key each row sees
    n_keys = int(last.max()) + 1
    keys = np.arange(n_keys)
    masked = keys[None, :] > last[:, None]
    Q = decode_bf16(q_bits[rows])                             # [r, nq, D]
    for kvh in range(nkv):
        K, V = gather_tokens(kf, vf, block_table, 0, n_keys, kvh, strides, bs, D)
        for h in range(kvh * G, (kvh + 1) * G):
            S = float(scale) * (Q[:, h, :] @ K.T)             # [r, n_keys]
            S[masked] = -np.inf
            m = S.max(axis=1, keepdims=True)
            p = np.exp(S - m)
            out[:, h, :] = (p @ V) / p.sum(axis=1, keepdims=True)
    return out
