"""Paged decode over an FP8 KV cache, FP64 (test infrastructure; see
``oracle/__init__.py``).

The attn_splitk page names FP8 paged-decode launches and an FP8 packed
kernel but prints neither the FP8 format nor how the cache is scaled.
Readings (parity of the scale semantics is unpinned by the pages):
  * elements are OCP FP8 E4M3 ("fn"): sign, 4 exponent bits with bias 7,
    3 mantissa bits; exponent field 0 holds subnormals (m / 8 * 2^-6); the
    code S.1111.111 is NaN; there are no infinities; the largest finite
    magnitude is 448;
  * the cache holds K / k_scale and V / v_scale for two per-tensor FP32
    scales: K = decode(k8) * k_scale, V = decode(v8) * v_scale;
  * q stays BF16, the output is BF16, everything else is the BF16 path's
    definition (``oracle.attention``).
"""
from __future__ import annotations

import numpy as np

from .attention import decode_bf16


def _decode_table() -> np.ndarray:
    out = np.empty(256, dtype=np.float64)
    for b in range(256):
        sign = -1.0 if b & 0x80 else 1.0
        e = (b >> 3) & 0xF
        m = b & 0x7
        if e == 0xF and m == 0x7:
            out[b] = np.nan
        elif e == 0:
            out[b] = sign * (m / 8.0) * 2.0 ** -6
        else:
            out[b] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return out


_E4M3 = _decode_table()


def decode_e4m3(codes: np.ndarray) -> np.ndarray:
    """E4M3 codes -> FP64 (exact)."""
    return _E4M3[np.asarray(codes, dtype=np.uint8)]


def paged_decode_fp8(q_bits, k8, v8, block_tables, seq_lens, scale, k_scale, v_scale):
    """One-shot paged decode with an FP8 cache: out [S, nq, D] FP64 (0 for an
    empty sequence).  Definition: s = scale * q . K, softmax, out = p V / l,
    with K and V decoded and multiplied by their scales in FP64."""
    S, nq, D = q_bits.shape
    nb, bs, nkv, _ = k8.shape
    G = nq // nkv
    q = decode_bf16(q_bits)
    out = np.zeros((S, nq, D), dtype=np.float64)
    for s in range(S):
        L = int(seq_lens[s])
        if L <= 0:
            continue
        t = np.arange(L)
        blk = block_tables[s, t // bs]
        K = decode_e4m3(k8[blk, t % bs]) * float(k_scale)     # [L, nkv, D]
        V = decode_e4m3(v8[blk, t % bs]) * float(v_scale)
        for h in range(nq):
            kvh = h // G
            sc = float(scale) * (K[:, kvh, :] @ q[s, h])
            p = np.exp(sc - sc.max())
            out[s, h] = (p @ V[:, kvh, :]) / p.sum()
    return out
