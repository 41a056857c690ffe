"""Pins of oracle.prefill (causal paged prefill) against things other than
itself: brute force, torch's FP64 scaled_dot_product_attention with an
explicit causal mask, closed forms, the decode oracle at the last position,
and invariances.  CPU only."""
import dataclasses
import math

import numpy as np
import pytest

import workloads as W
from oracle import attention as A
from oracle import prefill as PF


def _small(q_len, kv_len, q_offset, nq=4, nkv=2, D=8, bs=4, seed=11, canary=True):
    w = dataclasses.replace(W.WORKLOADS["prefill"], seed=seed, num_q_heads=nq, num_kv_heads=nkv,
                            head_dim=D, block_size=bs)
    return W.make_prefill(w, canary=canary, q_len=q_len, kv_len=kv_len, q_offset=q_offset)


def _f(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(float)


def _brute(p):
    """Pure-Python loops: exp without a max shift, fsum, positions by hand."""
    q_len, nq, D = p.q.shape
    nkv, bs = p.num_kv_heads, p.block_size
    out = np.zeros((q_len, nq, D))
    for i in range(q_len):
        for h in range(nq):
            kvh = h // (nq // nkv)
            qv = _f(p.q[i, h])
            ws, vs = [], []
            for j in range(p.kv_len):
                if j > p.q_offset + i:
                    break
                blk = p.block_table[j // bs]
                kv = _f(p.k_cache[blk, j % bs, kvh])
                vv = _f(p.v_cache[blk, j % bs, kvh])
                s = p.scale * math.fsum(float(a) * float(b) for a, b in zip(qv, kv))
                ws.append(math.exp(s))
                vs.append(vv)
            if ws:
                tot = math.fsum(ws)
                for d in range(D):
                    out[i, h, d] = math.fsum(w * v[d] for w, v in zip(ws, vs)) / tot
    return out


@pytest.mark.parametrize("q_len,kv_len,q_offset", [(5, 5, 0), (3, 9, 6), (4, 7, 1), (6, 4, 2)])
def test_brute_force(q_len, kv_len, q_offset):
    p = _small(q_len, kv_len, q_offset)
    got = PF.paged_prefill(p.q, p.k_cache, p.v_cache, p.block_table, p.kv_len, p.q_offset,
                           p.scale)
    np.testing.assert_allclose(got, _brute(p), rtol=1e-12, atol=1e-13)


def test_sdpa_with_causal_mask():
    torch = pytest.importorskip("torch")
    p = _small(24, 40, 16, nq=6, nkv=2, D=16, bs=8, canary=False)
    got = PF.paged_prefill(p.q, p.k_cache, p.v_cache, p.block_table, p.kv_len, p.q_offset,
                           p.scale)
    n = p.kv_len
    t = np.arange(n)
    blk = p.block_table[t // p.block_size]
    K = _f(p.k_cache[blk, t % p.block_size])                 # [n, nkv, D]
    V = _f(p.v_cache[blk, t % p.block_size])
    G = p.num_q_heads // p.num_kv_heads
    Kq = torch.tensor(np.repeat(K, G, axis=1)).permute(1, 0, 2)    # [nq, n, D]
    Vq = torch.tensor(np.repeat(V, G, axis=1)).permute(1, 0, 2)
    Q = torch.tensor(_f(p.q)).permute(1, 0, 2)                       # [nq, q_len, D]
    mask = torch.tensor(t[None, :] <= (p.q_offset + np.arange(p.q_len))[:, None])
    ref = torch.nn.functional.scaled_dot_product_attention(Q, Kq, Vq, attn_mask=mask,
                                                           scale=p.scale)
    np.testing.assert_allclose(got, ref.permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-13)


def test_first_row_is_the_first_value():
    """At q_offset 0, row 0 sees only key 0: p = 1, so out = v_0 exactly."""
    p = _small(8, 8, 0)
    got = PF.paged_prefill(p.q, p.k_cache, p.v_cache, p.block_table, p.kv_len, 0, p.scale)
    G = p.num_q_heads // p.num_kv_heads
    for h in range(p.num_q_heads):
        v0 = _f(p.v_cache[p.block_table[0], 0, h // G])
        assert np.array_equal(got[0, h], v0)


def test_last_position_equals_decode():
    """One query row at position kv_len - 1 sees the whole sequence: the
    decode oracle's result for that query."""
    p = _small(1, 37, 36, nq=8, nkv=2, D=32, bs=8)
    got = PF.paged_prefill(p.q, p.k_cache, p.v_cache, p.block_table, p.kv_len, p.q_offset,
                           p.scale)
    dec, _, _ = A.paged_decode(p.q, p.k_cache, p.v_cache, p.block_table[None, :],
                               np.array([p.kv_len], np.int32), p.scale)
    np.testing.assert_allclose(got, dec, rtol=1e-14, atol=0)


def test_empty_cache_gives_zeros():
    p = _small(3, 0, 0)
    got = PF.paged_prefill(p.q, p.k_cache, p.v_cache, p.block_table, 0, 0, p.scale)
    assert np.all(got == 0)


def test_future_keys_never_reach_a_row():
    """Poison every key / value after row i's position: rows up to i are
    unchanged (and finite)."""
    p = _small(6, 12, 4)
    base = PF.paged_prefill(p.q, p.k_cache, p.v_cache, p.block_table, p.kv_len, p.q_offset,
                            p.scale)
    i = 2
    k, v = p.k_cache.copy(), p.v_cache.copy()
    for j in range(p.q_offset + i + 1, p.kv_len):
        k[p.block_table[j // p.block_size], j % p.block_size] = W.BF16_QNAN
        v[p.block_table[j // p.block_size], j % p.block_size] = W.BF16_QNAN
    got = PF.paged_prefill(p.q, k, v, p.block_table, p.kv_len, p.q_offset, p.scale,
                           rows=np.arange(i + 1))
    assert np.all(np.isfinite(got))
    # (the two runs sum over different key counts, so BLAS may round differently)
    np.testing.assert_allclose(got, base[:i + 1], rtol=1e-14, atol=1e-15)


def test_block_relayout_invariance():
    p = _small(10, 21, 11, bs=4)
    base = PF.paged_prefill(p.q, p.k_cache, p.v_cache, p.block_table, p.kv_len, p.q_offset,
                            p.scale)
    n = -(-p.kv_len // p.block_size)
    perm = np.random.default_rng(3).permutation(p.num_blocks)
    k2, v2 = np.empty_like(p.k_cache), np.empty_like(p.v_cache)
    k2[perm] = p.k_cache
    v2[perm] = p.v_cache
    bt2 = p.block_table.copy()
    bt2[:n] = perm[p.block_table[:n]]
    got = PF.paged_prefill(p.q, k2, v2, bt2, p.kv_len, p.q_offset, p.scale)
    assert np.array_equal(got, base)
