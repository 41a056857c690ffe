"""Pins of the FP64 attention oracle (CPU only).

The oracle is checked against things other than itself:
  * brute force in pure Python (math.exp, math.fsum, no max subtraction,
    tokens found by walking the 4-D cache with plain indexing);
  * torch's scaled_dot_product_attention in FP64 on the CPU, with the GQA
    KV heads repeated (the library's own grouping convention);
  * closed forms (one token, two tokens, q = 0, scale = 0, equal keys,
    one dominant key, empty sequence);
  * invariances (block-table permutation with a matching pool relayout,
    the merge of per-split partials, scratch vs paged layout of the same data).
A plausible mistake (a dropped max shift that overflows, a wrong sign, the
wrong KV head for a q head, a transposed operand, an off-by-one in the
block/slot split) fails at least one of these.
"""
import math

import numpy as np
import pytest
import torch

import workloads as W
from oracle import attention as A
from oracle import geometry as g


def _tiny_random(seed, S=3, nq=4, nkv=2, D=8, bs=4, lens=(5, 1, 9), pool=12):
    rng = np.random.default_rng(seed)
    perm = rng.permutation(pool)
    nblk = [-(-L // bs) for L in lens]
    tables = np.full((S, max(nblk)), -1, np.int32)
    off = 0
    for s, n in enumerate(nblk):
        tables[s, :n] = perm[off:off + n]
        off += n
    q = W.f32_to_bf16_bits(rng.standard_normal((S, nq, D), np.float32))
    k = W.f32_to_bf16_bits(rng.standard_normal((pool, bs, nkv, D), np.float32))
    v = W.f32_to_bf16_bits(rng.standard_normal((pool, bs, nkv, D), np.float32))
    return q, k, v, tables, np.array(lens, np.int32)


def _f(bits):
    return float(W.bf16_bits_to_f32(np.array([bits], np.uint16))[0])


def _brute(q, k, v, tables, lens, scale):
    S, nq, D = q.shape
    _, bs, nkv, _ = k.shape
    G = nq // nkv
    out = [[None] * nq for _ in range(S)]
    for s in range(S):
        for h in range(nq):
            kvh = h // G
            ws, rows = [], []
            for t in range(int(lens[s])):
                blk = int(tables[s][t // bs])
                slot = t % bs
                dot = math.fsum(_f(q[s, h, d]) * _f(k[blk, slot, kvh, d]) for d in range(D))
                ws.append(math.exp(scale * dot))
                rows.append([_f(v[blk, slot, kvh, d]) for d in range(D)])
            if not ws:
                out[s][h] = [0.0] * D
                continue
            tot = math.fsum(ws)
            out[s][h] = [math.fsum(w * r[d] for w, r in zip(ws, rows)) / tot for d in range(D)]
    return np.array(out)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_matches_brute_force(seed):
    q, k, v, tables, lens = _tiny_random(seed)
    scale = float(np.float32(0.35))
    out, m, l = A.paged_decode(q, k, v, tables, lens, scale)
    ref = _brute(q, k, v, tables, lens, scale)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-13)


def test_matches_torch_sdpa_fp64_tiny_workload():
    inp = W.make_paged("tiny", canary=True)
    out, m, l = A.paged_decode(inp.q, inp.k_cache, inp.v_cache, inp.block_tables,
                               inp.seq_lens, inp.scale)
    G = inp.num_q_heads // inp.num_kv_heads
    for s in range(inp.num_seqs):
        L = int(inp.seq_lens[s])
        ids = inp.block_tables[s, :-(-L // inp.block_size)]
        kk = W.bf16_bits_to_f32(inp.k_cache[ids]).reshape(-1, inp.num_kv_heads, inp.head_dim)[:L]
        vv = W.bf16_bits_to_f32(inp.v_cache[ids]).reshape(-1, inp.num_kv_heads, inp.head_dim)[:L]
        Kt = torch.from_numpy(kk.astype(np.float64)).permute(1, 0, 2)       # [nkv, L, D]
        Vt = torch.from_numpy(vv.astype(np.float64)).permute(1, 0, 2)
        Kt = Kt.repeat_interleave(G, dim=0)
        Vt = Vt.repeat_interleave(G, dim=0)
        Qt = torch.from_numpy(W.bf16_bits_to_f32(inp.q[s]).astype(np.float64))[:, None, :]
        ref = torch.nn.functional.scaled_dot_product_attention(
            Qt[None], Kt[None], Vt[None], scale=inp.scale)[0, :, 0, :].numpy()
        np.testing.assert_allclose(out[s], ref, rtol=1e-12, atol=1e-12)
        assert not np.isnan(out[s]).any()       # NaN canaries never reached


def test_single_token_is_its_value():
    q, k, v, tables, lens = _tiny_random(3, lens=(1, 1, 1))
    out, m, l = A.paged_decode(q, k, v, tables, lens, 0.7)
    for s in range(3):
        for h in range(4):
            blk = tables[s, 0]
            np.testing.assert_array_equal(out[s, h], A.decode_bf16(v[blk, 0, h // 2]))
            assert l[s, h] == 1.0


def test_two_token_closed_form():
    # q = a e0, k0 = b0 e0, k1 = b1 e0 -> s_i = scale a b_i; out = v0 + sigmoid(s1 - s0) (v1 - v0)
    D, bs = 8, 4
    q = np.zeros((1, 1, D), np.float32); q[0, 0, 0] = 2.0
    k = np.zeros((1, bs, 1, D), np.float32); k[0, 0, 0, 0] = 1.5; k[0, 1, 0, 0] = -0.5
    v = np.zeros((1, bs, 1, D), np.float32); v[0, 0, 0, :] = 1.0; v[0, 1, 0, :] = 3.0
    tables = np.array([[0]], np.int32)
    lens = np.array([2], np.int32)
    scale = 0.5
    out, m, l = A.paged_decode(W.f32_to_bf16_bits(q), W.f32_to_bf16_bits(k),
                               W.f32_to_bf16_bits(v), tables, lens, scale)
    s0, s1 = 0.5 * 2.0 * 1.5, 0.5 * 2.0 * -0.5
    w1 = 1.0 / (1.0 + math.exp(s0 - s1))
    np.testing.assert_allclose(out[0, 0], 1.0 + w1 * 2.0, rtol=1e-15)
    assert m[0, 0] == s0
    np.testing.assert_allclose(l[0, 0], 1.0 + math.exp(s1 - s0), rtol=1e-15)


def test_dominant_key_selects_its_value():
    # a large positive score wins (softmax, not softmin, and no sign slip)
    q, k, v, tables, lens = _tiny_random(4, lens=(9, 9, 9))
    q[:] = W.f32_to_bf16_bits(np.zeros(q.shape, np.float32))
    q[:, :, 0] = W.f32_to_bf16_bits(np.array([4.0], np.float32))[0]
    k[:, :, :, 0] = W.f32_to_bf16_bits(np.array([0.0], np.float32))[0]
    blk = tables[1, 1]
    k[blk, 2, :, 0] = W.f32_to_bf16_bits(np.array([64.0], np.float32))[0]   # token 6 of seq 1
    out, _, _ = A.paged_decode(q, k, v, tables, lens, 1.0)
    for h in range(4):
        np.testing.assert_allclose(out[1, h], A.decode_bf16(v[blk, 2, h // 2]), atol=1e-100)


@pytest.mark.parametrize("case", ["q_zero", "scale_zero", "keys_equal"])
def test_uniform_weights_give_mean_of_values(case):
    q, k, v, tables, lens = _tiny_random(5, lens=(7, 3, 11))
    scale = 0.9
    if case == "q_zero":
        q[:] = 0
    elif case == "scale_zero":
        scale = 0.0
    else:
        k[:] = k[0, 0, 0, :]
    out, _, l = A.paged_decode(q, k, v, tables, lens, scale)
    for s in range(3):
        L = int(lens[s])
        for h in range(4):
            vals = np.array([A.decode_bf16(v[tables[s][t // 4], t % 4, h // 2]) for t in range(L)])
            np.testing.assert_allclose(out[s, h], vals.mean(axis=0), rtol=1e-13, atol=1e-15)
            np.testing.assert_allclose(l[s, h], L, rtol=1e-13)


def test_empty_sequence():
    q, k, v, tables, lens = _tiny_random(6, lens=(0, 5, 0))
    out, m, l = A.paged_decode(q, k, v, tables, lens, 0.5)
    for s in (0, 2):
        assert np.all(out[s] == 0) and np.all(m[s] == -np.inf) and np.all(l[s] == 0)
    assert np.all(np.isfinite(out[1]))


def test_gqa_head_mapping():
    # every KV head holds a constant value row; q head h must see kv head h // G
    q, k, v, tables, lens = _tiny_random(7, S=1, nq=6, nkv=3, lens=(10,), pool=4)
    for kvh in range(3):
        v[:, :, kvh, :] = W.f32_to_bf16_bits(np.array([kvh + 1.0], np.float32))[0]
    out, _, _ = A.paged_decode(q, k, v, tables, lens, 0.3)
    for h in range(6):
        np.testing.assert_allclose(out[0, h], h // 2 + 1.0, rtol=1e-14)


def test_large_scores_do_not_overflow():
    # the max shift keeps exp finite where a naive exp(s) overflows
    q, k, v, tables, lens = _tiny_random(8)
    out, m, l = A.paged_decode(q, k, v, tables, lens, 2000.0)
    assert np.all(np.isfinite(out)) and np.all(l >= 1.0)


def test_block_permutation_invariance():
    inp = W.make_paged("tiny", canary=True)
    base, m0, l0 = A.paged_decode(inp.q, inp.k_cache, inp.v_cache, inp.block_tables,
                                  inp.seq_lens, inp.scale)
    rng = np.random.default_rng(99)
    perm = rng.permutation(inp.num_blocks)        # new location of every block
    k2 = np.empty_like(inp.k_cache); v2 = np.empty_like(inp.v_cache)
    k2[perm] = inp.k_cache
    v2[perm] = inp.v_cache
    t2 = np.where(inp.block_tables >= 0, perm[np.maximum(inp.block_tables, 0)], -1).astype(np.int32)
    out, m, l = A.paged_decode(inp.q, k2, v2, t2, inp.seq_lens, inp.scale)
    np.testing.assert_array_equal(out, base)
    np.testing.assert_array_equal(m, m0)
    np.testing.assert_array_equal(l, l0)


@pytest.mark.parametrize("n", [1, 2, 4, 16])
def test_split_partials_merge_to_one_pass(n):
    inp = W.make_paged("tiny", canary=True)
    args = (inp.q, inp.k_cache, inp.v_cache, inp.block_tables, inp.seq_lens, inp.scale)
    out, m, l = A.paged_decode(*args)
    po, pm, pl = A.split_partials(*args, n)
    S, nq = m.shape
    for s in range(S):
        ranges = g.split_ranges(int(inp.seq_lens[s]), n, inp.block_size)
        for h in range(nq):
            for i, (b, e) in enumerate(ranges):
                if e == b:
                    assert pm[s, h, i] == -np.inf and pl[s, h, i] == 0
                    assert np.all(po[s, h, i] == 0)
            live = [i for i, (b, e) in enumerate(ranges) if e > b]
            M = max(pm[s, h, i] for i in live)
            w = {i: math.exp(pm[s, h, i] - M) for i in live}
            Ls = math.fsum(w[i] * pl[s, h, i] for i in live)
            O = sum(w[i] * po[s, h, i] for i in live)
            assert M == m[s, h]
            np.testing.assert_allclose(Ls, l[s, h], rtol=1e-13)
            np.testing.assert_allclose(O / Ls, out[s, h], rtol=1e-12, atol=1e-13)


def test_scratch_layout_agrees_with_paged_layout():
    w = W.Workload(name="t", seed=11, num_seqs=5, num_q_heads=8, num_kv_heads=2,
                   head_dim=16, block_size=8, seq_lens=(0, 1, 7, 8, 29), layout="scratch",
                   tile_capacity=2)
    sc = W.make_scratch(w, canary=True)
    out, m, l, o = A.tiled_state(sc.q, sc.pool, sc.slot_tables, sc.seq_lens)
    # the same data in the paged layout [block, slot, kv_head, dim]
    kp = np.ascontiguousarray(sc.pool[:, 0].transpose(0, 2, 1, 3))
    vp = np.ascontiguousarray(sc.pool[:, 1].transpose(0, 2, 1, 3))
    out2, m2, l2 = A.paged_decode(sc.q, kp, vp, sc.slot_tables, sc.seq_lens, A.tiled_scale(16))
    np.testing.assert_array_equal(out, out2)
    np.testing.assert_array_equal(m, m2)
    np.testing.assert_array_equal(l, l2)
    assert A.tiled_scale(256) == 0.0625
    assert np.all(out[0] == 0) and np.all(l[0] == 0)


def test_generator_recipe():
    inp = W.make_paged("tiny", canary=True)
    assert list(inp.seq_lens) == [37, 100]
    assert inp.k_cache.shape == (32, 16, 2, 128)
    # blocks are a seeded permutation of the pool, handed out in sequence order
    perm = np.random.default_rng(0).permutation(32)
    assert list(inp.block_tables[0, :3]) == list(perm[:3])
    assert list(inp.block_tables[1, :7]) == list(perm[3:10])
    assert np.all(inp.block_tables[0, 3:] == -1)
    # tail slots past the sequence end hold NaN canaries
    last = inp.block_tables[0, 2]
    assert np.all(np.isnan(W.bf16_bits_to_f32(inp.k_cache[last, 37 - 32:])))
    assert not np.any(np.isnan(W.bf16_bits_to_f32(inp.k_cache[last, :37 - 32])))
    lens = W.draw_seq_lens(W.WORKLOADS["batch"])
    assert lens.min() >= 512 and lens.max() <= 4096 and len(lens) == 32
    lens = W.draw_seq_lens(W.WORKLOADS["tiled"])
    assert list(lens[:6]) == [0, 1, 31, 32, 2048, 16384] and lens[127] == 0
    # RNE to bf16: 1 + 2^-8 is a tie and goes to even (1.0); 1 + 3*2^-8 rounds up
    x = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -2.5, np.nan], np.float32)
    b = W.f32_to_bf16_bits(x)
    assert list(b[:3]) == [0x3F80, 0x3F82, 0xC020] and b[3] == 0x7FC0
