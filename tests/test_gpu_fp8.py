"""GPU parity of the paged decode over an FP8 (OCP E4M3) KV cache against the
FP64 oracle, through the C ABI.  Needs an MI355X.

Exact checks use what the arithmetic fixes: E4M3 values decode exactly to
BF16 / FP32, a power-of-two scale multiplies exactly, and a one-token
sequence returns its V row times v_scale."""
import dataclasses

import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

import workloads as W
from oracle import attention as A
from oracle import fp8 as F
from tests.gpu_util import (PagedFP8OnDevice, assert_ml_close, assert_out_close, host_bf16,
                            host_bits, say)

import paged_decode_attention_splitk_amd as P

CU = 256


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _ref(f, rows=None):
    if rows is None:
        return F.paged_decode_fp8(f.q, f.k8, f.v8, f.block_tables, f.seq_lens, f.scale,
                                  f.k_scale, f.v_scale)
    rows = list(rows)
    return F.paged_decode_fp8(f.q[rows], f.k8, f.v8, f.block_tables[rows], f.seq_lens[rows],
                              f.scale, f.k_scale, f.v_scale)


@pytest.mark.parametrize("n", [1, 4])
def test_tiny_workload(n):
    say(f"[fp8 tiny] splits={n}")
    f = W.make_paged_fp8("tiny", canary=True)     # E4M3 NaN codes in unused blocks and tails
    dev = PagedFP8OnDevice(f)
    rc, out, _ = dev.run(n)
    assert rc == P.PDA_OK
    assert_out_close(host_bf16(out), _ref(f))


def test_batch_shape_auto_splits():
    """The batch decode shape (32 seqs, U[512, 4096], 32 q / 8 kv, D 128) with
    an FP8 cache under the Auto split count; every output element checked."""
    n = P.pda_auto_splits(CU, 32)
    say(f"[fp8 batch] splits={n}")
    f = W.make_paged_fp8("batch", canary=True)
    dev = PagedFP8OnDevice(f)
    rc, out, _ = dev.run(n)
    assert rc == P.PDA_OK
    assert_out_close(host_bf16(out), _ref(f))
    _, out2, _ = dev.run(n)
    assert np.array_equal(host_bits(out), host_bits(out2))


def test_partials_power_of_two_scales():
    """With power-of-two scales the cache's values are exact in BF16, so the
    workspace m / l / o of every split match the BF16 oracle's partials on
    those values."""
    w = dataclasses.replace(W.WORKLOADS["tiny"], seed=11, seq_lens=(37, 300))
    f = W.make_paged_fp8(w, canary=True, k_scale=0.25, v_scale=0.5)
    n = 4
    dev = PagedFP8OnDevice(f)
    rc, out, ws = dev.run(n)
    assert rc == P.PDA_OK
    kb = W.f32_to_bf16_bits((F.decode_e4m3(f.k8) * f.k_scale).astype(np.float32))
    vb = W.f32_to_bf16_bits((F.decode_e4m3(f.v8) * f.v_scale).astype(np.float32))
    S, nq, D = f.num_seqs, f.num_q_heads, f.head_dim
    po, pm, pl = A.split_partials(f.q, kb, vb, f.block_tables, f.seq_lens, f.scale, n)
    wsn = ws.cpu().numpy().reshape(S, nq, n, D + 2).astype(np.float64)
    assert_ml_close(wsn[..., D], pm, "workspace m")
    assert_ml_close(wsn[..., D + 1], pl, "workspace l")
    live = pl > 0
    assert_out_close(wsn[..., :D][live] / wsn[..., D + 1][live][:, None],
                     po[live] / pl[live][:, None], "workspace o / l")
    assert_out_close(host_bf16(out), _ref(f))


@pytest.mark.parametrize("lens", [(1, 1, 1), (0, 5, 0, 16), (15, 16, 17, 63, 64, 65, 1000)])
def test_edge_lengths(lens):
    say(f"[fp8 edge] lens={lens}")
    base = W.Workload(name="edge8", seed=17, num_seqs=len(lens), num_q_heads=8, num_kv_heads=2,
                      head_dim=128, block_size=16, seq_lens=tuple(lens))
    f = W.make_paged_fp8(base, canary=True)
    dev = PagedFP8OnDevice(f)
    ref = _ref(f)
    G = f.num_q_heads // f.num_kv_heads
    for n in (1, 3, 16):
        rc, out, _ = dev.run(n)
        assert rc == P.PDA_OK
        bits = host_bits(out)
        assert_out_close(host_bf16(out), ref, f"splits={n}")
        for s, L in enumerate(lens):
            if L == 0:
                assert np.all(bits[s] == 0)
            if L == 1:
                # one token: p = 1 and l = 1, so out = BF16(FP32(v_0 * v_scale))
                v0 = F.decode_e4m3(f.v8[f.block_tables[s, 0], 0]).astype(np.float32)
                want = W.f32_to_bf16_bits(v0 * np.float32(f.v_scale))
                for h in range(f.num_q_heads):
                    assert np.array_equal(bits[s, h], want[h // G])


@pytest.mark.parametrize("D,nq,nkv", [(64, 4, 4), (128, 6, 1), (256, 16, 2), (128, 40, 4)])
def test_other_shapes(D, nq, nkv):
    say(f"[fp8 shape] D={D} nq={nq} nkv={nkv}")
    base = W.Workload(name="shape8", seed=18, num_seqs=3, num_q_heads=nq, num_kv_heads=nkv,
                      head_dim=D, block_size=32, seq_lens=(100, 700, 33))
    f = W.make_paged_fp8(base, canary=True, k_scale=0.013, v_scale=0.021)
    dev = PagedFP8OnDevice(f)
    ref = _ref(f)
    for n in (1, 5):
        rc, out, _ = dev.run(n)
        assert rc == P.PDA_OK
        assert_out_close(host_bf16(out), ref, f"splits={n}")


def test_scale_identities_exact():
    """Power-of-two changes of the scales act exactly: 2 * v_scale doubles
    every output value, and (scale / 2, 2 * k_scale) gives the same bytes."""
    base = W.Workload(name="scl8", seed=19, num_seqs=6, num_q_heads=16, num_kv_heads=4,
                      head_dim=128, block_size=16, len_range=(1, 900))
    f = W.make_paged_fp8(base, canary=True)
    dev = PagedFP8OnDevice(f)
    for n in (1, 4):
        _, out, _ = dev.run(n)
        _, out_v2, _ = dev.run(n, v_scale=2 * f.v_scale)
        _, out_k2, _ = dev.run(n, scale=f.scale / 2, k_scale=2 * f.k_scale)
        a = host_bf16(out)
        assert np.array_equal(host_bf16(out_v2), 2 * a)
        assert np.array_equal(host_bits(out_k2), host_bits(out))


def test_batch_invariance():
    """A sequence's output bytes are the same alone and co-batched."""
    base = W.Workload(name="inv8", seed=20, num_seqs=48, num_q_heads=32, num_kv_heads=8,
                      head_dim=128, block_size=16, len_range=(1, 2048))
    f = W.make_paged_fp8(base, canary=True)
    dev = PagedFP8OnDevice(f)
    for n in (P.pda_auto_splits(CU, 32), 5):
        say(f"[fp8 invariance] splits={n}")
        _, out, _ = dev.run(n)
        full = host_bits(out)
        for s in range(f.num_seqs):
            _, one, _ = dev.run(n, rows=[s])
            assert np.array_equal(host_bits(one)[0], full[s]), f"seq {s} differs alone (n={n})"


def test_flags():
    f = W.make_paged_fp8("tiny", canary=True)   # 8 q / 2 kv heads, D 128: no packing
    dev = PagedFP8OnDevice(f)
    rc, _, _ = dev.run(4, flags=P.PDA_DECODE_PACKED)
    assert rc == P.PDA_NOT_APPLICABLE
    rc, out_d, _ = dev.run(4, flags=P.PDA_DECODE_DEFAULT)
    assert rc == P.PDA_OK
    _, out_u, _ = dev.run(4)
    assert np.array_equal(host_bits(out_d), host_bits(out_u))


@pytest.mark.parametrize("bs", [16, 32])
def test_packed_fp8_edges(bs):
    """The GQA-packed MFMA kernel's FP8 form (8 q heads x head_dim 256 per
    workgroup), one split and split-K, on edge lengths."""
    lens = (0, 1, 15, 16, 17, 100, 333, 2000)
    say(f"[fp8 packed edges] bs={bs}")
    base = W.Workload(name="pedge8", seed=21, num_seqs=len(lens), num_q_heads=16,
                      num_kv_heads=2, head_dim=256, block_size=bs, seq_lens=lens)
    f = W.make_paged_fp8(base, canary=True, k_scale=0.011, v_scale=0.017)
    dev = PagedFP8OnDevice(f)
    ref = _ref(f)
    for n in (1, 2, 5, 16):
        rc, out, _ = dev.run(n, flags=P.PDA_DECODE_PACKED)
        assert rc == P.PDA_OK
        assert_out_close(host_bf16(out), ref, f"packed fp8 n={n}")
        assert np.all(host_bits(out)[0] == 0)


def test_packed_fp8_partials_and_invariance():
    """Packed FP8 split-K partials with power-of-two scales against the BF16
    oracle's partials on the same (exact) values; batch invariance."""
    base = W.Workload(name="ppart8", seed=22, num_seqs=6, num_q_heads=32, num_kv_heads=4,
                      head_dim=256, block_size=16, len_range=(1, 3000))
    f = W.make_paged_fp8(base, canary=True, k_scale=0.125, v_scale=0.25)
    dev = PagedFP8OnDevice(f)
    n = 4
    rc, out, ws = dev.run(n, flags=P.PDA_DECODE_PACKED)
    assert rc == P.PDA_OK
    kb = W.f32_to_bf16_bits((F.decode_e4m3(f.k8) * f.k_scale).astype(np.float32))
    vb = W.f32_to_bf16_bits((F.decode_e4m3(f.v8) * f.v_scale).astype(np.float32))
    S, nq, D = f.num_seqs, f.num_q_heads, f.head_dim
    po, pm, pl = A.split_partials(f.q, kb, vb, f.block_tables, f.seq_lens, f.scale, n)
    wsn = ws.cpu().numpy().reshape(S, nq, n, D + 2).astype(np.float64)
    assert_ml_close(wsn[..., D], pm, "packed workspace m")
    assert_ml_close(wsn[..., D + 1], pl, "packed workspace l")
    live = pl > 0
    assert_out_close(wsn[..., :D][live] / wsn[..., D + 1][live][:, None],
                     po[live] / pl[live][:, None], "packed workspace o / l")
    assert_out_close(host_bf16(out), _ref(f), "packed fp8 split-K")
    for nn in (1, n):
        _, full, _ = dev.run(nn, flags=P.PDA_DECODE_PACKED)
        for s in (0, 3, 5):
            _, one, _ = dev.run(nn, rows=[s], flags=P.PDA_DECODE_PACKED)
            assert np.array_equal(host_bits(one)[0], host_bits(full)[s]), (nn, s)


_DEFAULT_CHILD_FP8 = r"""
import sys
sys.path.insert(0, sys.argv[1])
import numpy as np, torch
import paged_decode_attention_splitk_amd as P
import workloads as W
from tests.gpu_util import PagedFP8OnDevice, host_bits
assert P.pda_gqa_pack_enabled()
base = W.Workload(name="pdef8", seed=23, num_seqs=3, num_q_heads=16, num_kv_heads=2,
                  head_dim=256, block_size=16, seq_lens=(5, 300, 1000))
dev = PagedFP8OnDevice(W.make_paged_fp8(base, canary=True))
_, d, _ = dev.run(1, flags=P.PDA_DECODE_DEFAULT)
_, pk, _ = dev.run(1, flags=P.PDA_DECODE_PACKED)
_, up, _ = dev.run(1)
assert np.array_equal(host_bits(d), host_bits(pk))
assert not np.array_equal(host_bits(pk), host_bits(up))
# split launches stay unpacked under the default
_, d4, _ = dev.run(4, flags=P.PDA_DECODE_DEFAULT)
_, u4, _ = dev.run(4)
assert np.array_equal(host_bits(d4), host_bits(u4))
print("fp8 default->packed ok", flush=True)
"""


def test_default_flag_with_pack_switched_on_in_env():
    """With the pack switch on in the environment, the FP8 default dispatch
    takes the packed kernel on non-split launches of the packed shape only,
    as for BF16 caches."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    env = dict(os.environ, METRALE_ATTN_DECODE_GQA_PACK="on")
    say("[fp8 default flag, pack on] child process")
    r = subprocess.run([sys.executable, "-c", _DEFAULT_CHILD_FP8, root], env=env, cwd=root,
                       capture_output=True, text=True, timeout=240)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]
    assert "fp8 default->packed ok" in r.stdout
