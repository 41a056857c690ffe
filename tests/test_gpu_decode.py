"""GPU parity of the one-shot paged decode (split-K kernel + merge) against
the FP64 oracle, through the C ABI.  Needs an MI355X."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

import workloads as W
from oracle import attention as A
from oracle import geometry as g
from tests.gpu_util import (PagedOnDevice, assert_ml_close, assert_out_close, host_bf16,
                            host_bits, say)

import paged_decode_attention_splitk_amd as P

CU = 256   # the workloads are stated for 256 compute units


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _check_partials(dev, ws, n):
    inp = dev.inp
    S, nq, D = inp.num_seqs, inp.num_q_heads, inp.head_dim
    w = ws.cpu().numpy().reshape(S, nq, n, D + 2).astype(np.float64)
    po, pm, pl = A.split_partials(inp.q, inp.k_cache, inp.v_cache, inp.block_tables,
                                  inp.seq_lens, inp.scale, n)
    assert_ml_close(w[..., D], pm, "workspace m")
    assert_ml_close(w[..., D + 1], pl, "workspace l")
    live = pl > 0
    assert_out_close(w[..., :D][live] / w[..., D + 1][live][:, None],
                     po[live] / pl[live][:, None], "workspace o / l")


@pytest.mark.parametrize("n", [1, 4])
def test_tiny_workload(n):
    say(f"[tiny] splits={n}")
    inp = W.make_paged("tiny", canary=True)        # NaN canaries in unused blocks and tails
    dev = PagedOnDevice(inp)
    rc, out, ws = dev.run(n)
    assert rc == P.PDA_OK
    ref, m, l = A.paged_decode(inp.q, inp.k_cache, inp.v_cache, inp.block_tables,
                               inp.seq_lens, inp.scale)
    assert_out_close(host_bf16(out), ref)
    if n > 1:
        _check_partials(dev, ws, n)


def test_batch_workload_auto_full_size():
    n = P.pda_auto_splits(CU, 32)
    assert n == 16
    say(f"[batch] splits={n} device CUs={P.pda_device_cu_count(0)}")
    inp = W.make_paged("batch", canary=True)
    dev = PagedOnDevice(inp)
    rc, out, ws = dev.run(n)
    ref, m, l = A.paged_decode(inp.q, inp.k_cache, inp.v_cache, inp.block_tables,
                               inp.seq_lens, inp.scale)
    assert_out_close(host_bf16(out), ref)
    # workspace m / l / o of every split of every sequence
    _check_partials(dev, ws, n)
    # the same call again gives the same bytes, and so does each row alone
    _, out2, _ = dev.run(n)
    assert np.array_equal(host_bits(out), host_bits(out2))
    _each_row_alone(dev, host_bits(out), n, "batch")


def test_long_sequence_clamped_splits():
    n = P.pda_auto_splits(CU, 24)
    assert n == g.MAX_DECODE_SPLITS == 16
    say(f"[long] splits={n}")
    inp = W.make_paged("long", canary=True)
    dev = PagedOnDevice(inp)
    rc, out, ws = dev.run(n)
    ref, m, l = A.paged_decode(inp.q, inp.k_cache, inp.v_cache, inp.block_tables,
                               inp.seq_lens, inp.scale)
    assert_out_close(host_bf16(out), ref)
    _check_partials(dev, ws, n)


_PACKED_REF = {}


def _packed_reference(inp):
    """The oracle's output for every row of the packed workload (computed
    once per module: about 4 s on the host)."""
    if "out" not in _PACKED_REF:
        ref, _, _ = A.paged_decode(inp.q, inp.k_cache, inp.v_cache, inp.block_tables,
                                   inp.seq_lens, inp.scale)
        _PACKED_REF["out"] = ref
    return _PACKED_REF["out"]


def _each_row_alone(dev, full, n, what, **kw):
    """Every row's output bytes alone equal its bytes in the whole batch."""
    for s in range(dev.inp.num_seqs):
        _, one, _ = dev.run(n, rows=[s], **kw)
        assert np.array_equal(host_bits(one)[0], full[s]), f"{what}: seq {s} differs alone"


@pytest.mark.parametrize("n", [1, 16])
def test_packed_shape_unpacked_path(n):
    """The unpacked split-K path on the packed workload (64 sequences of
    1K-8K tokens, 32 q / 4 kv heads, head dim 256): all 64 rows against the
    oracle, and each row alone vs co-batched."""
    say(f"[packed-shape unpacked] splits={n}")
    inp = W.make_paged("packed", canary=True)
    dev = PagedOnDevice(inp)
    rc, out, ws = dev.run(n)
    assert rc == P.PDA_OK
    assert_out_close(host_bf16(out), _packed_reference(inp), f"unpacked splits={n}")
    _each_row_alone(dev, host_bits(out), n, f"unpacked splits={n}")


@pytest.mark.parametrize("lens", [(1, 1, 1), (0, 5, 0, 16), (15, 16, 17, 63, 64, 65, 1000)])
def test_edge_lengths(lens):
    say(f"[edge] lens={lens}")
    base = W.Workload(name="edge", seed=7, num_seqs=len(lens), num_q_heads=8, num_kv_heads=2,
                      head_dim=128, block_size=16, seq_lens=tuple(lens))
    inp = W.make_paged(base, canary=True)
    dev = PagedOnDevice(inp)
    ref, _, _ = A.paged_decode(inp.q, inp.k_cache, inp.v_cache, inp.block_tables, inp.seq_lens,
                               inp.scale)
    for n in (1, 3, 16):
        rc, out, ws = dev.run(n)
        got = host_bf16(out)
        assert_out_close(got, ref, f"splits={n}")
        for s, L in enumerate(lens):
            if L == 0:
                assert np.all(host_bits(out)[s] == 0)
            if L == 1:
                # one token: p = 1, l = 1, so out is v_0 exactly
                blk = inp.block_tables[s, 0]
                v0 = inp.v_cache[blk, 0]
                G = inp.num_q_heads // inp.num_kv_heads
                for h in range(inp.num_q_heads):
                    assert np.array_equal(host_bits(out)[s, h], v0[h // G])


@pytest.mark.parametrize("D,nq,nkv", [(64, 4, 4), (128, 6, 1), (256, 16, 2), (128, 40, 4)])
def test_other_shapes(D, nq, nkv):
    say(f"[shape] D={D} nq={nq} nkv={nkv}")
    base = W.Workload(name="shape", seed=8, num_seqs=3, num_q_heads=nq, num_kv_heads=nkv,
                      head_dim=D, block_size=32, seq_lens=(100, 700, 33))
    inp = W.make_paged(base, canary=True, scale=0.07)
    dev = PagedOnDevice(inp)
    ref, _, _ = A.paged_decode(inp.q, inp.k_cache, inp.v_cache, inp.block_tables, inp.seq_lens,
                               inp.scale)
    for n in (1, 5):
        rc, out, ws = dev.run(n)
        assert_out_close(host_bf16(out), ref, f"splits={n}")


@pytest.mark.parametrize("bs,D", [(64, 128), (128, 64), (48, 256)])
def test_larger_blocks(bs, D):
    """Block sizes past one group of tokens (several groups per block, and a
    non-power-of-two block), with ragged tails, at 1, 7 and 16 splits."""
    say(f"[blocks] bs={bs} D={D}")
    lens = (1, bs - 1, bs, bs + 1, 5 * bs + 3, 2000)
    base = W.Workload(name="blocks", seed=15, num_seqs=len(lens), num_q_heads=8, num_kv_heads=2,
                      head_dim=D, block_size=bs, seq_lens=lens)
    inp = W.make_paged(base, canary=True)
    dev = PagedOnDevice(inp)
    ref, _, _ = A.paged_decode(inp.q, inp.k_cache, inp.v_cache, inp.block_tables, inp.seq_lens,
                               inp.scale)
    for n in (1, 7, 16):
        rc, out, ws = dev.run(n)
        assert rc == P.PDA_OK
        assert_out_close(host_bf16(out), ref, f"bs={bs} splits={n}")
        if n > 1:
            _check_partials(dev, ws, n)


def test_many_sequences_maximum_splits():
    """A large batch (600 sequences: the unranked schedule past 64) of short
    and empty sequences at the split ceiling, sampled rows against the
    oracle, and every output row alone vs co-batched for a sample."""
    base = W.Workload(name="many", seed=16, num_seqs=600, num_q_heads=16, num_kv_heads=2,
                      head_dim=128, block_size=16, len_range=(0, 300))
    inp = W.make_paged(base, canary=True)
    dev = PagedOnDevice(inp)
    n = P.pda_max_decode_splits()
    say(f"[many] seqs=600 splits={n}")
    rc, out, _ = dev.run(n)
    assert rc == P.PDA_OK
    rows = [0, 1, 63, 64, 65, 299, 598, 599]
    sub = W.subset_paged(inp, rows)
    ref, _, _ = A.paged_decode(sub.q, sub.k_cache, sub.v_cache, sub.block_tables, sub.seq_lens,
                               sub.scale)
    assert_out_close(host_bf16(out)[rows], ref, "many")
    full = host_bits(out)
    for s in rows:
        _, one, _ = dev.run(n, rows=[s])
        assert np.array_equal(host_bits(one)[0], full[s]), f"seq {s} differs alone"
    empty = np.flatnonzero(inp.seq_lens == 0)
    assert np.all(full[empty] == 0)


def test_batch_invariance_auto_and_pinned():
    """Each sequence's output bytes are the same alone and co-batched with
    127 others, under Auto and Pinned split counts."""
    base = W.Workload(name="inv", seed=9, num_seqs=128, num_q_heads=32, num_kv_heads=8,
                      head_dim=128, block_size=16, len_range=(1, 2048))
    inp = W.make_paged(base, canary=True)
    dev = PagedOnDevice(inp)
    for n in (P.pda_num_splits(P.PDA_SPLITK_AUTO, 0, CU, 32, 128, 0),
              P.pda_num_splits(P.PDA_SPLITK_PINNED, 5, CU, 32, 128, 0)):
        say(f"[invariance] splits={n}")
        _, out, _ = dev.run(n)
        full = host_bits(out)
        for s in range(128):
            _, one, _ = dev.run(n, rows=[s])
            assert np.array_equal(host_bits(one)[0], full[s]), f"seq {s} differs alone (n={n})"


def test_packed_mfma_workload():
    """GQA-packed MFMA kernel (8 q heads x head_dim 256 per workgroup, one
    split) on the packed workload, against the oracle and the unpacked path."""
    say("[packed mfma]")
    inp = W.make_paged("packed", canary=True)
    assert P.pda_gqa_pack_shape_ok(32, 4, 256)
    dev = PagedOnDevice(inp)
    rc, out, _ = dev.run(1, packed=True)
    assert rc == P.PDA_OK
    ref = _packed_reference(inp)
    got = host_bf16(out)
    assert_out_close(got, ref, "packed")
    _, out_u, _ = dev.run(1)
    assert_out_close(host_bf16(out_u), ref, "unpacked")
    # batch invariance of the packed launch, every row
    _each_row_alone(dev, host_bits(out), 1, "packed", packed=True)


def test_packed_split_k_workload():
    """The packed kernel's split-K form (this library's extension) at the Auto
    split count on the packed workload: all 64 rows against the oracle, the
    workspace m / l of every split of every row against the oracle's split
    partials, and each row alone vs co-batched."""
    inp = W.make_paged("packed", canary=True)
    n = P.pda_auto_splits(CU, inp.num_q_heads)
    say(f"[packed split-K] splits={n}")
    dev = PagedOnDevice(inp)
    rc, out, ws = dev.run(n, packed=True)
    assert rc == P.PDA_OK
    assert_out_close(host_bf16(out), _packed_reference(inp), "packed split-K")
    S, nq, D = inp.num_seqs, inp.num_q_heads, inp.head_dim
    wsn = ws.cpu().numpy().reshape(S, nq, n, D + 2).astype(np.float64)
    say("[packed split-K] oracle split partials, all rows")
    po, pm, pl = A.split_partials(inp.q, inp.k_cache, inp.v_cache, inp.block_tables,
                                  inp.seq_lens, inp.scale, n)
    assert_ml_close(wsn[..., D], pm, "packed workspace m")
    assert_ml_close(wsn[..., D + 1], pl, "packed workspace l")
    live = pl > 0
    assert_out_close(wsn[..., :D][live] / wsn[..., D + 1][live][:, None],
                     po[live] / pl[live][:, None], "packed workspace o / l")
    _each_row_alone(dev, host_bits(out), n, "packed split-K", packed=True)


@pytest.mark.parametrize("bs", [16, 32])
def test_packed_mfma_edges(bs):
    lens = (0, 1, 15, 16, 17, 100, 333)
    say(f"[packed edges] bs={bs}")
    base = W.Workload(name="pedge", seed=14, num_seqs=len(lens), num_q_heads=16, num_kv_heads=2,
                      head_dim=256, block_size=bs, seq_lens=lens)
    inp = W.make_paged(base, canary=True)
    dev = PagedOnDevice(inp)
    rc, out, _ = dev.run(1, packed=True)
    assert rc == P.PDA_OK
    ref, _, _ = A.paged_decode(inp.q, inp.k_cache, inp.v_cache, inp.block_tables, inp.seq_lens,
                               inp.scale)
    assert_out_close(host_bf16(out), ref, "packed edges")
    assert np.all(host_bits(out)[0] == 0)
    # the split-K form: same workspace partials as the oracle's splits, merged
    for n in (2, 5, 16):
        rc, out_n, ws = dev.run(n, packed=True)
        assert rc == P.PDA_OK
        assert_out_close(host_bf16(out_n), ref, f"packed split-K n={n}")
        assert np.all(host_bits(out_n)[0] == 0)
        _check_partials(dev, ws, n)


def test_legacy_negative_control():
    """Under Legacy the split count follows the batch once it passes
    max_decode_seqs, so a sequence's split-K state (its workspace partials,
    and with them the rounding of its output) depends on what it is batched
    with; under Auto the output bytes do not (attn_splitk page: the module
    comment and its invariants).  Both stay within tolerance of the oracle.
    The BF16 outputs of two split counts differ by FP32 rounding only, so on a
    small batch they may or may not differ in a visible bit; the partials
    always do."""
    base = W.Workload(name="legacy", seed=15, num_seqs=16, num_q_heads=8, num_kv_heads=2,
                      head_dim=128, block_size=16, len_range=(300, 1200))
    inp = W.make_paged(base, canary=True)
    dev = PagedOnDevice(inp)
    ref, _, _ = A.paged_decode(inp.q, inp.k_cache, inp.v_cache, inp.block_tables, inp.seq_lens,
                               inp.scale)
    rows = [0, 1, 2, 3]
    mds = 4   # max_decode_seqs
    n_small = P.pda_num_splits(P.PDA_SPLITK_LEGACY, 0, CU, 8, len(rows), mds)
    n_big = P.pda_num_splits(P.PDA_SPLITK_LEGACY, 0, CU, 8, 16, mds)
    assert (n_small, n_big) == (8, 2)        # 256 // (8 * 4), 256 // (8 * 16)
    say(f"[legacy control] splits {n_small} / {n_big}")
    _, small, ws_small = dev.run(n_small, rows=rows)
    _, big, ws_big = dev.run(n_big)
    assert_out_close(host_bf16(small), ref[rows], "legacy, 4 rows")
    assert_out_close(host_bf16(big), ref, "legacy, 16 rows")
    D, nq = inp.head_dim, inp.num_q_heads
    a = ws_small.cpu().numpy().reshape(len(rows), nq, n_small, D + 2)[0]
    b = ws_big.cpu().numpy().reshape(16, nq, n_big, D + 2)[0]
    # sequence 0's first split covers a different token range in the two
    # batches, so its (m, l) differ
    assert not np.array_equal(a[:, 0, D:], b[:, 0, D:])
    flips = int((host_bits(small) != host_bits(big)[rows]).sum())
    say(f"[legacy control] output elements that differ: {flips}")
    n_a4 = P.pda_num_splits(P.PDA_SPLITK_AUTO, 0, CU, 8, len(rows), mds)
    n_a16 = P.pda_num_splits(P.PDA_SPLITK_AUTO, 0, CU, 8, 16, mds)
    assert n_a4 == n_a16
    _, a_small, _ = dev.run(n_a4, rows=rows)
    _, a_big, _ = dev.run(n_a16)
    assert np.array_equal(host_bits(a_small), host_bits(a_big)[rows])


def _pack_shape_inputs():
    base = W.Workload(name="pdefault", seed=16, num_seqs=5, num_q_heads=16, num_kv_heads=2,
                      head_dim=256, block_size=16, seq_lens=(7, 100, 257, 16, 1000))
    return W.make_paged(base, canary=True)


def test_default_flag_follows_gqa_pack_switch():
    """PDA_DECODE_DEFAULT runs the packed kernel exactly when
    pda_gqa_pack_enabled() (resolved once per process) and the launch is one
    it serves; otherwise the unpacked path, and never NOT_APPLICABLE."""
    inp = _pack_shape_inputs()
    dev = PagedOnDevice(inp)
    rc, d1, _ = dev.run(1, flags=P.PDA_DECODE_DEFAULT)
    assert rc == P.PDA_OK
    _, pk, _ = dev.run(1, packed=True)
    _, up, _ = dev.run(1)
    want = pk if P.pda_gqa_pack_enabled() else up
    assert np.array_equal(host_bits(d1), host_bits(want))
    # a split launch never takes the packed kernel
    rc, d4, _ = dev.run(4, flags=P.PDA_DECODE_DEFAULT)
    assert rc == P.PDA_OK
    _, u4, _ = dev.run(4)
    assert np.array_equal(host_bits(d4), host_bits(u4))


_DEFAULT_CHILD = r"""
import sys
sys.path.insert(0, sys.argv[1])
import numpy as np, torch
import paged_decode_attention_splitk_amd as P
from tests.gpu_util import PagedOnDevice, host_bits
from tests.test_gpu_decode import _pack_shape_inputs
assert P.pda_gqa_pack_enabled()
dev = PagedOnDevice(_pack_shape_inputs())
_, d, _ = dev.run(1, flags=P.PDA_DECODE_DEFAULT)
_, pk, _ = dev.run(1, packed=True)
_, up, _ = dev.run(1)
assert np.array_equal(host_bits(d), host_bits(pk))
assert not np.array_equal(host_bits(pk), host_bits(up))
print("default->packed ok", flush=True)
"""


def test_default_flag_with_pack_switched_on_in_env():
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    env = dict(os.environ, METRALE_ATTN_DECODE_GQA_PACK="on")
    say("[default flag, pack on] child process")
    r = subprocess.run([sys.executable, "-c", _DEFAULT_CHILD, root], env=env, cwd=root,
                       capture_output=True, text=True, timeout=240)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]
    assert "default->packed ok" in r.stdout
