"""GPU parity of the fold kernel's parts form: one-shot launches that give a
sequence few (KV head, split) items split each item over several
workgroups, whose last one to finish combines their records.  Checked
against the FP64 oracle, for batch invariance (a sequence's bytes alone and
co-batched, also across runs of sequences that the library launches
separately), and for repeatability (the arrival tickets are back at zero
after every launch).  The GQA-packed MFMA kernel's non-split launch and the
tiled step have the same form (the tiled one with the running state joining
the combine), checked at several tile capacities.  Needs an MI355X."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

import workloads as W
from oracle import attention as A
from tests.gpu_util import (PagedFP8OnDevice, PagedOnDevice, ScratchOnDevice, assert_ml_close,
                            assert_out_close, host_bf16, host_bits, say)

import paged_decode_attention_splitk_amd as P


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _partials_close(inp, ws, n):
    S, nq, D = inp.num_seqs, inp.num_q_heads, inp.head_dim
    w = ws.cpu().numpy().reshape(S, nq, n, D + 2).astype(np.float64)
    po, pm, pl = A.split_partials(inp.q, inp.k_cache, inp.v_cache, inp.block_tables,
                                  inp.seq_lens, inp.scale, n)
    assert_ml_close(w[..., D], pm, "workspace m")
    assert_ml_close(w[..., D + 1], pl, "workspace l")
    live = pl > 0
    assert_out_close(w[..., :D][live] / w[..., D + 1][live][:, None],
                     po[live] / pl[live][:, None], "workspace o / l")


# 24 q / 4 kv heads at D 128 (the long-sequence shape): at 16 splits a
# sequence has 64 items, so an item may use 4 workgroups; at 1 and 3 splits
# 8.  An item uses one part per 128 of its blocks, up to that: the
# 40000-token sequence 2 (16 splits), 7 (3 splits) or 8 (1 split); the
# 9000-token one 1, 2 or 5.  Lengths: empty, ragged tails, a split shorter
# than a part.
@pytest.mark.parametrize("n", [16, 3, 1])
def test_oneshot_parts_few_items(n):
    w = W.Workload(name="parts", seed=21, num_seqs=4, num_q_heads=24, num_kv_heads=4,
                   head_dim=128, block_size=16, seq_lens=(0, 40000, 17, 9000))
    inp = W.make_paged(w, canary=True)
    dev = PagedOnDevice(inp)
    say(f"[parts one-shot] splits={n} lens={list(inp.seq_lens)}")
    rc, out, ws = dev.run(n)
    assert rc == P.PDA_OK
    ref, _, _ = A.paged_decode(inp.q, inp.k_cache, inp.v_cache, inp.block_tables,
                               inp.seq_lens, inp.scale)
    assert_out_close(host_bf16(out), ref, "parts out")
    if n > 1:
        _partials_close(inp, ws, n)
    full = host_bits(out)
    assert np.all(full[0] == 0)
    # a second launch finds the tickets at zero: same bytes
    _, again, _ = dev.run(n)
    assert np.array_equal(host_bits(again), full)
    for s in range(4):
        _, one, _ = dev.run(n, rows=[s])
        assert np.array_equal(host_bits(one)[0], full[s]), f"seq {s} differs alone (n={n})"


def test_oneshot_parts_in_several_launches():
    """45 sequences at the long-sequence shape, one of 40000 tokens (so an
    item may use 2 parts at 16 splits), need more part records than one
    launch may use, so the library launches runs of them (40 rows, then 5);
    each row still matches the oracle and its bytes alone."""
    w = W.Workload(name="parts-runs", seed=22, num_seqs=45, num_q_heads=24, num_kv_heads=4,
                   head_dim=128, block_size=16, len_range=(0, 700), forced=((3, 40000),))
    inp = W.make_paged(w, canary=True)
    dev = PagedOnDevice(inp)
    n = 16
    say(f"[parts runs] seqs=45 splits={n}")
    rc, out, _ = dev.run(n)
    assert rc == P.PDA_OK
    rows = [0, 1, 3, 38, 39, 40, 41, 44]
    sub = W.subset_paged(inp, rows)
    ref, _, _ = A.paged_decode(sub.q, sub.k_cache, sub.v_cache, sub.block_tables, sub.seq_lens,
                               sub.scale)
    assert_out_close(host_bf16(out)[rows], ref, "parts runs out")
    full = host_bits(out)
    for s in rows:
        _, one, _ = dev.run(n, rows=[s])
        assert np.array_equal(host_bits(one)[0], full[s]), f"seq {s} differs alone"


# tiled launches: capacity 16 gives 1 part per tile, 32 gives 2, 40 and 128
# give 3; a sequence's tile of n blocks uses one part per 16 of them, up to
# that (so 1-block tail tiles fold in one workgroup)
@pytest.mark.parametrize("cap", [16, 32, 40, 128])
def test_tiled_capacities(cap):
    w = W.Workload(name="tiled-parts", seed=23, num_seqs=8, num_q_heads=16, num_kv_heads=4,
                   head_dim=256, block_size=32,
                   seq_lens=(0, 1, 31, 32, 33, 700, 2100, 5000), layout="scratch",
                   tile_capacity=cap)
    sc = W.make_scratch(w, canary=True)
    dev = ScratchOnDevice(sc)
    say(f"[tiled capacity] capacity={cap}")
    rows = list(range(8))
    out, m, l, o = dev.run(cap)
    ref, rm, rl, ro = A.tiled_state(sc.q, sc.pool, sc.slot_tables, sc.seq_lens)
    assert_out_close(host_bf16(out), ref, "tiled out")
    assert_ml_close(m, rm, "state m")
    assert_ml_close(l, rl, "state l")
    live = rl > 0
    assert_out_close(o[live] / l[live][:, None], ro[live] / rl[live][:, None], "state o / l")
    full = host_bits(out)
    assert np.all(full[0] == 0)
    again, *_ = dev.run(cap)
    assert np.array_equal(host_bits(again), full)
    for s in rows:
        one, _, _, _ = dev.run(cap, rows=[s])
        assert np.array_equal(host_bits(one)[0], full[s]), f"seq {s} differs alone (cap={cap})"


def test_packed_parts_in_several_launches():
    """The packed MFMA kernel's non-split launch splits each (sequence, KV
    head) of 33 blocks or more over 2 workgroups; 300 sequences of the packed
    shape need more part records than one launch may use, so the library runs
    several launches.
    Sampled rows match the oracle, every sampled row has the same bytes
    alone, and a repeated call gives the same bytes (tickets back at 0)."""
    # most sequences are short (one part: under 64 blocks); the forced long
    # ones use 2 parts, on both sides of the launch boundary at 252 rows
    w = W.Workload(name="packed-runs", seed=24, num_seqs=300, num_q_heads=32, num_kv_heads=4,
                   head_dim=256, block_size=16, len_range=(0, 400),
                   forced=((0, 1500), (251, 1200), (252, 2000), (299, 900)))
    inp = W.make_paged(w, canary=True)
    dev = PagedOnDevice(inp)
    say("[packed parts runs] seqs=300")
    rc, out, _ = dev.run(1, packed=True)
    assert rc == P.PDA_OK
    rows = [0, 1, 150, 250, 251, 252, 253, 299]
    sub = W.subset_paged(inp, rows)
    ref, _, _ = A.paged_decode(sub.q, sub.k_cache, sub.v_cache, sub.block_tables, sub.seq_lens,
                               sub.scale)
    assert_out_close(host_bf16(out)[rows], ref, "packed parts runs")
    full = host_bits(out)
    _, again, _ = dev.run(1, packed=True)
    assert np.array_equal(host_bits(again), full)
    for s in rows:
        _, one, _ = dev.run(1, packed=True, rows=[s])
        assert np.array_equal(host_bits(one)[0], full[s]), f"packed seq {s} differs alone"


def test_part_users_interleaved():
    """Launches that hand records over (a few-item split-K fold, the packed
    non-split kernel, a tiled step) run one after another on one stream in
    several orders; each gives the bytes it gives alone, so none leaves a
    ticket or record behind that another one reads."""
    lw = W.Workload(name="mix-long", seed=25, num_seqs=2, num_q_heads=24, num_kv_heads=4,
                    head_dim=128, block_size=16, seq_lens=(3000, 1200))
    pw = W.Workload(name="mix-packed", seed=26, num_seqs=3, num_q_heads=32, num_kv_heads=4,
                    head_dim=256, block_size=16, seq_lens=(900, 40, 1700))
    tw = W.Workload(name="mix-tiled", seed=27, num_seqs=3, num_q_heads=16, num_kv_heads=4,
                    head_dim=256, block_size=32, seq_lens=(2500, 0, 700), layout="scratch",
                    tile_capacity=64)
    ld = PagedOnDevice(W.make_paged(lw, canary=True))
    pd = PagedOnDevice(W.make_paged(pw, canary=True))
    td = ScratchOnDevice(W.make_scratch(tw, canary=True))
    say("[parts interleaved]")
    base_l = host_bits(ld.run(3)[1])
    base_p = host_bits(pd.run(1, packed=True)[1])
    base_t = host_bits(td.run(64)[0])
    for order in ("lpt", "tpl", "ptl", "llpptt"):
        for c in order:
            if c == "l":
                assert np.array_equal(host_bits(ld.run(3)[1]), base_l), order
            elif c == "p":
                assert np.array_equal(host_bits(pd.run(1, packed=True)[1]), base_p), order
            else:
                assert np.array_equal(host_bits(td.run(64)[0]), base_t), order


# More shapes with several parts per item: head dim 64 with 8 heads per KV
# head (a 40000-token sequence at 4 splits: 5 parts per item), head dim 256
# with 2 heads per KV head (2 splits: 8 parts), each against the oracle and
# alone vs co-batched.
@pytest.mark.parametrize("D,nq,nkv,n", [(64, 16, 2, 4), (256, 8, 4, 2)])
def test_oneshot_parts_other_shapes(D, nq, nkv, n):
    w = W.Workload(name=f"parts-d{D}", seed=28, num_seqs=3, num_q_heads=nq, num_kv_heads=nkv,
                   head_dim=D, block_size=16, seq_lens=(40000, 300, 0))
    inp = W.make_paged(w, canary=True)
    dev = PagedOnDevice(inp)
    say(f"[parts shapes] D={D} nq={nq} nkv={nkv} splits={n}")
    rc, out, ws = dev.run(n)
    assert rc == P.PDA_OK
    ref, _, _ = A.paged_decode(inp.q, inp.k_cache, inp.v_cache, inp.block_tables,
                               inp.seq_lens, inp.scale)
    assert_out_close(host_bf16(out), ref, f"parts D={D}")
    if n > 1:
        _partials_close(inp, ws, n)
    full = host_bits(out)
    for s in range(3):
        _, one, _ = dev.run(n, rows=[s])
        assert np.array_equal(host_bits(one)[0], full[s]), f"seq {s} differs alone (D={D})"


def test_oneshot_parts_fp8():
    """The FP8 fold's parts form: the long-sequence shape with an E4M3 cache
    and a 40000-token sequence (2 parts per item at 16 splits) against the
    FP8 oracle, and alone vs co-batched."""
    from oracle import fp8 as F
    w = W.Workload(name="parts-fp8", seed=29, num_seqs=3, num_q_heads=24, num_kv_heads=4,
                   head_dim=128, block_size=16, seq_lens=(40000, 2000, 0))
    inp = W.make_paged_fp8(w, canary=True)
    dev = PagedFP8OnDevice(inp)
    say("[parts fp8] splits=16")
    rc, out, _ = dev.run(16)
    assert rc == P.PDA_OK
    ref = F.paged_decode_fp8(inp.q, inp.k8, inp.v8, inp.block_tables, inp.seq_lens, inp.scale,
                             inp.k_scale, inp.v_scale)
    assert_out_close(host_bf16(out), ref, "parts fp8")
    full = host_bits(out)
    for s in range(3):
        _, one, _ = dev.run(16, rows=[s])
        assert np.array_equal(host_bits(one)[0], full[s]), f"fp8 seq {s} differs alone"
