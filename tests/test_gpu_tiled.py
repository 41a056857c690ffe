"""GPU parity of the tiled state API (begin_step / step_tile / finalize)
against the FP64 oracle, and its batch invariance.  Needs an MI355X."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

import workloads as W
from oracle import attention as A
from tests.gpu_util import ScratchOnDevice, assert_ml_close, assert_out_close, host_bf16, host_bits, say

import paged_decode_attention_splitk_amd as P


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _check(sc, rows, out, m, l, o):
    ref, rm, rl, ro = A.tiled_state(sc.q[rows], sc.pool, sc.slot_tables[rows], sc.seq_lens[rows])
    assert_out_close(host_bf16(out), ref, "tiled out")
    assert_ml_close(m, rm, "state m")
    assert_ml_close(l, rl, "state l")
    live = rl > 0
    assert_out_close(o[live] / l[live][:, None], ro[live] / rl[live][:, None], "state o / l")


def test_small_scratch_layout_several_tiles():
    w = W.Workload(name="tiled-small", seed=12, num_seqs=7, num_q_heads=16, num_kv_heads=4,
                   head_dim=256, block_size=32, seq_lens=(0, 1, 31, 32, 33, 700, 2100),
                   layout="scratch", tile_capacity=4)
    say("[tiled small]")
    sc = W.make_scratch(w, canary=True)
    dev = ScratchOnDevice(sc)
    rows = list(range(7))
    out, m, l, o = dev.run(4)
    _check(sc, rows, out, m, l, o)
    assert np.all(host_bits(out)[0] == 0)


def test_tiled_workload_full_size():
    """The tiled workload at full size (128 sequences, 0-16K tokens, head dim
    256, 64-block tiles): every sequence's output and final (m, l, o) state
    against the oracle, and every sequence's output bytes alone equal to its
    bytes co-batched with the other 127."""
    w = W.WORKLOADS["tiled"]
    say("[tiled full] generating")
    sc = W.make_scratch(w, canary=True)
    dev = ScratchOnDevice(sc)
    say("[tiled full] running")
    out, m, l, o = dev.run(w.tile_capacity)
    say("[tiled full] oracle, all 128 sequences")
    _check(sc, list(range(w.num_seqs)), out, m, l, o)
    full = host_bits(out)
    say("[tiled full] each sequence alone")
    for s in range(w.num_seqs):
        one, _, _, _ = dev.run(w.tile_capacity, rows=[s])
        assert np.array_equal(host_bits(one)[0], full[s]), f"seq {s} differs alone"
    assert np.all(full[sc.seq_lens == 0] == 0)


def test_begin_step_bounds_and_reuse():
    w = W.Workload(name="tiled-reuse", seed=13, num_seqs=3, num_q_heads=8, num_kv_heads=2,
                   head_dim=128, block_size=16, seq_lens=(50, 0, 300), layout="scratch",
                   tile_capacity=2)
    sc = W.make_scratch(w, canary=True)
    dev = ScratchOnDevice(sc)
    t = P.TiledAttention(3, 8, 2, 128, 16, 2)
    with pytest.raises(P.PdaError):
        t.begin_step(4)
    # two steps on the same handle: the state is reset by begin_step
    a, *_ = dev.run(2, handle=t)
    b, m, l, o = dev.run(2, handle=t)
    assert np.array_equal(host_bits(a), host_bits(b))
    _check(sc, [0, 1, 2], b, m, l, o)
    t.close()
