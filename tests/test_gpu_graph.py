"""The decode calls, the tiled step and the causal prefill inside a captured
HIP graph (torch.cuda.CUDAGraph on the library's stream argument): every
replay, with eager work and synchronisations between replays, gives the
eager bytes.  Needs an MI355X."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

import dataclasses

import workloads as W
from tests.gpu_util import PagedOnDevice, ScratchOnDevice, dev_i32, dev_u16, host_bits, say

import paged_decode_attention_splitk_amd as P


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _capture(fn):
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()   # warm-up outside the graph
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


# 1 packed: the packed kernel's 2 parts (sequences of 33 blocks or more);
# 4 packed: its split-K form; "long": 24 q / 4 kv heads at D 128 with a
# 40000-token sequence, whose items use 2 parts at 16 splits and 8 at 1
@pytest.mark.parametrize("n,flags", [(1, "unpacked"), (16, "unpacked"), (1, "packed"),
                                     (4, "packed"), (16, "long"), (1, "long")])
def test_decode_graph_replays(n, flags):
    say(f"[graph] splits={n} {flags}")
    if flags == "long":
        base = W.Workload(name="graph-long", seed=32, num_seqs=3, num_q_heads=24,
                          num_kv_heads=4, head_dim=128, block_size=16,
                          seq_lens=(40000, 9000, 300))
    else:
        base = W.Workload(name="graph", seed=30, num_seqs=12, num_q_heads=32, num_kv_heads=4,
                          head_dim=256, block_size=16, len_range=(1, 1500))
    inp = W.make_paged(base, canary=True)
    dev = PagedOnDevice(inp)
    S, nq, D = inp.num_seqs, inp.num_q_heads, inp.head_dim
    fl = P.PDA_DECODE_PACKED if flags == "packed" else P.PDA_DECODE_UNPACKED
    out = torch.empty((S, nq, D), dtype=torch.bfloat16, device="cuda")
    wsf = P.pda_workspace_slots(S, nq, n, D) if n > 1 else 0
    ws = torch.zeros(max(wsf, 1), dtype=torch.float32, device="cuda")

    def call():
        P.pda_paged_decode(dev.q, dev.k, dev.v, dev.bt, dev.lens, out, ws if wsf else None, wsf,
                           S, nq, inp.num_kv_heads, D, inp.block_size, dev.bt.shape[1],
                           inp.num_blocks, inp.scale, n, fl)

    call()
    torch.cuda.synchronize()
    eager = host_bits(out).copy()
    g = _capture(call)
    for r in range(3):
        out.fill_(0)                     # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host_bits(out), eager), f"replay {r} differs"
        call()                           # an eager call between replays
        torch.cuda.synchronize()
        assert np.array_equal(host_bits(out), eager)


def test_tiled_step_graph_replays():
    """begin_step (a fill kernel, no memset), step_tile and finalize of the
    tiled API in one graph."""
    sc = W.make_scratch(W.Workload(name="tgraph", seed=31, num_seqs=6, num_q_heads=16,
                                   num_kv_heads=4, head_dim=256, block_size=32,
                                   len_range=(0, 3000), layout="scratch", tile_capacity=64),
                        canary=True)
    dev = ScratchOnDevice(sc)
    S = sc.num_seqs
    h = P.TiledAttention(S, sc.num_q_heads, sc.num_kv_heads, sc.head_dim, sc.block_size, 64)
    strides = h.scratch_pool_strides()
    k_ptr = dev.pool.data_ptr()
    v_ptr = k_ptr + dev.v_off_bytes
    calls = W.plan_tiles([sc.slot_tables[s] for s in range(S)],
                         [int(x) for x in sc.seq_lens], sc.block_size, 64)
    tiles = [(dev_i32(np.array(tb, np.int32).reshape(S, 64)), dev_i32(np.array(cnt, np.int32)),
              lbvs) for tb, cnt, lbvs in calls]
    out = torch.empty((S, sc.num_q_heads, sc.head_dim), dtype=torch.bfloat16, device="cuda")
    say(f"[graph tiled] calls={len(tiles)}")

    def step():
        h.begin_step(S)
        for tbd, cd, lbvs in tiles:
            h.step_tile(dev.q, k_ptr, v_ptr, sc.num_slots, tbd, cd, S, strides, lbvs)
        h.finalize(out, S)

    step()
    torch.cuda.synchronize()
    eager = host_bits(out).copy()
    g = _capture(step)
    for r in range(3):
        out.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host_bits(out), eager), f"replay {r} differs"
        step()
        torch.cuda.synchronize()
    h.close()


# the causal prefill (a kernel launch only): both staging forms, block size
# 16 (uniform block base per 16-row piece) and 8 (per-row table reads)
@pytest.mark.parametrize("bs", [16, 8])
def test_prefill_graph_replays(bs):
    w = dataclasses.replace(W.WORKLOADS["prefill"], seed=33, num_q_heads=16, num_kv_heads=2,
                            block_size=bs)
    pi = W.make_prefill(w, canary=True, q_len=300, kv_len=1000, q_offset=700)
    q, k, v = dev_u16(pi.q), dev_u16(pi.k_cache), dev_u16(pi.v_cache)
    bt = dev_i32(pi.block_table)
    out = torch.empty((pi.q_len, pi.num_q_heads, pi.head_dim), dtype=torch.bfloat16,
                      device="cuda")
    say(f"[graph prefill] bs={bs}")

    def call():
        P.pda_paged_prefill(q, k, v, out, bt, pi.q_len, pi.kv_len, pi.q_offset,
                            pi.num_q_heads, pi.num_kv_heads, pi.head_dim, pi.block_size,
                            len(pi.block_table), pi.num_blocks, pi.scale)

    call()
    torch.cuda.synchronize()
    eager = host_bits(out).copy()
    g = _capture(call)
    for r in range(3):
        out.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host_bits(out), eager), f"replay {r} differs"
        call()
        torch.cuda.synchronize()
        assert np.array_equal(host_bits(out), eager)
