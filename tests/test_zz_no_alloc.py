"""GPU test of pda_paged_decode_noalloc, the entry point that allocates
nothing (its split-K workspace is the library's per-GPU scratch array):
through the C ABI, its output bytes equal pda_paged_decode's with a
caller-owned workspace, and both are within tolerance of the FP64 oracle, on
two calls in a row (the second smaller, so it runs over the first call's
scratch contents).  Needs an MI355X."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

import workloads as W
from oracle import attention as A
from tests.gpu_util import PagedOnDevice, assert_out_close, host_bf16, host_bits, say

import paged_decode_attention_splitk_amd as P


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _noalloc(dev, n, flags=P.PDA_DECODE_UNPACKED):
    inp = dev.inp
    S, nq, D = inp.num_seqs, inp.num_q_heads, inp.head_dim
    out = torch.full((S, nq, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    rc = P.pda_paged_decode_noalloc(dev.q, dev.k, dev.v, dev.bt, dev.lens, out, S, nq,
                                    inp.num_kv_heads, D, inp.block_size, dev.bt.shape[1],
                                    inp.num_blocks, inp.scale, n, flags)
    torch.cuda.synchronize()
    return rc, out


def _reference(inp):
    ref, _, _ = A.paged_decode(inp.q, inp.k_cache, inp.v_cache, inp.block_tables,
                               inp.seq_lens, inp.scale)
    return ref


def test_noalloc_matches_workspace_entry_point_two_calls():
    # call 1: the batch decode shape (32 sequences of 512-4096 tokens, 32 q / 8
    # kv heads, D 128) at 16 splits -- 2129920 scratch floats
    big = PagedOnDevice(W.make_paged("batch", canary=True))
    n1 = P.pda_auto_splits(256, 32)
    say(f"[noalloc] call 1: batch, splits={n1}")
    rc, out1 = _noalloc(big, n1)
    assert rc == P.PDA_OK
    rc, want1, _ = big.run(n1)
    assert rc == P.PDA_OK
    assert np.array_equal(host_bits(out1), host_bits(want1))
    assert_out_close(host_bf16(out1), _reference(big.inp))

    # call 2: the tiny shape (2 sequences, 8 q / 2 kv heads) at 4 splits, over
    # the scratch the first call left behind
    small = PagedOnDevice(W.make_paged("tiny", canary=True))
    say("[noalloc] call 2: tiny, splits=4")
    rc, out2 = _noalloc(small, 4)
    assert rc == P.PDA_OK
    rc, want2, _ = small.run(4)
    assert rc == P.PDA_OK
    assert np.array_equal(host_bits(out2), host_bits(want2))
    assert_out_close(host_bf16(out2), _reference(small.inp))


def test_noalloc_parts_and_single_split():
    # the long single sequence (131072 tokens) splits each item into parts;
    # one split uses no scratch
    inp = W.make_paged("long", canary=False)
    dev = PagedOnDevice(inp)
    n = P.pda_auto_splits(256, inp.num_q_heads)
    for splits in (n, 1):
        say(f"[noalloc] long, splits={splits}")
        rc, got = _noalloc(dev, splits)
        assert rc == P.PDA_OK
        rc, want, _ = dev.run(splits)
        assert rc == P.PDA_OK
        assert np.array_equal(host_bits(got), host_bits(want))
    assert_out_close(host_bf16(got), _reference(inp))


def test_noalloc_refuses_a_workspace_past_its_scratch():
    # 64 sequences x 32 heads x 16 splits x 130 floats = 4259840 > 4194304;
    # every buffer is sized for the call (zero lengths), so even a launch
    # would stay in bounds
    S, nq, nkv, D, bs, mb, nb = 64, 32, 8, 128, 16, 4, 8
    q = torch.zeros((S, nq, D), dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros((nb, bs, nkv, D), dtype=torch.bfloat16, device="cuda")
    bt = torch.zeros((S, mb), dtype=torch.int32, device="cuda")
    lens = torch.zeros((S,), dtype=torch.int32, device="cuda")
    out = torch.empty((S, nq, D), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(P.PdaError) as e:
        P.pda_paged_decode_noalloc(q, kv, kv, bt, lens, out, S, nq, nkv, D, bs, mb, nb,
                                   D ** -0.5, 16)
    assert e.value.code == P.PDA_EINVAL
    assert "workspace" in P.pda_last_error()
    # 63 sequences fit (4193280 floats)
    assert P.pda_paged_decode_noalloc(q, kv, kv, bt, lens, out, S - 1, nq, nkv, D, bs, mb, nb,
                                      D ** -0.5, 16) == P.PDA_OK
    torch.cuda.synchronize()
    assert not host_bits(out[:S - 1]).any()   # zero-length sequences give 0


def test_noalloc_replays_in_a_hip_graph():
    # the callers it is for include code under graph capture: the call
    # captures (it launches kernels only) and every replay, with eager work
    # and synchronisations between, gives the eager bytes
    inp = W.make_paged("tiny", canary=True)
    dev = PagedOnDevice(inp)
    S, nq, D = inp.num_seqs, inp.num_q_heads, inp.head_dim
    rc, want = _noalloc(dev, 4)
    assert rc == P.PDA_OK
    out = torch.zeros((S, nq, D), dtype=torch.bfloat16, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        P.pda_paged_decode_noalloc(dev.q, dev.k, dev.v, dev.bt, dev.lens, out, S, nq,
                                   inp.num_kv_heads, D, inp.block_size, dev.bt.shape[1],
                                   inp.num_blocks, inp.scale, 4, stream=s.cuda_stream)
    torch.cuda.synchronize()
    for r in range(3):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        say(f"[noalloc graph] replay {r}")
        assert np.array_equal(host_bits(out), host_bits(want))
        _noalloc(dev, 16)   # eager use of the same scratch between replays
