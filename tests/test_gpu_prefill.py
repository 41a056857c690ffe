"""GPU parity of the causal paged prefill kernel (pda_paged_prefill) against
the FP64 oracle, through the C ABI.  Needs an MI355X."""
import dataclasses

import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

import workloads as W
from oracle import prefill as PF
from tests.gpu_util import assert_out_close, dev_i32, dev_u16, host_bf16, host_bits, say

import paged_decode_attention_splitk_amd as P


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _run(pi, out=None):
    q, k, v = dev_u16(pi.q), dev_u16(pi.k_cache), dev_u16(pi.v_cache)
    bt = dev_i32(pi.block_table)
    if out is None:
        out = torch.empty((pi.q_len, pi.num_q_heads, pi.head_dim), dtype=torch.bfloat16,
                          device="cuda")
    rc = P.pda_paged_prefill(q, k, v, out, bt, pi.q_len, pi.kv_len, pi.q_offset,
                             pi.num_q_heads, pi.num_kv_heads, pi.head_dim, pi.block_size,
                             len(pi.block_table), pi.num_blocks, pi.scale)
    torch.cuda.synchronize()
    return rc, out


def _small(q_len, kv_len, q_offset, nq=16, nkv=2, bs=16, seed=21):
    w = dataclasses.replace(W.WORKLOADS["prefill"], seed=seed, num_q_heads=nq, num_kv_heads=nkv,
                            block_size=bs)
    return W.make_prefill(w, canary=True, q_len=q_len, kv_len=kv_len, q_offset=q_offset)


@pytest.mark.parametrize("q_len,kv_len,q_offset,nq,nkv,bs", [
    (1, 1, 0, 8, 8, 16),
    (17, 17, 0, 16, 2, 16),
    (130, 130, 0, 16, 2, 16),        # two row tiles, ragged
    (100, 300, 200, 16, 2, 32),      # chunked: rows 200..299
    (64, 50, 0, 8, 4, 16),           # rows past the cache see its 50 keys
    (257, 700, 443, 8, 1, 8),        # odd block size, one KV head
    (300, 1000, 700, 32, 4, 16),
])
def test_small_against_oracle(q_len, kv_len, q_offset, nq, nkv, bs):
    say(f"[prefill] q_len={q_len} kv_len={kv_len} q_offset={q_offset} nq={nq} nkv={nkv} bs={bs}")
    pi = _small(q_len, kv_len, q_offset, nq, nkv, bs)
    rc, out = _run(pi)
    assert rc == P.PDA_OK
    ref = PF.paged_prefill(pi.q, pi.k_cache, pi.v_cache, pi.block_table, pi.kv_len, pi.q_offset,
                           pi.scale)
    assert_out_close(host_bf16(out), ref, "prefill")


def test_first_row_is_v0_and_repeatable():
    pi = _small(40, 40, 0)
    _, out = _run(pi)
    G = pi.num_q_heads // pi.num_kv_heads
    bits = host_bits(out)
    for h in range(pi.num_q_heads):
        assert np.array_equal(bits[0, h], pi.v_cache[pi.block_table[0], 0, h // G])
    _, out2 = _run(pi)
    assert np.array_equal(bits, host_bits(out2))


def test_not_applicable_launches_nothing():
    pi = _small(8, 8, 0)
    q, k, v = dev_u16(pi.q), dev_u16(pi.k_cache), dev_u16(pi.v_cache)
    bt = dev_i32(pi.block_table)
    out = torch.zeros((8, pi.num_q_heads, 256), dtype=torch.bfloat16, device="cuda")
    args = (q, k, v, out, bt, 8, 8, 0, pi.num_q_heads, pi.num_kv_heads)
    tail = (pi.block_size, len(pi.block_table), pi.num_blocks, pi.scale)
    assert P.pda_paged_prefill(*args, 128, *tail) == P.PDA_NOT_APPLICABLE          # head dim
    assert P.pda_paged_prefill(*args, 256, *tail, sliding_window=4) == P.PDA_NOT_APPLICABLE
    torch.cuda.synchronize()
    assert torch.count_nonzero(out.view(torch.int16)).item() == 0


@pytest.mark.parametrize("name,rows", [
    ("prefill", [0, 1, 127, 128, 1000, 2047, 4095]),
    ("prefill_chunk", [0, 5, 1023, 2047]),
])
def test_workload_sampled_rows(name, rows):
    say(f"[prefill workload] {name}")
    pi = W.make_prefill(name, canary=True)
    rc, out = _run(pi)
    assert rc == P.PDA_OK
    ref = PF.paged_prefill(pi.q, pi.k_cache, pi.v_cache, pi.block_table, pi.kv_len, pi.q_offset,
                           pi.scale, rows=rows)
    assert_out_close(host_bf16(out)[rows], ref, name)
