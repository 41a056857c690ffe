"""Helpers for the GPU parity tests: upload generated inputs with torch, run
the HIP path through the C-ABI binding, and compare with the oracle.

Tolerances (from the target statement of this library):
  BF16 outputs: |gpu - oracle| <= 1.6e-2 + 1e-2 * |oracle|, elementwise;
  FP32 m and l: |gpu - oracle| <= 1e-4 * |oracle| (+1e-6 when |oracle| < 1e-2),
                with -inf and 0 matched exactly.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import paged_decode_attention_splitk_amd as P
import workloads as W

ATOL_OUT, RTOL_OUT = 1.6e-2, 1e-2
RTOL_ML = 1e-4


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev_u16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to("cuda").view(torch.bfloat16)


def dev_i32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to("cuda")


def host_bf16(t: torch.Tensor) -> np.ndarray:
    """bf16 device tensor -> float64 numpy (exact)."""
    u = t.detach().view(torch.int16).cpu().numpy().view(np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def assert_out_close(gpu: np.ndarray, ref: np.ndarray, what: str = "out"):
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite GPU values"
    err = np.abs(gpu - ref)
    bound = ATOL_OUT + RTOL_OUT * np.abs(ref)
    bad = err > bound
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} elements outside tolerance; "
                             f"max err {err.max():.3e}; first {idx.tolist()} "
                             f"gpu {gpu[tuple(idx[0])]} ref {ref[tuple(idx[0])]}")


def assert_ml_close(gpu: np.ndarray, ref: np.ndarray, what: str):
    gpu = np.asarray(gpu, np.float64)
    ninf = ref == -np.inf
    assert np.array_equal(gpu == -np.inf, ninf), f"{what}: -inf pattern differs"
    zero = ref == 0
    assert np.array_equal(gpu[~ninf] == 0, zero[~ninf]), f"{what}: zero pattern differs"
    fin = ~ninf & ~zero
    r = ref[fin]
    tol = RTOL_ML * np.abs(r) + np.where(np.abs(r) < 1e-2, 1e-6, 0.0)
    err = np.abs(gpu[fin] - r)
    assert np.all(err <= tol), f"{what}: max rel err {np.max(err / np.maximum(np.abs(r), 1e-30)):.3e}"


class PagedOnDevice:
    """Device copies of a PagedInputs batch."""

    def __init__(self, inp):
        self.inp = inp
        self.q = dev_u16(inp.q)
        self.k = dev_u16(inp.k_cache)
        self.v = dev_u16(inp.v_cache)
        self.bt = dev_i32(inp.block_tables)
        self.lens = dev_i32(inp.seq_lens)

    def run(self, num_splits, packed=False, rows=None, out=None, ws=None, flags=None):
        """Run pda_paged_decode; ``rows`` restricts to a subset of sequences
        (their q rows / table rows / lengths, against the same pool).
        ``flags`` (a PDA_DECODE_* value) overrides ``packed``."""
        inp = self.inp
        q, bt, lens = self.q, self.bt, self.lens
        if rows is not None:
            idx = torch.as_tensor(rows, device="cuda", dtype=torch.long)
            q, bt, lens = q[idx].contiguous(), bt[idx].contiguous(), lens[idx].contiguous()
        S = q.shape[0]
        nq, D = inp.num_q_heads, inp.head_dim
        if out is None:
            out = torch.empty((S, nq, D), dtype=torch.bfloat16, device="cuda")
        wsf = P.pda_workspace_slots(S, nq, num_splits, D) if num_splits > 1 else 0
        if ws is None and wsf:
            ws = torch.full((wsf,), float("nan"), dtype=torch.float32, device="cuda")
        rc = P.pda_paged_decode(q, self.k, self.v, bt, lens, out, ws, wsf, S, nq,
                                inp.num_kv_heads, D, inp.block_size, bt.shape[1],
                                inp.num_blocks, inp.scale, num_splits,
                                flags if flags is not None else
                                (P.PDA_DECODE_PACKED if packed else P.PDA_DECODE_UNPACKED))
        torch.cuda.synchronize()
        return rc, out, ws


class ScratchOnDevice:
    """Device copies of a ScratchInputs batch (pool uploaded once)."""

    def __init__(self, sc):
        self.sc = sc
        self.q = dev_u16(sc.q)
        self.pool = dev_u16(sc.pool)
        self.v_off_bytes = 2 * sc.num_kv_heads * sc.block_size * sc.head_dim

    def run(self, tile_capacity, rows=None, handle=None):
        """Fold the sequences ``rows`` (default: all) through the tiled API
        with the plan of workloads.plan_tiles; returns (out bf16 tensor, m, l, o)."""
        sc = self.sc
        rows = list(range(sc.num_seqs)) if rows is None else list(rows)
        S = len(rows)
        q = self.q[torch.as_tensor(rows, device="cuda", dtype=torch.long)].contiguous()
        own = handle is None
        if own:
            handle = P.TiledAttention(max(S, 1), sc.num_q_heads, sc.num_kv_heads, sc.head_dim,
                                      sc.block_size, tile_capacity)
        strides = handle.scratch_pool_strides()
        k_ptr = self.pool.data_ptr()
        v_ptr = k_ptr + self.v_off_bytes
        calls = W.plan_tiles([sc.slot_tables[s] for s in rows],
                             [int(sc.seq_lens[s]) for s in rows], sc.block_size, tile_capacity)
        handle.begin_step(S)
        keep = []
        for tb, cnt, lbvs in calls:
            tbd = dev_i32(np.array(tb, np.int32).reshape(S, tile_capacity))
            cd = dev_i32(np.array(cnt, np.int32))
            keep.append((tbd, cd))
            handle.step_tile(q, k_ptr, v_ptr, sc.num_slots, tbd, cd, S, strides, lbvs)
        out = torch.empty((S, sc.num_q_heads, sc.head_dim), dtype=torch.bfloat16, device="cuda")
        handle.finalize(out, S)
        torch.cuda.synchronize()
        m_p, l_p, o_p = handle.state()
        nqs = S * sc.num_q_heads
        m = _read_f32(m_p, nqs).reshape(S, sc.num_q_heads)
        l = _read_f32(l_p, nqs).reshape(S, sc.num_q_heads)
        o = _read_f32(o_p, nqs * sc.head_dim).reshape(S, sc.num_q_heads, sc.head_dim)
        if own:
            handle.close()
        del keep
        return out, m, l, o


def _read_f32(ptr: int, n: int) -> np.ndarray:
    import ctypes
    host = np.empty(n, np.float32)
    if n == 0:
        return host
    hip = ctypes.CDLL("libamdhip64.so.7")   # the copy torch already loaded
    hip.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
    hip.hipMemcpy.restype = ctypes.c_int
    rc = hip.hipMemcpy(host.ctypes.data, ptr, n * 4, 2)   # hipMemcpyDeviceToHost
    assert rc == 0, rc
    return host


def dev_u8(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to("cuda")


class PagedFP8OnDevice:
    """Device copies of a PagedFP8Inputs batch."""

    def __init__(self, inp):
        self.inp = inp
        self.q = dev_u16(inp.q)
        self.k = dev_u8(inp.k8)
        self.v = dev_u8(inp.v8)
        self.bt = dev_i32(inp.block_tables)
        self.lens = dev_i32(inp.seq_lens)

    def run(self, num_splits, rows=None, flags=None, scale=None, k_scale=None, v_scale=None):
        """Run pda_paged_decode_fp8 (optionally on a subset of sequences);
        returns (rc, out, ws).  A non-OK return code is returned, not raised."""
        inp = self.inp
        q, bt, lens = self.q, self.bt, self.lens
        if rows is not None:
            idx = torch.as_tensor(rows, device="cuda", dtype=torch.long)
            q, bt, lens = q[idx].contiguous(), bt[idx].contiguous(), lens[idx].contiguous()
        S = q.shape[0]
        nq, D = inp.num_q_heads, inp.head_dim
        out = torch.empty((S, nq, D), dtype=torch.bfloat16, device="cuda")
        wsf = P.pda_workspace_slots(S, nq, num_splits, D) if num_splits > 1 else 0
        ws = (torch.full((wsf,), float("nan"), dtype=torch.float32, device="cuda")
              if wsf else None)
        try:
            rc = P.pda_paged_decode_fp8(
                q, self.k, self.v, bt, lens, out, ws, wsf, S, nq, inp.num_kv_heads, D,
                inp.block_size, bt.shape[1], inp.num_blocks,
                inp.scale if scale is None else scale,
                inp.k_scale if k_scale is None else k_scale,
                inp.v_scale if v_scale is None else v_scale, num_splits,
                P.PDA_DECODE_UNPACKED if flags is None else flags)
        except P.PdaError as e:
            return e.code, out, ws
        torch.cuda.synchronize()
        return rc, out, ws
