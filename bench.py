"""Decode-step benchmark of the MI355X paged-decode attention library.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload batch]

A step is one whole decode pass over one batch: the split-K fold kernel
(q.K^T, online softmax, P.V for every split) and the merge kernel, issued as
the library's two C-ABI calls pda_splitk_partials + pda_splitk_merge (which
is exactly what pda_paged_decode issues).  Inputs are resident in HBM before
the timed region; the KV pool is held in several identical copies used in
rotation, so no step finds its 301 MB of K/V in the 256 MB Infinity Cache
left behind by the step before it.

The default workload is batch decode: 32 sequences, lengths uniform in
[512, 4096] (seed 1), 32 q / 8 kv heads, head_dim 128, block size 16, BF16
N(0,1) data in a shuffled pool, split count from the Auto policy on 256 CUs
(16).  Prints one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
CU_COUNT = 256                 # the workloads are stated for 256 compute units
METRIC = "decode-attention µs/step + achieved HBM GB/s (% of MI355X peak), 32 seqs × 4K ctx"
CSRC = os.path.join(ROOT, "paged_decode_attention_splitk_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")


def alg_bytes(inp, n_splits, kv_elem=2):
    """Algorithmic HBM bytes of one decode step and of its two kernels.

    fold:  K and V of every valid token (num_kv_heads * head_dim * kv_elem B
           each: 2 for BF16, 1 for an E4M3 cache),
           q, the block-table entries and lengths read, the workspace written;
    merge: the workspace read, the BF16 output written.
    """
    import numpy as np
    lens = inp.seq_lens.astype(np.int64)
    S, nq, D = inp.q.shape
    nkv, bs = inp.num_kv_heads, inp.block_size
    kv = int(lens.sum()) * nkv * D * kv_elem * 2
    q = S * nq * D * 2
    tables = int(((lens + bs - 1) // bs).sum()) * 4 + S * 4
    ws = S * nq * n_splits * (D + 2) * 4 if n_splits > 1 else 0
    out = S * nq * D * 2
    fold = kv + q + tables + ws
    merge = ws + out
    return {"kv": kv, "fold": fold, "merge": merge, "step": fold + merge}


def _src_hash(path):
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def load_traffic(profile, kernel):
    """HBM bytes per launch of `kernel` from the committed counter summary
    profiles/<profile>_traffic.json (rocprofv3 FETCH_SIZE / WRITE_SIZE,
    copy-calibrated), or None when missing or taken from a different kernel
    source than the one built here."""
    try:
        rec = json.load(open(os.path.join(PROFILES, f"{profile}_traffic.json")))
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256_16") != _src_hash(os.path.join(CSRC, rec.get("source_file", ""))):
        return None
    if kernel is None:
        return (rec.get("per_step") or {}).get("fold_hbm_bytes_per_step")
    return (rec.get("kernels", {}).get(kernel) or {}).get("hbm_bytes_per_launch")


def profile_of(args, n):
    """(profile name, kernel) of the committed counter summary for the
    kernel a paged bench leg reports, or (None, None) for other settings."""
    fp8 = "true" if args.fp8 else "false"
    if args.workload == "batch" and not args.packed and n == 16:
        return ("fold_fp8_batch" if args.fp8 else "fold_batch",
                f"fold_kernel<0, 128, 4, {fp8}, false>")
    if args.workload == "long" and not args.packed and n == 16:
        return ("long_fp8" if args.fp8 else "long", f"fold_kernel<0, 128, 6, {fp8}, true>")
    if args.workload == "packed" and args.packed and n == 1:
        return ("packed_fp8_nosplit" if args.fp8 else "packed_nosplit",
                f"packed_kernel<false, 8, {fp8}, true>")
    if args.workload == "packed" and args.packed and n == 16 and not args.fp8:
        return "packed_splitk16", "packed_kernel<true, 2, false, false>"
    if args.workload == "packed" and not args.packed and n == 16 and not args.fp8:
        return "unpacked_auto16", "fold_kernel<0, 256, 8, false, false>"
    return None, None


# Inputs the oracle's worker processes read: set before the pool forks, so
# every worker inherits them (copy-on-write) instead of receiving a copy.
_CPU_INP = None
_CPU_FP8 = False


def _oracle_item(item):
    """One work item of the oracle baseline: the query heads of one (sequence,
    KV head) for a BF16 cache, or one whole sequence for an FP8 cache (the
    FP8 oracle works per sequence).  Returns that part of the output."""
    from oracle import attention as A
    from oracle import fp8 as F
    inp = _CPU_INP
    s, kvh = item
    if _CPU_FP8:
        sl = slice(s, s + 1)
        return F.paged_decode_fp8(inp.q[sl], inp.k8, inp.v8, inp.block_tables[sl],
                                  inp.seq_lens[sl], inp.scale, inp.k_scale, inp.v_scale)[0]
    G = inp.q.shape[1] // inp.num_kv_heads
    heads = [(s, h) for h in range(kvh * G, (kvh + 1) * G)]
    out, _, _ = A.paged_decode(inp.q, inp.k_cache, inp.v_cache, inp.block_tables, inp.seq_lens,
                               inp.scale, heads=heads)
    return out[s, kvh * G:(kvh + 1) * G]


def _worker_init():
    from threadpoolctl import threadpool_limits
    threadpool_limits(1)   # one BLAS thread per process: the pool supplies the parallelism


def cpu_baseline(inp, seconds, fp8=False, single_seconds=5.0, max_workers=16):
    """The FP64 oracle, unchanged, on the host cores: a pool of processes, one
    per usable core (at most ``max_workers``), over the batch's (sequence, KV
    head) items, repeated over the whole batch until ``seconds`` have passed
    (at least once); then the same oracle on one thread with one BLAS thread,
    for ``single_seconds``.  Must run before this process touches the GPU:
    the pool is forked.  Returns a dict of timings and core counts."""
    import multiprocessing as mp

    from threadpoolctl import threadpool_limits

    from oracle import attention as A
    from oracle import fp8 as F
    global _CPU_INP, _CPU_FP8
    _CPU_INP, _CPU_FP8 = inp, fp8
    affinity = len(os.sched_getaffinity(0))
    workers = max(1, min(affinity, max_workers))
    S = inp.q.shape[0]
    items = [(s, 0) for s in range(S)] if fp8 else \
        [(s, kvh) for s in range(S) for kvh in range(inp.num_kv_heads)]
    ctx = mp.get_context("fork")
    with ctx.Pool(workers, initializer=_worker_init) as pool:
        pool.map(_oracle_item, items[:workers], chunksize=1)   # workers up and warm
        reps, t0 = 0, time.perf_counter()
        while True:
            pool.map(_oracle_item, items, chunksize=1)
            reps += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                break
    par_s = el / reps
    reps1, t0 = 0, time.perf_counter()
    with threadpool_limits(1):
        while True:
            if fp8:
                F.paged_decode_fp8(inp.q, inp.k8, inp.v8, inp.block_tables, inp.seq_lens,
                                   inp.scale, inp.k_scale, inp.v_scale)
            else:
                A.paged_decode(inp.q, inp.k_cache, inp.v_cache, inp.block_tables,
                               inp.seq_lens, inp.scale)
            reps1 += 1
            el1 = time.perf_counter() - t0
            if el1 >= single_seconds:
                break
    return {"step_s": par_s, "reps": reps, "workers": workers, "items": len(items),
            "affinity": affinity, "cpu_count": os.cpu_count(),
            "single_step_s": el1 / reps1, "single_reps": reps1}


def calibrate_copy():
    """Three plain 1 GiB device-to-device copies: what a counter reads for
    them scales the same counter of the kernels in a counter run."""
    import torch
    src = torch.empty(1 << 29, dtype=torch.int16, device="cuda")   # 1 GiB
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def tiled_bench(args, K):
    """The tiled state API on the scratch-pool workload: a step is
    begin_step, every step_tile call of the workloads.plan_tiles schedule, finalize.
    Returns the JSON record (without cpu_baseline)."""
    import numpy as np
    import torch

    import paged_decode_attention_splitk_amd as P
    import workloads as W

    sc = W.make_scratch(args.workload, canary=False)
    S, nq, D = sc.q.shape
    nkv, bs, cap = sc.num_kv_heads, sc.block_size, sc.workload.tile_capacity
    lens = sc.seq_lens.astype(np.int64)
    calls = W.plan_tiles([sc.slot_tables[s] for s in range(S)], [int(x) for x in lens], bs, cap)
    q = torch.from_numpy(np.ascontiguousarray(sc.q).view(np.int16)).cuda()
    pool = torch.from_numpy(np.ascontiguousarray(sc.pool).view(np.int16)).cuda()
    k_ptr = pool.data_ptr()
    v_ptr = k_ptr + 2 * nkv * bs * D
    dev_calls = [(torch.tensor(np.array(tb, np.int32).reshape(S, cap)).cuda(),
                  torch.tensor(np.array(cnt, np.int32)).cuda(), lbvs) for tb, cnt, lbvs in calls]
    out = torch.empty((S, nq, D), dtype=torch.int16, device="cuda")
    h = P.TiledAttention(S, nq, nkv, D, bs, cap)
    strides = h.scratch_pool_strides()
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream

    def tiles(_i=0):
        for tb, cnt, lbvs in dev_calls:
            h.step_tile(q, k_ptr, v_ptr, sc.num_slots, tb, cnt, S, strides, lbvs, stream=sp)

    def step(_i=0):
        h.begin_step(S, stream=sp)
        tiles()
        h.finalize(out, S, stream=sp)

    if args.calibrate_copy:
        calibrate_copy()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if args.profile_steps:
        for _ in range(args.profile_steps):
            step()
        torch.cuda.synchronize()
        return {"profile_steps": args.profile_steps, "workload": args.workload}

    def timed(fn):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record(stream)
        for i in range(K):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / K, (time.perf_counter() - t0) * 1e3 / K

    gpu_ms, ms_per_step = timed(step)
    tiles_ms, _ = timed(tiles)

    # the same step captured once in a HIP graph and replayed (the library
    # launches kernels only, so the step captures as a whole)
    cap_stream = torch.cuda.Stream()
    cap_stream.wait_stream(stream)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=cap_stream):
        cs = cap_stream.cuda_stream
        h.begin_step(S, stream=cs)
        for tb, cnt, lbvs in dev_calls:
            h.step_tile(q, k_ptr, v_ptr, sc.num_slots, tb, cnt, S, strides, lbvs, stream=cs)
        h.finalize(out, S, stream=cs)
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    g0 = torch.cuda.Event(enable_timing=True)
    g1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    g0.record(stream)
    for _ in range(K):
        graph.replay()
    g1.record(stream)
    torch.cuda.synchronize()
    graph_wall_ms = (time.perf_counter() - t0) * 1e3 / K
    graph_ms = g0.elapsed_time(g1) / K
    # algorithmic bytes: valid K/V once; per active (call, sequence) its q,
    # its tile-table entries and a read + write of its (m, l, o) state; the
    # fill pass writes the state, finalize reads l, o and writes out
    kv = int(lens.sum()) * nkv * D * 2 * 2
    state_slot = nq * (D + 2) * 4
    tiles_b = kv
    for tb, cnt, lbvs in calls:
        active = [c for c in cnt if c > 0]
        tiles_b += len(active) * (nq * D * 2 + 2 * state_slot + 4) + 4 * int(sum(active))
    begin_b = S * state_slot
    fin_b = S * nq * (D + 1) * 4 + S * nq * D * 2
    step_b = tiles_b + begin_b + fin_b
    value = step_b / (ms_per_step * 1e-3) / 1e9
    achieved = tiles_b / (tiles_ms * 1e-3) / 1e9
    return {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": K, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": sc.workload.description, "num_seqs": S, "num_q_heads": nq,
                   "num_kv_heads": nkv, "head_dim": D, "block_size": bs, "tile_capacity": cap,
                   "total_tokens": int(lens.sum()), "step_tile_calls": len(calls),
                   "algorithmic_bytes_per_step": step_b},
        "us_per_step": round(ms_per_step * 1e3, 2),
        "pct_of_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "gpu_event_us_per_step": round(gpu_ms * 1e3, 2),
        "graph_replay_us_per_step": round(graph_wall_ms * 1e3, 2),
        "graph_replay_gpu_event_us_per_step": round(graph_ms * 1e3, 2),
        "kernels_us": {"step_tile_all_calls": round(tiles_ms * 1e3, 2)},
        "roofline": {"kernel": f"tiled fold (fold_kernel<2,{D},{min(nq // nkv, 8)}>), all calls",
                     "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": load_traffic("tiled", None),
                     "algorithmic_bytes_per_step": tiles_b},
    }


def prefill_bench(args, K):
    """Causal paged prefill of one sequence (pda_paged_prefill); reported in
    TFLOP/s of the causal attention (q.k and P.V, 2 flops per multiply-add,
    every unmasked (row, key) pair) against the bf16 MFMA peak."""
    import numpy as np
    import torch

    import paged_decode_attention_splitk_amd as P
    import workloads as W

    pi = W.make_prefill(args.workload, canary=False)
    ql, nq, D = pi.q.shape
    nkv, bs = pi.num_kv_heads, pi.block_size
    up = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()
    q, k, v = up(pi.q), up(pi.k_cache), up(pi.v_cache)
    bt = torch.from_numpy(pi.block_table).cuda()
    out = torch.empty((ql, nq, D), dtype=torch.int16, device="cuda")
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream

    def step(_i=0):
        rc = P.pda_paged_prefill(q, k, v, out, bt, ql, pi.kv_len, pi.q_offset, nq, nkv, D, bs,
                                 len(pi.block_table), pi.num_blocks, pi.scale, stream=sp)
        assert rc == P.PDA_OK

    if args.calibrate_copy:
        calibrate_copy()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if args.profile_steps:
        for _ in range(args.profile_steps):
            step()
        torch.cuda.synchronize()
        return {"profile_steps": args.profile_steps, "workload": args.workload}
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(K):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / K
    gpu_ms = e0.elapsed_time(e1) / K
    keys = np.minimum(pi.q_offset + np.arange(ql) + 1, pi.kv_len).astype(np.int64)
    flops = 4.0 * nq * D * float(keys.sum())
    tflops = flops / (gpu_ms * 1e-3) / 1e12
    kv_bytes = pi.kv_len * nkv * D * 2 * 2
    # block sizes that are multiples of 16 take the uniform-staging instance
    kname = f"prefill_kernel<{'true' if bs % 16 == 0 else 'false'}>"
    return {
        "metric": "causal paged prefill TFLOP/s", "value": round(flops / (ms * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s", "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": pi.workload.description, "q_len": ql, "kv_len": pi.kv_len,
                   "q_offset": pi.q_offset, "num_q_heads": nq, "num_kv_heads": nkv,
                   "head_dim": D, "block_size": bs, "flops_per_step": flops},
        "us_per_step": round(ms * 1e3, 2), "gpu_event_us_per_step": round(gpu_ms * 1e3, 2),
        "roofline": {"kernel": f"causal prefill ({kname})", "bound": "mfma",
                     "achieved": round(tflops, 2), "peak": 2500.0, "unit": "TFLOP/s",
                     "frac": round(tflops / 2500.0, 4),
                     "traffic": load_traffic("prefill_4096" if args.workload == "prefill"
                                             else args.workload, kname),
                     "kv_bytes_per_step": kv_bytes},
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="batch")
    ap.add_argument("--splits", type=int, default=0, help="pin a split count (default: Auto)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--copies", type=int, default=0, help="KV pool copies (default: >= 1 GB)")
    ap.add_argument("--packed", action="store_true",
                    help="run the GQA-packed MFMA kernel (single split; packed workload shape)")
    ap.add_argument("--fp8", action="store_true",
                    help="FP8 (E4M3) KV cache of the same shape (pda_*_fp8 entry points)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 1 GiB device copy (for counter scaling)")
    ap.add_argument("--profile-steps", type=int, default=0,
                    help="for counter runs: only the warm-up and this many steps (every "
                         "one on a cold KV copy), then a short JSON line")
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py runs on one GPU only: this library has no multi-GPU path "
              "(see the sharding note in DESIGN.md); use --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np

    import workloads as W

    layout = W.WORKLOADS[args.workload].layout
    inp = cpu = None
    if layout == "paged":
        inp = (W.make_paged_fp8(args.workload, canary=False) if args.fp8 else
               W.make_paged(args.workload, canary=False))
        if not args.no_cpu:
            # before anything touches the GPU: the oracle's pool is forked
            cpu = cpu_baseline(inp, args.cpu_seconds, args.fp8)

    import torch

    import paged_decode_attention_splitk_amd as P

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    dev_cus = P.pda_device_cu_count(0)

    if layout == "scratch":
        rec = tiled_bench(args, args.steps)
        print(json.dumps(rec), flush=True)
        return
    if layout == "prefill":
        rec = prefill_bench(args, args.steps)
        print(json.dumps(rec), flush=True)
        return

    k_host, v_host = (inp.k8, inp.v8) if args.fp8 else (inp.k_cache, inp.v_cache)
    S, nq, D = inp.q.shape
    nkv, bs = inp.num_kv_heads, inp.block_size
    n = args.splits or P.pda_num_splits(P.PDA_SPLITK_AUTO, 0, CU_COUNT, nq, S, 0)
    if args.packed:
        if not P.pda_gqa_pack_shape_ok(nq, nkv, D):
            sys.exit(f"--packed needs 8 q heads per kv head at head_dim 256 (got {nq}/{nkv}/{D})")
        n = args.splits or 1   # the packed kernels' own (non-split) launch unless pinned
    ab = alg_bytes(inp, n, 1 if args.fp8 else 2)
    copies = args.copies or max(1, math.ceil(1.0e9 / ab["kv"]))

    def up(a):
        a = np.ascontiguousarray(a)
        return torch.from_numpy(a if a.dtype == np.uint8 else a.view(np.int16)).cuda()

    q = up(inp.q)
    bt = torch.from_numpy(inp.block_tables).cuda()
    lens = torch.from_numpy(inp.seq_lens).cuda()
    ks = [up(k_host) for _ in range(copies)]
    vs = [up(v_host) for _ in range(copies)]
    wsf = P.pda_workspace_slots(S, nq, n, D)
    ws = torch.empty(max(wsf, 1), dtype=torch.float32, device="cuda")
    out = torch.empty((S, nq, D), dtype=torch.int16, device="cuda")
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    mb = bt.shape[1]

    flags = P.PDA_DECODE_PACKED if args.packed else P.PDA_DECODE_UNPACKED

    def partials(i):
        if args.fp8:
            if n == 1:
                rc = P.pda_paged_decode_fp8(q, ks[i % copies], vs[i % copies], bt, lens, out,
                                            None, 0, S, nq, nkv, D, bs, mb, inp.num_blocks,
                                            inp.scale, inp.k_scale, inp.v_scale, 1, flags, sp)
                assert rc == P.PDA_OK
            else:
                P.pda_splitk_partials_fp8(q, ks[i % copies], vs[i % copies], bt, lens, ws, wsf,
                                          S, nq, nkv, D, bs, mb, inp.num_blocks, inp.scale,
                                          inp.k_scale, inp.v_scale, n, flags, sp)
        elif n == 1:
            rc = P.pda_paged_decode(q, ks[i % copies], vs[i % copies], bt, lens, out, None, 0, S,
                                    nq, nkv, D, bs, mb, inp.num_blocks, inp.scale, 1, flags, sp)
            assert rc == P.PDA_OK
        else:
            P.pda_splitk_partials(q, ks[i % copies], vs[i % copies], bt, lens, ws, wsf, S, nq,
                                  nkv, D, bs, mb, inp.num_blocks, inp.scale, n, flags, sp)

    def merge():
        if n > 1:
            P.pda_splitk_merge(ws, wsf, out, S, nq, D, n, sp)

    def decode(i):
        """One whole step through the one-shot entry point (split-K: the
        fold launch, then the merge launch)."""
        wsp, wsn = (ws, wsf) if n > 1 else (None, 0)
        if args.fp8:
            rc = P.pda_paged_decode_fp8(q, ks[i % copies], vs[i % copies], bt, lens, out, wsp,
                                        wsn, S, nq, nkv, D, bs, mb, inp.num_blocks, inp.scale,
                                        inp.k_scale, inp.v_scale, n, flags, sp)
        else:
            rc = P.pda_paged_decode(q, ks[i % copies], vs[i % copies], bt, lens, out, wsp, wsn,
                                    S, nq, nkv, D, bs, mb, inp.num_blocks, inp.scale, n, flags,
                                    sp)
        assert rc == P.PDA_OK

    if args.calibrate_copy:
        calibrate_copy()

    if args.profile_steps:
        for i in range(args.warmup):
            decode(i)
        for i in range(args.profile_steps):
            decode(args.warmup + i)
        torch.cuda.synchronize()
        print(json.dumps({"profile_steps": args.profile_steps, "workload": args.workload,
                          "kv_pool_copies": copies, "packed": args.packed, "fp8": args.fp8,
                          "num_splits": n}), flush=True)
        return

    for i in range(args.warmup):
        decode(i)
        partials(i)
        merge()
    torch.cuda.synchronize()

    K = args.steps

    enqueue_ms = [0.0]

    def timed(fn):
        """Average ms of fn(i) over K calls, from HIP events on the launch
        stream around the whole run, and the host wall clock of the run
        (the host's own time to issue the K calls is kept in enqueue_ms)."""
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record(stream)
        for i in range(K):
            fn(i)
        enqueue_ms[0] = (time.perf_counter() - t0) * 1e3 / K
        e1.record(stream)
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) * 1e3 / K
        return e0.elapsed_time(e1) / K, wall

    # the timed region: K whole decode steps through pda_paged_decode
    gpu_ms, ms_per_step = timed(decode)
    host_enqueue_ms = enqueue_ms[0]
    # each kernel on its own, back to back, for its average duration
    fold_avg, _ = timed(partials)
    merge_avg, _ = timed(lambda i: merge())
    # warm: the same pool every step (K/V partly served from the Infinity Cache)
    warm_ms, _ = timed(lambda i: decode(0))

    # per-step distribution: an event pair around each of K steps (outside
    # the timed region above; the events add a little to each step)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(K)]
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(evs):
        a.record(stream)
        decode(i)
        b.record(stream)
    torch.cuda.synchronize()
    per_step = np.sort(np.array([a.elapsed_time(b) * 1e3 for a, b in evs]))
    pct = lambda q: round(float(np.percentile(per_step, q)), 2)

    # achievable-bandwidth context on this machine: a plain 1 GiB device copy
    src = torch.empty(1 << 29, dtype=torch.int16, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record(stream)
    for _ in range(5):
        dst.copy_(src)
    c1.record(stream)
    torch.cuda.synchronize()
    copy_gbs = 2 * (1 << 30) * 5 / (c0.elapsed_time(c1) * 1e-3) / 1e9   # read + write
    # and a plain 1 GiB read (torch's sum over int64: one pass, a few bytes out)
    rd = src.view(torch.int64)
    rd.sum()
    c0.record(stream)
    for _ in range(5):
        rd.sum()
    c1.record(stream)
    torch.cuda.synchronize()
    read_gbs = (1 << 30) * 5 / (c0.elapsed_time(c1) * 1e-3) / 1e9
    del src, dst, rd

    value = ab["step"] / (ms_per_step * 1e-3) / 1e9
    # the dominant kernel: the fold (or the packed kernel); with one split it
    # also writes the output itself
    kern_bytes = ab["fold"] + (ab["merge"] if n == 1 else 0)
    achieved = kern_bytes / (fold_avg * 1e-3) / 1e9
    profile, kernel = profile_of(args, n)
    traffic = load_traffic(profile, kernel) if profile else None
    rec = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3 kv, bf16 q/out" if args.fp8 else "bf16",
        "data": "synthetic",
        "config": {
            "workload": inp.workload.description,
            "num_seqs": S, "num_q_heads": nq, "num_kv_heads": nkv, "head_dim": D,
            "block_size": bs, "total_tokens": int(inp.seq_lens.sum()),
            "seq_len_min": int(inp.seq_lens.min()), "seq_len_max": int(inp.seq_lens.max()),
            "num_splits": n, "policy_cu_count": CU_COUNT, "device_cu_count": dev_cus,
            "kv_pool_copies": copies, "algorithmic_bytes_per_step": ab["step"],
            "kv_cache": "fp8 e4m3, per-tensor scales" if args.fp8 else "bf16",
        },
        "us_per_step": round(ms_per_step * 1e3, 2),
        "pct_of_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "gpu_event_us_per_step": round(gpu_ms * 1e3, 2),
        # the host's time to issue one step (binding + two launches): well
        # under the step, so the timed loop is bound by the GPU, not the host
        "host_enqueue_us_per_step": round(host_enqueue_ms * 1e3, 2),
        "warm_us_per_step": round(warm_ms * 1e3, 2),
        "step_us_percentiles": {"p10": pct(10), "p50": pct(50), "p90": pct(90)},
        "copy_1GiB_GBps": round(copy_gbs, 1),
        "read_1GiB_GBps": round(read_gbs, 1),
        "kernels_us": {"splitk_fold": round(fold_avg * 1e3, 2),
                       "splitk_merge": round(merge_avg * 1e3, 2)},
        "roofline": {
            "kernel": kernel or ("GQA-packed MFMA decode (packed_kernel)" if args.packed
                                 else "split-K fold (fold_kernel)"),
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "traffic_from": (f"profiles/{profile}_traffic.json: rocprofv3 FETCH_SIZE and "
                             "WRITE_SIZE of cold dispatches in their own runs, scaled by a "
                             "1 GiB device copy; not measured in this run"
                             if traffic is not None else None),
            "algorithmic_bytes_per_launch": kern_bytes,
        },
    }
    if args.packed:
        # algorithmic MFMA work: q.k and p.v, 2 flops per multiply-add, for
        # the real heads only (the kernel pads 8 heads to 16)
        flops = 4.0 * int(inp.seq_lens.sum()) * nq * D
        tflops = flops / (fold_avg * 1e-3) / 1e12
        rec["mfma"] = {"tflops": round(tflops, 2), "peak_bf16_tflops": 2500.0,
                       "utilisation": round(tflops / 2500.0, 5)}
    if cpu is not None:
        rec["cpu_baseline"] = {
            "value": round(ab["step"] / cpu["step_s"] / 1e9, 4),
            "unit": "GB/s",
            "cores": cpu["workers"],
            "kind": "oracle",
            "sample": f"the whole {S}-sequence batch, FP64 numpy oracle (unchanged) in "
                      f"{cpu['workers']} processes over {cpu['items']} "
                      f"{'sequence' if args.fp8 else '(sequence, KV head)'} items, one BLAS "
                      f"thread each, {cpu['reps']} repetition(s); "
                      f"{cpu['step_s'] * 1e3:.1f} ms per step",
            "ms_per_step": round(cpu["step_s"] * 1e3, 2),
            "os_cpu_count": cpu["cpu_count"],
            "affinity_cores": cpu["affinity"],
            "single_thread_ms": round(cpu["single_step_s"] * 1e3, 2),
            "single_thread_value": round(ab["step"] / cpu["single_step_s"] / 1e9, 4),
        }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
