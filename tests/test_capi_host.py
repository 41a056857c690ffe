"""Host-side checks of the C-ABI library (CPU only; nothing is launched).

* the library loads without a GPU and exports every function declared in
  include/pda.h;
* the geometry functions agree bit-exactly with the oracle's formulas over
  sweeps of their inputs;
* argument validation rejects bad calls before any HIP call;
* the tile planner covers every token exactly once, in order.
"""
import os
import re

import numpy as np
import pytest

import paged_decode_attention_splitk_amd as P
import workloads as W
from oracle import geometry as g

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "pda.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(pda_[a-z0-9_]+)\s*\(", src)))


def test_every_declared_symbol_is_exported_and_bound():
    names = _declared()
    assert len(names) >= 30
    for n in names:
        assert hasattr(P._lib, n), n          # dlsym succeeds
        assert n in P.EXPORTED, n              # and the binding declares it
        assert callable(getattr(P, n)), n      # with a same-named Python function


def test_constants():
    assert P.pda_max_decode_splits() == g.MAX_DECODE_SPLITS
    assert P.pda_splitk_target_waves() == g.SPLITK_TARGET_WAVES
    assert P.pda_gqa_pack_width() == g.DECODE_GQA_PACK_WIDTH
    assert P.pda_gqa_pack_head_dim() == g.DECODE_GQA_PACK_HEAD_DIM
    assert P.pda_min_kv_per_split() == g.PD_MIN_KV_PER_SPLIT
    assert P.pda_max_head_dim() == g.MAX_HEAD_DIM


def test_split_count_functions_bit_exact():
    for cu in list(range(0, 520, 7)) + [48, 132, 148, 256, 304, 2**31]:
        for nq in range(0, 129):
            assert P.pda_auto_splits(cu, nq) == g.auto_splits(cu, nq), (cu, nq)
            for ref in (0, 1, 3, 8, 64, 512):
                assert P.pda_legacy_splits(cu, nq, ref) == g.legacy_splits(cu, nq, ref)
    for seqs in range(0, 513, 17):
        for mx in (0, 1, 8, 64, 256):
            assert P.pda_split_ref_seqs(seqs, mx) == g.split_ref_seqs(seqs, mx)
    for pin in list(range(0, 65)) + [2**32 - 1]:
        assert P.pda_pinned_splits(pin) == g.pinned_splits(pin)
    for pol in (0, 1, 2, 3, -1):
        for pin in (0, 4, 99):
            for cu, nq, seqs, mx in [(256, 32, 32, 64), (132, 1, 1, 8), (48, 24, 300, 256),
                                     (256, 0, 1, 1)]:
                assert (P.pda_num_splits(pol, pin, cu, nq, seqs, mx)
                        == g.num_splits(pol, pin, cu, nq, seqs, mx))


def test_sizes_and_gate_bit_exact():
    for rows in (0, 1, 32, 128, 10**6):
        for nq in (1, 8, 24, 32, 128):
            for n in (1, 4, 16):
                for D in (64, 128, 256):
                    assert P.pda_workspace_slots(rows, nq, n, D) == g.workspace_slots(rows, nq, n, D)
    for nq in range(0, 80):
        for nkv in range(0, 12):
            for D in (64, 128, 255, 256, 512):
                assert P.pda_gqa_pack_shape_ok(nq, nkv, D) == g.gqa_pack_shape_ok(nq, nkv, D)
    for nkv in range(0, 17):
        for seqs in range(0, 300, 7):
            assert P.pda_gqa_pack_ctas(nkv, seqs) == g.gqa_pack_ctas(nkv, seqs)
    for L in list(range(0, 400)) + [4096, 8002, 16384, 131072, 2**31 - 1]:
        for n in (1, 2, 3, 4, 13, 16):
            for bs in (16, 32, 48):
                assert P.pda_split_chunk(L, n, bs) == g.split_chunk(L, n, bs), (L, n, bs)
    for dims in [(128, 16, 4, 256, 32, 64), (32, 32, 8, 128, 16, 8), (1, 8, 2, 64, 16, 1)]:
        _, nq, nkv, D, bs, _ = dims
        assert P.pda_tiled_paged_strides(dims) == g.paged_strides(bs, nkv, D)
        assert P.pda_tiled_scratch_pool_strides(dims) == g.scratch_pool_strides(bs, nkv, D)


FAKE = 1 << 20   # 16-byte aligned non-null value; validation rejects before any use


def _decode(**kw):
    a = dict(q=FAKE, k_cache=FAKE, v_cache=FAKE, block_tables=FAKE, seq_lens=FAKE, out=FAKE,
             workspace=FAKE, workspace_floats=10**9, num_seqs=2, num_q_heads=8, num_kv_heads=2,
             head_dim=128, block_size=16, max_blocks_per_seq=8, num_blocks=32, scale=0.1,
             num_splits=4, flags=0, stream=0)
    a.update(kw)
    return P.pda_paged_decode(**a)


@pytest.mark.parametrize("bad", [
    dict(num_kv_heads=0), dict(num_q_heads=7), dict(num_q_heads=0), dict(head_dim=96),
    dict(head_dim=512), dict(block_size=8), dict(block_size=0), dict(num_splits=0),
    dict(num_splits=17), dict(workspace=None), dict(workspace_floats=100), dict(q=None),
    dict(out=None), dict(block_tables=None), dict(k_cache=FAKE + 2), dict(workspace=FAKE + 4),
    dict(max_blocks_per_seq=0), dict(num_blocks=0), dict(flags=4), dict(scale=float("nan")),
    dict(scale=float("inf")),
])
def test_decode_rejects_bad_arguments(bad):
    with pytest.raises(P.PdaError) as e:
        _decode(**bad)
    assert e.value.code == P.PDA_EINVAL
    assert P.pda_last_error()


def test_packed_not_applicable_launches_nothing():
    # shapes outside the packed gate, with one split or several
    assert _decode(flags=P.PDA_DECODE_PACKED) == P.PDA_NOT_APPLICABLE
    assert _decode(flags=P.PDA_DECODE_PACKED, num_q_heads=32, num_kv_heads=4, head_dim=128,
                   num_splits=2) == P.PDA_NOT_APPLICABLE
    assert _decode(flags=P.PDA_DECODE_PACKED, num_q_heads=24, num_kv_heads=4, head_dim=256,
                   num_splits=1) == P.PDA_NOT_APPLICABLE
    assert "not applicable" in P.pda_last_error()
    assert P.pda_splitk_partials(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 10**9, 2, 8, 2, 128, 16, 8,
                                 32, 0.1, 2, P.PDA_DECODE_PACKED, 0) == P.PDA_NOT_APPLICABLE
    with pytest.raises(P.PdaError):
        _decode(flags=3)


def test_empty_batch_is_a_no_op():
    assert _decode(num_seqs=0) == P.PDA_OK
    assert P.pda_splitk_merge(FAKE, 0, FAKE, 0, 8, 128, 4, 0) == P.PDA_OK


def test_merge_and_partials_validation():
    with pytest.raises(P.PdaError):
        P.pda_splitk_merge(FAKE, 10, FAKE, 2, 8, 128, 4, 0)       # workspace too small
    with pytest.raises(P.PdaError):
        P.pda_splitk_merge(FAKE, 10**9, FAKE, 2, 8, 100, 4, 0)    # head dim
    with pytest.raises(P.PdaError):
        P.pda_splitk_partials(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 10**9, 2, 8, 2, 128, 16, 8, 32,
                              0.1, 1, 0, 0)                       # partials need >= 2 splits


def test_tiled_validate():
    ok = (128, 16, 4, 256, 32, 64)
    assert P.pda_tiled_validate(ok) == P.PDA_OK
    for bad in [(128, 16, 0, 256, 32, 64), (128, 16, 3, 256, 32, 64), (128, 16, 4, 257, 32, 64),
                (128, 16, 4, 512, 32, 64), (128, 16, 4, 96, 32, 64), (128, 16, 4, 256, 24, 64),
                (0, 16, 4, 256, 32, 64), (128, 16, 4, 256, 32, 0)]:
        with pytest.raises(P.PdaError) as e:
            P.pda_tiled_validate(bad)
        assert e.value.code == P.PDA_EINVAL
    with pytest.raises(P.PdaError):
        P.pda_tiled_create((128, 16, 3, 256, 32, 64))


def _fold_plan(calls, S):
    seen = [[] for _ in range(S)]
    for tb, cnt, lbvs in calls:
        for s in range(S):
            for j in range(cnt[s]):
                valid = lbvs if j == cnt[s] - 1 else None
                seen[s].append((tb[s][j], valid))
    return seen


@pytest.mark.parametrize("bs,cap", [(32, 64), (16, 3), (32, 1)])
def test_plan_tiles_covers_every_token_once_in_order(bs, cap):
    rng = np.random.default_rng(5)
    lens = [0, 1, bs - 1, bs, 2 * bs + 3, 7 * bs, 200, 1000]
    tables = []
    nxt = 0
    for L in lens:
        n = -(-L // bs)
        tables.append(list(range(nxt, nxt + n)) + [-1] * 3)
        nxt += n
    calls = W.plan_tiles(tables, lens, bs, cap)
    for tb, cnt, lbvs in calls:
        assert 1 <= lbvs <= bs and all(0 <= c <= cap for c in cnt)
    seen = _fold_plan(calls, len(lens))
    for s, L in enumerate(lens):
        toks = []
        for blk, valid in seen[s]:
            nvalid = bs if valid is None else valid
            toks += [(blk, k) for k in range(nvalid)]
        expect = [(tables[s][t // bs], t % bs) for t in range(L)]
        assert toks == expect, s


def test_prefill_gate_and_validation():
    assert P.pda_prefill_applies(32, 4, 256)
    assert not P.pda_prefill_applies(32, 4, 128)
    assert not P.pda_prefill_applies(32, 4, 256, causal=False)
    assert not P.pda_prefill_applies(32, 4, 256, sliding_window=512)
    assert not P.pda_prefill_applies(30, 4, 256)
    assert not P.pda_prefill_applies(32, 0, 256)

    def pf(**kw):
        a = dict(q=FAKE, k_cache=FAKE, v_cache=FAKE, out=FAKE, block_table=FAKE, q_len=16,
                 kv_len=16, q_offset=0, num_q_heads=8, num_kv_heads=2, head_dim=256,
                 block_size=16, max_blocks=1, num_blocks=1, scale=0.0625, sliding_window=0,
                 stream=0)
        a.update(kw)
        return P.pda_paged_prefill(**a)

    # not applicable: nothing is checked further, nothing launched
    assert pf(q_len=0) == P.PDA_NOT_APPLICABLE
    assert pf(head_dim=128) == P.PDA_NOT_APPLICABLE
    assert pf(sliding_window=8) == P.PDA_NOT_APPLICABLE
    assert pf(num_q_heads=7) == P.PDA_NOT_APPLICABLE
    for bad in (dict(q=0), dict(block_table=0), dict(block_size=0), dict(num_blocks=0),
                dict(kv_len=17), dict(q_offset=2**31 - 8), dict(scale=float("nan"))):
        with pytest.raises(P.PdaError) as e:
            pf(**bad)
        assert e.value.code == P.PDA_EINVAL


def _decode_fp8(**kw):
    a = dict(q=FAKE, k_cache=FAKE, v_cache=FAKE, block_tables=FAKE, seq_lens=FAKE, out=FAKE,
             workspace=FAKE, workspace_floats=10**9, num_seqs=2, num_q_heads=8, num_kv_heads=2,
             head_dim=128, block_size=16, max_blocks_per_seq=8, num_blocks=32, scale=0.1,
             k_scale=0.01, v_scale=0.02, num_splits=4, flags=0, stream=0)
    a.update(kw)
    return P.pda_paged_decode_fp8(**a)


@pytest.mark.parametrize("bad", [
    dict(num_kv_heads=0), dict(num_q_heads=7), dict(head_dim=96), dict(block_size=8),
    dict(num_splits=0), dict(num_splits=17), dict(workspace=None), dict(workspace_floats=100),
    dict(q=None), dict(v_cache=None), dict(out=None), dict(k_cache=FAKE + 2), dict(flags=4),
    dict(scale=float("nan")), dict(k_scale=float("inf")), dict(v_scale=float("nan")),
])
def test_decode_fp8_rejects_bad_arguments(bad):
    with pytest.raises(P.PdaError) as e:
        _decode_fp8(**bad)
    assert e.value.code == P.PDA_EINVAL
    assert P.pda_last_error()


def test_decode_fp8_packed_not_applicable_and_empty():
    # the packed FP8 kernel has the BF16 one's gate
    assert _decode_fp8(flags=P.PDA_DECODE_PACKED) == P.PDA_NOT_APPLICABLE
    assert _decode_fp8(flags=P.PDA_DECODE_PACKED, num_q_heads=24, num_kv_heads=4,
                       head_dim=256, num_splits=1) == P.PDA_NOT_APPLICABLE
    assert P.pda_splitk_partials_fp8(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 10**9, 2, 8, 2, 128, 16,
                                     8, 32, 0.1, 0.01, 0.02, 2, P.PDA_DECODE_PACKED,
                                     0) == P.PDA_NOT_APPLICABLE
    assert _decode_fp8(num_seqs=0) == P.PDA_OK
    assert P.pda_splitk_partials_fp8(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 10**9, 0, 8, 2, 128, 16,
                                     8, 32, 0.1, 0.01, 0.02, 2, 0, 0) == P.PDA_OK
    for bad in (dict(n=1), dict(ks=float("nan"))):
        with pytest.raises(P.PdaError):
            P.pda_splitk_partials_fp8(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 10**9, 2, 8, 2, 128, 16,
                                      8, 32, 0.1, bad.get("ks", 0.01), 0.02, bad.get("n", 2), 0,
                                      0)


def test_missing_library_fails_loudly(tmp_path):
    """Without libpda.so the binding refuses to import (no CPU fallback)."""
    import shutil
    import subprocess
    import sys
    pkg = tmp_path / "paged_decode_attention_splitk_amd"
    pkg.mkdir()
    shutil.copy(os.path.join(os.path.dirname(P.__file__), "__init__.py"), pkg / "__init__.py")
    code = ("import sys; sys.path.insert(0, %r)\n"
            "try:\n"
            "    import paged_decode_attention_splitk_amd\n"
            "except ImportError as e:\n"
            "    print('refused:', e); sys.exit(0)\n"
            "sys.exit(1)\n") % str(tmp_path)
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "no CPU fallback" in r.stdout


CSRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                    "paged_decode_attention_splitk_amd", "csrc")


def _constexpr_int(src, name):
    m = re.search(rf"constexpr\s+int\s+{name}\s*=\s*(\d+)\s*;", src)
    assert m, f"no 'constexpr int {name} = N;' in the source"
    return int(m.group(1))


def test_kernel_sources_declare_the_dispatched_pack_shape():
    """The packed kernel is compiled for the width and head dim that the host
    gate dispatches to it, and says so in a static_assert ("Module
    attn_splitk": DECODE_GQA_PACK_WIDTH, DECODE_GQA_PACK_HEAD_DIM; the page
    pins the kernel sources' declared width to the dispatch width with a
    test).  Likewise the prefill kernel's head dim and its gate."""
    packed = open(os.path.join(CSRC, "decode_packed.hip")).read()
    assert _constexpr_int(packed, "kG") == P.pda_gqa_pack_width() == g.DECODE_GQA_PACK_WIDTH
    assert _constexpr_int(packed, "kD") == P.pda_gqa_pack_head_dim() == 256
    assert re.search(r"static_assert\(\s*kG\s*==\s*\(int\)kGqaPackWidth", packed)
    assert re.search(r"static_assert\(\s*kD\s*==\s*\(int\)kGqaPackHeadDim", packed)
    # the gate admits exactly the compiled shape
    G, D = _constexpr_int(packed, "kG"), _constexpr_int(packed, "kD")
    assert P.pda_gqa_pack_shape_ok(4 * G, 4, D)
    assert not P.pda_gqa_pack_shape_ok(4 * (G + 1), 4, D)
    assert not P.pda_gqa_pack_shape_ok(4 * G, 4, D // 2)
    prefill = open(os.path.join(CSRC, "prefill.hip")).read()
    Dp = _constexpr_int(prefill, "kD")
    assert re.search(r"static_assert\(\s*kD\s*==\s*\(int\)kPrefillHeadDim", prefill)
    assert P.pda_prefill_applies(32, 4, Dp)
    assert not P.pda_prefill_applies(32, 4, Dp // 2)
    # the fold kernel's widest head group is the pack width
    kernels = open(os.path.join(CSRC, "pda_kernels.h")).read()
    assert _constexpr_int(kernels, "kMaxHeadsPerGroup") == P.pda_gqa_pack_width()


def _noalloc(**kw):
    a = dict(q=FAKE, k_cache=FAKE, v_cache=FAKE, block_tables=FAKE, seq_lens=FAKE, out=FAKE,
             num_seqs=2, num_q_heads=8, num_kv_heads=2, head_dim=128, block_size=16,
             max_blocks_per_seq=8, num_blocks=32, scale=0.1, num_splits=4, flags=0, stream=0)
    a.update(kw)
    return P.pda_paged_decode_noalloc(**a)


@pytest.mark.parametrize("bad", [
    dict(num_kv_heads=0), dict(head_dim=96), dict(block_size=8), dict(num_splits=0),
    dict(num_splits=17), dict(q=None), dict(out=None), dict(k_cache=FAKE + 2),
    # 64 x 32 heads x 16 splits x (128 + 2) floats is past the 4 Mi-float scratch
    dict(num_seqs=64, num_q_heads=32, num_kv_heads=8, num_splits=16),
])
def test_noalloc_rejects_bad_arguments_before_any_hip_call(bad):
    with pytest.raises(P.PdaError) as e:
        _noalloc(**bad)
    assert e.value.code == P.PDA_EINVAL
    assert P.pda_last_error()


def test_noalloc_empty_batch_is_a_no_op():
    assert _noalloc(num_seqs=0) == P.PDA_OK
