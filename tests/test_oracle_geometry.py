"""Pins of the oracle's launch-geometry formulas (CPU only).

Each test checks ``oracle.geometry`` against something other than itself:
numbers printed on the pages (``tests/golden/attn_splitk_examples.json``),
invariants the pages state, or numpy's own layout arithmetic.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import geometry as g

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                     "attn_splitk_examples.json")))


def test_auto_printed_examples():
    ex = GOLDEN["auto_ask_one_head_132_sms"]
    assert g.auto_splits_ask(ex["sm_count"], ex["num_q_heads"]) == ex["value"]
    # the ceiling exists because of that ask: the clamped value is the ceiling
    assert g.auto_splits(ex["sm_count"], ex["num_q_heads"]) == g.MAX_DECODE_SPLITS
    ex = GOLDEN["auto_splits_24_heads_148_sms"]
    # printed as what Auto asks for, and not clamped by the ceiling
    assert g.auto_splits_ask(ex["sm_count"], ex["num_q_heads"]) == ex["value"]
    assert g.auto_splits(ex["sm_count"], ex["num_q_heads"]) == ex["value"]
    # ceil, not floor or round: 296/24 = 12.33 -> 13
    assert math.floor(2 * 148 / 24) == 12


def test_auto_bounds_and_batch_independence():
    for sm in (1, 48, 132, 148, 256, 304, 512):
        for nq in range(1, 129):
            a = g.auto_splits(sm, nq)
            assert 1 <= a <= g.MAX_DECODE_SPLITS
            # Auto aims at WAVES waves of workgroups with one sequence in flight:
            # unless clamped, a * nq covers at least 2 * sm and overshoots by < nq
            if 1 < a < g.MAX_DECODE_SPLITS:
                assert 2 * sm <= a * nq < 2 * sm + nq
            for seqs in (1, 7, 128):
                # Auto and Pinned depend only on (sm_count, num_q_heads) and the pin
                assert g.num_splits(g.AUTO, 0, sm, nq, seqs, 64) == a
                assert g.num_splits(g.PINNED, 5, sm, nq, seqs, 64) == 5
    assert g.auto_splits(256, 0) == 0


def test_ceiling_reading_fits_the_pages():
    # at least the unclamped 13 of the 148-SM example, and below the 22 that a
    # 24-head model asks for on 256 CUs (which must be clamped)
    assert 13 <= g.MAX_DECODE_SPLITS < g.auto_splits_ask(256, 24) == 22


def test_pinned_clamp():
    assert g.pinned_splits(0) == 1
    assert g.pinned_splits(1) == 1
    assert g.pinned_splits(4) == 4
    assert g.pinned_splits(g.MAX_DECODE_SPLITS) == g.MAX_DECODE_SPLITS
    assert g.pinned_splits(10_000) == g.MAX_DECODE_SPLITS


def test_legacy_rule_properties():
    # one split once the reference batch alone fills the SMs
    assert g.legacy_splits(132, 32, 8) == 1
    assert g.legacy_splits(132, 132, 1) == 1
    # below that, the integer quotient: never overshoots the SM count
    for sm in (48, 132, 148, 256):
        for nq in (1, 2, 8, 24, 32):
            for ref in (1, 2, 3, 4):
                cur = nq * ref
                v = g.legacy_splits(sm, nq, ref)
                if cur >= sm:
                    assert v == 1
                else:
                    assert v >= 1 and v * cur <= sm < (v + 1) * cur
    # not clamped to the ceiling (only the other policies are)
    assert g.legacy_splits(132, 1, 1) == 132 > g.MAX_DECODE_SPLITS
    # only Legacy reads the batch: past max_decode_seqs the count moves
    assert g.split_ref_seqs(3, 8) == 8 and g.split_ref_seqs(20, 8) == 20
    a = g.num_splits(g.LEGACY, 0, 256, 4, 1, 8)
    b = g.num_splits(g.LEGACY, 0, 256, 4, 32, 8)
    assert a == 256 // 32 and b == 256 // 128 and a != b
    assert g.legacy_splits(256, 0, 5) == 0


def test_workspace_slots_matches_array_size():
    for rows, nq, n, D in [(32, 32, 16, 128), (1, 24, 16, 128), (2, 8, 4, 128), (5, 3, 1, 64)]:
        ws = np.empty((rows, nq, n, D + 2), dtype=np.float32)
        assert g.workspace_slots(rows, nq, n, D) == ws.size


def test_gqa_pack_gate_and_ctas():
    assert GOLDEN["gqa_pack_head_dim"]["value"] == g.DECODE_GQA_PACK_HEAD_DIM
    assert g.gqa_pack_shape_ok(32, 4, 256)
    assert g.gqa_pack_shape_ok(8, 1, 256)
    assert not g.gqa_pack_shape_ok(32, 4, 128)      # other head dims refused
    assert not g.gqa_pack_shape_ok(24, 4, 256)      # ratio 6 != width
    assert not g.gqa_pack_shape_ok(64, 4, 256)      # ratio 16 != width
    assert not g.gqa_pack_shape_ok(0, 0, 256)
    ex = GOLDEN["gqa_pack_ctas_cover_48_sms"]
    first = min(n for n in range(1, 100) if g.gqa_pack_ctas(ex["num_kv_heads"], n) >= ex["sm_count"])
    assert first == ex["first_num_seqs_covering"]
    # a PACK_WIDTH-fold cut from the unpacked q_heads * seqs
    assert g.gqa_pack_ctas(4, 12) * g.DECODE_GQA_PACK_WIDTH == 32 * 12


def test_strides_match_numpy_layouts():
    for bs, nkv, D in [(16, 8, 128), (32, 4, 256), (16, 2, 128), (8, 3, 64)]:
        paged = np.empty((5, bs, nkv, D), dtype=np.uint16)
        st = [s // 2 for s in paged.strides]
        assert g.paged_strides(bs, nkv, D) == (st[0], st[1], st[2])
        pool = np.empty((5, 2, nkv, bs, D), dtype=np.uint16)
        st = [s // 2 for s in pool.strides]
        assert g.scratch_pool_strides(bs, nkv, D) == (st[0], st[3], st[2])
        assert g.scratch_pool_v_offset(bs, nkv, D) == st[1]


def test_split_partition_reading():
    # parity unpinned (no value printed); check the rule's own invariants
    for L in list(range(0, 300)) + [4096, 131072, 8002]:
        for n in (1, 2, 4, 13, 16):
            for bs in (16, 32):
                rs = g.split_ranges(L, n, bs)
                assert len(rs) == n
                c = g.split_chunk(L, n, bs)
                assert c % bs == 0 and c >= g.PD_MIN_KV_PER_SPLIT
                live = [(b, e) for b, e in rs if e > b]
                # the live splits come first and tile [0, L) in order, no gaps
                assert rs[:len(live)] == live
                covered = [t for b, e in live for t in range(b, e)] if L < 5000 else None
                if covered is not None:
                    assert covered == list(range(L))
                assert sum(e - b for b, e in live) == L
                assert all(b % bs == 0 for b, _ in live)          # block-aligned starts
                assert all(e - b == c for b, e in live[:-1])      # all but the last are full
                assert len(live) == -(-L // c) <= n
    # the values used by the tiny workload with pin 4
    assert g.split_ranges(37, 4, 16) == [(0, 37), (37, 37), (37, 37), (37, 37)]
    assert g.split_ranges(100, 4, 16) == [(0, 64), (64, 100), (100, 100), (100, 100)]


def test_tiled_dims_and_bytes():
    ex = GOLDEN["max_head_dim"]
    assert g.MAX_HEAD_DIM == ex["value"]
    assert g.tiled_dims_error(128, 16, 4, 256, 32, 64) is None
    assert g.tiled_dims_error(128, 16, 4, 257, 32, 64) is not None
    assert g.tiled_dims_error(128, 16, 3, 128, 32, 64) is not None
    assert g.tiled_dims_error(128, 16, 0, 128, 32, 64) is not None
    m, l, o, out = g.tiled_state_bytes(128, 16, 256)
    assert (m, l) == (128 * 16 * 4,) * 2
    assert o == np.empty((128, 16, 256), np.float32).nbytes
    assert out == np.empty((128, 16, 256), np.uint16).nbytes
    assert int(GOLDEN["neg_inf_f32_bits"]["value"], 16) == g.NEG_INF_F32_BITS
    assert np.array([g.NEG_INF_F32_BITS], np.uint32).view(np.float32)[0] == -np.inf
