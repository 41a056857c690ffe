"""Pins of oracle.fp8: the E4M3 decoding against values fixed by the OCP FP8
definition, the generator's quantiser round trip, and the FP8 decode against
the BF16 oracle on the same (exactly representable) values.  CPU only."""
import dataclasses

import numpy as np
import pytest

import workloads as W
from oracle import attention as A
from oracle import fp8 as F


@pytest.mark.parametrize("code,value", [
    (0x00, 0.0), (0x80, -0.0), (0x38, 1.0), (0xB8, -1.0), (0x7E, 448.0), (0xFE, -448.0),
    (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9), (0x08, 2.0 ** -6), (0x39, 1.125),
    (0x40, 2.0), (0x3F, 1.875), (0x77, 240.0), (0x78, 256.0),
])
def test_e4m3_values(code, value):
    got = F.decode_e4m3(np.array([code]))[0]
    assert got == value and np.signbit(got) == np.signbit(value)


def test_e4m3_nan_codes_and_count():
    d = F.decode_e4m3(np.arange(256))
    assert np.isnan(d[0x7F]) and np.isnan(d[0xFF])
    assert np.isnan(d).sum() == 2
    finite = d[~np.isnan(d)]
    assert np.max(finite) == 448 and np.min(finite) == -448
    # 127 distinct non-negative magnitudes, strictly increasing with the code
    assert np.all(np.diff(d[:127]) > 0)


def test_quantiser_round_trip():
    x = np.random.default_rng(1).standard_normal(20000) * 50
    q = W.f32_to_e4m3_bits(x)
    back = F.decode_e4m3(q)
    a = np.minimum(np.abs(x), 448.0)
    # nearest representable: within half the gap to the next code
    mags = F.decode_e4m3(np.arange(127))
    i = np.clip(np.searchsorted(mags, a), 1, 126)
    gap = mags[i] - mags[i - 1]
    assert np.all(np.abs(np.abs(back) - a) <= gap / 2 + 1e-18)
    assert np.all(np.sign(back[np.abs(back) > 0]) == np.sign(x[np.abs(back) > 0]))


def test_matches_bf16_oracle_on_exact_values():
    """E4M3 values times a power-of-two scale are exact in BF16, so the BF16
    oracle on those values is the same definition."""
    w = dataclasses.replace(W.WORKLOADS["tiny"], seed=3)
    f = W.make_paged_fp8(w, canary=False, k_scale=0.25, v_scale=0.5)
    got = F.paged_decode_fp8(f.q, f.k8, f.v8, f.block_tables, f.seq_lens, f.scale, f.k_scale,
                             f.v_scale)
    kb = W.f32_to_bf16_bits((F.decode_e4m3(f.k8) * f.k_scale).astype(np.float32))
    vb = W.f32_to_bf16_bits((F.decode_e4m3(f.v8) * f.v_scale).astype(np.float32))
    ref, _, _ = A.paged_decode(f.q, kb, vb, f.block_tables, f.seq_lens, f.scale)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)


def test_scale_semantics():
    """Doubling v_scale doubles the output; k_scale multiplies the scores
    exactly as the softmax scale does."""
    f = W.make_paged_fp8("tiny", canary=False)
    args = (f.q, f.k8, f.v8, f.block_tables, f.seq_lens)
    base = F.paged_decode_fp8(*args, f.scale, f.k_scale, f.v_scale)
    np.testing.assert_allclose(F.paged_decode_fp8(*args, f.scale, f.k_scale, 2 * f.v_scale),
                               2 * base, rtol=1e-13)
    np.testing.assert_allclose(F.paged_decode_fp8(*args, 2 * f.scale, f.k_scale, f.v_scale),
                               F.paged_decode_fp8(*args, f.scale, 2 * f.k_scale, f.v_scale),
                               rtol=1e-12)
