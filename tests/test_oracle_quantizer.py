"""Pins of the oracle's scalar quantizer (vector-wise absmax, round to nearest even).

"LLM.int8()" page, abstract: vector-wise quantization with one normalization constant
per vector; "nuQmm" report page, GPTQ statement under "Large-model Quantization":
round to the nearest quantization level.  The reading: the absmax s maps to 127 and
q = round-half-even(127 x / s).

The pins below do not re-type the oracle's fp32 op sequence.  They compare with the
exact real-valued rule computed by numpy in float64 (np.rint is round-half-even), and
allow a disagreement only where 127 x / s lies within the fp32 sequence's own rounding
error of a half-integer; on scales where that sequence is exact (s = 127 * 2^e) no
disagreement at all is allowed, which pins the tie rule.
"""
import numpy as np
import pytest

import oracle
from tests.indep import f32_of

ALL16 = np.arange(65536, dtype=np.uint32).astype(np.uint16)


def _finite(dt):
    v = f32_of(ALL16, dt)
    return v[np.isfinite(v)]


def _scales(dt):
    vals = np.abs(_finite(dt))
    # below 2^-120 the fp32 constant 127/s overflows: outside the quantizer's contract
    vals = np.unique(vals[vals >= 2.0**-120])
    rng = np.random.default_rng(1)
    pick = list(rng.choice(vals, 150, replace=False))
    pick += [1.0, 2.0, 0.5, 127.0, 6.0, 60.0, 1.0 / 64]
    if dt == "fp16":
        pick += [2.0**-24, 3 * 2.0**-24, 2.0**-14, 65504.0]
    else:
        pick += [2.0**-100, 2.0**100, 3.0e38]
    return np.array(sorted(set(np.float32(p) for p in pick)), np.float32)


@pytest.mark.parametrize("dt", ["fp16", "bf16"])
def test_quantizer_matches_exact_rounding_exhaustive(dt):
    xs = _finite(dt)
    total = disagree = 0
    for s in _scales(dt):
        x = xs[np.abs(xs) <= s]
        q = oracle.quantize(x, s).astype(np.int64)
        e = 127.0 * x.astype(np.float64) / np.float64(s)   # exact rule in float64
        ref = np.rint(e)
        assert np.all(np.abs(q) <= 127)
        # the absmax maps to +-127
        assert oracle.quantize(np.array([s, -s], np.float32), s).tolist() == [127, -127]
        d = q != ref
        if d.any():
            # only near-ties may differ, and by one step
            frac = np.abs(e[d] - np.floor(e[d]) - 0.5)
            assert np.all(frac <= 2e-5 * np.maximum(1.0, np.abs(e[d]))), (s, x[d][:4], q[d][:4], ref[d][:4])
            assert np.all(np.abs(q[d] - ref[d]) == 1)
        total += x.size
        disagree += int(d.sum())
    assert total > 1_000_000
    assert disagree <= total * 1e-4


@pytest.mark.parametrize("dt", ["fp16", "bf16"])
@pytest.mark.parametrize("e", [-6, -3, 0, 2, 5])
def test_quantizer_exact_on_power_of_two_scales(dt, e):
    # s = 127 * 2^e: 127/s = 2^-e exactly, so x*inv is exact and q must be rint(127x/s) everywhere
    s = np.float32(127.0 * 2.0**e)
    xs = _finite(dt)
    x = xs[np.abs(xs) <= s]
    q = oracle.quantize(x, s).astype(np.int64)
    ref = np.rint(x.astype(np.float64) * 2.0**-e)
    assert np.array_equal(q, ref)


def test_quantizer_ties_go_to_even():
    x = np.array([0.5, 1.5, 2.5, -0.5, -1.5, 62.5, -62.5, 126.5, 3.5], np.float32)
    assert oracle.quantize(x, 127.0).tolist() == [0, 2, 2, 0, -2, 62, -62, 126, 4]


def test_quantizer_zero_scale_and_zero_input():
    assert oracle.inv_scale(0.0) == 0.0
    assert oracle.quantize(np.array([0.0, -0.0], np.float32), 0.0).tolist() == [0, 0]
    assert oracle.quantize(np.array([0.0, -0.0], np.float32), 3.0).tolist() == [0, 0]


def test_quantizer_error_bound_and_monotone():
    rng = np.random.default_rng(2)
    for _ in range(50):
        x = rng.standard_normal(4096).astype(np.float32) * np.float32(rng.uniform(0.01, 100))
        s = np.float32(np.max(np.abs(x)))
        q = oracle.quantize(x, s)
        err = np.abs(x.astype(np.float64) - q.astype(np.float64) * np.float64(s) / 127.0)
        assert np.all(err <= np.float64(s) / 254.0 * (1 + 2.0**-20))
        order = np.argsort(x, kind="stable")
        assert np.all(np.diff(q[order].astype(np.int64)) >= 0)
        assert np.array_equal(oracle.quantize(-x, s), -q)
