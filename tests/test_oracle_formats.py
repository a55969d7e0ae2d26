"""Pins of the oracle's 16-bit <-> fp32 conversions against numpy (fp16) and torch (bf16).

Widening must be exact for every pattern; narrowing must be round-to-nearest-even
(the conversion both sides of the parity check use for the output Y).
"""
import numpy as np
import pytest

import oracle
from tests.indep import bits_of, f32_of

ALL16 = np.arange(65536, dtype=np.uint32).astype(np.uint16)


@pytest.mark.parametrize("dt", ["fp16", "bf16"])
def test_widening_every_pattern(dt):
    got = oracle.to_f32(ALL16, dt)
    ref = f32_of(ALL16, dt)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def _narrowing_cases(dt, seed=0):
    rng = np.random.default_rng(seed)
    vals = f32_of(ALL16, dt)
    fin = vals[np.isfinite(vals)].astype(np.float64)
    fin = np.unique(fin)
    mids = (fin[:-1] + fin[1:]) / 2.0  # exact ties between neighbours (exact in float64)
    mids32 = mids.astype(np.float32)
    cases = [vals[np.isfinite(vals)], mids32,
             np.nextafter(mids32, np.float32(np.inf)), np.nextafter(mids32, np.float32(-np.inf)),
             rng.integers(0, 2**32, 2_000_000, dtype=np.uint64).astype(np.uint32).view(np.float32),
             np.array([65504.0, 65519.996, 65520.0, 65536.0, 1e9, -65520.0, 2.0**-24, 2.0**-25,
                       3 * 2.0**-26, 2.0**-26, 0.0, -0.0, np.inf, -np.inf], np.float32)]
    out = np.concatenate([c.astype(np.float32) for c in cases])
    return out[~np.isnan(out)]


@pytest.mark.parametrize("dt", ["fp16", "bf16"])
def test_narrowing_round_to_nearest_even(dt):
    f = _narrowing_cases(dt)
    got = oracle.from_f32(f, dt)
    ref = bits_of(f, dt)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, (dt, f[bad[:5]], got[bad[:5]], ref[bad[:5]])


@pytest.mark.parametrize("dt", ["fp16", "bf16"])
def test_narrowing_nan_stays_nan(dt):
    f = np.array([np.nan, -np.nan, np.float32(np.nan) * 2], np.float32)
    back = f32_of(oracle.from_f32(f, dt), dt)
    assert np.all(np.isnan(back))
