"""A seeded sweep of shapes over every routing region, each case compared with the oracle
element by element (tests/parity.py has the bars).

The hand-picked cases elsewhere pin each path at its edges; these draw M, K, N, the
dtype, the threshold and the injected outlier columns from one seeded generator, so that
the library's own choices (one-launch, slab or tiled X pass; small-batch or tiled product
kernel; stream-K and half tiles or whole tiles) meet ragged sizes they were not tuned on.
Every case prints its draw and the route the library reports before it runs."""
import numpy as np
import pytest

import int8_quantized_matmul_rowwise_amd as lm
import workloads
from tests import parity

pytestmark = pytest.mark.gpu

# (rows, K range, N range, oracle multiply-adds at most) per region; K a multiple of 16 and
# N of 8 (the boundary's rule)
_REGIONS = [
    ((1, 128), (16, 20000), (8, 3000), 4e9),         # small batches: one-launch or slab X pass
    ((129, 640), (16, 3000), (8, 1600), 4e9),        # tiled: detection, compaction, row coding
    ((24, 112), (2048, 6144), (12000, 24000), 2e10),  # narrow batches on wide weights: slab X pass,
                                                      # stream-K and half tiles, or the small-batch kernel
    ((113, 128), (8192, 12288), (11000, 16000), 2e10),  # half tiles after the row-coding X pass
    ((1, 700), (16, 4000), (8, 2400), 4e9),          # anywhere
]
_CASES = 40


def _draw(i):
    rng = np.random.default_rng(1000 + i)
    (m0, m1), (k0, k1), (n0, n1), macs = _REGIONS[i % len(_REGIONS)]
    while True:
        M = int(rng.integers(m0, m1 + 1))
        K = 16 * int(rng.integers(max(1, k0 // 16), k1 // 16 + 1))
        N = 8 * int(rng.integers(max(1, n0 // 8), n1 // 8 + 1))
        if M * K * N <= macs:
            break
    dt = "fp16" if rng.integers(2) else "bf16"
    tau = float(rng.choice([6.0, 6.0, 6.0, 3.0, np.inf, 0.0], p=[0.3, 0.2, 0.2, 0.15, 0.1, 0.05]))
    n_out = int(rng.integers(0, 13))
    return M, K, N, dt, tau, n_out


@pytest.mark.parametrize("i", range(_CASES))
def test_seeded_shape_sweep(i):
    M, K, N, dt, tau, n_out = _draw(i)
    route = "small-batch" if lm.int8_matmul_workspace_layout(M, K, N)["small_batch"] else "tiled"
    print(f"\n[case] sweep {i}: {M}x{K}x{N} {dt} tau={tau} injected={n_out} -> {route}", flush=True)
    x, _ = workloads.make_x(M, K, dt, n_outliers=min(n_out, K), outlier_range=(6.5, 40.0), seed=i, wid=61)
    w = workloads.make_w(K, N, dt, sigma=0.02, seed=i, wid=61)
    st = parity.run_case(x, w, tau)
    if tau == np.inf:
        assert st["n_outliers"] == 0 and st["n_ulp_flips"] == 0
    if tau == 0.0:
        assert st["n_outliers"] == int((np.abs(workloads.bits(x) & 0x7FFF) > 0).any(axis=0).sum())
