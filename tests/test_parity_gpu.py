"""Parity of the HIP path with the CPU oracle (through the C-ABI), on seeded inputs.

Small and medium cases compare every element; the full-size workloads compare the
whole X pass and sampled rows of the products, in the same launch configuration the
benchmark times.  See tests/parity.py for the bars."""
import numpy as np
import pytest
import torch

import int8_quantized_matmul_rowwise_amd as lm
import oracle
import workloads
from tests import parity
from tests.indep import bits_of, f32_of
from tests.test_oracle_pipeline import _lattice_case

pytestmark = pytest.mark.gpu


def _case(M, K, N, dt, n_out=3, seed=0, rng=(6.5, 40.0), w_sigma=0.02):
    x, _ = workloads.make_x(M, K, dt, n_outliers=min(n_out, K), outlier_range=rng, seed=seed, wid=60)
    w = workloads.make_w(K, N, dt, sigma=w_sigma, seed=seed, wid=60)
    return x, w


def _banner(msg):
    print(f"\n[case] {msg}", flush=True)


def test_tiny_workload():
    x, w, cols, wl = workloads.make_workload("tiny")
    _banner("tiny 32x256x128 fp16")
    st = parity.run_case(x, w, wl.tau)
    assert st["n_outliers"] == 2


@pytest.mark.parametrize("dt", ["fp16", "bf16"])
def test_ragged_medium(dt):
    # several 256x256 tiles and a ragged tail in M, N and K (K = 8 * 128 + 16)
    _banner(f"ragged 300x1040x520 {dt}")
    x, w = _case(300, 1040, 520, dt, n_out=5, seed=1)
    st = parity.run_case(x, w, 6.0)
    assert st["n_outliers"] >= 5


@pytest.mark.parametrize("M,K,N,dt", [(1, 16, 8, "fp16"), (1, 4096, 264, "bf16"), (16, 8192, 512, "bf16"),
                                      (64, 1040, 264, "fp16"), (65, 1040, 264, "bf16"), (33, 32784, 24, "fp16"),
                                      (257, 272, 264, "fp16"), (513, 128, 8, "bf16"), (7, 32, 1032, "fp16"),
                                      # small batches: one-workgroup X pass (M*K <= 32768) with waves that
                                      # straddle rows (K = 800: 100 chunks per row), at and just past its
                                      # size limit, and the two slab launches past it (16, 32 and 64 rows
                                      # held per lane; K not a multiple of the 512-column slab)
                                      (40, 800, 136, "bf16"), (64, 512, 264, "fp16"), (64, 528, 264, "fp16"),
                                      (40, 3200, 136, "bf16"), (64, 4096, 264, "bf16"), (24, 2064, 136, "fp16"),
                                      (32, 16400, 40, "bf16"), (17, 1552, 8, "fp16"),
                                      # two rows at the largest small-batch K; a ragged last slab and a
                                      # half-filled last bitmap word (K % 32 = 16)
                                      (2, 32768, 8, "bf16"), (5, 7440, 24, "fp16"),
                                      # small batches with N wide enough that they take the tiled kernel
                                      (24, 1024, 36864, "fp16"), (48, 512, 28672, "bf16"),
                                      # the small-batch kernel with two 16-column groups per workgroup
                                      # (1, 2 and 4 row groups; 4 and 8 waves; a ragged last group)
                                      (16, 2048, 16384, "fp16"), (32, 1024, 8192, "fp16"),
                                      (64, 512, 16384, "bf16"), (40, 800, 8200, "bf16"),
                                      # the small-batch path at its largest K, with a ragged K, and the
                                      # tiled path just past it
                                      (2, 65536, 8, "bf16"), (16, 40976, 24, "fp16"), (8, 65552, 16, "fp16"),
                                      # 65 to 128 rows on the small-batch path (5 to 8 row groups), one
                                      # of them through the one-workgroup X pass
                                      (80, 1024, 512, "fp16"), (128, 2048, 264, "bf16"), (100, 304, 136, "fp16"),
                                      # the fewest rows that take the blocked copy of the codes (8), through
                                      # the slab launches with K % 64 = 16, and a partial row group (12)
                                      # through the one-workgroup X pass
                                      (8, 4112, 72, "bf16"), (12, 2048, 40, "fp16"),
                                      # 128 rows on the small-batch path only because the stream-K
                                      # grid of the tiled path would fill under half the chip
                                      (128, 2064, 7424, "fp16"),
                                      # up to 128 rows on the tiled path: stream-K ragged in M, N and K;
                                      # 256 tiles (no stream-K); stream-K over 64 tiles with the row
                                      # coding (past 112 rows)
                                      (100, 2064, 20000, "bf16"), (16, 2048, 65536, "fp16"),
                                      (128, 1040, 16384, "bf16"),
                                      # row coding holding 12 chunks per thread (one workgroup per row)
                                      (300, 20496, 264, "fp16")])
def test_edge_shapes(M, K, N, dt):
    _banner(f"edge {M}x{K}x{N} {dt}")
    x, w = _case(M, K, N, dt, n_out=2, seed=M + K + N)
    parity.run_case(x, w, 6.0)


@pytest.mark.parametrize("M,K,N,n_out,dt", [(96, 2048, 20000, 40, "bf16"), (64, 1024, 65536, 300, "fp16"),
                                             (112, 4112, 16400, 64, "fp16"),
                                             # more groups of 64 weight rows than gather workgroups:
                                             # each takes every 4096th group
                                             (16, 256, 300000, 40, "bf16")])
def test_mid_batches_tiled_many_outliers(M, K, N, n_out, dt):
    # up to 112 rows on the tiled path (the slab X pass) with many outlier columns: the W_O
    # gather looks each column up by its rank in the bitmap (several per bitmap word, up to
    # ten rounds of 32)
    _banner(f"mid tiled {M}x{K}x{N} {dt}, {n_out} outlier columns")
    assert not lm.int8_matmul_workspace_layout(M, K, N)["small_batch"]
    x, w = _case(M, K, N, dt, n_out=n_out, seed=M + N)
    st = parity.run_case(x, w, 6.0)
    assert st["n_outliers"] >= n_out


@pytest.mark.parametrize("K,dt", [(128, "fp16"), (256, "bf16"), (400, "fp16"), (336, "bf16")])
def test_several_tiles_per_workgroup(K, dt):
    # 17 x 21 = 357 tiles of 256 x 256 on 256 workgroups: some take two tiles, and the
    # operand loads run one (K = 128: one stage per tile) or two tiles ahead; ragged in M,
    # N and K (400 and 336: a partial last stage).  Rows sampled in the first, a middle
    # and the last row tile, C compared exactly.
    M, N = 4200, 5256
    _banner(f"several tiles per workgroup {M}x{K}x{N} {dt}")
    x, w = _case(M, K, N, dt, n_out=4, seed=K)
    rng = np.random.default_rng(K)
    rows = np.unique(np.concatenate([[0, 255, 256, 2047, 4095, 4096, M - 1], rng.integers(0, M, 5)]))
    st = parity.run_case(x, w, 6.0, rows=rows)
    assert st["n_outliers"] >= 4


def test_k_zero_on_the_tiled_path():
    # M > 64 takes the tiled kernel's launcher: K = 0 is the empty sum (Y = +0, C = F = 0)
    _banner("K=0, M=300, N=264")
    X = torch.zeros(300, 0, dtype=torch.float16, device="cuda")
    Wq = torch.zeros(264, 0, dtype=torch.int8, device="cuda")
    s_w = torch.zeros(264, device="cuda")
    Y = lm.int8_matmul(X, Wq, s_w, 6.0, Y=torch.full((300, 264), 5.0, dtype=torch.float16, device="cuda"))
    C, F, _ = lm.int8_matmul_accumulators(X, Wq, 6.0)
    torch.cuda.synchronize()
    assert not Y.view(torch.int16).any() and not C.any() and not F.view(torch.int32).any()
    # 64 rows, N wide enough for the tiled kernel
    _banner("K=0, M=64, N=65536")
    X = torch.zeros(64, 0, dtype=torch.bfloat16, device="cuda")
    Wq = torch.zeros(65536, 0, dtype=torch.int8, device="cuda")
    s_w = torch.zeros(65536, device="cuda")
    Y = lm.int8_matmul(X, Wq, s_w, 6.0, Y=torch.full((64, 65536), 5.0, dtype=torch.bfloat16, device="cuda"))
    torch.cuda.synchronize()
    assert not Y.view(torch.int16).any()


@pytest.mark.parametrize("dt", ["fp16", "bf16"])
def test_threshold_exactly_tau_is_not_an_outlier(dt):
    _banner(f"x == tau {dt}")
    x, w = _case(64, 256, 136, dt, n_out=0, seed=3)
    x[5, 17] = 6.0
    x[9, 200] = -6.0
    x[11, 33] = 7.5
    st = parity.run_case(x, w, 6.0)
    assert st["n_outliers"] == 1


@pytest.mark.parametrize("dt", ["fp16", "bf16"])
@pytest.mark.parametrize("M", [4, 80])  # small-batch slab detection and the tiled path's detection
def test_detection_threshold_sweep(dt, M):
    """The outlier set against the oracle with every finite magnitude in one column each
    (random signs, spread over the rows) and thresholds at 0, the smallest subnormal, a
    representable value, a value strictly between two representable ones, the largest
    finite value and +inf."""
    top = 0x7C00 if dt == "fp16" else 0x7F80  # +inf's pattern; every magnitude below is finite
    K = 32768
    rng = np.random.default_rng(11)
    mags = np.arange(top, dtype=np.uint32)
    signs = rng.integers(0, 2, top).astype(np.uint32) << 15
    Xb = np.zeros((M, K), np.uint16)
    Xb[mags % M, mags] = (mags | signs).astype(np.uint16)
    X = workloads.from_bits(Xb, dt).cuda()
    Wq = torch.zeros((8, K), dtype=torch.int8, device="cuda")
    six = float(f32_of(bits_of(np.array([6.0]), dt), dt)[0])
    between = float(np.nextafter(np.float32(six), np.float32(7.0)))  # not representable in 16 bits
    largest = float(f32_of(np.array([top - 1], np.uint16), dt)[0])
    tiny = float(f32_of(np.array([1], np.uint16), dt)[0])
    for tau in (0.0, tiny, six, between, largest, float("inf")):
        _banner(f"detection sweep {dt} M={M} tau={tau!r}")
        ws = lm.int8_matmul_prepare(X, Wq, tau)
        torch.cuda.synchronize()
        v = lm.workspace_views(ws, M, K, 8, X.dtype)
        O = oracle.outlier_columns(Xb, dt, tau)
        assert v["n_outliers"] == O.size, (tau, v["n_outliers"], O.size)
        assert np.array_equal(v["outliers"].cpu().numpy(), O), tau


@pytest.mark.parametrize("dt", ["fp16", "bf16"])
@pytest.mark.parametrize("M", [40, 130])  # small-batch path and tiled path
def test_tau_zero_every_column_is_an_outlier(dt, M):
    # the degenerate 16-bit path: n_O = K (nine 32-wide chunks), C = 0, s_x = 0
    _banner(f"tau=0 {dt} M={M}")
    x, w = _case(M, 272, 72, dt, n_out=0, seed=4)
    st = parity.run_case(x, w, 0.0)
    assert st["n_outliers"] == 272


@pytest.mark.parametrize("dt", ["fp16", "bf16"])
def test_tau_inf_pure_vectorwise_is_bitwise(dt):
    _banner(f"tau=inf {dt}")
    x, w = _case(96, 512, 264, dt, n_out=4, seed=5)
    st = parity.run_case(x, w, float("inf"))
    assert st["n_outliers"] == 0 and st["n_ulp_flips"] == 0


def test_zero_rows_and_zero_weight_columns():
    _banner("zero rows / columns")
    x, w = _case(50, 320, 80, "fp16", n_out=2, seed=6)
    x[3] = 0
    x[10, :] = 0
    w[:, 7] = 0
    w[:, 64] = 0
    parity.run_case(x, w, 6.0)


@pytest.mark.parametrize("dt", ["fp16", "bf16"])
@pytest.mark.parametrize("M", [13, 70, 140])  # small-batch path (one and five row groups) and tiled path
def test_lattice_closed_form_exact_on_gpu(dt, M):
    # power-of-two lattice: every step is exact, so Y must equal RN_T(exact) bitwise,
    # outlier part included (its sums are exact integers in any order)
    _banner(f"lattice {dt} M={M}")
    for seed in range(4):
        xl, wl_, tau, exact, cols = _lattice_case(dt, seed, M=M, K=320, N=136, out_cols=(3, 20, 41, 300))
        X = workloads.from_bits(bits_of(xl, dt), dt)
        W = workloads.from_bits(bits_of(wl_, dt), dt)
        Wq, s_w = lm.int8_quantize_weight(W.cuda())
        Y = lm.int8_matmul(X.cuda(), Wq, s_w, tau)
        with np.errstate(over="ignore"):
            ref = bits_of(exact.astype(np.float32), dt)
        assert np.array_equal(parity.to_bits(Y), ref), seed


def test_empty_batch_and_empty_features():
    _banner("M=0, K=0, N=0")
    Wq = torch.zeros(8, 64, dtype=torch.int8, device="cuda")
    s_w = torch.ones(8, device="cuda")
    Y = lm.int8_matmul(torch.zeros(0, 64, dtype=torch.float16, device="cuda"), Wq, s_w, 6.0)
    assert Y.shape == (0, 8)
    X = torch.randn(5, 0).to(torch.bfloat16).cuda()
    W = torch.zeros(0, 16, dtype=torch.bfloat16, device="cuda")
    Wq0, s0 = lm.int8_quantize_weight(W)
    assert torch.all(s0 == 0)
    Y = lm.int8_matmul(X, Wq0, s0, 6.0, Y=torch.full((5, 16), 7.0, dtype=torch.bfloat16, device="cuda"))
    torch.cuda.synchronize()
    assert torch.all(Y == 0) and not torch.signbit(Y.float()).any()
    # the X pass of an empty feature dimension: no outlier columns, every row scale 0
    ws = torch.full((lm.int8_matmul_workspace_bytes(5, 0, 16),), 0x55, dtype=torch.uint8, device="cuda")
    lm.int8_matmul_prepare(X, Wq0, 6.0, workspace=ws)
    torch.cuda.synchronize()
    v = lm.workspace_views(ws, 5, 0, 16, X.dtype)
    assert v["n_outliers"] == 0 and torch.all(v["s_x"] == 0)
    Y = lm.int8_matmul(torch.randn(4, 32).half().cuda(), torch.zeros(0, 32, dtype=torch.int8, device="cuda"),
                       torch.zeros(0, device="cuda"), 6.0)
    assert Y.shape == (4, 0)


def test_determinism_and_stats():
    _banner("determinism + stats")
    x, w = _case(200, 1024, 384, "bf16", n_out=6, seed=7)
    Xd, Wd = x.cuda(), w.cuda()
    Wq, s_w = lm.int8_quantize_weight(Wd)
    Y1 = lm.int8_matmul(Xd, Wq, s_w, 6.0)
    Y2 = lm.int8_matmul(Xd, Wq, s_w, 6.0)
    torch.cuda.synchronize()
    assert torch.equal(Y1.view(torch.int16), Y2.view(torch.int16))
    n, cols = lm.int8_matmul_stats(Xd, 6.0)
    O = oracle.outlier_columns(workloads.bits(x), "bf16", 6.0)
    assert n == O.size and np.array_equal(cols.cpu().numpy(), O)
    n0, _ = lm.int8_matmul_stats(Xd, float("inf"))
    assert n0 == 0


def test_outputs_outside_y_untouched():
    # canaries around Y: the kernels write exactly M x N elements
    _banner("canaries")
    x, w = _case(70, 256, 136, "fp16", n_out=2, seed=8)
    Wq, s_w = lm.int8_quantize_weight(w.cuda())
    buf = torch.full((70 * 136 + 2048,), 12345.0, dtype=torch.float16, device="cuda")
    Y = buf[1024:1024 + 70 * 136].view(70, 136)
    lm.int8_matmul(x.cuda(), Wq, s_w, 6.0, Y=Y)
    torch.cuda.synchronize()
    assert torch.all(buf[:1024] == 12345.0) and torch.all(buf[1024 + 70 * 136:] == 12345.0)


_FULL = {}


def _full_inputs(name):
    if name not in _FULL:
        _FULL.clear()
        _FULL[name] = workloads.make_workload(name)
    return _FULL[name]


@pytest.mark.parametrize("name", ["ffn_up", "decode", "qkv_175b", "ffn_down"])
def test_full_size_workload_sampled(name):
    x, w, cols, wl = _full_inputs(name)
    _banner(f"full size {name} {wl.M}x{wl.K}x{wl.N} {wl.dtype}")
    # one seeded row in every 256-row tile of the product kernel's schedule, plus the first and last
    rng = np.random.default_rng(11)
    tiles = np.arange(0, wl.M, 256)
    rows = (np.unique(np.concatenate([[0, wl.M - 1], tiles + rng.integers(0, np.minimum(256, wl.M - tiles))]))
            if wl.M > 16 else None)
    st = parity.run_case(x, w, wl.tau, rows=rows)
    assert st["n_outliers"] >= len(cols)
    print(f"[stats] {name}: {st}", flush=True)


def test_two_stage_calls_equal_the_one_call():
    _banner("prepare + products == int8_matmul")
    x, w = _case(130, 512, 264, "bf16", n_out=3, seed=9)
    Xd = x.cuda()
    Wq, s_w = lm.int8_quantize_weight(w.cuda())
    Y1 = lm.int8_matmul(Xd, Wq, s_w, 6.0)
    ws = lm.int8_matmul_prepare(Xd, Wq, 6.0)
    Y2 = lm.int8_matmul_products(130, 512, torch.bfloat16, Wq, s_w, ws)
    Y3 = lm.int8_matmul_products(130, 512, torch.bfloat16, Wq, s_w, ws)  # the workspace is reusable
    torch.cuda.synchronize()
    assert torch.equal(Y1.view(torch.int16), Y2.view(torch.int16))
    assert torch.equal(Y1.view(torch.int16), Y3.view(torch.int16))


# ---- exhaustive quantizer sweeps on the GPU: every finite 16-bit value under ~40 scales

def _finite_patterns(dt):
    p = np.arange(65536, dtype=np.uint32)
    exp_mask = 0x7C00 if dt == "fp16" else 0x7F80
    return p[(p & exp_mask) != exp_mask].astype(np.uint16)


def _sweep_scales(dt):
    """About 40 magnitudes (as 15-bit patterns): evenly spread over the finite range, plus the
    smallest allowed scale, powers of two and the largest finite value.  For bf16 the
    scales stay at or above 2^-120, below which 127/s leaves fp32 (outside the contract)."""
    top = 0x7BFF if dt == "fp16" else 0x7F7F
    low = 0x0001 if dt == "fp16" else 0x0380
    base = np.linspace(low, top, 32).astype(np.int64)
    pow2 = (np.array([0x3C00, 0x4400, 0x5800, 0x0400], np.int64) if dt == "fp16"
            else np.array([0x3F80, 0x4300, 0x4780, 0x0400], np.int64))
    extra = np.array([low, top, low + 1, top - 1], np.int64)
    return np.unique(np.concatenate([base, pow2, extra]))[:40]


def _sweep_rows(dt, width=None):
    """Rows whose absmax is each scale s, holding every finite value of magnitude <= s
    (both signs).  width: split each scale's values over rows of at most `width` columns,
    each row carrying s itself.  Returns 16-bit patterns, zero padded, K a multiple of 16."""
    pats = _finite_patterns(dt)
    mag = (pats & 0x7FFF).astype(np.int64)
    rows = []
    for s in _sweep_scales(dt):
        vals = pats[mag <= s]
        if width is None:
            rows.append(vals)
        else:
            for k in range(0, vals.size, width - 1):
                rows.append(np.concatenate([[np.uint16(s)], vals[k:k + width - 1]]))
    K = int(-(-max(r.size for r in rows) // 16) * 16)
    X = np.zeros((len(rows), K), np.uint16)
    for i, r in enumerate(rows):
        X[i, :r.size] = r
    return X


@pytest.mark.parametrize("dt", ["fp16", "bf16"])
@pytest.mark.parametrize("layout", ["two_reads", "hold16", "hold8", "hold4", "small_batch"])
def test_row_quantizer_exhaustive_sweep(dt, layout):
    """X side: s_x and every code bitwise against the oracle, tau = inf (no outliers),
    through each row-coding configuration: rows longer than the register hold (read
    twice), rows held in registers at each hold size (K <= 32768, 16384, 8192; M > 128),
    and the small-batch launch (64 rows)."""
    width = {"two_reads": None, "hold16": 32768, "hold8": 16384, "hold4": 8192, "small_batch": 32768}[layout]
    Xb = _sweep_rows(dt, width)
    if layout == "small_batch":
        Xb = Xb[:64]
    else:
        while Xb.shape[0] <= 128:  # past the small-batch switch
            Xb = np.concatenate([Xb, Xb[::-1]])
    M, K = Xb.shape
    _banner(f"row quantizer sweep {dt} {layout}: {M} x {K}")
    X = workloads.from_bits(Xb, dt).cuda()
    Wq = torch.zeros((8, K), dtype=torch.int8, device="cuda")
    ws = lm.int8_matmul_prepare(X, Wq, float("inf"))
    torch.cuda.synchronize()
    v = lm.workspace_views(ws, M, K, 8, X.dtype)
    O = oracle.outlier_columns(Xb, dt, float("inf"))
    assert O.size == 0 and v["n_outliers"] == 0
    Xq_o, s_x_o, _ = oracle.quantize_rows(Xb, dt, O)
    assert np.array_equal(v["s_x"].cpu().numpy().view(np.uint32), s_x_o.view(np.uint32)), "s_x differs"
    xq = v["Xq"].cpu().numpy()
    bad = np.argwhere(xq != Xq_o)
    assert bad.size == 0, f"Xq differs at {bad[:5].tolist()} (of {len(bad)})"
    # every nonzero row maps its absmax to +-127
    assert np.all(np.abs(xq.astype(np.int32)).max(axis=1) == 127)


@pytest.mark.parametrize("dt", ["fp16", "bf16"])
def test_weight_quantizer_exhaustive_sweep(dt):
    """W side: the same value sets as the columns of W (K x N), Wq and s_w bitwise."""
    Wb = np.ascontiguousarray(_sweep_rows(dt).T)
    K, N = Wb.shape
    N8 = -(-N // 8) * 8
    Wb = np.concatenate([Wb, np.zeros((K, N8 - N), np.uint16)], axis=1)
    _banner(f"weight quantizer sweep {dt}: {K} x {N8}")
    Wq, s_w = lm.int8_quantize_weight(workloads.from_bits(Wb, dt).cuda())
    torch.cuda.synchronize()
    Wq_o, s_w_o = oracle.quantize_weight(Wb, dt)
    assert np.array_equal(s_w.cpu().numpy().view(np.uint32), s_w_o.view(np.uint32)), "s_w differs"
    bad = np.argwhere(Wq.cpu().numpy() != Wq_o)
    assert bad.size == 0, f"Wq differs at {bad[:5].tolist()} (of {len(bad)})"
