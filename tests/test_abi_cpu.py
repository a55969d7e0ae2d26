"""The C-ABI boundary on the CPU: the library loads, exports every function its header
declares, sizes its workspace, and rejects bad arguments before any GPU work (these
calls return before the first HIP call, so they run without a GPU)."""
import ctypes
import math
import re

import pytest

import int8_quantized_matmul_rowwise_amd as L

INF = float("inf")
A16 = 0x10000  # a fake, 16-byte-aligned device address: never dereferenced by these calls


def _declared_functions():
    src = open(L.HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\**\s*([a-z_0-9]+)\s*\(", src, flags=re.M)))


def test_library_exports_every_declared_function():
    names = _declared_functions()
    assert set(names) >= {"int8_quantize_weight", "int8_matmul", "int8_matmul_stats",
                          "int8_matmul_workspace_bytes", "int8_matmul_workspace_layout",
                          "int8_matmul_accumulators", "llmint8_status_string"}
    lib = ctypes.CDLL(L.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(L._SIGNATURES)


def test_status_strings():
    for s in (0, -1, -2, -3, -4, 7):
        assert L.status_string(s).startswith("LLMINT8")


def test_workspace_layout_regions_fit_and_align():
    for (M, K, N) in [(1, 16, 8), (32, 256, 128), (300, 1040, 520), (4096, 12288, 36864), (0, 64, 8), (5, 0, 8),
                      (16, 8192, 8192)]:
        lay = L.int8_matmul_workspace_layout(M, K, N)
        assert lay["total"] == L.int8_matmul_workspace_bytes(M, K, N)
        assert lay["xq_pitch"] % 256 == 0 and lay["xq_pitch"] >= K
        assert lay["xo_pitch"] % 32 == 0 and lay["xo_pitch"] >= K
        # the small-batch product kernel gathers Wq[:,O] itself: no W_O region then
        wo = 0 if lay["small_batch"] else 2 * N * lay["xo_pitch"]
        regions = sorted([(lay["xq"], M * lay["xq_pitch"]), (lay["s_x"], 4 * M), (lay["n_outliers"], 4),
                          (lay["outliers"], 4 * K), (lay["xo"], 2 * M * lay["xo_pitch"]),
                          (lay["wo"], wo), (lay["scratch"], 4 * math.ceil(K / 32))])
        for (o, n), (o2, _) in zip(regions, regions[1:]):
            assert o % 256 == 0 and o + n <= o2
        assert regions[-1][0] + regions[-1][1] <= lay["total"]


def test_workspace_views_of_both_paths():
    # the views of a workspace (a host buffer here) for a small-batch and a tiled layout
    import torch
    for (M, K, N, small) in [(40, 1040, 264, True), (300, 1040, 520, False), (16, 8192, 8192, True)]:
        lay = L.int8_matmul_workspace_layout(M, K, N)
        assert lay["small_batch"] == small
        ws = torch.zeros(lay["total"], dtype=torch.uint8)
        v = L.workspace_views(ws, M, K, N, torch.float16)
        assert v["Xq"].shape == (M, K) and v["s_x"].numel() == M and v["n_outliers"] == 0
        assert (v["WO"] is None) == small


def _mm(**kw):
    a = dict(X=A16, M=4, K=64, dt=0, Wq=A16 * 2, s_w=A16 * 3, N=8, tau=6.0, Y=A16 * 4 + 0x100000,
             ws=A16 * 0x1000, wsb=1 << 30, stream=None)
    a.update(kw)
    return L.lib().int8_matmul(a["X"], a["M"], a["K"], a["dt"], a["Wq"], a["s_w"], a["N"], a["tau"], a["Y"],
                               a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(dt=2), L.EINVAL), (dict(M=-1), L.EINVAL), (dict(K=-16), L.EINVAL), (dict(N=-8), L.EINVAL),
    (dict(K=24), L.EINVAL), (dict(N=12), L.EINVAL), (dict(K=133152), L.ERANGE),
    (dict(tau=float("nan")), L.EINVAL), (dict(tau=-1.0), L.EINVAL),
    (dict(X=None), L.EINVAL), (dict(X=A16 + 8), L.EINVAL), (dict(Wq=None), L.EINVAL), (dict(Y=None), L.EINVAL),
    (dict(Y=A16 + 2), L.EINVAL), (dict(s_w=None), L.EINVAL), (dict(ws=None), L.EWORKSPACE), (dict(wsb=100), L.EWORKSPACE),
    (dict(Y=A16), L.EINVAL),  # Y overlaps X
])
def test_matmul_rejects(kw, code):
    assert _mm(**kw) == code


def test_matmul_empty_batch_is_a_noop():
    assert _mm(M=0, X=None, ws=None, wsb=0) == L.OK


def test_quantize_weight_rejects():
    q = L.lib().int8_quantize_weight
    assert q(A16, 64, 8, 3, A16 * 2, A16 * 4, None) == L.EINVAL
    assert q(A16, 60, 8, 0, A16 * 2, A16 * 4, None) == L.EINVAL
    assert q(A16, 64, 9, 0, A16 * 2, A16 * 4, None) == L.EINVAL
    assert q(None, 64, 8, 0, A16 * 2, A16 * 4, None) == L.EINVAL
    assert q(A16, 64, 8, 0, A16 * 2, None, None) == L.EINVAL
    assert q(A16, 64, 8, 0, A16 + 64, A16 * 4, None) == L.EINVAL     # Wq overlaps W
    assert q(A16, 200000, 8, 0, A16 * 2, A16 * 4, None) == L.ERANGE
    assert q(None, 64, 0, 0, None, None, None) == L.OK                # N = 0: nothing to do


def test_stats_rejects():
    s = L.lib().int8_matmul_stats
    n = ctypes.c_int32(-5)
    assert s(A16, 4, 64, 0, 6.0, None, None, A16 * 4, 1 << 20, None) == L.EINVAL
    assert s(A16, 4, 64, 0, float("nan"), ctypes.byref(n), None, A16 * 4, 1 << 20, None) == L.EINVAL
    assert s(A16, 4, 64, 0, 6.0, ctypes.byref(n), None, A16 * 4, 10, None) == L.EWORKSPACE
    assert s(A16, 4, 60, 0, 6.0, ctypes.byref(n), None, A16 * 4, 1 << 20, None) == L.EINVAL
    assert s(None, 0, 64, 0, 6.0, ctypes.byref(n), None, None, 0, None) == L.OK and n.value == 0


def test_accumulators_rejects():
    a = L.lib().int8_matmul_accumulators
    assert a(A16, 4, 64, 0, A16 * 2, 8, 6.0, None, A16 * 8, A16 * 16, 1 << 30, None) == L.EINVAL
    assert a(A16, 4, 64, 1, A16 * 2, 8, -2.0, A16 * 4, A16 * 8, A16 * 16, 1 << 30, None) == L.EINVAL


def test_binding_fails_loudly_without_gpu_tensors():
    import torch
    with pytest.raises(TypeError):
        L.int8_matmul(torch.zeros(4, 64, dtype=torch.float16), torch.zeros(8, 64, dtype=torch.int8),
                      torch.zeros(8), 6.0)


def test_blockwise_codec_rejects():
    qz, dq = L.lib().int8_blockwise_quantize, L.lib().int8_blockwise_dequantize
    X, Q, S = A16, A16 * 64, A16 * 128  # disjoint fake device buffers for n = 4096
    for block in (0, 32, 96, 100, 8192, -64):
        assert qz(X, 4096, block, Q, S, None) == L.EINVAL
        assert dq(Q, S, 4096, block, X, None) == L.EINVAL
    assert qz(X, -1, 2048, Q, S, None) == L.EINVAL
    assert qz(None, 4096, 2048, Q, S, None) == L.EINVAL
    assert qz(X, 4096, 2048, None, S, None) == L.EINVAL
    assert qz(X, 4096, 2048, Q, None, None) == L.EINVAL
    assert qz(X + 8, 4096, 2048, Q, S, None) == L.EINVAL        # x not 16-byte aligned
    assert qz(X, 4096, 2048, Q + 2, S, None) == L.EINVAL        # q not 4-byte aligned
    assert qz(X, 4096, 2048, X + 64, S, None) == L.EINVAL       # q overlaps x
    assert qz(X, 4096, 2048, Q, Q + 1024, None) == L.EINVAL     # absmax overlaps q
    assert dq(Q, S, 4096, 2048, Q - 64, None) == L.EINVAL       # x overlaps q
    assert dq(Q, S, 4096, 2048, X + 4, None) == L.EINVAL        # x not 16-byte aligned
    assert qz(None, 0, 2048, None, None, None) == L.OK           # empty: nothing to do
    assert dq(None, None, 0, 64, None, None) == L.OK


def test_fixed_outlier_entry_points_reject():
    wf, mf = L.lib().int8_quantize_weight_fixed, L.lib().int8_matmul_fixed
    kb = L.lib().int8_quantize_weight_fixed_workspace_bytes
    assert kb(64) >= 8 and kb(-1) == 0
    W, Wq, S, O, WO, WS = A16, A16 * 64, A16 * 128, A16 * 192, A16 * 256, A16 * 320
    assert wf(W, 64, 8, 0, O, -1, Wq, S, WO, WS, 1 << 16, None) == L.EINVAL      # n_O < 0
    assert wf(W, 64, 8, 0, O, 65, Wq, S, WO, WS, 1 << 16, None) == L.EINVAL      # n_O > K
    assert wf(W, 64, 8, 0, None, 3, Wq, S, WO, WS, 1 << 16, None) == L.EINVAL    # no list
    assert wf(W, 64, 8, 0, O, 3, Wq, S, None, WS, 1 << 16, None) == L.EINVAL     # no W_O
    assert wf(W, 64, 8, 0, O + 2, 3, Wq, S, WO, WS, 1 << 16, None) == L.EINVAL   # list misaligned
    assert wf(W, 64, 8, 0, O, 3, Wq, S, WO, WS, 4, None) == L.EWORKSPACE          # workspace too small
    assert wf(W, 64, 8, 0, O, 3, Wq, S, WO, WO + 16, 1 << 16, None) == L.EINVAL  # workspace overlaps W_O
    assert wf(W, 60, 8, 0, O, 3, Wq, S, WO, WS, 1 << 16, None) == L.EINVAL       # K % 16
    assert wf(None, 64, 0, 0, None, 0, None, None, None, None, 0, None) == L.OK  # N = 0
    X, Y = A16, A16 * 512
    big = 1 << 30
    assert mf(X, 4, 64, 0, O, -1, Wq, S, WO, 8, Y, WS, big, None) == L.EINVAL
    assert mf(X, 4, 64, 0, O, 65, Wq, S, WO, 8, Y, WS, big, None) == L.EINVAL
    assert mf(X, 4, 64, 0, None, 2, Wq, S, WO, 8, Y, WS, big, None) == L.EINVAL
    assert mf(X, 4, 64, 0, O, 2, Wq, S, None, 8, Y, WS, big, None) == L.EINVAL
    assert mf(X, 4, 64, 0, O, 2, Wq, S, WO, 8, Y, WS, 16, None) == L.EWORKSPACE
    assert mf(X, 4, 64, 0, O, 2, Wq, S, WO, 8, WO + 64, WS, big, None) == L.EINVAL  # Y overlaps W_O
    assert mf(X, 4, 64, 2, O, 2, Wq, S, WO, 8, Y, WS, big, None) == L.EINVAL        # dtype
    assert mf(None, 0, 64, 0, None, 0, Wq, S, None, 8, None, None, 0, None) == L.OK  # M = 0


def test_group_entry_points_reject():
    wg, mg = L.lib().int8_quantize_weight_group, L.lib().int8_matmul_group
    wb = L.lib().int8_matmul_group_workspace_bytes
    MB = 0x100000
    W, Wq, S, X, Y, WS = MB, 2 * MB, 3 * MB, 4 * MB, 5 * MB, 8 * MB
    need = wb(4, 1024, 128)
    assert need >= 4 * 1024 + 2 * 4 * 4 * 8 and need % 256 == 0
    assert wb(4, 1024, 100) == 0 and wb(-1, 1024, 128) == 0 and wb(4, 1024, 2048) == 0
    for G in (0, 64, 100, 192, -128, 8192):
        assert wg(W, 8192, 8, 0, G, Wq, S, None) == L.EINVAL, G
        assert mg(X, 4, 8192, 0, G, Wq, S, 8, Y, WS, 1 << 30, None) == L.EINVAL, G
    assert wg(W, 384, 8, 0, 256, Wq, S, None) == L.EINVAL                       # G does not divide K
    assert wg(W, 1024, 8, 2, 128, Wq, S, None) == L.EINVAL                      # dtype
    assert wg(None, 1024, 8, 0, 128, Wq, S, None) == L.EINVAL
    assert wg(W, 1024, 8, 0, 128, Wq + 8, S, None) == L.EINVAL                  # Wq not 16-byte aligned
    assert wg(W, 1024, 8, 0, 128, W + 64, S, None) == L.EINVAL                  # Wq overlaps W
    assert wg(W, 1024, 0, 0, 128, None, None, None) == L.OK                     # N = 0
    assert mg(X, 4, 1024, 0, 128, Wq, S, 8, Y, WS, need - 1, None) == L.EWORKSPACE
    assert mg(X, 4, 1024, 0, 128, Wq, S, 8, Y, WS + 16, need + 256, None) == L.EWORKSPACE  # not 256-aligned
    assert mg(X, 4, 1024, 0, 128, Wq, S, 8, None, WS, need, None) == L.EINVAL   # no Y
    assert mg(X, 4, 1024, 0, 128, Wq, S, 8, X + 64, WS, need, None) == L.EINVAL  # Y overlaps X
    assert mg(X, 4, 1024, 0, 128, Wq, S, 8, Y, X, need, None) == L.EINVAL       # workspace overlaps X
    assert mg(None, 4, 1024, 0, 128, Wq, S, 8, Y, WS, need, None) == L.EINVAL
    assert mg(X, 4, 1040, 0, 128, Wq, S, 8, Y, WS, 1 << 30, None) == L.EINVAL  # G does not divide K
    assert mg(X, 4, 1024, 0, 128, Wq, S, 12, Y, WS, 1 << 30, None) == L.EINVAL  # N % 8
    assert mg(None, 0, 1024, 0, 128, Wq, S, 8, None, None, 0, None) == L.OK     # M = 0
    assert mg(X, 4, 1024, 0, 128, Wq, S, 0, None, None, 0, None) == L.OK        # N = 0


def test_group_route_query():
    q = L.int8_matmul_group_small_batch
    assert q(16, 8192, 8192, 1024) and q(1, 1024, 264, 128)
    assert not q(4096, 12288, 36864, 1024) and not q(300, 1024, 264, 128)
    assert L.lib().int8_matmul_group_small_batch(16, 8192, 8192, 100) == L.EINVAL


def test_group_two_stage_entry_points_reject():
    pg, gp = L.lib().int8_matmul_group_prepare, L.lib().int8_matmul_group_products
    need = L.lib().int8_matmul_group_workspace_bytes(4, 1024, 128)
    MB = 0x100000
    X, Wq, S, Y, WS = MB, 2 * MB, 3 * MB, 5 * MB, 8 * MB
    assert pg(X, 4, 1024, 0, 100, WS, need, None) == L.EINVAL            # group size
    assert pg(X, 4, 1024, 0, 128, WS, need - 1, None) == L.EWORKSPACE
    assert pg(None, 4, 1024, 0, 128, WS, need, None) == L.EINVAL
    assert pg(X, 4, 1024, 0, 128, X + 256, need, None) == L.EINVAL       # workspace overlaps X
    assert pg(None, 0, 1024, 0, 128, None, 0, None) == L.OK              # M = 0
    assert gp(4, 1024, 0, 128, Wq, S, 8, Y, WS, need - 1, None) == L.EWORKSPACE
    assert gp(4, 1024, 0, 128, Wq, S, 8, None, WS, need, None) == L.EINVAL
    assert gp(4, 1024, 0, 128, None, S, 8, Y, WS, need, None) == L.EINVAL
    assert gp(4, 1024, 0, 128, Wq, S, 8, WS + 256, WS, need, None) == L.EINVAL  # Y overlaps the workspace
    assert gp(4, 1024, 0, 128, Wq, S, 0, None, None, 0, None) == L.OK    # N = 0
