"""Parity of the block-wise absmax int8 codec's HIP kernels with the CPU oracle (through the
C ABI): codes, block scales and the decode, bit for bit."""
import numpy as np
import pytest
import torch

import int8_quantized_matmul_rowwise_amd as lm
import oracle
import workloads

pytestmark = pytest.mark.gpu

BLOCKS = [64, 128, 256, 512, 1024, 2048, 4096]


def _check(x: torch.Tensor, block: int, rows=None):
    n = x.numel()
    q, a = lm.int8_blockwise_quantize(x.cuda(), block)
    xr = lm.int8_blockwise_dequantize(q, a, block)
    torch.cuda.synchronize()
    q_o, a_o = oracle.block_quantize(x.numpy(), block)
    assert np.array_equal(a.cpu().numpy().view(np.uint32), a_o.view(np.uint32)), "absmax differs"
    qg = q.cpu().numpy().ravel()
    bad = np.argwhere(qg != q_o)
    assert bad.size == 0, f"codes differ at {bad[:5].ravel().tolist()} (of {bad.size})"
    xr_o = oracle.block_dequantize(q_o, a_o, block)
    assert np.array_equal(xr.cpu().numpy().ravel().view(np.uint32), xr_o.view(np.uint32)), "decode differs"
    return n


@pytest.mark.parametrize("block", BLOCKS)
def test_codec_parity_ragged(block):
    print(f"\n[case] codec block {block}", flush=True)
    for n in (block * 37, block * 37 + 5, block * 3 + 4 * 7 + 3, block - 1, 1, 3, 4, 5):
        _check(workloads.make_state(n, seed=n % 97), block)


def test_codec_lattice_round_trip_exact_on_gpu():
    block = 256
    rng = np.random.default_rng(3)
    nb = 200
    k = rng.integers(-127, 128, nb * block).astype(np.int64)
    k[::block] = 127
    e = rng.integers(-40, 41, nb)
    x = torch.from_numpy((k * np.exp2(np.repeat(e, block))).astype(np.float32))
    q, a = lm.int8_blockwise_quantize(x.cuda(), block)
    xr = lm.int8_blockwise_dequantize(q, a, block)
    assert np.array_equal(q.cpu().numpy().astype(np.int64), k)
    assert torch.equal(xr.cpu().view(torch.int32), x.view(torch.int32))


def test_codec_zero_blocks_and_tiny_values():
    x = workloads.make_state(2048 * 6, seed=5)
    x[2048:4096] = 0.0
    x[4096:6144] *= 1e-30  # subnormal products in the decode
    _check(x, 2048)


def test_codec_full_size_sampled():
    """The benchmarked size (2^26 of the 2^28 elements, to bound host time), every block."""
    n = 1 << 26
    print(f"\n[case] codec full size n={n}", flush=True)
    _check(workloads.make_state(n, seed=0), 2048)
