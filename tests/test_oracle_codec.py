"""Pins of the oracle's block-wise absmax int8 codec (talk summary "llama3-model-quantization",
Key Points, 8-bit optimizers: per-block normalisation by the block maximum, 8-bit values).

None of these re-types the codec: they check closed forms on exactly representable
lattices, agreement with the scalar quantizer (pinned exhaustively elsewhere) block by
block, the error bound, exact symmetries, and degenerate shapes."""
import numpy as np
import pytest

import oracle

BLOCKS = [1, 7, 64, 256, 2048]


def _state(n, seed, tail=0.001):
    """Optimizer-state-like values: N(0, 1e-3) with a thin tail of large entries."""
    rng = np.random.default_rng(seed)
    x = rng.normal(0.0, 1e-3, n).astype(np.float32)
    k = rng.random(n) < tail
    x[k] = (rng.choice([-1.0, 1.0], k.sum()) * rng.uniform(0.01, 0.5, k.sum())).astype(np.float32)
    return x


@pytest.mark.parametrize("block", [16, 64, 2048])
def test_codec_lattice_round_trip_is_exact(block):
    # x = k * 2^e, |k| <= 127, each block holding +-127 * 2^e: RN32(127/s) = 2^-e and
    # RN32(s/127) = 2^e exactly, so the codes are k and the decode returns x bit for bit.
    rng = np.random.default_rng(block)
    nb = 40
    n = nb * block - block // 3  # ragged last block
    k = rng.integers(-127, 128, n).astype(np.int64)
    e = rng.integers(-30, 31, nb)
    for b in range(nb):
        lo = b * block
        k[lo] = 127 * (1 if rng.random() < 0.5 else -1)
    x = (k * np.exp2(np.repeat(e, block)[:n])).astype(np.float32)
    q, absmax = oracle.block_quantize(x, block)
    assert np.array_equal(q.astype(np.int64), k)
    assert np.array_equal(absmax, (127.0 * np.exp2(e)).astype(np.float32))
    assert np.array_equal(oracle.block_dequantize(q, absmax, block).view(np.uint32), x.view(np.uint32))


@pytest.mark.parametrize("block", BLOCKS)
def test_codec_blocks_use_the_scalar_quantizer(block):
    x = _state(5000 + 13, seed=block)
    q, absmax = oracle.block_quantize(x, block)
    nb = -(-x.size // block)
    assert absmax.size == nb
    for b in range(nb):
        xb = x[b * block:(b + 1) * block]
        assert absmax[b] == np.max(np.abs(xb))
        assert np.array_equal(q[b * block:(b + 1) * block], oracle.quantize(xb, float(absmax[b])))


@pytest.mark.parametrize("block", BLOCKS)
def test_codec_error_bound_and_range(block):
    x = _state(20000, seed=7 + block)
    q, absmax = oracle.block_quantize(x, block)
    xr = oracle.block_dequantize(q, absmax, block)
    s = np.repeat(absmax, block)[:x.size].astype(np.float64)
    assert np.all(np.abs(q.astype(np.int32)) <= 127)
    # half a step plus the rounding of the scale and of the products (relative 2^-20)
    assert np.all(np.abs(xr.astype(np.float64) - x) <= s / 254.0 * (1 + 2.0**-20) + s * 2.0**-20)
    nb = absmax.size
    qm = np.array([np.abs(q[b * block:(b + 1) * block].astype(np.int32)).max() for b in range(nb)])
    assert np.all(qm[absmax > 0] == 127)


def test_codec_symmetries():
    block = 256
    x = _state(10 * block + 5, seed=3)
    q, a = oracle.block_quantize(x, block)
    xr = oracle.block_dequantize(q, a, block)
    qn, an = oracle.block_quantize(-x, block)
    assert np.array_equal(qn, -q) and np.array_equal(an, a)
    q2, a2 = oracle.block_quantize(x * np.float32(8.0), block)
    assert np.array_equal(q2, q) and np.array_equal(a2, a * np.float32(8.0))
    assert np.array_equal(oracle.block_dequantize(q2, a2, block), xr * np.float32(8.0))
    # blocks are independent: changing block 3 leaves every other block's codes alone
    y = x.copy()
    y[3 * block:4 * block] *= np.float32(50.0)
    qy, ay = oracle.block_quantize(y, block)
    keep = np.ones(x.size, bool)
    keep[3 * block:4 * block] = False
    assert np.array_equal(qy[keep], q[keep]) and np.array_equal(np.delete(ay, 3), np.delete(a, 3))
    # a permutation inside a block permutes its codes
    perm = np.random.default_rng(1).permutation(block)
    z = x.copy()
    z[:block] = x[:block][perm]
    qz, _ = oracle.block_quantize(z, block)
    assert np.array_equal(qz[:block], q[:block][perm])


def test_codec_degenerate_shapes():
    # one element per block: every nonzero element codes to +-127 and decodes to itself
    x = _state(300, seed=5)
    q, a = oracle.block_quantize(x, 1)
    assert np.array_equal(np.abs(q[x != 0].astype(np.int32)), np.full((x != 0).sum(), 127))
    assert np.array_equal(a, np.abs(x))
    # a block of zeros: scale 0, codes 0, decode +0
    z = np.zeros(100, np.float32)
    qz, az = oracle.block_quantize(z, 64)
    assert not qz.any() and not az.any() and not oracle.block_dequantize(qz, az, 64).any()
    # block larger than the tensor: one block
    q1, a1 = oracle.block_quantize(x, 4096)
    assert a1.size == 1 and a1[0] == np.abs(x).max()
    # empty tensor
    q0, a0 = oracle.block_quantize(np.zeros(0, np.float32), 64)
    assert q0.size == 0 and a0.size == 0
