"""Pins of the oracle's binary (1-bit) matrices against what the pages and the
mathematics fix, not against the oracle's own formulas:

* the level is the mean of the positive half of N(0, 1) (numerical
  integration) and the fixed point of the 2-level Lloyd-Max iteration;
* eight codes per byte, LSB first: a hand-made byte, and the packer against
  an explicit per-bit formula;
* the encoder keeps the sign of each rotated coordinate (dense float64
  rotation), a zero group encodes to code 0 and norm 0;
* the product equals n * c * sum(+-xr) written out with explicit loops;
* the int8 code book of the W2A8 product is +-127.
"""
import math

import numpy as np
import pytest
from scipy import integrate

import cq_inputs
import oracle


def test_binary_level_is_the_half_normal_mean():
    phi = lambda z: math.exp(-0.5 * z * z) / math.sqrt(2 * math.pi)
    num, _ = integrate.quad(lambda z: z * phi(z), 0, math.inf, epsabs=0, epsrel=1e-12)
    den, _ = integrate.quad(phi, 0, math.inf, epsabs=0, epsrel=1e-12)
    mean = num / den
    assert abs(oracle.binary_level() - mean) < 1e-12
    # the 2-level Lloyd-Max fixed point of N(0, 1) is +-E[Z | Z > 0]
    lm = oracle.gaussian_lloyd_max(2)
    assert np.allclose(lm, [-mean, mean], rtol=0, atol=1e-12)
    assert oracle.binary_level32() == np.float32(mean / math.sqrt(128))
    assert oracle.codebook_for(1).tolist() == [-oracle.binary_level32(), oracle.binary_level32()]
    with pytest.raises(ValueError):
        oracle.codebook_for(1, [0.0, 1.0])


def test_binary_sizes():
    assert oracle.storage_bits(1) == 1
    assert oracle.bits_per_weight(1) == 1.125
    # 130 columns pad to 256: 32 bytes of bits and 2 norms per row
    assert oracle.blob_bytes(1, 128, 3, 130) == 3 * 32 + 3 * 2 * 2


def test_binary_pack_hand_example():
    codes = np.array([[1, 0, 1, 1, 0, 0, 0, 1, 0, 1, 1, 1, 1, 1, 1, 0]], dtype=np.uint8)
    packed = oracle.pack_codes(codes, 1)
    assert packed.tolist() == [[0b10001101, 0b01111110]]
    assert np.array_equal(oracle.unpack_codes(packed, 1, 16), codes)


def test_binary_pack_matches_per_bit_formula():
    rng = np.random.default_rng(3)
    codes = rng.integers(0, 2, size=(5, 384)).astype(np.uint8)
    packed = oracle.pack_codes(codes, 1)
    assert packed.shape == (5, 48)
    for r in range(5):
        for col in range(384):
            assert (int(packed[r, col // 8]) >> (col % 8)) & 1 == codes[r, col]
    assert np.array_equal(oracle.unpack_codes(packed, 1, 384), codes)


def test_binary_encoder_keeps_the_sign():
    w = cq_inputs.master(120, 1, 6, 300)
    codes, norms = oracle.encode(w, 1)
    wp = np.zeros((6, 384))
    wp[:, :300] = w
    r = (wp.reshape(6, 3, 128) @ oracle.hadamard()).reshape(6, 384)
    assert np.all(np.abs(r) > 1e-9)  # no coordinate near the threshold in this draw
    assert np.array_equal(codes, (r > 0).astype(np.uint8))
    n = np.sqrt((r.reshape(6, 3, 128) ** 2).sum(-1))
    assert np.allclose(norms.astype(np.float64), n, rtol=2 ** -10, atol=0)
    # a zero group: every coordinate ties between -c and +c, the smaller
    # index (code 0) wins, and the norm is 0
    z = np.zeros((1, 128), np.float32)
    cz, nz = oracle.encode(z, 1)
    assert np.all(cz == 0) and nz[0, 0] == 0


def test_binary_product_closed_form():
    rows, cols = 5, 300
    blob = oracle.quantize(cq_inputs.master(121, 1, rows, cols), 1)
    x = cq_inputs.activations(121, 1, 2, cols)
    got = oracle.matvec(blob, 1, rows, cols, x)
    kpad = 384
    packed = blob[: rows * kpad // 8].reshape(rows, kpad // 8)
    norms = blob[rows * kpad // 8:].view("<f2").reshape(rows, 3).astype(np.float64)
    c = float(oracle.binary_level32())
    for b in range(2):
        xp = [float(v) for v in x[b]] + [0.0] * (kpad - cols)
        for r in range(rows):
            total = 0.0
            for g in range(3):
                s = 0.0
                for j in range(128):
                    xr = sum(xp[128 * g + k] * (-1) ** bin(k & j).count("1") for k in range(128)) / math.sqrt(128)
                    col = 128 * g + j
                    bit = (int(packed[r, col >> 3]) >> (col & 7)) & 1
                    s += (c if bit else -c) * xr
                total += norms[r, g] * s
            assert abs(got[b, r] - total) <= 1e-12 * (1 + abs(total))


def test_binary_int8_codebook():
    c8, sc = oracle.codebook_int8(1)
    c = oracle.binary_level32()
    assert c8.tolist() == [-127, 127]
    assert sc == np.float32(c / np.float32(127.0))
    assert abs(127 * float(sc) - float(c)) <= float(sc) / 2
