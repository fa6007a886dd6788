"""Pins of the CQ-W2A8 oracle (oracle/w2a8.py) against what the pages and the
arithmetic fix, independently of the oracle's own formulas:

* the fp32 butterfly is the fast form of the Sylvester matrix: exact on
  integer inputs, and within its rounding bound of the float64 rotation;
* int8 activations: the group's absmax lands on +-127, round half to even,
  |x - q sx| <= sx / 2, zero groups, power-of-two scale invariance;
* the int8 codebook: maxabs lands on +-127, |c - c8 sc| <= sc / 2, and the
  ternary crumbs' integers;
* the product: exact assembly on the int8 grid, and the quantisation error
  bound against the exact float64 product (a dropped or doubled scale, a
  wrong sign or a transposed operand breaks one of these).
"""
import math

import numpy as np
import pytest

import cq_inputs
import oracle


def test_butterfly_is_the_sylvester_transform_on_integers():
    # sums of integers below 2^24 are exact in fp32: the butterfly must give
    # S.x exactly, then one fp32 multiply by fp32(1/sqrt(128))
    rng = np.random.default_rng(1)
    x = rng.integers(-1000, 1001, size=(3, 384)).astype(np.float32)
    S = oracle.sylvester(128).astype(np.int64)
    exact = (x.astype(np.int64).reshape(3, 3, 128) @ S).reshape(3, 384)
    want = exact.astype(np.float32) * np.float32(1.0 / math.sqrt(128))
    assert np.array_equal(oracle.rotate_acts_fp32(x), want)
    assert oracle.INV_SQRT_GROUP_F32 == np.float32(0.08838834764831845)


def test_butterfly_error_bound_against_float64_rotation():
    # each of the 7 stages rounds values bounded by the group's L1 norm: the
    # fp32 result is within 2^-16 * ||x_g||_1 / sqrt(128) of H.x (a generous
    # bound; any wrong pairing or sign is off by O(||x_g||))
    x = cq_inputs.activations(7, 0, 4, 1000)
    got = oracle.rotate_acts_fp32(x).astype(np.float64)
    ref = oracle.rotate_acts(x)
    xp = np.zeros((4, 1024))
    xp[:, :1000] = x
    l1 = np.repeat(np.abs(xp).reshape(4, 8, 128).sum(-1), 128, axis=1)
    assert np.all(np.abs(got - ref) <= 2.0 ** -16 * l1 / math.sqrt(128))


def test_int8_activation_half_even_example():
    # absmax 127 gives sx = 1 exactly, so q is x rounded half to even
    g = np.zeros(128, dtype=np.float32)
    g[:8] = [127.0, 2.5, -2.5, 3.5, 0.5, -0.5, 1.5, -126.5]
    q, sx = oracle.quantize_acts_int8(g[None, :])
    assert sx[0, 0] == np.float32(1.0)
    assert q[0, :8].tolist() == [127, 2, -2, 4, 0, 0, 2, -126]
    assert np.all(q[0, 8:] == 0)


def test_int8_activation_properties():
    xr = oracle.rotate_acts_fp32(cq_inputs.activations(7, 1, 3, 2048))
    q, sx = oracle.quantize_acts_int8(xr)
    v = xr.reshape(3, 16, 128).astype(np.float64)
    qv = q.reshape(3, 16, 128)
    # the absmax element of every group maps to +-127 and nothing exceeds it
    assert np.all(np.max(np.abs(qv), axis=-1) == 127)
    # dequantised values are within half a step (plus the fp32 quotient's rounding)
    s = sx.astype(np.float64)[..., None]
    assert np.all(np.abs(v - qv * s) <= s * (0.5 + 1e-6))
    # a power-of-two scale of x scales sx and leaves q unchanged
    q2, sx2 = oracle.quantize_acts_int8(xr * np.float32(8.0))
    assert np.array_equal(q2, q) and np.array_equal(sx2, sx * np.float32(8.0))
    # an all-zero group has sx = 0 and q = 0
    z = xr.copy()
    z[1, 128:256] = 0
    qz, sxz = oracle.quantize_acts_int8(z)
    assert sxz[1, 1] == 0 and np.all(qz[1, 128:256] == 0)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_int8_codebook(bits):
    levels = cq_inputs.codebook(bits)
    c8, sc = oracle.codebook_int8(bits, levels)
    lv = np.asarray(levels, np.float64)
    assert np.max(np.abs(c8)) == 127 and abs(int(c8[np.argmax(np.abs(lv))])) == 127
    assert np.all(np.abs(lv - c8 * float(sc)) <= float(sc) * (0.5 + 1e-6))
    assert np.all(np.diff(c8) > 0)  # the order of the levels survives


def test_int8_codebook_ternary_is_the_crumb_integers():
    c8, sc = oracle.codebook_int8(5)
    assert c8.tolist() == [0, 1, -2, -1]
    assert sc == oracle.ternary_level32()


def _grid_matrix(bits, rows, cols, seed):
    # a matrix whose levels lie on the int8 grid of their own scale: the
    # codebook quantisation is then exact
    c8_target = {2: [-127, -40, 40, 127], 4: list(range(-120, 121, 16))[:15] + [127]}[bits]
    levels = np.asarray(c8_target, np.float32) * np.float32(1e-3)
    w = cq_inputs.master(seed, bits, rows, cols)
    return oracle.quantize(w, bits, levels), levels


@pytest.mark.parametrize("bits", [2, 4])
def test_product_is_exact_on_the_int8_grid(bits):
    # int8 codes and per-group scales in, dense float64 product of the
    # dequantised operands out: the assembly adds no error of its own
    rows, cols = 9, 384
    blob, levels = _grid_matrix(bits, rows, cols, 40 + bits)
    c8, sc = oracle.codebook_int8(bits, levels)
    assert np.allclose(c8 * float(sc), levels, rtol=1e-6, atol=0)
    rng = np.random.default_rng(bits)
    xq = rng.integers(-128, 128, size=(2, 384))
    sx = rng.uniform(0.5, 2.0, size=(2, 3)).astype(np.float32)
    got = oracle.w2a8_from_quantized(blob, bits, rows, cols, xq, sx, levels)
    # dense rotated-domain reference: w_rot = c8[q] * sc * n, x_rot = xq * sx
    packed, norms = oracle.split_blob(blob, bits, rows, cols)
    codes = oracle.unpack_codes(packed, bits, 384)
    w_rot = c8[codes] * float(sc) * np.repeat(norms.astype(np.float32).astype(np.float64), 128, axis=1)
    x_rot = xq * np.repeat(sx.astype(np.float64), 128, axis=1)
    assert np.allclose(got, x_rot @ w_rot.T, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("bits", [1, 2, 3, 4, 5])
def test_product_within_the_quantisation_bound(bits):
    # per group: |<c, xr> - sc sx <c8, q>| <= max|c| * sum|xr - sx q|
    #            + max|c - sc c8| * sx * sum|q| + the fp32 rotation error;
    # summed with the norms, against the exact float64 product
    rows, cols = 24, 1000
    levels = cq_inputs.codebook(bits)
    blob = oracle.quantize(cq_inputs.master(50, bits, rows, cols), bits, levels)
    x = cq_inputs.activations(50, bits, 3, cols)
    got = oracle.matvec_w2a8(blob, bits, rows, cols, x, levels)
    exact = oracle.matvec(blob, bits, rows, cols, x, levels)
    xr = oracle.rotate_acts_fp32(x).astype(np.float64)
    q, sx = oracle.quantize_acts_int8(oracle.rotate_acts_fp32(x))
    c8, sc = oracle.codebook_int8(bits, levels)
    lv = (np.array([0.0, 1.0, -2.0, -1.0]) * float(sc)) if bits == 5 else oracle.codebook_for(bits, levels).astype(np.float64)
    cmax, cerr = np.max(np.abs(lv)), np.max(np.abs(lv - c8 * float(sc)))
    s = np.repeat(sx.astype(np.float64), 128, axis=1)
    act_err = np.abs(xr - q * s).reshape(3, 8, 128).sum(-1)             # sum |xr - sx q| per group
    qsum = (np.abs(q) * s).reshape(3, 8, 128).sum(-1)                    # sx * sum|q| per group
    rot_err = 2.0 ** -16 * np.abs(np.pad(x, ((0, 0), (0, 24)))).reshape(3, 8, 128).sum(-1)
    per_group = cmax * (act_err + rot_err) + cerr * qsum                 # [batch, group]
    _, norms = oracle.split_blob(blob, bits, rows, cols)
    bound = per_group @ norms.astype(np.float64).T                       # [batch, rows]
    assert np.all(np.abs(got - exact) <= bound * (1 + 1e-9) + 1e-12)
    # and the bound discriminates: a flipped sign or a doubled scale breaks it
    assert np.max(np.abs(got - exact)) > 0
    assert np.any(np.abs(-got - exact) > bound) and np.any(np.abs(2 * got - exact) > bound)
