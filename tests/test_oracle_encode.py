"""Pins of the oracle's encoder: a literal per-coordinate loop, codebook-point
round trips, the tie rule, zero groups, scale invariance, padding, overflow,
non-idempotence and the Gaussian distortion the Lloyd-Max levels promise."""
import math

import numpy as np
import pytest

import cq_inputs
import oracle
from conftest import golden


def _brute_group(w, levels):
    """Per-coordinate reading of the encoder steps in plain Python floats."""
    n = len(w)
    r = [sum(float(w[k]) * (-1) ** bin(k & j).count("1") for k in range(n)) / math.sqrt(n) for j in range(n)]
    norm = math.sqrt(sum(v * v for v in r))
    q = []
    for v in r:
        u = v / max(norm, 1e-12)
        best = 0
        for j in range(1, len(levels)):
            if abs(u - float(levels[j])) < abs(u - float(levels[best])):
                best = j
        q.append(best)
    return q, norm


@pytest.mark.parametrize("bits,kind", [(2, "empirical"), (3, "empirical"), (4, "empirical"),
                                       (2, "gaussian"), (4, "gaussian"), (5, None)])
def test_matches_literal_loop(bits, kind):
    levels = None if bits == 5 else cq_inputs.codebook(bits, kind)
    lv = oracle.codebook_for(bits, levels)
    w = cq_inputs.master(90, bits, 2, 256)
    codes, norms = oracle.encode(w, bits, levels)
    crumb = {0: 3, 1: 0, 2: 1}
    for r in range(2):
        for g in range(2):
            q, n = _brute_group(w[r, 128 * g:128 * (g + 1)], lv)
            if bits == 5:
                q = [crumb[i] for i in q]
            assert codes[r, 128 * g:128 * (g + 1)].tolist() == q
            assert norms[r, g] == np.float16(np.float32(n))


@pytest.mark.parametrize("bits,kind", [(2, "gaussian"), (3, "gaussian"), (4, "gaussian"), (2, "empirical")])
def test_codebook_points_round_trip(bits, kind):
    # w = (s * c[q]) . H rotates back to s*c[q]: the encoder must return q and norm s*|c[q]|
    # whenever every normalised level c_{q_i}/|c[q]| stays inside its own cell.
    lv = cq_inputs.codebook(bits, kind).astype(np.float64)
    rng = np.random.default_rng(bits)
    H = oracle.hadamard()
    for trial in range(20):
        q = rng.integers(0, len(lv), size=128)
        v = lv[q]
        scaled = v / np.linalg.norm(v)
        mids = (lv[:-1] + lv[1:]) / 2
        if not np.array_equal(np.searchsorted(mids, scaled), q):
            continue
        s = 2.0 ** rng.integers(-6, 3)
        w = (s * v) @ H
        codes, norms = oracle.encode(w[None, :].astype(np.float32), bits, lv.astype(np.float32))
        assert codes[0].tolist() == q.tolist()
        assert abs(float(norms[0, 0]) - s * np.linalg.norm(v)) <= 2.0 ** -10 * s * np.linalg.norm(v)


def test_ties_go_to_the_smaller_index():
    # a constant group rotates to (a, 0, ..., 0) exactly; u = 0 is equidistant
    # from -0.125 and +0.125, and the smaller index (1) must win.
    levels = np.array([-0.25, -0.125, 0.125, 0.25], dtype=np.float32)
    w = np.full((1, 128), 0.03, dtype=np.float32)
    codes, norms = oracle.encode(w, 2, levels)
    assert codes[0, 0] == 3
    assert codes[0, 1:].tolist() == [1] * 127
    assert norms[0, 0] == np.float16(np.float32(0.03 * math.sqrt(128)))


@pytest.mark.parametrize("bits", [2, 3, 4, 5])
def test_zero_group(bits):
    levels = None if bits == 5 else cq_inputs.codebook(bits)
    codes, norms = oracle.encode(np.zeros((2, 256), np.float32), bits, levels)
    assert np.all(norms == 0)
    if bits == 5:
        assert np.all(codes == 0)  # crumb of the 0 level
    else:
        lv = levels.astype(np.float64)
        assert np.all(codes == int(np.argmin(np.abs(lv))))
    assert np.all(oracle.dequantize(oracle.make_blob(oracle.pack_codes(codes, bits), norms),
                                    bits, 2, 256, levels) == 0)


@pytest.mark.parametrize("bits", [2, 4, 5])
def test_power_of_two_scale_invariance(bits):
    levels = None if bits == 5 else cq_inputs.codebook(bits)
    w = cq_inputs.master(91, bits, 4, 384)
    c1, n1 = oracle.encode(w, bits, levels)
    c2, n2 = oracle.encode(w * np.float32(4.0), bits, levels)
    assert np.array_equal(c1, c2)
    assert np.array_equal(n1.astype(np.float32) * 4, n2.astype(np.float32))


def test_padding_is_zero_fill():
    w = cq_inputs.master(92, 0, 3, 200)
    wp = np.zeros((3, 256), np.float32)
    wp[:, :200] = w
    a = oracle.encode(w, 2, cq_inputs.codebook(2))
    b = oracle.encode(wp, 2, cq_inputs.codebook(2))
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_fp16_norm_overflow_stores_infinity():
    w = np.full((1, 128), 1.0e4, dtype=np.float32)
    _, norms = oracle.encode(w, 4, cq_inputs.codebook(4))
    assert np.isinf(norms[0, 0]) and norms[0, 0] > 0


def test_requantisation_is_not_idempotent():
    # The quantised direction is not unit length, so re-encoding w_hat rescales
    # each norm by |c[q]| ...
    levels = cq_inputs.codebook(2)
    w = cq_inputs.master(93, 0, 8, 512)
    codes, norms = oracle.encode(w, 2, levels)
    blob = oracle.make_blob(oracle.pack_codes(codes, 2), norms)
    w_hat = oracle.dequantize(blob, 2, 8, 512, levels).astype(np.float32)
    _, norms2 = oracle.encode(w_hat, 2, levels)
    cnorm = np.linalg.norm(levels.astype(np.float64)[codes].reshape(8, 4, 128), axis=-1)
    assert np.allclose(norms2.astype(np.float64), norms.astype(np.float64) * cnorm, rtol=2e-3, atol=0)
    assert np.any(np.abs(cnorm - 1) > 1e-3)
    # ... and can move codes: with levels (-1/4, -1/8, 1/8, 1/4), a direction of 127
    # coordinates at 0.07 and one large one stores codes (2, ..., 2, 3); the
    # reconstruction's direction c[q]/|c[q]| puts the large coordinate at 0.175,
    # nearer 1/8 than 1/4.
    lv = np.array([-0.25, -0.125, 0.125, 0.25], dtype=np.float32)
    u = np.full(128, 0.07)
    u[0] = np.sqrt(1 - 127 * 0.07 ** 2)
    g = (u @ oracle.hadamard())[None, :].astype(np.float32)
    c1, n1 = oracle.encode(g, 2, lv)
    assert c1[0, 0] == 3 and np.all(c1[0, 1:] == 2)
    again = oracle.dequantize(oracle.make_blob(oracle.pack_codes(c1, 2), n1), 2, 1, 128, lv)
    c2, _ = oracle.encode(again.astype(np.float32), 2, lv)
    assert c2[0, 0] == 2 and np.all(c2[0, 1:] == 2)


@pytest.mark.parametrize("bits,L", [(2, 4), (3, 8), (4, 16), (5, 3)])
def test_distortion_and_code_frequencies_follow_the_gaussian_quantiser(bits, L):
    g = golden("max1960_gaussian.json")
    levels = None if bits == 5 else cq_inputs.codebook(bits, "gaussian")
    rows, cols = 256, 1024
    w = cq_inputs.master(94, bits, rows, cols)
    codes, norms = oracle.encode(w, bits, levels)
    blob = oracle.make_blob(oracle.pack_codes(codes, bits), norms)
    w_hat = oracle.dequantize(blob, bits, rows, cols, levels)
    d = np.sum((w - w_hat) ** 2) / np.sum(w.astype(np.float64) ** 2)
    assert abs(d - g["levels"][str(L)]["mse"]) / g["levels"][str(L)]["mse"] < 0.03
    # fraction of coordinates in each cell ~ Gaussian cell probabilities
    from scipy import stats
    if bits == 5:
        a = oracle.ternary_level()
        probs = np.diff(stats.norm.cdf([-np.inf, -a / 2, a / 2, np.inf]))
        freq = np.array([np.mean(codes == 3), np.mean(codes == 0), np.mean(codes == 1)])
    else:
        c = oracle.gaussian_lloyd_max(L)
        probs = np.diff(stats.norm.cdf(np.concatenate([[-np.inf], (c[:-1] + c[1:]) / 2, [np.inf]])))
        freq = np.bincount(codes.ravel(), minlength=L) / codes.size
    assert np.max(np.abs(freq - probs)) < 0.01
