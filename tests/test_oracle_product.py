"""Pins of the oracle's products: the rotated-activation identity by brute
force, the Hadamard-column probe, linearity, Parseval, the end-to-end
quantisation error, and the bf16 variant against its analytic bound."""
import numpy as np
import pytest

import cq_inputs
import oracle


def _butterfly(v):
    v = np.array(v, dtype=np.float64)
    h = 1
    while h < v.shape[-1]:
        for i in range(0, v.shape[-1], 2 * h):
            a = v[..., i:i + h].copy()
            b = v[..., i + h:i + 2 * h].copy()
            v[..., i:i + h] = a + b
            v[..., i + h:i + 2 * h] = a - b
        h *= 2
    return v / np.sqrt(v.shape[-1])


def _blob(cfg, bits, rows, cols, kind="empirical"):
    levels = None if bits == 5 else cq_inputs.codebook(bits, kind)
    w = cq_inputs.master(cfg, bits, rows, cols)
    return oracle.quantize(w, bits, levels), levels, w


@pytest.mark.parametrize("bits", [2, 3, 4, 5])
def test_rotated_activation_identity(bits):
    rows, cols = 6, 300
    blob, levels, _ = _blob(95, bits, rows, cols)
    x = cq_inputs.activations(95, bits, 3, cols)
    y = oracle.matvec(blob, bits, rows, cols, x, levels)
    # sum_g n_g <c[q_g], H x_g>, with the butterfly rotation and explicit loops
    packed, norms = oracle.split_blob(blob, bits, rows, cols)
    kpad = 384
    vals = oracle.level_values(oracle.unpack_codes(packed, bits, kpad), bits, levels)
    xp = np.zeros((3, kpad))
    xp[:, :cols] = x
    xr = _butterfly(xp.reshape(3, 3, 128))
    for b in range(3):
        for r in range(rows):
            acc = 0.0
            for g in range(3):
                acc += float(norms[r, g]) * float(np.dot(vals[r, 128 * g:128 * (g + 1)], xr[b, g]))
            scale = np.linalg.norm(oracle.dequantize(blob, bits, rows, cols, levels)[r]) * np.linalg.norm(x[b])
            assert abs(acc - y[b, r]) <= 1e-13 * scale


@pytest.mark.parametrize("bits", [2, 3, 4, 5])
def test_hadamard_column_probe_reads_back_each_index(bits):
    rows, cols = 5, 256
    blob, levels, _ = _blob(96, bits, rows, cols)
    packed, norms = oracle.split_blob(blob, bits, rows, cols)
    codes = oracle.unpack_codes(packed, bits, 256)
    vals = oracle.level_values(codes, bits, levels)
    H = oracle.hadamard()
    for g in (0, 1):
        for j in (0, 1, 2, 3, 7, 8, 63, 64, 127):
            x = np.zeros((1, cols))
            x[0, 128 * g:128 * (g + 1)] = H @ np.eye(128)[j]
            y = oracle.matvec(blob, bits, rows, cols, x, levels)[0]
            expect = norms[:, g].astype(np.float64) * vals[:, 128 * g + j]
            assert np.allclose(y, expect, rtol=0, atol=1e-14)


def test_linearity_zero_and_parseval():
    rows, cols = 7, 512
    blob, levels, _ = _blob(97, 2, rows, cols)
    x1 = cq_inputs.activations(97, 1, 1, cols)
    x2 = cq_inputs.activations(97, 2, 1, cols)
    y1 = oracle.matvec(blob, 2, rows, cols, x1, levels)
    y2 = oracle.matvec(blob, 2, rows, cols, x2, levels)
    y12 = oracle.matvec(blob, 2, rows, cols, x1.astype(np.float64) + 2 * x2.astype(np.float64), levels)
    assert np.allclose(y12, y1 + 2 * y2, rtol=0, atol=1e-12)
    assert np.all(oracle.matvec(blob, 2, rows, cols, np.zeros((1, cols)), levels) == 0)
    packed, norms = oracle.split_blob(blob, 2, rows, cols)
    vals = oracle.level_values(oracle.unpack_codes(packed, 2, 512), 2, levels).reshape(rows, 4, 128)
    w_hat = oracle.dequantize(blob, 2, rows, cols, levels).reshape(rows, 4, 128)
    assert np.allclose(np.linalg.norm(w_hat, axis=-1),
                       norms.astype(np.float64) * np.linalg.norm(vals, axis=-1), rtol=1e-14, atol=0)


@pytest.mark.parametrize("bits,min_cos", [(2, 0.92), (3, 0.975), (4, 0.993), (5, 0.88)])
def test_end_to_end_error_matches_quantiser_distortion(bits, min_cos):
    # y_quantised vs the unquantised product W.x: cosine ~ sqrt(1 - D_L)
    rows, cols = 256, 1024
    blob, levels, w = _blob(98, bits, rows, cols, "gaussian" if bits != 5 else "empirical")
    x = cq_inputs.activations(98, bits, 1, cols)
    y = oracle.matvec(blob, bits, rows, cols, x, levels)[0]
    exact = w.astype(np.float64) @ x[0].astype(np.float64)
    cos = y @ exact / np.linalg.norm(y) / np.linalg.norm(exact)
    assert min_cos < cos < 0.9999


def test_gemm_rows_equal_matvec_and_row_subsets():
    rows, cols = 9, 256
    blob, levels, _ = _blob(99, 4, rows, cols)
    X = cq_inputs.activations(99, 0, 4, cols)
    C = oracle.gemm(blob, 4, rows, cols, X, levels)
    for m in range(4):
        assert np.allclose(C[m], oracle.matvec(blob, 4, rows, cols, X[m:m + 1], levels)[0], rtol=0, atol=1e-15)
    ids = np.array([0, 4, 8])
    assert np.allclose(oracle.gemm(blob, 4, rows, cols, X, levels, row_ids=ids), C[:, ids], rtol=0, atol=1e-15)


def test_bf16_round_matches_torch():
    import torch
    rng = np.random.default_rng(5)
    x = (rng.standard_normal(10000) * 10.0 ** rng.integers(-5, 5, 10000)).astype(np.float32)
    # exact ties: bf16 value + half an ulp
    base = oracle.bf16_round(x[:100])
    ties = (base.view(np.uint32) + np.uint32(0x8000)).view(np.float32)
    x = np.concatenate([x, ties, -ties, [0.0, -0.0, 1.0, 65504.0]]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(oracle.bf16_round(x).view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_bf16_variant_within_analytic_bound(bits):
    rows, cols, M = 16, 512, 8
    blob, levels, _ = _blob(100, bits, rows, cols)
    X = cq_inputs.activations(100, bits, M, cols, "f16")
    C = oracle.gemm(blob, bits, rows, cols, X, levels)
    Cb = oracle.gemm_bf16(blob, bits, rows, cols, X, levels)
    wn = np.linalg.norm(oracle.dequantize(blob, bits, rows, cols, levels), axis=1)
    xn = np.linalg.norm(X.astype(np.float64), axis=1)
    assert np.all(np.abs(Cb - C) <= 7.8e-3 * np.outer(xn, wn))
    cos = np.sum(Cb * C) / np.linalg.norm(Cb) / np.linalg.norm(C)
    assert cos > 0.9999


def test_ternary_crumbs_sign_extend():
    a = float(oracle.ternary_level32())
    assert oracle.level_values(np.array([0, 1, 2, 3]), 5).tolist() == [0.0, a, -2 * a, -a]


@pytest.mark.parametrize("bits", [2, 3, 4, 5])
def test_gather_rows_by_definition(bits):
    # each gathered element by explicit loops over the Sylvester matrix:
    # w_hat[r, 128 g + k] = sum_j c[q[r, 128 g + j]] * n[r, g] * S[j, k] / sqrt(128)
    rows, cols = 5, 200
    blob, levels, _ = _blob(96, bits, rows, cols)
    ids = [4, 0, 4, -1, 5, 2]
    got = oracle.gather_rows(blob, bits, rows, cols, ids, levels)
    packed, norms = oracle.split_blob(blob, bits, rows, cols)
    codes = oracle.unpack_codes(packed, bits, 256)
    S = oracle.sylvester(128)
    for i, r in enumerate(ids):
        if not 0 <= r < rows:
            assert np.all(np.isnan(got[i]))  # ids outside the matrix give NaN rows
            continue
        vals = oracle.level_values(codes[r], bits, levels)
        for k in range(0, cols, 37):
            g, kk = divmod(k, 128)
            want = sum(vals[128 * g + j] * float(np.float32(norms[r, g])) * S[j, kk] for j in range(128))
            assert abs(got[i, k] - want / np.sqrt(128)) <= 1e-12
    assert np.array_equal(got[0], got[2])  # a repeated id repeats the row


def test_gather_rows_times_x_is_the_matvec():
    rows, cols = 9, 300
    blob, levels, _ = _blob(97, 2, rows, cols)
    x = cq_inputs.activations(97, 0, 2, cols)
    ids = np.array([8, 3, 3, 0])
    g = oracle.gather_rows(blob, 2, rows, cols, ids, levels)
    y = oracle.matvec(blob, 2, rows, cols, x, levels)
    assert np.allclose(x.astype(np.float64) @ g.T, y[:, ids], rtol=1e-12, atol=1e-12)


# --- pins of gemm_bf16's rounding points --------------------------------------
#
# gemm_bf16 rounds the rotated activation X' = fp32(H.x) and the weight operand
# V = fp32(level) * fp32(norm) (the product in fp32) to bf16, nearest even, and
# sums the products in float64.  The hand-made case below puts X' and V on and
# off bf16 ties, so that every plausible slip -- rounding only X', only V,
# neither, V before the norm multiply, or ties away from zero instead of to
# even -- gives a different, hand-computed result.

def _bf16_by_hand(v):
    """bf16 round to nearest, ties to even, by way of the significand: v =
    m * 2^e with m in [0.5, 1); keep 8 significant bits with Python's round
    (which rounds halves to even).  Normal finite values only."""
    import math
    if v == 0.0:
        return 0.0
    m, e = math.frexp(v)
    return math.ldexp(round(m * 256.0), e - 8)


def _tie_case():
    # levels of a 2-bit code book (inputs of the method): 0 for the unused
    # columns, and two values whose products with the norms sit on or off
    # bf16 ties (bf16 spacing in [1, 2) is 2^-7)
    levels = np.array([-1.0, 0.0, 1.00390625, 1.01171875], dtype=np.float32)
    rows, cols = 2, 128
    codes = np.ones((rows, cols), dtype=np.uint8)  # level 0
    codes[:, 0], codes[:, 1] = 2, 3
    norms = np.array([[1.5], [1.0]], dtype=np.float16)
    blob = oracle.make_blob(oracle.pack_codes(codes, 2), norms)
    # x = H v, so that the rotated activation is v (exact in fp32 after the
    # float64 rotation: x is constant on the Hadamard columns' signs)
    v = np.zeros(cols)
    v[0], v[1] = 1.005859375, 1.00390625  # 128.75 ulps (rounds up); an exact tie (to even: down)
    x = (oracle.hadamard() @ v)[None, :]
    return blob, levels, rows, cols, x


def test_gemm_bf16_tie_case_by_hand():
    blob, levels, rows, cols, x = _tie_case()
    C = oracle.gemm_bf16(blob, 2, rows, cols, x, levels)
    # X' = bf16(1.005859375) = 1.0078125, bf16(1.00390625) = 1.0 (tie to even)
    # row 0 (norm 1.5): V = bf16(1.505859375) = 1.5078125, bf16(1.517578125) = 1.515625
    # row 1 (norm 1.0): V = bf16(1.00390625) = 1.0 (tie, even), bf16(1.01171875) = 1.015625 (tie, even)
    want = [1.0078125 * 1.5078125 + 1.0 * 1.515625, 1.0078125 * 1.0 + 1.0 * 1.015625]
    assert C.shape == (1, 2) and C[0].tolist() == want


def test_gemm_bf16_rounding_slips_all_differ():
    blob, levels, rows, cols, x = _tie_case()
    got = oracle.gemm_bf16(blob, 2, rows, cols, x, levels)[0]
    c = [1.00390625, 1.01171875]
    v = [1.005859375, 1.00390625]
    n = [1.5, 1.0]

    def product(rx, rv, v_before_norm=False, rnd=_bf16_by_hand):
        out = []
        for r in range(2):
            acc = 0.0
            for k in range(2):
                xk = rnd(v[k]) if rx else v[k]
                if v_before_norm:
                    vk = rnd(c[k]) * n[r]
                else:
                    vk = rnd(float(np.float32(c[k]) * np.float32(n[r]))) if rv else c[k] * n[r]
                acc += xk * vk
            out.append(acc)
        return out

    variants = {
        "both": product(True, True),
        "x only": product(True, False),
        "v only": product(False, True),
        "neither": product(False, False),
        "v before norm": product(True, True, v_before_norm=True),
        "ties away": product(True, True, rnd=math_half_up),
    }
    vals = [tuple(v_) for v_ in variants.values()]
    assert len(set(vals)) == len(vals), variants
    assert got.tolist() == variants["both"]


def math_half_up(v):
    """bf16 rounding with ties away from zero (positive values): the slip
    the tie case must catch."""
    import math
    m, e = math.frexp(v)
    return math.ldexp(math.floor(m * 256.0 + 0.5), e - 8)


@pytest.mark.parametrize("bits", [2, 3, 4, 5])
def test_gemm_bf16_equals_an_explicit_loop(bits):
    rows, cols, M = 3, 256, 2
    blob, levels, _ = _blob(101, bits, rows, cols)
    X = cq_inputs.activations(101, bits, M, cols, "f16")
    got = oracle.gemm_bf16(blob, bits, rows, cols, X, levels)
    packed, norms = oracle.split_blob(blob, bits, rows, cols)
    vals = oracle.level_values(oracle.unpack_codes(packed, bits, cols), bits, levels)
    S = oracle.sylvester(128)
    for m in range(M):
        xr = [sum(float(X[m, 128 * (k // 128) + j]) * S[k % 128, j] for j in range(128)) / np.sqrt(128)
              for k in range(cols)]
        for r in range(rows):
            acc = 0.0
            for k in range(cols):
                w = float(np.float32(vals[r, k]) * np.float32(norms[r, k // 128]))
                acc += _bf16_by_hand(float(np.float32(xr[k]))) * _bf16_by_hand(w)
            assert abs(acc - got[m, r]) <= 1e-12 * max(1.0, abs(acc)), (m, r)


@pytest.mark.parametrize("bits", [1, 2, 3, 4, 5])
def test_matvec_rotated_equals_the_dense_product(bits):
    # the rotated-activation route (used for full-size parity) against the
    # dense reconstruction, on every row range
    rows, cols = 40, 700
    blob, levels, _ = _blob(102, bits, rows, cols)
    x = cq_inputs.activations(102, bits, 3, cols)
    dense = oracle.matvec(blob, bits, rows, cols, x, levels)
    for r0, r1 in [(0, rows), (0, 1), (13, 29), (39, 40)]:
        got = oracle.matvec_rotated(blob, bits, rows, cols, x, levels, row0=r0, row1=r1)
        assert np.allclose(got, dense[:, r0:r1], rtol=0, atol=1e-13 * np.max(np.abs(dense)))


@pytest.mark.parametrize("bits", [2, 4, 5])
def test_matvec_rotated_row_norms_are_the_dense_row_norms(bits):
    rows, cols = 20, 500
    blob, levels, _ = _blob(103, bits, rows, cols)
    x = cq_inputs.activations(103, bits, 1, cols)
    _, rn = oracle.matvec_rotated(blob, bits, rows, cols, x, levels, row0=4, row1=17, row_norms=True)
    dense = np.linalg.norm(oracle.dequantize(blob, bits, rows, cols, levels), axis=1)
    assert np.allclose(rn, dense[4:17], rtol=1e-13, atol=0)
