"""The operand arithmetic of the fp16 matrix-core matvec kernels, emulated on
the CPU and held against the oracle on the inputs of ``precision_cases``
(activations lined up with weight rows, rows of one or two groups, group
norms in fp16's subnormal range, norms spanning six decades).

The kernels' arithmetic, as include/cq.h documents it: the rotated
activation of each batch row is scaled by the power of two 2^e that puts its
largest |value| in [2^14, 2^15) and held as two fp16 values, hi = fp16(a)
and lo = fp16(a - hi); each stored code's level is scaled by 2^sl (largest
|level| in [2^14, 2^15)) and held the same way (binary and ternary levels are
integer multiples of one level and exact); the products of the fp16 parts
are exact, each group is summed on its own, and the sum is multiplied by
fp32(float(norm) * 2^-sl) and by 2^-e.  The emulation forms the same operand
values with NumPy's fp16 rounding (nearest even) and adds the exact products
in float64; the kernels' fp32 sums of one group (128 terms, a few hundred
ulps at most) are not modelled.

Two checks per case: the present scheme stays far inside the fp32 bar, and
the scheme it replaced -- one fp16 operand fp16(level * norm) and one fp16
activation -- exceeds the bar on the aligned and small-norm cases, so these
inputs do reach the errors they are there to reach.
"""
import numpy as np
import pytest

import oracle
import precision_cases as pc


def f16(a):
    return np.asarray(a, dtype=np.float32).astype(np.float16).astype(np.float64)


def pow2_exponent(m):
    """e with m * 2^e in [2^14, 2^15), clamped to [-100, 100]; 0 for m = 0."""
    if not (m > 0) or not np.isfinite(m):
        return 0
    _, e = np.frexp(m)  # m < 2^e
    return int(np.clip(15 - e, -100, 100))


def code_levels32(bits, levels):
    """fp32 level of each stored code."""
    sb = oracle.storage_bits(bits)
    return oracle.level_values(np.arange(1 << sb), bits, levels).astype(np.float32)


def _rotated32(x):
    return oracle.rotate_acts(x).astype(np.float32)


def emulate_split(blob, bits, rows, cols, x, levels):
    packed, norms = oracle.split_blob(blob, bits, rows, cols)
    kpad = oracle.padded_cols(cols)
    codes = oracle.unpack_codes(packed, bits, kpad)
    lv = code_levels32(bits, levels)
    if bits in (1, 5):
        unit = np.float32(lv[1])                      # +c, or the ternary a
        mult = {1: [-1.0, 1.0], 5: [0.0, 1.0, -2.0, -1.0]}[bits]
        b_val = np.array(mult)                        # exact in fp16
        lscale = unit
    else:
        sl = pow2_exponent(float(np.max(np.abs(lv))))
        s = (lv.astype(np.float64) * 2.0 ** sl).astype(np.float32)
        hi = f16(s)
        lo = f16(s.astype(np.float64) - hi)
        b_val = hi + lo
        lscale = np.float32(2.0 ** -sl)
    B = b_val[codes].reshape(rows, kpad // 128, 128)
    nf = (norms.astype(np.float32) * lscale).astype(np.float32).astype(np.float64)  # [rows, groups]
    xr = _rotated32(x)
    y = np.zeros((xr.shape[0], rows))
    for b in range(xr.shape[0]):
        e = pow2_exponent(float(np.max(np.abs(xr[b]))))
        a = (xr[b].astype(np.float64) * 2.0 ** e).astype(np.float32)
        a_hi = f16(a)
        a_lo = f16(a.astype(np.float64) - a_hi)
        A = (a_hi + a_lo).reshape(kpad // 128, 128)
        S = np.einsum("rgk,gk->rg", B, A)
        y[b] = (S * nf).sum(axis=1) * 2.0 ** -e
    return y


def emulate_single_fp16(blob, bits, rows, cols, x, levels):
    packed, norms = oracle.split_blob(blob, bits, rows, cols)
    kpad = oracle.padded_cols(cols)
    codes = oracle.unpack_codes(packed, bits, kpad)
    lv = code_levels32(bits, levels)
    n32 = np.repeat(norms.astype(np.float32), 128, axis=1)
    V = f16(lv[codes] * n32)                          # fp16(level * norm), the product in fp32
    xr = _rotated32(x)
    y = np.zeros((xr.shape[0], rows))
    for b in range(xr.shape[0]):
        e = pow2_exponent(float(np.max(np.abs(xr[b]))))
        A = f16(xr[b].astype(np.float64) * 2.0 ** e)
        y[b] = (V @ A) * 2.0 ** -e
    return y


CPU_CASES = ["aligned:512x512", "aligned:512x128", "aligned:8192x512", "aligned:32768x256",
             "sigma1e-4:512x512", "sigma1e-5:512x512", "sigma1e-6:512x512", "mixed:512x1024"]


@pytest.mark.parametrize("bits", [1, 2, 3, 4, 5])
@pytest.mark.parametrize("name", CPU_CASES)
def test_split_operands_meet_the_fp32_bar(name, bits):
    rows, cols = (int(v) for v in name.split(":")[1].split("x"))
    blob, levels, x = pc.case(name, bits, 2)
    ref, wn, xn = pc.bar_terms(blob, bits, rows, cols, levels, x)
    y = emulate_split(blob, bits, rows, cols, x, levels)
    assert pc.err_over_bar(y, ref, wn, xn) <= 0.02


@pytest.mark.parametrize("name,bits", [("aligned:512x512", 2), ("aligned:512x128", 1), ("aligned:512x128", 3),
                                       ("aligned:32768x256", 2), ("sigma1e-5:512x512", 2),
                                       ("sigma1e-6:512x512", 4), ("mixed:512x1024", 5)])
def test_single_fp16_operands_fail_the_bar(name, bits):
    rows, cols = (int(v) for v in name.split(":")[1].split("x"))
    blob, levels, x = pc.case(name, bits, 1)
    ref, wn, xn = pc.bar_terms(blob, bits, rows, cols, levels, x)
    assert pc.err_over_bar(emulate_single_fp16(blob, bits, rows, cols, x, levels), ref, wn, xn) > 1.0
