"""CQ-W2A8 oracle: the integer decode product the pages deploy.

TEST INFRASTRUCTURE ONLY (see the package docstring).

[cact-format post, "How the kernel reads it"]: the kernel rotates each
128-group of the activation, quantises the rotated group to int8 with one
scale per group, looks up int8 centroids by the packed indices, accumulates
with an int8 dot product, and multiplies once per group by the weight norm
times the activation scale times the codebook scale.  The exporter calls this
CQ-W2A8 (2-bit weights, 8-bit activations, groups of 128).
[OpenNeedle reference, Cactus 2-bit kernel]: the activation is Hadamard
rotated, then quantised per group by absmax to int8; the codebook is mapped
to int8 by maxabs/127; the int8 dot is scaled by the activation scale, the
codebook scale and the fp16 norm.  [OpenNeedle reference, activation fake-quant note]:
the activation scale is absmax/127, values are rounded and clamped to
[-128, 127].

Readings (also listed in the design notes):
* R14 -- the int8 decisions depend on the fp32 value of the rotated group.
  The pages fix an fp32 butterfly in registers but not its order; both sides
  use the radix-2 butterfly in stride order 1, 2, ..., 64 with every sum and
  difference rounded to fp32, then one fp32 multiply by fp32(1/sqrt(128))
  (``rotate_acts_fp32``).
* R15 -- activation scale sx = fp32(absmax / 127) (IEEE division); code
  q = clamp(round_half_even(fp32(x / sx)), -128, 127); a group whose absmax
  is 0 has sx = 0 and q = 0.  Activations are finite.
* R16 -- codebook scale sc = fp32(max|c| / 127); c8 = round_half_even(
  fp32(c / sc)), within [-127, 127].
* R17 -- ternary crumbs sign-extend straight to integers in the kernel
  [cact-format post, "Cactus Quants"]: c8 is the crumb's value {0, 1, -2, -1}
  and sc is the fp32 ternary level a / sqrt(128).
* R18 -- the per-group multiply and the sum over groups are real-number
  operations the pages do not round; here they are float64 (the GPU uses
  fp32, compared within its rounding bound).
"""

import math

import numpy as np

from .cq import GROUP, TERNARY_MARKER, codebook_for, padded_cols, split_blob, ternary_level32, unpack_codes

__all__ = ["INV_SQRT_GROUP_F32", "rotate_acts_fp32", "quantize_acts_int8", "codebook_int8",
           "w2a8_group_terms", "w2a8_from_quantized", "matvec_w2a8"]

INV_SQRT_GROUP_F32 = np.float32(1.0 / math.sqrt(GROUP))
"""fp32(1/sqrt(128)), the one scaling multiply of the butterfly (R14)."""


def _pad32(x, group):
    x = np.asarray(x, dtype=np.float32)
    if x.ndim == 1:
        x = x[None, :]
    kpad = padded_cols(x.shape[1], group)
    out = np.zeros((x.shape[0], kpad), dtype=np.float32)
    out[:, : x.shape[1]] = x
    return out


def rotate_acts_fp32(x, group=GROUP):
    """fp32 rotated activations as the butterfly computes them (R14), x
    zero-padded to whole groups; float32 [batch, cols_pad].

    Stage h (h = 1, 2, 4, ..., group/2) replaces each pair (v[i], v[i+h]),
    i & h == 0, by (v[i] + v[i+h], v[i] - v[i+h]), in fp32 [cact-format post,
    "How the kernel reads it": a fast Walsh-Hadamard butterfly per group]; the
    result is then multiplied by fp32(1/sqrt(group)).
    """
    xp = _pad32(x, group)
    b, kpad = xp.shape
    v = xp.reshape(b, kpad // group, group)
    h = 1
    while h < group:
        pairs = v.reshape(b, kpad // group, group // (2 * h), 2, h)
        lo, hi = pairs[:, :, :, 0, :], pairs[:, :, :, 1, :]
        v = np.stack([lo + hi, lo - hi], axis=3).reshape(b, kpad // group, group)
        h *= 2
    inv = np.float32(1.0 / math.sqrt(group))
    return (v * inv).astype(np.float32).reshape(b, kpad)


def quantize_acts_int8(xr, group=GROUP):
    """Per-group int8 activations (R15): returns (q int64 [batch, cols_pad],
    sx float32 [batch, groups])."""
    xr = np.asarray(xr, dtype=np.float32)
    b, kpad = xr.shape
    v = xr.reshape(b, kpad // group, group)
    amax = np.max(np.abs(v), axis=-1)
    sx = (amax / np.float32(127.0)).astype(np.float32)
    safe = np.where(sx > 0, sx, np.float32(1.0)).astype(np.float32)
    t = (v / safe[..., None]).astype(np.float32)
    q = np.clip(np.rint(t), -128, 127).astype(np.int64)
    q = np.where(sx[..., None] > 0, q, 0)
    return q.reshape(b, kpad), sx


def codebook_int8(bits, levels=None, group=GROUP):
    """int8 value of every stored code and the codebook scale (R16, R17):
    returns (c8 int64 [2^b'], sc float32)."""
    if bits == TERNARY_MARKER:
        return np.array([0, 1, -2, -1], dtype=np.int64), np.float32(ternary_level32(group))
    lv = codebook_for(bits, levels, group).astype(np.float32)
    sc = np.float32(np.max(np.abs(lv)) / np.float32(127.0))
    c8 = np.rint((lv / sc).astype(np.float32)).astype(np.int64)
    return c8, sc


def w2a8_group_terms(blob, bits, rows, cols, xq, sx, levels=None, group=GROUP, row_ids=None):
    """The per-group terms (float(n[r, g]) * sx[b, g] * sc) * sum_k c8[q[r, g, k]] * xq[b, g, k],
    float64 [batch, rows, groups]: the integer dot exact (int64), the scaling
    in float64 [cact-format post, "How the kernel reads it"]."""
    packed, norms = split_blob(blob, bits, rows, cols, group)
    if row_ids is not None:
        packed, norms = packed[row_ids], norms[row_ids]
    kpad = padded_cols(cols, group)
    ng = kpad // group
    n = packed.shape[0]
    c8, sc = codebook_int8(bits, levels, group)
    w8 = c8[unpack_codes(packed, bits, kpad).astype(np.int64)].reshape(n, ng, group)
    xq = np.asarray(xq, dtype=np.int64).reshape(-1, ng, group)
    nb = xq.shape[0]
    dots = np.zeros((nb, n, ng), dtype=np.int64)
    for g in range(ng):
        dots[:, :, g] = xq[:, g, :] @ w8[:, g, :].T
    scale = (norms.astype(np.float32).astype(np.float64)[None, :, :]
             * np.asarray(sx, dtype=np.float64).reshape(nb, 1, ng) * float(sc))
    return scale * dots.astype(np.float64)


def w2a8_from_quantized(blob, bits, rows, cols, xq, sx, levels=None, group=GROUP, row_ids=None):
    """y[b, r] = the sum over groups of ``w2a8_group_terms``, float64."""
    return np.sum(w2a8_group_terms(blob, bits, rows, cols, xq, sx, levels, group, row_ids), axis=-1)


def matvec_w2a8(blob, bits, rows, cols, x, levels=None, group=GROUP, row_ids=None):
    """The CQ-W2A8 decode product of activation x [batch, cols] (not
    rotated): R14 rotation, R15 quantisation, then ``w2a8_from_quantized``.
    float64 [batch, rows] (or [batch, len(row_ids)])."""
    xq, sx = quantize_acts_int8(rotate_acts_fp32(x, group), group)
    return w2a8_from_quantized(blob, bits, rows, cols, xq, sx, levels, group, row_ids)
