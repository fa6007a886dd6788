"""CQ oracle: Hadamard matrix, codebooks, encoder, bit packing, dequantisation
and the float64 matrix products.

Page names used in the citations are defined in the package docstring.  All
floating point is float64 except where a page fixes another precision (the
encoder's fp32 norm and the fp16 stored norm).  Nothing here is blocked, fused
or reordered beyond what the cited passage states.
"""

import math

import numpy as np

__all__ = [
    "GROUP", "TERNARY_MARKER", "TERNARY_LEVEL", "BINARY_MARKER",
    "sylvester", "hadamard", "storage_bits", "bits_per_weight",
    "padded_cols", "blob_bytes",
    "gaussian_lloyd_max", "ternary_level", "lloyd_max_empirical",
    "ternary_level32", "binary_level", "binary_level32", "codebook_for",
    "rotate_fp32", "nearest_level", "encode", "quantize",
    "pack_codes", "unpack_codes", "make_blob", "split_blob",
    "level_values", "dequantize", "gather_rows", "rotate_acts",
    "matvec", "matvec_rotated", "gemm", "bf16_round", "gemm_bf16",
]

GROUP = 128
"""Quantisation group along the reduction axis [cact-format post, "Cactus Quants"]."""

TERNARY_MARKER = 5
"""Record ``bits`` value that marks ternary weights; they are stored as 2-bit
crumbs, not 5-bit codes [needle.js tutorial, "Shared codebooks"; OpenNeedle
reference, file layout]."""

TERNARY_LEVEL = 1.2240064
"""Analytic ternary level before division by sqrt(group), as printed in
[needle.js tutorial, "Shared codebooks"]."""

BINARY_MARKER = 1
"""Record ``bits`` value of binary weights, one bit per weight, eight per
byte [cact-format post, "Cactus Quants"].  Reading: the pages name binary
weights and their packing but no marker; 1, the number of bits stored, is
the plainest."""


# --------------------------------------------------------------------------
# Hadamard matrix

def sylvester(n):
    """Integer Sylvester-Hadamard matrix of order ``n`` (a power of two).

    Sylvester doubling: S_1 = [1], S_2m = [[S_m, S_m], [S_m, -S_m]]
    [OpenNeedle reference, Hadamard-MLP formulas: H is the orthogonal
    Sylvester/Walsh-Hadamard matrix].  Reading: the CQ rotation uses this
    natural (Sylvester) row order; the pages name the matrix but not its row
    order for CQ.
    """
    if n < 1 or n & (n - 1):
        raise ValueError("Hadamard order must be a power of two")
    s = np.ones((1, 1), dtype=np.int64)
    while s.shape[0] < n:
        s = np.block([[s, s], [s, -s]])
    return s


def hadamard(n=GROUP):
    """Normalised Walsh-Hadamard matrix H = S / sqrt(n), float64
    [cact-format post, "Cactus Quants"; OpenNeedle reference, CQ quantisation
    steps: H = Hadamard(128)/sqrt(128)]."""
    return sylvester(n).astype(np.float64) / math.sqrt(n)


# --------------------------------------------------------------------------
# Sizes

def storage_bits(bits):
    """Bits stored per index: ``bits`` for codebook widths 2/3/4 and for binary
    (1), and 2 for the ternary marker 5, whose values are 2-bit crumbs
    [cact-format post, "Cactus Quants"; OpenNeedle reference, file layout]."""
    if bits not in (BINARY_MARKER, 2, 3, 4, TERNARY_MARKER):
        raise ValueError(f"unsupported CQ bits {bits}")
    return 2 if bits == TERNARY_MARKER else bits


def bits_per_weight(bits, group=GROUP):
    """Index bits plus 16 norm bits per group: 2.125 at CQ2, 4.125 at CQ4
    [cact-format post, "Cactus Quants"; OpenNeedle reference, byte accounting]."""
    return storage_bits(bits) + 16.0 / group


def padded_cols(cols, group=GROUP):
    """Input length padded up to a multiple of the group
    [needle.js tutorial, "Anatomy of a CQ matrix"]."""
    return -(-cols // group) * group


def blob_bytes(bits, group, rows, cols):
    """Byte length of one CQ matrix blob: ``rows`` packed index rows of
    cols_pad*b/8 bytes, then rows*cols_pad/group fp16 norms
    [needle.js tutorial, "Anatomy of a CQ matrix"].  ``b`` is the storage width
    (2 for ternary crumbs).  Raises ``ValueError`` for invalid parameters."""
    b = storage_bits(bits)
    if group < 8 or group & (group - 1):
        raise ValueError("group must be a power of two >= 8")
    if rows < 0 or cols < 0:
        raise ValueError("negative shape")
    kpad = padded_cols(cols, group)
    return rows * (kpad * b // 8) + rows * (kpad // group) * 2


# --------------------------------------------------------------------------
# Codebooks

def _phi(t):
    return 0.0 if math.isinf(t) else math.exp(-0.5 * t * t) / math.sqrt(2.0 * math.pi)


def _Phi(t):
    return 0.5 * math.erfc(-t / math.sqrt(2.0))


def gaussian_lloyd_max(levels, iters=200000, tol=1e-15):
    """Lloyd-Max quantiser of N(0, 1) with ``levels`` levels, float64, ascending.

    The pages describe the CQ levels as Lloyd-Max centroids of a Gaussian
    [cact-format post, "Cactus Quants"; needle.js tutorial, "Shared codebooks"].
    Lloyd's alternation: thresholds at midpoints of adjacent centres, centres at
    the conditional means phi-differences / Phi-differences of their cells.
    """
    c = np.linspace(-2.0, 2.0, levels)
    for _ in range(iters):
        edges = [-math.inf] + [(c[j] + c[j + 1]) / 2 for j in range(levels - 1)] + [math.inf]
        new = np.array([(_phi(edges[j]) - _phi(edges[j + 1])) / (_Phi(edges[j + 1]) - _Phi(edges[j]))
                        for j in range(levels)])
        done = np.max(np.abs(new - c)) < tol
        c = new
        if done:
            break
    return c


def ternary_level():
    """Positive level ``a`` of the 3-level Lloyd-Max quantiser of N(0, 1).

    Levels {-a, 0, +a}, thresholds +-a/2, so a is the mean of N(0,1) above a/2:
    a = phi(a/2) / (1 - Phi(a/2)).  The pages print the result as 1.2240064
    [needle.js tutorial, "Shared codebooks"]; solved here by fixed-point
    iteration in float64.
    """
    a = 1.0
    for _ in range(1000):
        nxt = _phi(a / 2) / (1.0 - _Phi(a / 2))
        if abs(nxt - a) < 1e-16:
            return nxt
        a = nxt
    return a


def lloyd_max_empirical(levels, group=GROUP, n_samples=400_000, iters=200, seed=0):
    """Empirical Lloyd-Max codebook as the exporter builds it, fp32, ascending.

    [OpenNeedle reference, codebook generation]: Lloyd-Max on the samples
    RandomState(0).randn(400000) for 200 iterations, initial centres taken from
    quantiles, final centres divided by sqrt(group_size) and cast to FP32.
    Reading: the initial quantiles are at (i + 0.5)/levels, cells are split at
    midpoints of adjacent centres and each centre moves to its cell's mean.
    With these readings the 4-level result equals the printed CQ2 header values
    bit for bit.
    """
    s = np.random.RandomState(seed).randn(n_samples)
    c = np.quantile(s, (np.arange(levels) + 0.5) / levels)
    for _ in range(iters):
        cell = np.searchsorted((c[:-1] + c[1:]) / 2, s)
        c = np.bincount(cell, weights=s, minlength=levels) / np.bincount(cell, minlength=levels)
    return (c / math.sqrt(group)).astype(np.float32)


def ternary_level32(group=GROUP):
    """fp32 ternary level a / sqrt(group), with a = 1.2240064 as printed
    [needle.js tutorial, "Shared codebooks"].  Reading: divide in float64,
    then round once to fp32."""
    return np.float32(TERNARY_LEVEL / math.sqrt(group))


def binary_level():
    """Positive level of the 2-level Lloyd-Max quantiser of N(0, 1), float64.

    The pages say binary weights have a closed-form centroid and store no
    codebook for them [cact-format post, "Five regions", "Cactus Quants"].
    Reading: with the threshold at 0 (the midpoint of -c and +c) each level is
    the mean of its half of N(0, 1), E[Z | Z > 0] = sqrt(2/pi).
    """
    return math.sqrt(2.0 / math.pi)


def binary_level32(group=GROUP):
    """fp32 binary level sqrt(2/pi) / sqrt(group): the unit-sphere coordinates
    of a 128-group are N(0, 1/group) (the same division as the ternary and
    Lloyd-Max levels).  Reading: divide in float64, then round once to fp32."""
    return np.float32(binary_level() / math.sqrt(group))


def codebook_for(bits, levels=None, group=GROUP):
    """The fp32 ascending levels an index selects.

    Widths 2/3/4 take the caller's 4/8/16 levels (the file's embedded codebook
    is authoritative [OpenNeedle reference, codebook generation]).  The ternary
    marker uses the analytic {-a, 0, +a}/sqrt(group) and takes no levels
    [needle.js tutorial, "Shared codebooks"]; binary uses {-c, +c} of
    ``binary_level32`` and takes none either.
    """
    if bits == TERNARY_MARKER:
        if levels is not None:
            raise ValueError("ternary levels are analytic; pass levels=None")
        a = ternary_level32(group)
        return np.array([-a, 0.0, a], dtype=np.float32)
    if bits == BINARY_MARKER:
        # Reading: code 0 selects -c and code 1 selects +c (ascending, as the
        # codes of the other widths index ascending levels).
        if levels is not None:
            raise ValueError("binary levels are analytic; pass levels=None")
        c = binary_level32(group)
        return np.array([-c, c], dtype=np.float32)
    storage_bits(bits)
    lv = np.asarray(levels, dtype=np.float32)
    if lv.shape != (1 << bits,):
        raise ValueError(f"CQ{bits} needs {1 << bits} levels")
    if not np.all(np.diff(lv.astype(np.float64)) > 0):
        raise ValueError("levels must be strictly ascending")
    return lv


# --------------------------------------------------------------------------
# Encoder

def rotate_fp32(groups):
    """fp32 rotated coordinates r = w.H of each group (last axis).

    [OpenNeedle reference, CQ quantisation steps]: r = w H with the normalised
    Hadamard matrix, computed by the exporter in FP32.  Reading: r is the fp32
    rounding of (w.S) * sqrt(1/group), where w.S (a signed sum of fp32 values)
    is formed in float64 and the scaling is one float64 multiply.  This is the
    correctly rounded fp32 of w.H except within ~2^-29 of an fp32 rounding
    boundary, and it fixes one value for the decisions taken below.
    """
    g = groups.shape[-1]
    t = groups.astype(np.float64) @ sylvester(g).astype(np.float64)
    return (t * math.sqrt(1.0 / g)).astype(np.float32)


def nearest_level(u, levels):
    """Index of the level nearest to each coordinate; on equal distance the
    smaller index wins [OpenNeedle reference, CQ quantisation steps].

    Reading: the distances |u - c_j| between the fp32 values are compared
    exactly (float64 holds each difference of two fp32 values in this range
    exactly).  ``np.argmin`` returns the first minimum, which is the tie rule.
    """
    d = np.abs(u.astype(np.float64)[..., None] - np.asarray(levels, np.float32).astype(np.float64))
    return np.argmin(d, axis=-1)


# Ternary index (over ascending levels -a, 0, +a) -> stored 2-bit crumb.
# Reading of the garbled crumb description [cact-format post, "Cactus Quants":
# signed 2-bit crumbs that sign-extend]: the crumb is the two's-complement
# 2-bit value of the sign, so -1 -> 0b11, 0 -> 0b00, +1 -> 0b01.
_CRUMB_OF_INDEX = np.array([3, 0, 1], dtype=np.uint8)


def encode(w, bits, levels=None, group=GROUP, chunk_rows=256):
    """Quantise a float32 [rows, cols] matrix: stored codes and fp16 norms.

    [OpenNeedle reference, CQ quantisation steps], per row and per group of
    ``group`` weights along the input axis, the input zero-padded to a
    multiple of the group [needle.js tutorial, "Anatomy of a CQ matrix"]:

        r = w H                       (fp32, see ``rotate_fp32``)
        n = sqrt(sum(r^2))            FP32
        u = r / max(n, 1e-12)         with the unrounded (fp32) norm
        q_i = argmin_j |u_i - c_j|    ties to the smaller index
        n_store = float16(n)

    Reading: n is the fp32 rounding of the float64 norm of the fp32 r; u is
    the IEEE fp32 quotient; float16 rounds to nearest even (overflow -> inf).
    Returns ``codes`` uint8 [rows, cols_pad] (level indices, or ternary
    crumbs) and ``norms`` float16 [rows, cols_pad/group].
    """
    w = np.asarray(w, dtype=np.float32)
    rows, cols = w.shape
    kpad = padded_cols(cols, group)
    ng = kpad // group
    lv = codebook_for(bits, levels, group)
    codes = np.zeros((rows, kpad), dtype=np.uint8)
    norms = np.zeros((rows, ng), dtype=np.float16)
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        wp = np.zeros((r1 - r0, kpad), dtype=np.float32)
        wp[:, :cols] = w[r0:r1]
        r32 = rotate_fp32(wp.reshape(r1 - r0, ng, group))
        n32 = np.sqrt(np.sum(r32.astype(np.float64) ** 2, axis=-1)).astype(np.float32)
        u32 = r32 / np.maximum(n32, np.float32(1e-12))[..., None]
        idx = nearest_level(u32, lv)
        if bits == TERNARY_MARKER:
            idx = _CRUMB_OF_INDEX[idx]
        codes[r0:r1] = idx.reshape(r1 - r0, kpad)
        with np.errstate(over="ignore"):
            norms[r0:r1] = n32.astype(np.float16)
    return codes, norms


def quantize(w, bits, levels=None, group=GROUP):
    """Encode ``w`` into one CQ blob (uint8 array): packed rows then norms."""
    codes, norms = encode(w, bits, levels, group)
    return make_blob(pack_codes(codes, bits), norms)


# --------------------------------------------------------------------------
# Bit packing and the blob

def pack_codes(codes, bits):
    """Pack stored codes row by row.

    [OpenNeedle reference, file layout]: every 8 codes form the word
    sum(code[i] << (i*b)), emitted as b little-endian bytes; each row is one
    continuous LSB-first bitstream [cact-format post, "Cactus Quants"].
    """
    b = storage_bits(bits)
    codes = np.asarray(codes)
    rows, k = codes.shape
    if k % 8:
        raise ValueError("row length must be a multiple of 8 codes")
    if codes.size and int(codes.max()) >= (1 << b):
        raise ValueError("code out of range for the storage width")
    c = codes.astype(np.uint64).reshape(rows, k // 8, 8)
    word = np.zeros((rows, k // 8), dtype=np.uint64)
    for i in range(8):
        word |= c[:, :, i] << np.uint64(i * b)
    out = np.empty((rows, k // 8, b), dtype=np.uint8)
    for j in range(b):
        out[:, :, j] = (word >> np.uint64(8 * j)) & np.uint64(0xFF)
    return out.reshape(rows, k // 8 * b)


def unpack_codes(packed, bits, k):
    """Read the ``k`` stored codes of each packed row with the per-index
    formulas of [needle.js tutorial, "2-bit", "4-bit", "3-bit"]:

    * 2-bit: byte = row[col >> 2]; code = (byte >> ((col & 3)*2)) & 3
    * 4-bit: byte = row[col >> 1]; code = (byte >> ((col & 1)*4)) & 15
    * 3-bit: bit = 3*col; window = row[bit>>3] | row[(bit>>3)+1] << 8;
      code = (window >> (bit & 7)) & 7
    * 1-bit (reading: the same LSB-first stream at eight per byte
      [cact-format post, "Cactus Quants"]): byte = row[col >> 3];
      code = (byte >> (col & 7)) & 1

    Reading: the 3-bit window's second byte is taken as 0 past the end of the
    row; the last code never needs it, so no byte outside the row is read.
    """
    b = storage_bits(bits)
    p = np.asarray(packed, dtype=np.uint8).astype(np.int64)
    col = np.arange(k)
    if b == 1:
        return ((p[:, col >> 3] >> (col & 7)) & 1).astype(np.uint8)
    if b == 2:
        return ((p[:, col >> 2] >> ((col & 3) * 2)) & 3).astype(np.uint8)
    if b == 4:
        return ((p[:, col >> 1] >> ((col & 1) * 4)) & 15).astype(np.uint8)
    bit = col * 3
    byte = bit >> 3
    inside = byte + 1 < p.shape[1]
    hi = np.where(inside, p[:, np.minimum(byte + 1, p.shape[1] - 1)], 0)
    window = p[:, byte] | (hi << 8)
    return ((window >> (bit & 7)) & 7).astype(np.uint8)


def make_blob(packed, norms):
    """Blob = all packed index rows, then all fp16 norms, one per (output row,
    input group), row-major [needle.js tutorial, "Anatomy of a CQ matrix";
    OpenNeedle reference, file layout].  Reading: norms follow the last packed
    row directly, ordered [row][group], little-endian."""
    p = np.ascontiguousarray(packed, dtype=np.uint8).ravel()
    n = np.ascontiguousarray(norms, dtype="<f2").view(np.uint8).ravel()
    return np.concatenate([p, n])


def split_blob(blob, bits, rows, cols, group=GROUP):
    """Views (packed [rows, row_bytes] uint8, norms [rows, groups] float16).

    A blob whose length differs from packed + 2*normCount is rejected with
    "Inconsistent CQ matrix length" [needle.js tutorial, "Anatomy of a CQ
    matrix"]."""
    blob = np.asarray(blob, dtype=np.uint8).ravel()
    if blob.size != blob_bytes(bits, group, rows, cols):
        raise ValueError("Inconsistent CQ matrix length")
    kpad = padded_cols(cols, group)
    row_bytes = kpad * storage_bits(bits) // 8
    packed = blob[: rows * row_bytes].reshape(rows, row_bytes)
    norms = blob[rows * row_bytes:].view("<f2").reshape(rows, kpad // group)
    return packed, norms


# --------------------------------------------------------------------------
# Dequantisation and products

def level_values(codes, bits, levels=None, group=GROUP):
    """float64 level selected by each stored code.

    Widths 2/3/4: levels[code].  Ternary: the crumb sign-extends as a 2-bit
    two's-complement number and scales the analytic level
    [cact-format post, "Cactus Quants"].  Reading: crumb 0b10 sign-extends to
    -2 and so decodes to -2a; the encoder never writes it.
    """
    codes = np.asarray(codes).astype(np.int64)
    if bits == TERNARY_MARKER:
        s = np.where(codes >= 2, codes - 4, codes)
        return s.astype(np.float64) * float(ternary_level32(group))
    lv = codebook_for(bits, levels, group).astype(np.float64)
    return lv[codes]


def dequantize(blob, bits, rows, cols, levels=None, group=GROUP, row_ids=None):
    """Dense reconstruction, float64 [len(row_ids) or rows, cols_pad].

    rotated = codebook[index] * float32(norm); dense group = rotated . H
    [needle.js tutorial, "Reconstructing one group"; OpenNeedle reference,
    CQ quantisation steps: w_hat = (codebook[q] * float32(n_store)) H].
    """
    packed, norms = split_blob(blob, bits, rows, cols, group)
    if row_ids is not None:
        packed, norms = packed[row_ids], norms[row_ids]
    kpad = padded_cols(cols, group)
    ng = kpad // group
    n = packed.shape[0]
    vals = level_values(unpack_codes(packed, bits, kpad), bits, levels, group)
    rotated = vals.reshape(n, ng, group) * norms.astype(np.float32).astype(np.float64)[..., None]
    return (rotated @ hadamard(group)).reshape(n, kpad)


def gather_rows(blob, bits, rows, cols, ids, levels=None, group=GROUP):
    """Dense rows ``ids`` of the reconstruction, float64 [len(ids), cols].

    A row gather (embedding and engram tables) reconstructs the dense groups
    of the indexed rows only: rotated = codebook[index] * norm, dense group =
    rotated . H [needle.js tutorial, "Reconstructing one group" and "Keep the
    quantized views"; OpenNeedle reference, engine notes].  Reading: an id
    outside [0, rows) gives a row of NaN (the call refuses to invent a row).
    """
    ids = np.asarray(ids, dtype=np.int64).reshape(-1)
    out = np.full((ids.size, cols), np.nan)
    ok = (ids >= 0) & (ids < rows)
    if np.any(ok):
        out[ok] = dequantize(blob, bits, rows, cols, levels, group, row_ids=ids[ok])[:, :cols]
    return out


def _pad(x, group):
    x = np.asarray(x, dtype=np.float64)
    if x.ndim == 1:
        x = x[None, :]
    kpad = padded_cols(x.shape[1], group)
    out = np.zeros((x.shape[0], kpad), dtype=np.float64)
    out[:, : x.shape[1]] = x
    return out


def rotate_acts(x, group=GROUP):
    """Rotated activations x'_g = H.x_g of every group, x zero-padded, float64
    [cact-format post, "How the kernel reads it": each 128-lane group of the
    activation is rotated with the same Hadamard transform]."""
    xp = _pad(x, group)
    b, kpad = xp.shape
    return (xp.reshape(b, kpad // group, group) @ hadamard(group)).reshape(b, kpad)


def matvec(blob, bits, rows, cols, x, levels=None, group=GROUP, row_ids=None):
    """y[b, r] = sum_k w_hat[r, k] x[b, k], float64, through the dense
    dequantised matrix.  ``x`` is [batch, cols] (or [cols]); the result is
    [batch, rows] (or [batch, len(row_ids)])."""
    w_hat = dequantize(blob, bits, rows, cols, levels, group, row_ids)
    return _pad(x, group) @ w_hat.T


def matvec_rotated(blob, bits, rows, cols, x, levels=None, group=GROUP, row0=0, row1=None, row_norms=False):
    """y[b, r] for rows r in [row0, row1), float64, by the rotated-activation
    identity [OpenNeedle reference, rotated-activation identity]: for every
    group, dot(w_hat_g, x_g) = n_store * dot(codebook[q], H x_g), so

        y[b, r] = sum_g float32(n[r, g]) * sum_j c[q[r, g, j]] * (H x_g)[j]

    with H x_g computed once for all rows.  The same value as ``matvec`` up to
    float64 rounding order, without the dense reconstruction (the rows at
    full size are far too many for it).  With ``row_norms`` also returns
    ||w_hat_r||_2, which equals the norm of the rotated row (H is
    orthogonal: Parseval)."""
    packed, norms = split_blob(blob, bits, rows, cols, group)
    row1 = rows if row1 is None else row1
    kpad = padded_cols(cols, group)
    xr = rotate_acts(x, group)                      # [batch, kpad]
    vals = level_values(unpack_codes(packed[row0:row1], bits, kpad), bits, levels, group)
    wrot = vals * np.repeat(norms[row0:row1].astype(np.float32).astype(np.float64), group, axis=1)
    y = xr @ wrot.T
    if row_norms:
        return y, np.sqrt(np.sum(wrot * wrot, axis=1))
    return y


def gemm(blob, bits, rows, cols, X, levels=None, group=GROUP, row_ids=None):
    """C[m, r] = sum_k X[m, k] w_hat[r, k], float64 (C = X . W_hat^T)."""
    return matvec(blob, bits, rows, cols, X, levels, group, row_ids)


def bf16_round(x):
    """Round float32 values to bfloat16 (8-bit significand, round to nearest,
    ties to even); returned as float32 holding the bf16 value.  Finite inputs
    only."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = ((u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)) << np.uint64(16)
    return u.astype(np.uint32).view(np.float32)


def gemm_bf16(blob, bits, rows, cols, X, levels=None, group=GROUP, row_ids=None):
    """The product with the bf16 operand roundings of the matrix-core path.

    Rotated domain: C[m, r] = sum_g sum_k X'[m, g, k] V[r, g, k] with
    X' = bf16(fp32(H.x_g)) and V = bf16(fp32(c[q]) * fp32(n_store)); the
    products are summed in float64.  By the rotated-activation identity
    [OpenNeedle reference, rotated-activation identity] this equals ``gemm``
    up to the two bf16 roundings.
    """
    packed, norms = split_blob(blob, bits, rows, cols, group)
    if row_ids is not None:
        packed, norms = packed[row_ids], norms[row_ids]
    kpad = padded_cols(cols, group)
    n = packed.shape[0]
    lv = level_values(unpack_codes(packed, bits, kpad), bits, levels, group).astype(np.float32)
    n32 = np.repeat(norms.astype(np.float32), group, axis=1)
    V = bf16_round(lv * n32).astype(np.float64)
    Xr = bf16_round(rotate_acts(X, group).astype(np.float32)).astype(np.float64)
    return Xr @ V.reshape(n, kpad).T
