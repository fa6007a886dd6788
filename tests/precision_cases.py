"""Inputs that stress the fp32 accuracy of a CQ product.

The bar of an fp32-accumulate product is max |y - y_oracle| <= 1e-4 *
||w_hat_row|| * ||x|| for every (batch, row).  Random N(0, 1) activations
against N(0, 0.02^2) masters hide rounding errors that are the same for
every weight with the same code: they average out over a row.  These cases
do not let them:

* ``aligned``  -- activation rows equal to dequantised weight rows, so that
  every term of one row's sum has the same sign and y = ||w_hat_row||^2 is
  the bar's own scale (the tied-embedding logits of a hidden state close to
  a token's row);
* ``short``    -- rows of 128 or 256 columns (one or two groups: nothing to
  average over), many rows;
* ``sigma``    -- masters with sigma 1e-4, 1e-5, 1e-6: group norms down to
  fp16's subnormal range;
* ``mixed``    -- rows whose group norms span six decades.

Each case returns (blob, bits, rows, cols, levels, x).  Masters come from
``cq_inputs`` and are encoded by the oracle; where encoding would take too
long on the CPU, the packed codes are uniformly random bytes (any bytes are a
valid CQ matrix).  Test infrastructure only: it calls the oracle for inputs,
never the GPU library.
"""
import numpy as np

import cq_inputs
import oracle


def levels_for(bits):
    return None if bits in (1, 5) else cq_inputs.codebook(bits)


def encoded(cfg, bits, rows, cols, sigma=cq_inputs.WEIGHT_SIGMA):
    levels = levels_for(bits)
    w = cq_inputs.master(cfg, bits, rows, cols, sigma=sigma)
    return oracle.quantize(w, bits, levels), levels


def random_codes(cfg, bits, rows, cols, norm_scale=None):
    """A CQ matrix with uniformly random codes and N(0.226, 0.014^2) norms,
    times ``norm_scale[g]`` per group column when given."""
    kpad = oracle.padded_cols(cols)
    ng = kpad // oracle.GROUP
    row_bytes = kpad * oracle.storage_bits(bits) // 8
    packed = cq_inputs.random_bytes(cfg, bits, rows * row_bytes).reshape(rows, row_bytes)
    if bits == 5:
        # crumb 10 is never written by the encoder: map it to 00
        p = packed.copy()
        for sh in range(0, 8, 2):
            bad = ((p >> sh) & 3) == 2
            p[bad] &= np.uint8(~(3 << sh) & 0xFF)
        packed = p
    norms = cq_inputs.random_norms(cfg, bits, rows * ng).view(np.float16).reshape(rows, ng).astype(np.float32)
    if norm_scale is not None:
        norms = norms * np.asarray(norm_scale, dtype=np.float32)[None, :]
    return oracle.make_blob(packed, norms.astype(np.float16)), levels_for(bits)


def aligned_x(blob, bits, rows, cols, levels, batch, salt=0):
    """Activation rows equal to dequantised rows (fp32), one distinct row per
    batch element."""
    ids = (np.arange(batch) * 7919 + 13 + salt) % rows
    w = oracle.dequantize(blob, bits, rows, cols, levels, row_ids=ids)[:, :cols]
    return w.astype(np.float32)


def case(name, bits, batch):
    """The named case at width ``bits`` and ``batch`` activation rows."""
    kind, shape = name.split(":")
    rows, cols = (int(v) for v in shape.split("x"))
    cfg = 50 + bits
    if kind in ("aligned", "random"):
        if rows * cols > (1 << 22):
            blob, levels = random_codes(cfg, bits, rows, cols)
        else:
            blob, levels = encoded(cfg, bits, rows, cols)
    elif kind.startswith("sigma"):
        blob, levels = encoded(cfg, bits, rows, cols, sigma=float(kind[5:]))
    elif kind == "mixed":
        ng = oracle.padded_cols(cols) // oracle.GROUP
        blob, levels = random_codes(cfg, bits, rows, cols, norm_scale=10.0 ** -(np.arange(ng) % 6))
    else:
        raise ValueError(name)
    if kind == "random":
        x = cq_inputs.activations(cfg, rows, batch, cols)
    elif kind == "aligned" or batch == 1:
        x = aligned_x(blob, bits, rows, cols, levels, batch)
    else:
        # small norms and mixed norms: aligned rows, then random rows
        h = (batch + 1) // 2
        x = np.concatenate([aligned_x(blob, bits, rows, cols, levels, h),
                            cq_inputs.activations(cfg, rows, batch - h, cols)])
    return blob, levels, x


# Cases and the kernel each one reaches (batch 1 / batch 2..8):
#   512x512, 512x128, 8192x512, 262144x128, 32768x256  small-matrix kernel
#   1024x5120                                            batched matrix-core kernel
#   1024x8192                                            lookup tables (batch 1) / batched kernel
CASES = [
    "aligned:512x512", "aligned:512x128", "aligned:8192x512",
    "random:262144x128", "aligned:262144x128", "random:32768x256", "aligned:32768x256",
    "sigma1e-4:512x512", "sigma1e-5:512x512", "sigma1e-6:512x512",
    "mixed:512x1024", "aligned:1024x5120", "mixed:1024x5120", "aligned:1024x8192",
]


def bar_terms(blob, bits, rows, cols, levels, x):
    """(oracle y [batch, rows], ||w_hat_row||, ||x_b||), all float64."""
    ref = oracle.matvec(blob, bits, rows, cols, x, levels)
    wn = np.linalg.norm(oracle.dequantize(blob, bits, rows, cols, levels), axis=1)
    xn = np.linalg.norm(np.asarray(x, dtype=np.float64), axis=1)
    return ref, wn, xn


def err_over_bar(y, ref, wn, xn, tol=1e-4):
    bound = tol * np.outer(xn, wn)
    return float(np.max(np.abs(np.asarray(y, np.float64) - ref) / np.maximum(bound, 1e-300)))
