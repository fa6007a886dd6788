"""Seeded synthetic inputs shared by the oracle-side tests and the GPU path.

This module holds no arithmetic of the CQ method: it only draws random
numbers with fixed seeds, casts them to the dtypes the workloads name, and
loads stored codebook values.  Nothing here imports the oracle or the HIP
library.

Recipe (every draw is reproducible from its key alone):

* Keys are ``SeedSequence([config_id, tensor_id, role, chunk])`` for NumPy's
  default generator (PCG64).  ``role`` 0 is a weight master, 1 an activation.
* Weight masters are N(0, sigma^2) float32 with sigma = 0.02, drawn in
  independent chunks of ``CHUNK_ROWS`` rows, so any row range can be
  regenerated without drawing the rows before it.
* Activations are N(0, 1) float32; fp16 and bf16 activations are those draws
  rounded to nearest even.
* Codebooks: the printed 2-bit header values, and for 3/4-bit the values in
  ``tests/golden/codebooks.json`` (written by a script that runs the oracle's
  empirical Lloyd-Max procedure).
* Full-size product tests use uniformly random packed bytes and fp16 norms
  drawn around the norm of a N(0, 0.02^2) group: any bytes are a valid CQ
  matrix, and the oracle decodes the same bytes.
"""

import json
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

CHUNK_ROWS = 1024
WEIGHT_SIGMA = 0.02

_HERE = os.path.dirname(os.path.abspath(__file__))
_CODEBOOK_FILE = os.path.join(os.path.dirname(_HERE), "tests", "golden", "codebooks.json")

# The 2-bit codebook as printed by the OpenNeedle reference notes (header values).
CQ2_PRINTED = (-0.1331721395254135, -0.03990209102630615,
               0.04003528133034706, 0.13346044719219208)


def _gen(*key):
    return np.random.default_rng(np.random.SeedSequence([int(k) for k in key]))


def codebook(bits, kind="empirical"):
    """fp32 ascending levels for CQ ``bits`` (2, 3, 4); ``None`` for the
    ternary marker 5 and binary 1, whose levels are analytic.  ``kind`` is
    "empirical" (exporter procedure) or "gaussian" (analytic Lloyd-Max /
    sqrt(128))."""
    if bits in (1, 5):
        return None
    if bits == 2 and kind == "empirical":
        return np.array(CQ2_PRINTED, dtype=np.float32)
    with open(_CODEBOOK_FILE) as f:
        data = json.load(f)
    return np.array(data[kind][str(bits)], dtype=np.float32)


def master(config_id, tensor_id, rows, cols, r0=0, r1=None, sigma=WEIGHT_SIGMA, threads=8):
    """Rows [r0, r1) of the float32 weight master of shape [rows, cols]."""
    r1 = rows if r1 is None else r1
    if not (0 <= r0 <= r1 <= rows):
        raise ValueError("row range outside the matrix")
    out = np.empty((r1 - r0, cols), dtype=np.float32)
    chunks = range(r0 // CHUNK_ROWS, -(-r1 // CHUNK_ROWS)) if r1 > r0 else range(0)

    def fill(c):
        c0 = c * CHUNK_ROWS
        n = min(CHUNK_ROWS, rows - c0)
        block = _gen(config_id, tensor_id, 0, c).standard_normal((n, cols), dtype=np.float32)
        block *= np.float32(sigma)
        a, b = max(r0, c0), min(r1, c0 + n)
        out[a - r0:b - r0] = block[a - c0:b - c0]

    if threads > 1 and len(chunks) > 1:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(fill, chunks))
    else:
        for c in chunks:
            fill(c)
    return out


def activations(config_id, tensor_id, batch, cols, dtype="f32"):
    """N(0,1) activations [batch, cols] as float32 holding values of ``dtype``
    ("f32", "f16" or "bf16", rounded to nearest even from the fp32 draw)."""
    x = _gen(config_id, tensor_id, 1, 0).standard_normal((batch, cols), dtype=np.float32)
    return cast(x, dtype)


def cast(x, dtype):
    """Round float32 values to ``dtype`` and return them as float32."""
    x = np.asarray(x, dtype=np.float32)
    if dtype == "f32":
        return x
    if dtype == "f16":
        return x.astype(np.float16).astype(np.float32)
    if dtype == "bf16":
        import torch
        return torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    raise ValueError(dtype)


def random_bytes(config_id, tensor_id, nbytes):
    """``nbytes`` uniformly random bytes (uint8); stands in for packed CQ
    indices at sizes where encoding a master on the CPU would take minutes."""
    return _gen(config_id, tensor_id, 3, 0).integers(0, 256, size=nbytes, dtype=np.uint8)


def random_norms(config_id, tensor_id, n, mean=0.226, sd=0.014):
    """``n`` positive fp16 values drawn as N(mean, sd^2), returned as uint8
    bytes (little-endian fp16).  The defaults are the norm statistics of a
    128-group of N(0, 0.02^2) weights: 0.02 times a chi variable with 128
    degrees of freedom."""
    v = _gen(config_id, tensor_id, 4, 0).normal(mean, sd, size=n)
    v = np.maximum(v, mean / 8).astype(np.float16)
    return v.view(np.uint8)


def sample_rows(config_id, tensor_id, rows, n):
    """``n`` distinct sorted row indices in [0, rows), always including the
    first and last row."""
    if n >= rows:
        return np.arange(rows)
    pick = _gen(config_id, tensor_id, 2, 0).choice(rows, size=n, replace=False)
    return np.unique(np.concatenate([pick, [0, rows - 1]]))
