"""The C-ABI used from plain C99 (tests/c_client.c): the header compiles as
C, the client links against libcq.so and the HIP runtime, and on the GPU its
encoder and product agree with the oracle."""
import os
import subprocess

import numpy as np
import pytest

import cq_inputs
import oracle
from conftest import ROOT

LIB_DIR = os.path.join(ROOT, "hadamard_rotated_codebook_amd")
ROCM = "/opt/rocm"


def _build(tmp_path):
    if not os.path.exists(os.path.join(LIB_DIR, "libcq.so")):
        pytest.skip("libcq.so not built")
    exe = str(tmp_path / "c_client")
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"),
           os.path.join(ROOT, "tests", "c_client.c"), "-o", exe,
           "-L", LIB_DIR, "-lcq", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           "-Wl,-rpath," + LIB_DIR, "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    return exe


def test_c_client_compiles_and_links(tmp_path):
    exe = _build(tmp_path)
    assert os.access(exe, os.X_OK)


@pytest.mark.gpu
def test_c_client_matches_the_oracle(tmp_path):
    exe = _build(tmp_path)
    rows, cols, batch = 300, 1000, 3
    levels = cq_inputs.codebook(2)
    w = cq_inputs.master(130, 2, rows, cols)
    x = cq_inputs.activations(130, 2, batch, cols)
    with open(tmp_path / "in.bin", "wb") as f:
        f.write(np.array([rows, cols, batch], np.int64).tobytes())
        f.write(np.asarray(levels, np.float32).tobytes())
        f.write(w.astype(np.float32).tobytes())
        f.write(x.astype(np.float32).tobytes())
    r = subprocess.run([exe, str(tmp_path)], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr, flush=True)
    assert r.returncode == 0
    blob = np.fromfile(tmp_path / "blob.bin", np.uint8)
    y = np.fromfile(tmp_path / "y.bin", np.float32).reshape(batch, rows).astype(np.float64)
    # the encoder: the oracle's indices (this draw has no coordinate near a
    # decision boundary) and the same fp16 norms
    ref_blob = oracle.quantize(w, 2, levels)
    assert blob.size == ref_blob.size
    codes = oracle.unpack_codes(oracle.split_blob(blob, 2, rows, cols)[0], 2, 1024)
    ref_codes = oracle.unpack_codes(oracle.split_blob(ref_blob, 2, rows, cols)[0], 2, 1024)
    assert np.mean(codes == ref_codes) >= 0.9999
    # the product of the encoded matrix, within the fp32-path bar
    ref = oracle.matvec(blob, 2, rows, cols, x, levels)
    wn = np.linalg.norm(oracle.dequantize(blob, 2, rows, cols, levels), axis=1)
    bound = 1e-4 * np.outer(np.linalg.norm(x.astype(np.float64), axis=1), wn)
    assert np.all(np.abs(y - ref) <= bound)
