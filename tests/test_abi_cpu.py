"""The C-ABI library on the CPU: it loads, exports every entry point that
include/cq.h declares, and its host-side validation rejects bad arguments
before launching anything.  No call here reaches a kernel launch: every call
either fails validation or has nothing to do."""
import ctypes
import os
import re

import numpy as np
import pytest

import cq_inputs
import oracle
from conftest import ROOT

cq = pytest.importorskip("hadamard_rotated_codebook_amd", reason="libcq.so not built")
lib = cq._lib

OK, NULL, BITS, GROUP, SHAPE, LENGTH, CODEBOOK, DTYPE, WORKSPACE, ALIGN, HIP, OVERLAP, SCRATCH = range(13)
FAKE = 1 << 40  # a 256-byte aligned address that is never dereferenced on the host


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "cq.h")).read()
    return sorted(set(re.findall(r"^(?:cq_status|int32_t|const char \*)\s*(cq_\w+)\(", text, re.M)))


def test_every_declared_symbol_is_exported():
    names = _declared_functions()
    assert set(names) == {"cq_version", "cq_status_string", "cq_blob_bytes", "cq_workspace_bytes",
                          "cq_rotate_acts", "cq_matvec", "cq_rotate_matvec", "cq_rotate_matvec_noalloc",
                          "cq_rotate_multi_matvec",
                          "cq_rotate_multi_workspace_bytes", "cq_quantize_acts_int8", "cq_matvec_w2a8_quantized",
                          "cq_matvec_w2a8", "cq_gather_rows", "cq_gemm", "cq_quantize", "cq_quantize_rows",
                          "cq_kv_scores_workspace_bytes", "cq_kv_scores", "cq_matvec_t", "cq_kv_append", "cq_kv_attention",
                          "cq_read_probe"}
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_status_strings():
    assert cq.cq_version() == 10000
    for s in range(13):
        assert lib.cq_status_string(s).decode() != "unknown status"
    assert lib.cq_status_string(LENGTH).decode() == "Inconsistent CQ matrix length"
    assert lib.cq_status_string(99).decode() == "unknown status"


@pytest.mark.parametrize("bits", [1, 2, 3, 4, 5])
def test_blob_bytes_matches_oracle(bits):
    for rows, cols in [(0, 0), (1, 1), (3, 130), (512, 512), (65536, 16384), (7, 1000), (1 << 30, 128)]:
        assert cq.cq_blob_bytes(bits, rows, cols) == oracle.blob_bytes(bits, 128, rows, cols)


def _blob_status(bits, group, rows, cols):
    out = ctypes.c_uint64(12345)
    st = lib.cq_blob_bytes(bits, group, rows, cols, ctypes.byref(out))
    return st, out.value


def test_blob_bytes_errors_leave_output_untouched():
    assert _blob_status(0, 128, 1, 1) == (BITS, 12345)
    assert _blob_status(6, 128, 1, 1) == (BITS, 12345)
    assert _blob_status(2, 64, 1, 1) == (GROUP, 12345)
    assert _blob_status(2, 128, -1, 1) == (SHAPE, 12345)
    assert _blob_status(2, 128, 1, (1 << 30) + 1) == (SHAPE, 12345)
    assert lib.cq_blob_bytes(2, 128, 1, 1, None) == NULL


_DEFAULT = object()


def _matrix(bits=2, rows=4, cols=256, blob=FAKE, nbytes=None, levels=_DEFAULT):
    if levels is _DEFAULT:
        levels = None if bits == 5 else cq_inputs.codebook(bits)
    arr = None if levels is None else np.ascontiguousarray(levels, np.float32)
    ptr = None if arr is None else arr.ctypes.data_as(ctypes.POINTER(ctypes.c_float))
    nb = oracle.blob_bytes(bits, 128, rows, cols) if nbytes is None else nbytes
    m = cq._Matrix(bits, 128, rows, cols, ctypes.c_void_p(blob), nb, ptr)
    return m, arr


def _matvec(m, xr=FAKE + (1 << 30), batch=1, y=FAKE + (1 << 31)):
    return lib.cq_matvec(ctypes.byref(m), ctypes.c_void_p(xr), batch, ctypes.c_void_p(y), None, 0, None)


def _gemm(m, xr=FAKE + (1 << 30), mm=8, c=FAKE + (1 << 31)):
    return lib.cq_gemm(ctypes.byref(m), ctypes.c_void_p(xr), mm, ctypes.c_void_p(c), None, 0, None)


def test_matvec_and_gemm_validation():
    m, k = _matrix(bits=7, nbytes=0, levels=None)
    assert _matvec(m) == BITS and _gemm(m) == BITS
    m, k = _matrix(nbytes=oracle.blob_bytes(2, 128, 4, 256) - 1)
    assert _matvec(m) == LENGTH and _gemm(m) == LENGTH
    m, k = _matrix(blob=0)
    assert _matvec(m) == NULL
    m, k = _matrix(blob=FAKE + 8)
    assert _matvec(m) == ALIGN
    m, k = _matrix(levels=np.array([0.1, 0.0, 0.2, 0.3]))
    assert _matvec(m) == CODEBOOK and _gemm(m) == CODEBOOK
    m, k = _matrix(levels=np.array([0.0, 0.1, np.nan, 0.3]))
    assert _matvec(m) == CODEBOOK
    m, k = _matrix(levels=None)
    assert _matvec(m) == CODEBOOK
    m, k = _matrix(bits=5, levels=np.array([-1.0, 0.0, 1.0]))
    assert _matvec(m) == CODEBOOK
    m, k = _matrix()
    assert _matvec(m, batch=9) == SHAPE and _matvec(m, batch=-1) == SHAPE
    assert _gemm(m, mm=-1) == SHAPE
    assert _matvec(m, y=0) == NULL and _gemm(m, c=0) == NULL
    assert _matvec(m, xr=0) == NULL and _gemm(m, xr=0) == NULL
    assert _matvec(m, xr=FAKE + 4) == ALIGN and _gemm(m, xr=FAKE + 8) == ALIGN
    assert _matvec(m, y=FAKE + (1 << 31) + 2) == ALIGN
    # outputs overlapping an input
    assert _matvec(m, y=FAKE + 64) == OVERLAP
    assert _matvec(m, y=FAKE + (1 << 30) + 16) == OVERLAP
    assert _gemm(m, c=FAKE + (1 << 30)) == OVERLAP
    assert lib.cq_matvec(None, None, 1, None, None, 0, None) == NULL


def _rotate_matvec(m, x=FAKE + (1 << 30), batch=1, y=FAKE + (1 << 31), ws=None, wsb=0):
    return lib.cq_rotate_matvec(ctypes.byref(m), ctypes.c_void_p(x), batch, ctypes.c_void_p(y),
                                None if ws is None else ctypes.c_void_p(ws), wsb, None)


def test_rotate_matvec_validation():
    # the fused call checks like cq_matvec; x is [batch][cols] fp32 (4-byte aligned)
    m, k = _matrix(bits=7, nbytes=0, levels=None)
    assert _rotate_matvec(m) == BITS
    m, k = _matrix(levels=np.array([0.1, 0.0, 0.2, 0.3]))
    assert _rotate_matvec(m) == CODEBOOK
    m, k = _matrix()
    need = ctypes.c_uint64(7)
    # a small matrix with K in one slice: one launch that rotates x itself,
    # no workspace
    for batch in (1, 8):
        assert lib.cq_workspace_bytes(2, ctypes.byref(m), batch, ctypes.byref(need)) == OK and need.value == 0
    assert _rotate_matvec(m, batch=9) == SHAPE and _rotate_matvec(m, batch=-1) == SHAPE
    assert _rotate_matvec(m, batch=0) == OK
    assert _rotate_matvec(m, x=0) == NULL and _rotate_matvec(m, y=0) == NULL
    assert _rotate_matvec(m, x=FAKE + (1 << 30) + 2) == ALIGN
    assert _rotate_matvec(m, y=FAKE + (1 << 31) + 2) == ALIGN
    assert _rotate_matvec(m, y=FAKE + (1 << 30) + 16) == OVERLAP  # y on top of x
    assert _rotate_matvec(m, y=FAKE + 64) == OVERLAP  # y on top of the blob
    # small but K beyond one slice: the rotated activation goes to the workspace
    wide, _ = _matrix(rows=4, cols=5000)
    assert lib.cq_workspace_bytes(2, ctypes.byref(wide), 1, ctypes.byref(need)) == OK and need.value == 5120 * 4 + 2 * 4 * 4
    assert _rotate_matvec(wide) == WORKSPACE
    big, _ = _matrix(rows=1000, cols=16384)
    need = ctypes.c_uint64()
    assert lib.cq_workspace_bytes(0, ctypes.byref(big), 1, ctypes.byref(need)) == OK and need.value > 0
    assert _rotate_matvec(big) == WORKSPACE
    assert _rotate_matvec(big, ws=FAKE + (1 << 32), wsb=need.value - 1) == WORKSPACE
    assert _rotate_matvec(big, ws=FAKE + (1 << 32) + 4, wsb=need.value) == ALIGN
    assert _rotate_matvec(big, ws=FAKE + (1 << 30), wsb=need.value) == OVERLAP  # workspace on x
    assert lib.cq_rotate_matvec(None, None, 1, None, None, 0, None) == NULL


def _mats(*ms):
    arr = (cq._Matrix * max(len(ms), 1))()
    for i, m in enumerate(ms):
        arr[i] = m
    return arr


def _multi(ms, x=FAKE + (1 << 30), batch=1, ys=None, ws=None, wsb=0, n=None):
    ys = [FAKE + (1 << 31) + (i << 24) for i in range(len(ms))] if ys is None else ys
    yarr = (ctypes.c_void_p * max(len(ys), 1))(*ys)
    return lib.cq_rotate_multi_matvec(_mats(*ms), len(ms) if n is None else n, ctypes.c_void_p(x), batch, yarr,
                                      None if ws is None else ctypes.c_void_p(ws), wsb, None)


def _multi_ws(ms, batch=1, n=None):
    out = ctypes.c_uint64(7)
    st = lib.cq_rotate_multi_workspace_bytes(_mats(*ms), len(ms) if n is None else n, batch, ctypes.byref(out))
    return st, out.value


def test_rotate_multi_matvec_validation():
    # Q/K/V/gate-like: small matrices sharing cols, one launch, no workspace
    q, kq = _matrix(rows=512, cols=512)
    kk, kk_ = _matrix(bits=3, rows=256, cols=512)
    t5, _ = _matrix(bits=5, rows=7, cols=512)
    assert _multi_ws([q, kk, t5], batch=8) == (OK, 0)
    assert _multi([q, kk, t5], batch=0) == OK and _multi([], n=0) == OK
    assert _multi([q, kk], n=-1) == SHAPE and _multi([q], n=65) == SHAPE
    assert _multi([q, kk], batch=9) == SHAPE and _multi([q, kk], batch=-1) == SHAPE
    odd, _ = _matrix(rows=4, cols=384)
    assert _multi([q, odd]) == SHAPE and _multi_ws([q, odd])[0] == SHAPE  # unequal cols
    bad, _ = _matrix(levels=np.array([0.1, 0.0, 0.2, 0.3]), cols=512)
    assert _multi([q, bad]) == CODEBOOK and _multi_ws([q, bad])[0] == CODEBOOK
    short, _ = _matrix(rows=4, cols=512, nbytes=10)
    assert _multi([short, q]) == LENGTH
    assert lib.cq_rotate_multi_matvec(None, 2, ctypes.c_void_p(FAKE), 1, None, None, 0, None) == NULL
    assert lib.cq_rotate_multi_matvec(_mats(q), 1, ctypes.c_void_p(FAKE + (1 << 30)), 1, None, None, 0, None) == NULL
    assert lib.cq_rotate_multi_workspace_bytes(_mats(q), 1, 1, None) == NULL
    ys = [FAKE + (1 << 31), FAKE + (1 << 32)]
    assert _multi([q, kk], ys=[ys[0], 0]) == NULL
    assert _multi([q, kk], ys=[ys[0], ys[1] + 2]) == ALIGN
    assert _multi([q, kk], x=0) == NULL and _multi([q, kk], x=FAKE + (1 << 30) + 1) == ALIGN
    # outputs on top of x, a blob or one another
    assert _multi([q, kk], ys=[ys[0], FAKE + (1 << 30) + 64]) == OVERLAP
    assert _multi([q, kk], ys=[ys[0], FAKE + 128]) == OVERLAP
    assert _multi([q, kk], ys=[ys[0], ys[0] + 512 * 4 - 4]) == OVERLAP
    # a matrix with no rows needs no output pointer; cols == 0 zeroes outputs
    empty, _ = _matrix(rows=0, cols=512, blob=0)
    assert _multi_ws([empty, q]) == (OK, 0)
    # matrices past the small-matrix kernel (K beyond 4096, or over 2^26
    # weights) share one rotation in the workspace: the largest partial-sum
    # region (16-byte aligned), then batch x cols_pad floats
    big, _ = _matrix(rows=1000, cols=16384)
    wide, _ = _matrix(rows=4, cols=16384)
    part = 16 * 1000 * 4  # 2-bit tables: 1024 columns a slice
    assert _multi_ws([wide, big]) == (OK, part + 16384 * 4)
    q4, _ = _matrix(rows=512, cols=4096)
    big4, _ = _matrix(rows=16385, cols=4096)  # just over 2^26 weights: the tables at batch 1
    st, nb = _multi_ws([q4, big4])
    assert st == OK and nb == 4 * 16385 * 4 + 4096 * 4
    assert _multi_ws([q4, big4], batch=2) == (OK, 2 * 4096 * 4)  # the batched kernel: one slice
    assert _multi([q4, big4]) == WORKSPACE
    assert _multi([q4, big4], ws=FAKE + (1 << 33), wsb=nb - 1) == WORKSPACE
    assert _multi([q4, big4], ws=FAKE + (1 << 33) + 4, wsb=nb) == ALIGN
    assert _multi([q4, big4], ws=FAKE + (1 << 30), wsb=nb) == OVERLAP  # workspace on x
    assert _multi([q4, big4], ws=FAKE + (1 << 31), wsb=nb) == OVERLAP  # workspace on y[0]


WS = FAKE + (1 << 33)


def _w2a8(m, x=FAKE + (1 << 30), batch=1, y=FAKE + (1 << 31), ws=WS, wsb=1 << 20):
    return lib.cq_matvec_w2a8(ctypes.byref(m), ctypes.c_void_p(x), batch, ctypes.c_void_p(y), ctypes.c_void_p(ws),
                              wsb, None)


def _w2a8q(m, xq=FAKE + (1 << 30), sx=FAKE + (1 << 32), batch=1, y=FAKE + (1 << 31)):
    return lib.cq_matvec_w2a8_quantized(ctypes.byref(m), ctypes.c_void_p(xq), ctypes.c_void_p(sx), batch,
                                        ctypes.c_void_p(y), None)


def _qacts(x=FAKE + (1 << 30), batch=2, cols=300, xq=FAKE + (1 << 31), sx=FAKE + (1 << 32)):
    return lib.cq_quantize_acts_int8(ctypes.c_void_p(x), batch, cols, ctypes.c_void_p(xq), ctypes.c_void_p(sx), None)


def _w8ws(m, batch):
    out = ctypes.c_uint64(7)
    st = lib.cq_workspace_bytes(3, ctypes.byref(m), batch, ctypes.byref(out))
    return st, out.value


@pytest.mark.parametrize("call", [_w2a8, _w2a8q])
def test_matvec_w2a8_validation(call):
    m, k = _matrix(bits=7, nbytes=0, levels=None)
    assert call(m) == BITS
    m, k = _matrix(levels=np.array([0.1, 0.0, 0.2, 0.3]))
    assert call(m) == CODEBOOK
    m, k = _matrix(nbytes=10)
    assert call(m) == LENGTH
    m, k = _matrix()
    assert call(m, batch=9) == SHAPE and call(m, batch=-1) == SHAPE
    assert call(m, batch=0) == OK
    assert call(m, y=0) == NULL
    assert call(m, y=FAKE + (1 << 31) + 1) == ALIGN
    assert call(m, y=FAKE + (1 << 30) + 8) == OVERLAP and call(m, y=FAKE + 64) == OVERLAP
    # the whole quantised activation fits one workgroup: 16384 columns up
    # to batch 3, not 4; 14336 at batch 4, not 14464; 27264 at batch 1, not
    # 27392; 6528 at batch 8, not 6656
    wide, _ = _matrix(rows=4, cols=16384)
    assert call(wide, batch=4) == SHAPE
    assert call(wide, batch=3, y=0) == NULL  # past the shape check
    assert call(_matrix(rows=4, cols=14336)[0], batch=4, y=0) == NULL
    assert call(_matrix(rows=4, cols=14464)[0], batch=4) == SHAPE
    assert call(_matrix(rows=4, cols=27264)[0], batch=1, y=0) == NULL
    assert call(_matrix(rows=4, cols=27392)[0], batch=1) == SHAPE
    b8, _ = _matrix(rows=4, cols=6528)
    assert call(b8, batch=8, y=0) == NULL
    b8x, _ = _matrix(rows=4, cols=6656)
    assert call(b8x, batch=8) == SHAPE
    # nothing to do
    z, _ = _matrix(rows=0, blob=0)
    assert call(z) == OK


def test_matvec_w2a8_activation_and_workspace_checks():
    m, k = _matrix()
    assert _w2a8(m, x=0) == NULL and _w2a8(m, x=FAKE + (1 << 30) + 2) == ALIGN
    assert _w2a8q(m, xq=0) == NULL and _w2a8q(m, sx=0) == NULL
    assert _w2a8q(m, xq=FAKE + (1 << 30) + 8) == ALIGN and _w2a8q(m, sx=FAKE + (1 << 32) + 2) == ALIGN
    assert _w2a8q(m, y=FAKE + (1 << 32) + 4) == OVERLAP  # y on sx
    # workspace: batch x cols_pad int8, 256-aligned, then the fp32 scales
    assert _w8ws(m, 1) == (OK, 256 + 2 * 4)
    assert _w8ws(m, 3) == (OK, 768 + 3 * 2 * 4)
    assert _w8ws(m, 9)[0] == SHAPE
    wide, _ = _matrix(rows=4, cols=16384)
    assert _w8ws(wide, 4)[0] == SHAPE and _w8ws(wide, 2) == (OK, 32768 + 2 * 128 * 4)
    assert _w8ws(_matrix(rows=0, blob=0)[0], 1) == (OK, 0)
    assert _w2a8(m, ws=0) == WORKSPACE and _w2a8(m, wsb=263) == WORKSPACE
    assert _w2a8(m, ws=WS + 8) == ALIGN
    assert _w2a8(m, ws=FAKE + (1 << 30) + 64) == OVERLAP  # workspace on x
    assert _w2a8(m, ws=FAKE + (1 << 31)) == OVERLAP  # workspace on y
    assert _w2a8(m, ws=FAKE + 128) == OVERLAP  # workspace on the blob
    cz, _ = _matrix(cols=0)
    assert _w2a8(cz, ws=0, y=0) == NULL  # y still required where cols == 0


def test_quantize_acts_int8_validation():
    assert _qacts(batch=-1) == SHAPE and _qacts(cols=-1) == SHAPE and _qacts(cols=(1 << 30) + 1) == SHAPE
    assert _qacts(batch=0, x=0) == OK and _qacts(cols=0, xq=0) == OK
    assert _qacts(x=0) == NULL and _qacts(xq=0) == NULL and _qacts(sx=0) == NULL
    assert _qacts(x=FAKE + (1 << 30) + 2) == ALIGN and _qacts(xq=FAKE + (1 << 31) + 4) == ALIGN
    assert _qacts(sx=FAKE + (1 << 32) + 1) == ALIGN
    assert _qacts(xq=FAKE + (1 << 30) + 16) == OVERLAP  # xq on x
    assert _qacts(sx=FAKE + (1 << 31) + 512) == OVERLAP  # sx on xq (2 x 384 bytes)


def _gather(m, ids=FAKE + (1 << 30), n=4, out=FAKE + (1 << 31), dt=0):
    return lib.cq_gather_rows(ctypes.byref(m), ctypes.c_void_p(ids), n, ctypes.c_void_p(out), dt, None)


def test_gather_rows_validation():
    m, k = _matrix(bits=7, nbytes=0, levels=None)
    assert _gather(m) == BITS
    m, k = _matrix(levels=np.array([0.1, 0.0, 0.2, 0.3]))
    assert _gather(m) == CODEBOOK
    m, k = _matrix()
    assert _gather(m, dt=3) == DTYPE and _gather(m, dt=-1) == DTYPE
    assert _gather(m, n=-1) == SHAPE and _gather(m, n=(1 << 30) + 1) == SHAPE
    assert _gather(m, n=0) == OK
    assert _gather(m, ids=0) == NULL and _gather(m, out=0) == NULL
    assert _gather(m, ids=FAKE + (1 << 30) + 4) == ALIGN
    assert _gather(m, out=FAKE + (1 << 31) + 2) == ALIGN and _gather(m, out=FAKE + (1 << 31) + 1, dt=2) == ALIGN
    assert _gather(m, out=FAKE + (1 << 30) + 16) == OVERLAP  # out on top of ids
    assert _gather(m, out=FAKE + 32) == OVERLAP  # out on top of the blob
    z, _ = _matrix(rows=4, cols=0)
    assert _gather(z) == OK  # no columns: nothing to write


def test_nothing_to_do_returns_ok_without_launching():
    m, k = _matrix()
    assert _matvec(m, batch=0) == OK and _gemm(m, mm=0) == OK
    m, k = _matrix(rows=0, blob=0)
    assert _matvec(m) == OK and _gemm(m) == OK
    assert lib.cq_rotate_acts(ctypes.c_void_p(FAKE), 0, 0, 128, ctypes.c_void_p(FAKE), 0, None) == OK
    assert lib.cq_rotate_acts(ctypes.c_void_p(FAKE), 0, 4, 0, ctypes.c_void_p(FAKE), 0, None) == OK
    lv = cq_inputs.codebook(2)
    p = lv.ctypes.data_as(ctypes.POINTER(ctypes.c_float))
    assert lib.cq_quantize(None, 0, 128, 2, 128, p, None, 0, None) == OK


def test_rotate_validation():
    x, xr = ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE + (1 << 30))
    assert lib.cq_rotate_acts(x, 3, 1, 128, xr, 0, None) == DTYPE
    assert lib.cq_rotate_acts(x, 0, 1, 128, xr, 1, None) == DTYPE
    assert lib.cq_rotate_acts(x, 0, -1, 128, xr, 0, None) == SHAPE
    assert lib.cq_rotate_acts(None, 0, 1, 128, xr, 0, None) == NULL
    assert lib.cq_rotate_acts(ctypes.c_void_p(FAKE + 2), 0, 1, 128, xr, 0, None) == ALIGN
    assert lib.cq_rotate_acts(x, 0, 1, 128, ctypes.c_void_p(FAKE + (1 << 30) + 4), 0, None) == ALIGN
    assert lib.cq_rotate_acts(x, 0, 2, 128, ctypes.c_void_p(FAKE + 512), 0, None) == OVERLAP


def test_quantize_validation():
    lv = cq_inputs.codebook(2)
    p = lv.ctypes.data_as(ctypes.POINTER(ctypes.c_float))
    w, blob = ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE + (1 << 30))
    nb = oracle.blob_bytes(2, 128, 4, 256)
    assert lib.cq_quantize(w, 4, 256, 6, 128, p, blob, nb, None) == BITS
    assert lib.cq_quantize(w, 4, 256, 2, 64, p, blob, nb, None) == GROUP
    assert lib.cq_quantize(w, 4, 256, 2, 128, None, blob, nb, None) == CODEBOOK
    assert lib.cq_quantize(w, 4, 256, 2, 128, p, blob, nb + 1, None) == LENGTH
    assert lib.cq_quantize(None, 4, 256, 2, 128, p, blob, nb, None) == NULL
    assert lib.cq_quantize(w, 4, 256, 2, 128, p, ctypes.c_void_p(FAKE + (1 << 30) + 8), nb, None) == ALIGN
    assert lib.cq_quantize(w, 4, 256, 2, 128, p, ctypes.c_void_p(FAKE + 256), nb, None) == OVERLAP
    tern = ctypes.cast(None, ctypes.POINTER(ctypes.c_float))
    nb5 = oracle.blob_bytes(5, 128, 4, 256)
    assert lib.cq_quantize(w, 4, 256, 5, 128, p, blob, nb5, None) == CODEBOOK
    assert lib.cq_quantize(w, 4, 256, 5, 128, tern, blob, nb5 - 2, None) == LENGTH


def test_matvec_workspace_rules():
    # K beyond one slice needs a workspace: one partial sum per slice and row
    m, k = _matrix(rows=1000, cols=16384)
    need = ctypes.c_uint64()
    assert lib.cq_workspace_bytes(0, ctypes.byref(m), 1, ctypes.byref(need)) == OK
    nslice = 16  # 1024 columns of 2-bit byte tables per slice
    assert need.value == nslice * 1000 * 4  # one fp32 partial sum per slice and row
    ws = FAKE + (1 << 32)
    call = lambda w, n: lib.cq_matvec(ctypes.byref(m), ctypes.c_void_p(FAKE + (1 << 30)), 1,
                                      ctypes.c_void_p(FAKE + (1 << 31)), ctypes.c_void_p(w), n, None)
    assert call(0, 0) == WORKSPACE
    assert call(ws, need.value - 1) == WORKSPACE
    assert call(ws + 4, need.value) == ALIGN
    assert call(FAKE + (1 << 31) + 64, need.value) == OVERLAP  # workspace on top of y
    # batches of 2..8 run on the matrix-core kernel: 4096-column slices, one
    # partial sum per slice, batch vector and row
    for batch in (2, 5, 8):
        needb = ctypes.c_uint64()
        assert lib.cq_workspace_bytes(0, ctypes.byref(m), batch, ctypes.byref(needb)) == OK
        assert needb.value == 4 * batch * 1000 * 4
    # K within one slice of that kernel: no workspace
    m2, _ = _matrix(rows=1000, cols=4096)
    assert lib.cq_workspace_bytes(0, ctypes.byref(m2), 8, ctypes.byref(needb)) == OK and needb.value == 0


def test_workspace_bytes():
    m, k = _matrix()
    out = ctypes.c_uint64(7)
    assert lib.cq_workspace_bytes(0, ctypes.byref(m), 1, ctypes.byref(out)) == OK and out.value == 0
    assert lib.cq_workspace_bytes(1, ctypes.byref(m), 4096, ctypes.byref(out)) == OK
    assert lib.cq_workspace_bytes(0, ctypes.byref(m), 9, ctypes.byref(out)) == SHAPE
    assert lib.cq_workspace_bytes(5, ctypes.byref(m), 1, ctypes.byref(out)) == SHAPE
    assert lib.cq_workspace_bytes(6, ctypes.byref(m), 1, ctypes.byref(out)) == SHAPE
    assert lib.cq_workspace_bytes(-1, ctypes.byref(m), 1, ctypes.byref(out)) == SHAPE
    # empty K or no rows: nothing is launched, so no workspace (and no division by zero)
    for rows, cols in ((5, 0), (0, 256), (0, 0)):
        e, _ = _matrix(rows=rows, cols=cols)
        out.value = 7
        assert lib.cq_workspace_bytes(0, ctypes.byref(e), 8, ctypes.byref(out)) == OK and out.value == 0
    # the fused call: as cq_matvec at batch 1; at batch 2..8 also the rotated
    # activation, after the partial sums rounded up to 16 bytes
    m3, _ = _matrix(rows=1001, cols=16384)
    for batch in (1, 2, 8):
        a, b = ctypes.c_uint64(), ctypes.c_uint64()
        assert lib.cq_workspace_bytes(0, ctypes.byref(m3), batch, ctypes.byref(a)) == OK
        assert lib.cq_workspace_bytes(2, ctypes.byref(m3), batch, ctypes.byref(b)) == OK
        assert b.value == (a.value if batch == 1 else -(-a.value // 16) * 16 + batch * 16384 * 4)
    assert lib.cq_workspace_bytes(2, ctypes.byref(m3), 9, ctypes.byref(out)) == SHAPE
    # a K split over several slices needs partial sums
    big, _ = _matrix(rows=65536, cols=16384)
    assert lib.cq_workspace_bytes(0, ctypes.byref(big), 1, ctypes.byref(out)) == OK
    assert out.value > 0 and out.value % 16 == 0


def test_binding_has_the_c_names():
    for n in ("cq_blob_bytes", "cq_workspace_bytes", "cq_rotate_acts", "cq_matvec", "cq_rotate_matvec",
              "cq_rotate_multi_matvec", "cq_rotate_multi_workspace_bytes", "cq_quantize_acts_int8",
              "cq_matvec_w2a8_quantized", "cq_matvec_w2a8", "cq_gather_rows",
              "cq_gemm", "cq_quantize"):
        assert callable(getattr(cq, n))


def test_binary_matrices():
    # binary (bits 1): analytic levels, so levels must be NULL
    m, k = _matrix(bits=1, levels=np.array([-0.1, 0.1]))
    assert _matvec(m) == CODEBOOK
    m, k = _matrix(bits=1)
    assert k is None and m.blob_bytes == 4 * 32 + 4 * 2 * 2
    assert _matvec(m, y=0) == NULL  # past every matrix check
    assert _gemm(m, c=0) == NULL  # past every matrix check
    # batch 1: the lookup tables on 2048-column slices; batch 4: the matrix
    # cores on 4096-column slices, partial sums per vector
    big, _ = _matrix(bits=1, rows=65536, cols=16384)
    out1, out4 = ctypes.c_uint64(0), ctypes.c_uint64(0)
    assert lib.cq_workspace_bytes(0, ctypes.byref(big), 1, ctypes.byref(out1)) == OK
    assert lib.cq_workspace_bytes(0, ctypes.byref(big), 4, ctypes.byref(out4)) == OK
    assert out1.value == 8 * 65536 * 4 and out4.value == 4 * 4 * 65536 * 4
    # W2A8: the same limits as the other widths (both kernels decode binary)
    wide, _ = _matrix(bits=1, rows=4, cols=16384)
    assert _w2a8(wide, batch=3, y=0) == NULL and _w2a8(wide, batch=4) == SHAPE
    assert _w2a8(_matrix(bits=1, rows=4, cols=4096)[0], batch=5, y=0) == NULL
    assert _w2a8(_matrix(bits=1, rows=4, cols=27264)[0], batch=1, y=0) == NULL


def test_column_limits_are_shape_errors():
    # the kernels' 32-bit tile offsets bound cols_pad: a wider matrix is a
    # CQ_ERR_SHAPE from validation (nothing launched), not a launch failure
    gemm_max, mv_max = 1 << 22, 1 << 24
    m, k = _matrix(rows=1, cols=gemm_max + 1)
    assert _gemm(m) == SHAPE
    out = ctypes.c_uint64(7)
    assert lib.cq_workspace_bytes(cq.OP_GEMM, ctypes.byref(m), 8, ctypes.byref(out)) == SHAPE and out.value == 7
    m, k = _matrix(rows=1, cols=mv_max + 1)
    assert _matvec(m) == SHAPE and _rotate_matvec(m) == SHAPE
    for op in (cq.OP_MATVEC, cq.OP_ROTATE_MATVEC):
        assert lib.cq_workspace_bytes(op, ctypes.byref(m), 1, ctypes.byref(out)) == SHAPE and out.value == 7
    # at the limits the shape passes and validation goes on to the next check
    # (nothing is launched: the gemm's output overlaps its activation, the
    # matvec has no workspace for its K slices)
    m, k = _matrix(rows=1, cols=gemm_max)
    assert _gemm(m, c=FAKE + (1 << 30)) == OVERLAP
    m, k = _matrix(rows=1, cols=mv_max)
    assert _matvec(m, y=FAKE + (1 << 30)) == WORKSPACE


def test_gemm_ignores_its_workspace_arguments():
    # cq_gemm needs no scratch: the workspace query reports 0 and any
    # workspace pointer and size are accepted (validation reaches the same
    # overlap error with and without them)
    m, k = _matrix()
    out = ctypes.c_uint64(7)
    assert lib.cq_workspace_bytes(cq.OP_GEMM, ctypes.byref(m), 4096, ctypes.byref(out)) == OK and out.value == 0
    base = lib.cq_gemm(ctypes.byref(m), ctypes.c_void_p(FAKE + (1 << 30)), 8, ctypes.c_void_p(FAKE), None, 0, None)
    with_ws = lib.cq_gemm(ctypes.byref(m), ctypes.c_void_p(FAKE + (1 << 30)), 8, ctypes.c_void_p(FAKE),
                          ctypes.c_void_p(FAKE + 3), 5, None)
    assert base == with_ws == OVERLAP


def _noalloc(m, x=FAKE + (1 << 30), batch=1, y=FAKE + (1 << 31)):
    return lib.cq_rotate_matvec_noalloc(ctypes.byref(m), ctypes.c_void_p(x), batch, ctypes.c_void_p(y), None)


def test_noalloc_validation():
    # the checks of cq_rotate_matvec, then the static scratch's size: a call
    # that needs more than CQ_NOALLOC_SCRATCH_BYTES is refused before any
    # device call (65536 x 16384 fits at every batch; 2^20 rows do not)
    limit = 16 << 20
    m, k = _matrix(bits=7, nbytes=0, levels=None)
    assert _noalloc(m) == BITS
    m, k = _matrix()
    assert _noalloc(m, batch=9) == SHAPE and _noalloc(m, y=0) == NULL and _noalloc(m, y=FAKE + 64) == OVERLAP
    need = ctypes.c_uint64(0)
    for bits in (1, 2, 3, 4, 5):
        for batch in range(1, 9):
            m, k = _matrix(bits=bits, rows=65536, cols=16384)
            assert lib.cq_workspace_bytes(cq.OP_ROTATE_MATVEC, ctypes.byref(m), batch, ctypes.byref(need)) == OK
            assert need.value <= limit
    m, k = _matrix(rows=1 << 20, cols=16384)
    assert lib.cq_workspace_bytes(cq.OP_ROTATE_MATVEC, ctypes.byref(m), 1, ctypes.byref(need)) == OK
    assert need.value > limit
    assert _noalloc(m) == SCRATCH
    assert "static scratch" in lib.cq_status_string(SCRATCH).decode()
    # nothing to do: no device call at all
    m, k = _matrix(rows=0)
    assert _noalloc(m) == OK


def test_kv_cache_calls_validation():
    # cq_quantize_rows: the row range must lie inside the matrix
    m, k = _matrix(rows=256, cols=256)
    w = FAKE + (1 << 33)
    assert lib.cq_quantize_rows(ctypes.c_void_p(w), 1, ctypes.byref(m), 256, None) == SHAPE
    assert lib.cq_quantize_rows(ctypes.c_void_p(w), 2, ctypes.byref(m), 255, None) == SHAPE
    assert lib.cq_quantize_rows(ctypes.c_void_p(w), -1, ctypes.byref(m), 0, None) == SHAPE
    assert lib.cq_quantize_rows(ctypes.c_void_p(w), 1, ctypes.byref(m), -1, None) == SHAPE
    assert lib.cq_quantize_rows(ctypes.c_void_p(w), 0, ctypes.byref(m), 256, None) == OK  # nothing to do
    assert lib.cq_quantize_rows(None, 1, ctypes.byref(m), 0, None) == NULL
    assert lib.cq_quantize_rows(ctypes.c_void_p(w + 2), 1, ctypes.byref(m), 0, None) == ALIGN
    assert lib.cq_quantize_rows(ctypes.c_void_p(FAKE + 64), 1, ctypes.byref(m), 0, None) == OVERLAP
    bad, _ = _matrix(bits=7, nbytes=0, levels=None)
    assert lib.cq_quantize_rows(ctypes.c_void_p(w), 1, ctypes.byref(bad), 0, None) == BITS
    # cq_kv_scores: head geometry must match the cache width
    out = ctypes.c_uint64(7)
    for nq, nkv, hd in ((8, 4, 64), (12, 2, 128), (4, 4, 64)):
        assert lib.cq_kv_scores_workspace_bytes(ctypes.byref(m), nq, nkv, hd, ctypes.byref(out)) == (
            OK if nkv * hd == 256 else SHAPE)
    assert lib.cq_kv_scores_workspace_bytes(ctypes.byref(m), 8, 4, 64, ctypes.byref(out)) == OK
    assert out.value >= 8 * 256 * 4
    for nq, nkv, hd in ((6, 4, 64), (0, 4, 64), (8, 0, 64), (8, 4, 32), (512, 4, 64)):
        assert lib.cq_kv_scores_workspace_bytes(ctypes.byref(m), nq, nkv, hd, ctypes.byref(out)) == SHAPE
    q, sc, ws = FAKE + (1 << 33), FAKE + (1 << 34), FAKE + (1 << 35)
    call = lambda **kw: lib.cq_kv_scores(ctypes.byref(m), ctypes.c_void_p(kw.get("q", q)), 8, 4, 64,
                                         ctypes.c_void_p(kw.get("sc", sc)), ctypes.c_void_p(kw.get("ws", ws)),
                                         kw.get("wsb", 1 << 20), None)
    assert call(wsb=16) == WORKSPACE and call(ws=ws + 16) == ALIGN and call(sc=0) == NULL
    assert call(sc=q) == OVERLAP and call(ws=FAKE) == OVERLAP
    # cq_matvec_t: sizes and the workspace query (row chunks of 1024: a
    # 256-row cache needs none, 2500 rows three chunks of partial sums)
    assert lib.cq_workspace_bytes(cq.OP_MATVEC_T, ctypes.byref(m), 8, ctypes.byref(out)) == OK
    assert out.value == 0
    m3, lv3 = _matrix(rows=2500, cols=256)  # lv3 keeps the levels array alive
    assert lib.cq_workspace_bytes(cq.OP_MATVEC_T, ctypes.byref(m3), 8, ctypes.byref(out)) == OK
    assert out.value == 3 * 8 * 256 * 4
    assert lib.cq_workspace_bytes(cq.OP_MATVEC_T, ctypes.byref(m), 9, ctypes.byref(out)) == SHAPE
    big, _ = _matrix(rows=(1 << 20) + 1, cols=128)
    assert lib.cq_workspace_bytes(cq.OP_MATVEC_T, ctypes.byref(big), 1, ctypes.byref(out)) == SHAPE
    mt = lambda **kw: lib.cq_matvec_t(ctypes.byref(m3), ctypes.c_void_p(kw.get("p", q)), kw.get("b", 2),
                                      ctypes.c_void_p(kw.get("o", sc)), ctypes.c_void_p(kw.get("ws", ws)),
                                      kw.get("wsb", 1 << 20), None)
    assert mt(b=9) == SHAPE and mt(o=0) == NULL and mt(p=0) == NULL and mt(wsb=4) == WORKSPACE
    assert mt(o=q) == OVERLAP and mt(o=sc + 2) == ALIGN


def test_kv_attention_validation():
    # the fused step: both caches alike, a head inside one 128-group, 1 <= n <= rows
    K, kk = _matrix(rows=256, cols=256, blob=FAKE)
    V, kv = _matrix(rows=256, cols=256, blob=FAKE + (1 << 32))
    q, o = FAKE + (1 << 33), FAKE + (1 << 34)
    lib.cq_kv_attention.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int32,
                                    ctypes.c_int32, ctypes.c_int32, ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p]

    def call(k=K, v=V, n=256, qq=q, nq=8, nkv=4, hd=64, out=o):
        return lib.cq_kv_attention(ctypes.addressof(k), ctypes.addressof(v), n, qq, nq, nkv, hd, 0.125, out, None)

    for n in (0, -1, 257):
        assert call(n=n) == SHAPE
    assert call(nq=6) == SHAPE and call(nq=0) == SHAPE and call(nkv=0) == SHAPE and call(nq=512, nkv=4) == SHAPE
    assert call(nkv=4, hd=32) == SHAPE  # 4 x 32 != 256 columns
    W, kw = _matrix(rows=64, cols=96 * 2, blob=FAKE)
    W2, kw2 = _matrix(rows=64, cols=96 * 2, blob=FAKE + (1 << 32))
    assert call(k=W, v=W2, n=8, nq=2, nkv=2, hd=96) == SHAPE  # 96 does not divide 128
    K3, k3 = _matrix(bits=3, rows=256, cols=256, blob=FAKE)
    assert call(k=K3) == SHAPE  # different widths
    K2, k2 = _matrix(rows=128, cols=256, blob=FAKE)
    assert call(k=K2, n=100) == SHAPE  # different row counts
    assert call(qq=0) == NULL and call(out=0) == NULL
    assert call(qq=q + 2) == ALIGN and call(out=o + 2) == ALIGN
    assert call(out=q) == OVERLAP and call(out=FAKE + 64) == OVERLAP and call(out=FAKE + (1 << 32) + 64) == OVERLAP
    bad, _ = _matrix(bits=7, nbytes=0, levels=None)
    assert call(k=bad) == BITS


def test_kv_append_validation():
    K, kk = _matrix(rows=256, cols=256, blob=FAKE)
    V, kv = _matrix(rows=256, cols=256, blob=FAKE + (1 << 32))
    k, v = FAKE + (1 << 33), FAKE + (1 << 34)
    lib.cq_kv_append.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                 ctypes.c_int64, ctypes.c_void_p]

    def call(kk_=K, vv=V, ka=k, va=v, n=1, row0=0):
        return lib.cq_kv_append(ctypes.addressof(kk_), ctypes.addressof(vv), ka, va, n, row0, None)

    assert call(n=0, row0=256) == OK  # nothing to do
    assert call(row0=256) == SHAPE and call(n=2, row0=255) == SHAPE and call(n=-1) == SHAPE and call(row0=-1) == SHAPE
    V3, k3 = _matrix(bits=3, rows=256, cols=256, blob=FAKE + (1 << 32))
    assert call(vv=V3) == SHAPE  # widths differ
    Vs, ks = _matrix(rows=100, cols=256, blob=FAKE + (1 << 32))
    assert call(vv=Vs, row0=100) == SHAPE  # does not fit the smaller cache
    assert call(ka=0) == NULL and call(va=0) == NULL
    assert call(ka=k + 2) == ALIGN and call(va=v + 2) == ALIGN
    Vo, ko = _matrix(rows=256, cols=256, blob=FAKE + 64)
    assert call(vv=Vo) == OVERLAP  # the two blobs overlap
    assert call(ka=FAKE + 128) == OVERLAP and call(va=FAKE + (1 << 32) + 128) == OVERLAP
    bad, _ = _matrix(bits=7, nbytes=0, levels=None)
    assert call(kk_=bad) == BITS
