"""cq_rotate_matvec_noalloc (the entry point that allocates nothing: its
scratch is the library's static device array) against cq_rotate_matvec
through the C-ABI: the same results, bit for bit, on two calls in a row, the
second with a smaller input, so that it runs on what the first left in the
scratch.  Run by itself in a fresh process and after the other tests."""
import ctypes
import sys

import numpy as np
import pytest
import torch

import cq_inputs

pytestmark = pytest.mark.gpu
cq = pytest.importorskip("hadamard_rotated_codebook_amd")
DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _noalloc_raw(W, x, y):
    """The C entry point with raw pointers and the current stream."""
    m, keep = W._struct()
    st = cq._lib.cq_rotate_matvec_noalloc(ctypes.byref(m), ctypes.c_void_p(x.data_ptr()), x.shape[0],
                                          ctypes.c_void_p(y.data_ptr()),
                                          ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, cq._lib.cq_status_string(st).decode()


def _matrix(bits, rows, cols, seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    w = torch.randn((rows, cols), generator=g, device=DEV).mul_(0.02)
    return cq.cq_quantize(w, bits, cq_inputs.codebook(bits)), g


# (bits, rows, cols, batch) of the two calls, larger first, and the kernel
# each reaches: the lookup tables with 16 K slices of partial sums (4 MiB of
# scratch); the batched matrix-core kernel with the rotation and 2 slices
CASES = [
    [(2, 65536, 16384, 1), (4, 1024, 6000, 3)],
    [(4, 65536, 16384, 8), (5, 40000, 4096, 1)],
    [(3, 8192, 9000, 5), (1, 300, 640, 2)],
]


@pytest.mark.parametrize("calls", CASES)
def test_noalloc_matches_rotate_matvec(calls):
    for bits, rows, cols, batch in calls:
        say("noalloc", bits, rows, cols, batch)
        W, g = _matrix(bits, rows, cols, 7 * rows + cols)
        x = torch.randn((batch, cols), generator=g, device=DEV)
        ref = cq.cq_rotate_matvec(W, x)
        y = torch.full((batch, rows), float("nan"), device=DEV)
        _noalloc_raw(W, x, y)
        torch.cuda.synchronize()
        assert torch.equal(y, ref), (bits, rows, cols, batch)
        y2 = torch.full((batch, rows), float("nan"), device=DEV)
        cq.cq_rotate_matvec_noalloc(W, x, y2)  # the binding of the same entry point
        torch.cuda.synchronize()
        assert torch.equal(y2, ref)
        del W, x, ref, y, y2
    torch.cuda.empty_cache()
