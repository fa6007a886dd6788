"""GPU parity of every matvec route on inputs that defeat averaging
(``precision_cases``: activations lined up with weight rows, rows of one or
two groups, small group norms, norms spanning six decades), element by
element against the float64 oracle at the fp32 bar:

    |y - y_oracle| <= 1e-4 * ||w_hat_row||_2 * ||x||_2, cosine >= 0.99999.

Each case goes through cq_matvec (from cq_rotate_acts), cq_rotate_matvec and
cq_rotate_multi_matvec (with a second matrix of another shape in the same
call), at batch 1 and 8 (3 for the widest rows).
"""
import sys

import numpy as np
import pytest
import torch

import precision_cases as pc

pytestmark = pytest.mark.gpu
cq = pytest.importorskip("hadamard_rotated_codebook_amd")
DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _check(y, ref, wn, xn, what):
    y = np.asarray(y, dtype=np.float64)
    r = pc.err_over_bar(y, ref, wn, xn)
    assert r <= 1.0, f"{what}: max err/bound {r:.3g}"
    for b in range(ref.shape[0]):
        if np.linalg.norm(ref[b]) > 0:
            cos = y[b] @ ref[b] / np.linalg.norm(y[b]) / np.linalg.norm(ref[b])
            assert cos >= 0.99999, (what, b, cos)
    return r


@pytest.mark.parametrize("bits", [1, 2, 3, 4, 5])
@pytest.mark.parametrize("name", pc.CASES)
def test_matvec_routes_at_the_fp32_bar(name, bits):
    rows, cols = (int(v) for v in name.split(":")[1].split("x"))
    worst = 0.0
    for batch in (1, 3 if cols > 4096 else 8):
        say("precision", name, "bits", bits, "batch", batch)
        blob, levels, x = pc.case(name, bits, batch)
        ref, wn, xn = pc.bar_terms(blob, bits, rows, cols, levels, x)
        W = cq.CQMatrix(bits, rows, cols, torch.from_numpy(blob).to(DEV), levels)
        xd = torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
        y1 = cq.cq_matvec(W, cq.cq_rotate_acts(xd)).cpu().numpy()
        y2 = cq.cq_rotate_matvec(W, xd).cpu().numpy()
        # the shared-activation call, with a 64-row matrix of the same width
        # and columns in the same call
        blob2, levels2 = pc.random_codes(77, bits, 64, cols)
        W2 = cq.CQMatrix(bits, 64, cols, torch.from_numpy(blob2).to(DEV), levels2)
        y3, y4 = cq.cq_rotate_multi_matvec([W, W2], xd)
        torch.cuda.synchronize()
        worst = max(worst, _check(y1, ref, wn, xn, "cq_matvec"), _check(y2, ref, wn, xn, "cq_rotate_matvec"),
                    _check(y3.cpu().numpy(), ref, wn, xn, "cq_rotate_multi_matvec"))
        ref2, wn2, xn2 = pc.bar_terms(blob2, bits, 64, cols, levels2, x)
        _check(y4.cpu().numpy(), ref2, wn2, xn2, "cq_rotate_multi_matvec (second matrix)")
    say(f"  worst err/bound {worst:.3g}")
