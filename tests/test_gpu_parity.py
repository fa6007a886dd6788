"""GPU parity: every entry point of libcq against the float64 oracle on the
same seeded inputs, at sizes that span several tiles/phases with ragged tails,
plus the degenerate cases (empty batch, zero rows, zero cols).

Bars (fixed by the method's acceptance rule):
  fp32 paths      |y - y_oracle| <= 1e-4 * ||w_hat_row||_2 * ||x||_2, cosine >= 0.99999
  bf16 MFMA path  |C - C_oracle| <= 1e-2 * ||w_hat_row||_2 * ||x||_2, cosine >= 0.9999
  encoder         >= 99.99 % identical indices, mismatches within 1e-5 of a
                  decision boundary; fp16 norms identical
"""
import sys

import numpy as np
import pytest
import torch

import cq_inputs
import oracle

pytestmark = pytest.mark.gpu
cq = pytest.importorskip("hadamard_rotated_codebook_amd")
DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _levels(bits, kind="empirical"):
    return None if bits == 5 else cq_inputs.codebook(bits, kind)


def _to_dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.to(DEV)


def _cq_from_oracle(bits, rows, cols, cfg, kind="empirical"):
    levels = _levels(bits, kind)
    w = cq_inputs.master(cfg, bits, rows, cols)
    blob = oracle.quantize(w, bits, levels)
    return cq.CQMatrix(bits, rows, cols, _to_dev(blob), levels), blob, levels, w


def _check_fp32_product(y, ref, w_hat_norms, x_norms, tol=1e-4, min_cos=0.99999):
    y = y.astype(np.float64)
    bound = tol * np.outer(x_norms, w_hat_norms)
    err = np.abs(y - ref)
    assert np.all(err <= bound), f"max err/bound {np.max(err / np.maximum(bound, 1e-300)):.3g}"
    for b in range(ref.shape[0]):
        if np.linalg.norm(ref[b]) > 0:
            cos = y[b] @ ref[b] / np.linalg.norm(y[b]) / np.linalg.norm(ref[b])
            assert cos >= min_cos, cos


# ----------------------------------------------------------------- rotation

@pytest.mark.parametrize("xdt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("odt", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("batch,cols", [(1, 512), (3, 300), (5, 1000), (2, 16384), (7, 127)])
def test_rotate_acts(xdt, odt, batch, cols):
    say("rotate", xdt, odt, batch, cols)
    x = cq_inputs.activations(11, cols, batch, cols, xdt)
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[xdt]
    xr = cq.cq_rotate_acts(_to_dev(x, tdt), odt)
    torch.cuda.synchronize()
    got = xr.float().cpu().numpy().astype(np.float64)
    ref = oracle.rotate_acts(x)
    kpad = ref.shape[1]
    gnorm = np.linalg.norm(np.pad(x.astype(np.float64), ((0, 0), (0, kpad - cols))).reshape(batch, -1, 128), axis=-1)
    gnorm = np.repeat(gnorm, 128, axis=1)
    bound = 2e-6 * gnorm + (2.0 ** -8 * np.abs(ref) if odt == torch.bfloat16 else 0)
    assert np.all(np.abs(got - ref) <= bound)


def test_rotate_empty_inputs_are_noops():
    x = torch.zeros((0, 256), device=DEV)
    assert cq.cq_rotate_acts(x).shape == (0, 256)
    x = torch.zeros((3, 0), device=DEV)
    assert cq.cq_rotate_acts(x).shape == (3, 0)


# ------------------------------------------------------------------ matvec

@pytest.mark.parametrize("bits", [1, 2, 3, 4, 5])
@pytest.mark.parametrize("rows,cols,batch", [
    (512, 512, 1),       # the single 512x512 matvec workload
    (1000, 5000, 1),     # ragged rows, partial last phase
    (300, 9000, 3),      # several phases, batch split 2 + 1
    (257, 2048, 4),
    (64, 640, 8),        # batch split 4 + 4
    (1, 128, 5),
    (9, 16384, 2),
])
def test_matvec(bits, rows, cols, batch):
    say("matvec", bits, rows, cols, batch)
    W, blob, levels, _ = _cq_from_oracle(bits, rows, cols, 20 + batch)
    x = cq_inputs.activations(21, rows, batch, cols)
    xr = cq.cq_rotate_acts(_to_dev(x))
    y = cq.cq_matvec(W, xr)
    torch.cuda.synchronize()
    ref = oracle.matvec(blob, bits, rows, cols, x, levels)
    w_hat = np.linalg.norm(oracle.dequantize(blob, bits, rows, cols, levels), axis=1)
    _check_fp32_product(y.cpu().numpy(), ref, w_hat, np.linalg.norm(x.astype(np.float64), axis=1))


@pytest.mark.parametrize("bits", [2, 4])
def test_matvec_hadamard_column_probe(bits):
    # x_g = H e_j in one group: y_r = norm[r, g] * level(q[r, g, j]) up to the
    # rotation's rounding and one rounding of the lookup-table entry to fp16
    # (relative 2^-11) -- pins the GPU bit layout index by index (adjacent
    # levels differ by far more than that)
    rows, cols = 96, 384
    W, blob, levels, _ = _cq_from_oracle(bits, rows, cols, 30)
    packed, norms = oracle.split_blob(blob, bits, rows, cols)
    vals = oracle.level_values(oracle.unpack_codes(packed, bits, cols), bits, levels)
    H = oracle.hadamard()
    for g in range(3):
        for j in range(128):
            x = np.zeros((1, cols), np.float32)
            x[0, 128 * g:128 * (g + 1)] = H[:, j]
            y = cq.cq_matvec(W, cq.cq_rotate_acts(_to_dev(x)))
            expect = norms[:, g].astype(np.float64) * vals[:, 128 * g + j]
            got = y.cpu().numpy()[0].astype(np.float64)
            assert np.allclose(got, expect, rtol=2.0 ** -11, atol=1e-7 * np.max(np.abs(expect))), (g, j)


def test_matvec_degenerate_shapes():
    levels = cq_inputs.codebook(2)
    # cols == 0: every output is an empty sum
    W = cq.CQMatrix(2, 5, 0, torch.zeros(0, dtype=torch.uint8, device=DEV), levels)
    y = torch.full((2, 5), 7.0, device=DEV)
    cq.cq_matvec(W, torch.zeros((2, 0), device=DEV), out=y)
    assert torch.all(y == 0)
    # rows == 0 and batch == 0 write nothing
    W0 = cq.CQMatrix(2, 0, 256, torch.zeros(0, dtype=torch.uint8, device=DEV), levels)
    assert cq.cq_matvec(W0, torch.zeros((1, 256), device=DEV)).shape == (1, 0)
    W1, _, _, _ = _cq_from_oracle(2, 4, 256, 31)
    assert cq.cq_matvec(W1, torch.zeros((0, 256), device=DEV)).shape == (0, 4)
    # x = 0 gives y = 0
    y = cq.cq_matvec(W1, cq.cq_rotate_acts(torch.zeros((1, 256), device=DEV)))
    assert torch.all(y == 0)


def test_matvec_ternary_crumb_10_sign_extends():
    # crumb 0b10 decodes to -2a (never written by the encoder, but defined)
    rows, cols = 2, 128
    codes = np.full((rows, cols), 2, np.uint8)
    norms = np.ones((rows, 1), np.float16)
    blob = oracle.make_blob(oracle.pack_codes(codes, 5), norms)
    W = cq.CQMatrix(5, rows, cols, _to_dev(blob), None)
    x = cq_inputs.activations(32, 0, 1, cols)
    y = cq.cq_matvec(W, cq.cq_rotate_acts(_to_dev(x))).cpu().numpy()
    ref = oracle.matvec(blob, 5, rows, cols, x)
    _check_fp32_product(y, ref, np.linalg.norm(oracle.dequantize(blob, 5, rows, cols), axis=1),
                        np.linalg.norm(x.astype(np.float64), axis=1))


def test_matvec_workspace_reuse_across_shapes():
    # one workspace, filled with garbage first, serves calls with different
    # slice and row-block counts: its contents on entry must not matter
    shapes = [(4, 3000, 16384, 1), (2, 700, 16384, 3), (3, 5000, 9000, 1), (5, 64, 16384, 8), (4, 3000, 16384, 1)]
    ws = torch.full((1 << 24,), 0x7f, dtype=torch.uint8, device=DEV)  # 0x7f7f7f7f is a huge float
    for bits, rows, cols, batch in shapes:
        W, blob, levels, _ = _cq_from_oracle(bits, rows, cols, 34)
        x = cq_inputs.activations(34, rows, batch, cols)
        y = cq.cq_matvec(W, cq.cq_rotate_acts(_to_dev(x)), workspace=ws)
        ref = oracle.matvec(blob, bits, rows, cols, x, levels)
        w_hat = np.linalg.norm(oracle.dequantize(blob, bits, rows, cols, levels), axis=1)
        _check_fp32_product(y.cpu().numpy(), ref, w_hat, np.linalg.norm(x.astype(np.float64), axis=1))


def test_matvec_rejects_small_workspace():
    W, _, _, _ = _cq_from_oracle(2, 100, 16384, 35)
    xr = torch.zeros((1, 16384), device=DEV)
    need = cq.cq_workspace_bytes(0, W, 1)
    assert need > 0
    with pytest.raises(cq.CQError) as e:
        cq.cq_matvec(W, xr, workspace=torch.zeros(need - 16, dtype=torch.uint8, device=DEV))
    assert e.value.status == 8


def _random_cq(bits, rows, cols, cfg):
    """A full-size CQ matrix from seeded random bytes (no encoder involved):
    returns the device matrix and the host blob the oracle decodes."""
    kpad = oracle.padded_cols(cols)
    packed = cq_inputs.random_bytes(cfg, bits, rows * kpad * oracle.storage_bits(bits) // 8)
    norms = cq_inputs.random_norms(cfg, bits, rows * (kpad // 128))
    blob = np.concatenate([packed, norms])
    assert blob.size == oracle.blob_bytes(bits, 128, rows, cols)
    return cq.CQMatrix(bits, rows, cols, _to_dev(blob), _levels(bits)), blob


def _row_subset(blob, bits, rows, cols, pick):
    packed, norms = oracle.split_blob(blob, bits, rows, cols)
    return oracle.make_blob(packed[pick], norms[pick])


@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("batch", [1, 3])
def test_matvec_very_long_rows(bits, batch):
    # K = 65613 (a ragged last group): 65 (CQ2) or 129 (CQ4) table slices at batch 1 and
    # 17 matrix-core slices at batch 3, all added by the combine kernel
    rows, cols = 200, 65613
    say("matvec long rows", bits, batch)
    W, blob, levels, _ = _cq_from_oracle(bits, rows, cols, 140 + batch)
    x = cq_inputs.activations(140, bits, batch, cols)
    y = cq.cq_rotate_matvec(W, _to_dev(x)).cpu().numpy()
    ref = oracle.matvec(blob, bits, rows, cols, x, levels)
    w_hat = np.linalg.norm(oracle.dequantize(blob, bits, rows, cols, levels), axis=1)
    _check_fp32_product(y, ref, w_hat, np.linalg.norm(x.astype(np.float64), axis=1))


def _oracle_rows_parallel(fn, rows, chunk=1024, threads=16):
    """fn(r0, r1) over row chunks in a thread pool (the oracle's NumPy work
    releases the GIL); results concatenated along the last axis."""
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(threads) as ex:
        parts = list(ex.map(lambda r0: fn(r0, min(rows, r0 + chunk)), range(0, rows, chunk)))
    return parts


@pytest.mark.parametrize("bits", [1, 2, 3, 4, 5])
def test_matvec_full_size_all_rows(bits):
    # the 65536 x 16384 workload in the launch configuration the benchmark
    # times, every row against the oracle (its rotated-activation route, in
    # row chunks); CQ2 also at batch 8, binary at batch 3
    rows, cols = 65536, 16384
    say("matvec full size", bits)
    W, blob = _random_cq(bits, rows, cols, 60)
    levels = _levels(bits)
    batches = {2: (1, 8), 1: (1, 3)}.get(bits, (1,))
    xs = [cq_inputs.activations(60, 100 * b + bits, b, cols) for b in batches]
    ys = [cq.cq_matvec(W, cq.cq_rotate_acts(_to_dev(x))).cpu().numpy() for x in xs]
    del W
    torch.cuda.empty_cache()
    xall = np.concatenate(xs)
    parts = _oracle_rows_parallel(
        lambda r0, r1: oracle.matvec_rotated(blob, bits, rows, cols, xall, levels, row0=r0, row1=r1,
                                             row_norms=True), rows)
    ref = np.concatenate([p[0] for p in parts], axis=1)
    w_hat = np.concatenate([p[1] for p in parts])
    say("  oracle done")
    at = 0
    for x, y in zip(xs, ys):
        _check_fp32_product(y, ref[at:at + x.shape[0]], w_hat, np.linalg.norm(x.astype(np.float64), axis=1))
        at += x.shape[0]


def test_matvec_is_deterministic():
    W, _, _, _ = _cq_from_oracle(2, 2000, 16384, 33)
    xr = cq.cq_rotate_acts(_to_dev(cq_inputs.activations(33, 0, 1, 16384)))
    a = cq.cq_matvec(W, xr).clone()
    b = cq.cq_matvec(W, xr)
    assert torch.equal(a, b)


@pytest.mark.parametrize("bits", [1, 2, 3, 4, 5])
@pytest.mark.parametrize("rows,cols,batch", [(700, 16384, 1), (300, 5000, 1), (257, 9000, 3), (129, 1003, 8), (64, 128, 2)])
def test_rotate_matvec_equals_rotate_then_matvec(bits, rows, cols, batch):
    # the fused call rotates inside the product's kernels with the same
    # butterfly: bit-identical to cq_rotate_acts + cq_matvec, and within the
    # fp32 bar of the oracle (odd cols exercise the unvectorised loads)
    say("rotate_matvec", bits, rows, cols, batch)
    W, blob, levels, _ = _cq_from_oracle(bits, rows, cols, 80 + batch)
    x = cq_inputs.activations(81, rows, batch, cols)
    xd = _to_dev(x)
    fused = cq.cq_rotate_matvec(W, xd)
    two = cq.cq_matvec(W, cq.cq_rotate_acts(xd))
    torch.cuda.synchronize()
    assert torch.equal(fused, two)
    ref = oracle.matvec(blob, bits, rows, cols, x, levels)
    w_hat = np.linalg.norm(oracle.dequantize(blob, bits, rows, cols, levels), axis=1)
    _check_fp32_product(fused.cpu().numpy(), ref, w_hat, np.linalg.norm(x.astype(np.float64), axis=1))


def test_rotate_matvec_full_size():
    # the 65536 x 16384 CQ2 workload at batch 1 and 8, in the benchmark's
    # launch configuration, against the two-call path
    rows, cols = 65536, 16384
    say("rotate_matvec full size")
    W, _ = _random_cq(2, rows, cols, 61)
    for batch in (1, 8):
        xd = _to_dev(cq_inputs.activations(61, batch, batch, cols))
        assert torch.equal(cq.cq_rotate_matvec(W, xd), cq.cq_matvec(W, cq.cq_rotate_acts(xd)))
    del W
    torch.cuda.empty_cache()


def _oracle_check(W, blob, levels, x, y):
    ref = oracle.matvec(blob, W.bits, W.rows, W.cols, x, levels)
    w_hat = np.linalg.norm(oracle.dequantize(blob, W.bits, W.rows, W.cols, levels), axis=1)
    _check_fp32_product(y.cpu().numpy(), ref, w_hat, np.linalg.norm(x.astype(np.float64), axis=1))


@pytest.mark.parametrize("batch", [1, 3, 8])
@pytest.mark.parametrize("cols", [512, 300, 3000, 4096])
def test_rotate_multi_matvec_one_launch(batch, cols):
    # small matrices of every width sharing x: one launch per width, the
    # kernel rotating x itself; ten 2-bit matrices take two launches of at
    # most eight.  Each output equals the two-call path bit for bit (same
    # fp16 staging, scale and product order) and the oracle within the fp32 bar.
    say("multi one launch", batch, cols)
    specs = [(2, 512), (3, 256), (4, 130), (5, 37), (2, 1)] + [(2, 128 + 17 * i) for i in range(9)]
    mats = [_random_cq(bits, rows, cols, 500 + i) for i, (bits, rows) in enumerate(specs)]
    x = cq_inputs.activations(84, cols + batch, batch, cols)
    xd = _to_dev(x)
    Ws = [W for W, _ in mats]
    assert cq.cq_rotate_multi_workspace_bytes(Ws, batch) == 0
    ys = cq.cq_rotate_multi_matvec(Ws, xd)
    xr = cq.cq_rotate_acts(xd)
    for (W, blob), y in zip(mats, ys):
        assert torch.equal(y, cq.cq_matvec(W, xr)), (W.bits, W.rows)
        assert torch.equal(y, cq.cq_rotate_matvec(W, xd)), (W.bits, W.rows)
        _oracle_check(W, blob, _levels(W.bits), x, y)


@pytest.mark.parametrize("batch", [1, 4])
@pytest.mark.parametrize("cols,specs", [
    # 131073 x 512 is just over 2^26 weights: the lookup tables at batch 1,
    # the batched kernel at 4, with one shared rotation; the rest run in one
    # launch per width
    (512, [(2, 512), (4, 131073), (2, 256), (5, 300)]),
    (5000, [(2, 100), (3, 1000), (4, 2000)]),  # K beyond 4096: all share one rotation
    (640, [(1, 300), (2, 200), (1, 5000)]),     # binary matrices take the shared rotation
])
def test_rotate_multi_matvec_mixed_paths(batch, cols, specs):
    say("multi mixed", batch, cols)
    mats = [_random_cq(bits, rows, cols, 600 + i) for i, (bits, rows) in enumerate(specs)]
    x = cq_inputs.activations(85, cols + batch, batch, cols)
    xd = _to_dev(x)
    Ws = [W for W, _ in mats]
    ws = torch.full((max(cq.cq_rotate_multi_workspace_bytes(Ws, batch), 16),), 0x7F, dtype=torch.uint8, device=DEV)
    ys = cq.cq_rotate_multi_matvec(Ws, xd, workspace=ws)
    xr = cq.cq_rotate_acts(xd)
    for (W, blob), y in zip(mats, ys):
        assert torch.equal(y, cq.cq_matvec(W, xr)), (W.bits, W.rows)
        if W.rows > 20000:  # the oracle on sampled rows
            pick = cq_inputs.sample_rows(85, W.bits, W.rows, 64)
            sub = _row_subset(blob, W.bits, W.rows, cols, pick)
            ref = oracle.matvec(sub, W.bits, len(pick), cols, x, W.levels)
            w_hat = np.linalg.norm(oracle.dequantize(sub, W.bits, len(pick), cols, W.levels), axis=1)
            _check_fp32_product(y.cpu().numpy()[:, pick], ref, w_hat, np.linalg.norm(x.astype(np.float64), axis=1))
        else:
            _oracle_check(W, blob, _levels(W.bits), x, y)


def test_rotate_multi_matvec_degenerate():
    W1, _ = _random_cq(2, 64, 256, 700)
    W0 = cq.CQMatrix(2, 0, 256, torch.empty(0, dtype=torch.uint8, device=DEV), _levels(2))
    x = _to_dev(cq_inputs.activations(86, 0, 2, 256))
    ys = cq.cq_rotate_multi_matvec([W0, W1], x)
    assert ys[0].shape == (2, 0) and torch.equal(ys[1], cq.cq_rotate_matvec(W1, x))
    assert cq.cq_rotate_multi_matvec([], x) == []
    e = cq.cq_rotate_multi_matvec([W1], x[:0])
    assert e[0].shape == (0, 64)
    # cols == 0: every output is zero
    Wz = cq.CQMatrix(3, 5, 0, torch.empty(0, dtype=torch.uint8, device=DEV), _levels(3))
    y = torch.full((2, 5), float("nan"), device=DEV)
    cq.cq_rotate_multi_matvec([Wz], torch.empty((2, 0), device=DEV), outs=[y])
    assert torch.equal(y, torch.zeros_like(y))


def test_needle_layer_multi_and_graph():
    # a Needle decode layer as the library serves it: Q/K/V/gate in one
    # shared-activation call, out in its own; against the oracle, then the
    # pair captured in a HIP graph and replayed (eager work and syncs
    # between replays) bit for bit
    say("needle layer multi")
    cols = 512
    specs = [(2, 512), (2, 256), (2, 256), (2, 512)]
    mats = [_cq_from_oracle(bits, rows, cols, 710 + i)[:3] for i, (bits, rows) in enumerate(specs)]
    Wo, blob_o, lev_o, _ = _cq_from_oracle(2, 512, cols, 719)
    x_in, x_out = cq_inputs.activations(87, 0, 1, cols), cq_inputs.activations(87, 1, 1, cols)
    xi, xo = _to_dev(x_in), _to_dev(x_out)
    ys = cq.cq_rotate_multi_matvec([m[0] for m in mats], xi)
    yo = cq.cq_rotate_matvec(Wo, xo)
    for (W, blob, levels), y in zip(mats, ys):
        _oracle_check(W, blob, levels, x_in, y)
    _oracle_check(Wo, blob_o, lev_o, x_out, yo)
    ref = [y.clone() for y in ys] + [yo.clone()]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        cq.cq_rotate_multi_matvec([m[0] for m in mats], xi, outs=ys)
        cq.cq_rotate_matvec(Wo, xo, out=yo)
    for i in range(4):
        for y in ys + [yo]:
            y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(ys + [yo], ref):
            assert torch.equal(a, b), i
    del g


# ------------------------------------------------------------ W2A8 (int8)

def _check_w2a8(y, blob, bits, rows, cols, x, levels, row_ids=None):
    # integer dots exact on both sides, same int8 decisions: the GPU's fp32
    # per-group products and sums are within (groups + 8) * 2^-23 of the sum
    # of the terms' magnitudes (twice the fp32 accumulation bound)
    xq, sx = oracle.quantize_acts_int8(oracle.rotate_acts_fp32(x))
    terms = oracle.w2a8_group_terms(blob, bits, rows, cols, xq, sx, levels, row_ids=row_ids)
    ref = terms.sum(-1)
    bound = (terms.shape[-1] + 8) * 2.0 ** -23 * np.abs(terms).sum(-1) + 1e-30
    err = np.abs(y.astype(np.float64) - ref)
    assert np.all(err <= bound), f"max err/bound {np.max(err / bound):.3g}"


def test_rotation_is_the_oracle_butterfly_bit_for_bit():
    # the int8 decisions of W2A8 take the fp32 rotation; the GPU's butterfly
    # and the oracle's fp32 butterfly must agree in every bit
    for batch, cols in ((1, 512), (3, 1000), (2, 16384)):
        x = cq_inputs.activations(90, cols, batch, cols)
        got = cq.cq_rotate_acts(_to_dev(x)).cpu().numpy()
        assert np.array_equal(got.view(np.uint32), oracle.rotate_acts_fp32(x).view(np.uint32)), (batch, cols)


@pytest.mark.parametrize("batch,cols,offset", [
    (1, 16384, 0), (3, 1000, 0), (11, 300, 1), (8, 6528, 0), (2, 128, 1), (1, 1, 0),
])
def test_quantize_acts_int8_is_the_oracle_bit_for_bit(batch, cols, offset):
    # the int8 activations and their scales: every byte and every bit of the
    # scales as the oracle's (same fp32 rotation, IEEE division, half-even);
    # offset 1 makes x unaligned for vector loads
    say("quantize acts int8", batch, cols, offset)
    x = cq_inputs.activations(96, cols, batch, cols)
    x[0, : min(cols, 128)] = 0.0  # an all-zero group: scale 0, codes 0
    if batch > 2:
        x[2, :5] *= 1e4  # a group dominated by a few values
    buf = torch.zeros(batch * cols + offset, dtype=torch.float32, device=DEV)
    xd = buf[offset:].view(batch, cols)
    xd.copy_(_to_dev(x))
    xq, sx = cq.cq_quantize_acts_int8(xd)
    want_q, want_sx = oracle.quantize_acts_int8(oracle.rotate_acts_fp32(x))
    assert np.array_equal(xq.cpu().numpy().astype(np.int64), want_q)
    assert np.array_equal(sx.cpu().numpy().view(np.uint32), want_sx.view(np.uint32))


@pytest.mark.parametrize("bits", [1, 2, 3, 4, 5])
@pytest.mark.parametrize("rows,cols,batch", [(700, 2048, 1), (129, 8192, 2), (64, 640, 8), (300, 16384, 1)])
def test_matvec_w2a8_quantized_any_int8(bits, rows, cols, batch):
    # the product alone on int8 activations the oracle draws (the full range,
    # -128 included) and arbitrary positive scales; same inputs on both sides
    say("w2a8 quantized", bits, rows, cols, batch)
    W, blob = _random_cq(bits, rows, cols, 97 + batch)
    levels = _levels(bits)
    kpad = oracle.padded_cols(cols)
    rng = np.random.default_rng(rows + bits)
    xq = rng.integers(-128, 128, size=(batch, kpad)).astype(np.int8)
    sx = rng.uniform(1e-3, 2e-2, size=(batch, kpad // 128)).astype(np.float32)
    y = cq.cq_matvec_w2a8_quantized(W, _to_dev(xq), _to_dev(sx)).cpu().numpy()
    terms = oracle.w2a8_group_terms(blob, bits, rows, cols, xq, sx, levels)
    bound = (terms.shape[-1] + 8) * 2.0 ** -23 * np.abs(terms).sum(-1) + 1e-30
    err = np.abs(y.astype(np.float64) - terms.sum(-1))
    assert np.all(err <= bound), f"max err/bound {np.max(err / bound):.3g}"


@pytest.mark.parametrize("bits", [1, 2, 3, 4, 5])
@pytest.mark.parametrize("rows,cols,batch", [
    (512, 512, 1), (300, 1000, 3), (257, 2048, 2), (64, 640, 8), (1, 128, 1),
    (1000, 16384, 1), (9, 16384, 2), (33, 6528, 8), (130, 5000, 4),
    (100, 768, 1), (45, 1536, 2), (77, 4096, 1), (5, 8192, 2),
    (20, 16384, 3), (17, 14336, 4), (3, 27264, 1),
])
def test_matvec_w2a8(bits, rows, cols, batch):
    say("w2a8", bits, rows, cols, batch)
    W, blob = _random_cq(bits, rows, cols, 91 + batch)
    levels = _levels(bits)
    x = cq_inputs.activations(92, rows, batch, cols)
    y = cq.cq_matvec_w2a8(W, _to_dev(x)).cpu().numpy()
    _check_w2a8(y, blob, bits, rows, cols, x, levels)


@pytest.mark.parametrize("bits", [1, 2, 4])
def test_matvec_w2a8_full_size_sampled_rows(bits):
    # the 65536 x 16384 workload in the benchmark's launch configuration;
    # the oracle on sampled rows
    rows, cols = 65536, 16384
    say("w2a8 full size", bits)
    W, blob = _random_cq(bits, rows, cols, 93)
    levels = _levels(bits)
    pick = cq_inputs.sample_rows(93, bits, rows, 48)
    sub = _row_subset(blob, bits, rows, cols, pick)
    x = cq_inputs.activations(93, bits, 1, cols)
    y = cq.cq_matvec_w2a8(W, _to_dev(x)).cpu().numpy()
    _check_w2a8(y[:, pick], sub, bits, len(pick), cols, x, levels)
    del W
    torch.cuda.empty_cache()


def test_matvec_w2a8_degenerate_and_limits():
    W, blob = _random_cq(2, 70, 256, 94)
    x = _to_dev(cq_inputs.activations(94, 0, 2, 256))
    assert cq.cq_matvec_w2a8(W, x[:0]).shape == (0, 70)
    # an all-zero activation: every group scale is 0 and so is y
    assert torch.equal(cq.cq_matvec_w2a8(W, torch.zeros_like(x)), torch.zeros((2, 70), device=DEV))
    Wz = cq.CQMatrix(4, 3, 0, torch.empty(0, dtype=torch.uint8, device=DEV), _levels(4))
    y = torch.full((2, 3), float("nan"), device=DEV)
    cq.cq_matvec_w2a8(Wz, torch.empty((2, 0), device=DEV), out=y)
    assert torch.equal(y, torch.zeros_like(y))
    Wb, _ = _random_cq(2, 8, 16384, 95)
    with pytest.raises(cq.CQError) as e:
        cq.cq_matvec_w2a8(Wb, torch.zeros((4, 16384), device=DEV))
    assert e.value.status == 4  # CQ_ERR_SHAPE: the quantised activation exceeds one workgroup's LDS
    a = cq.cq_matvec_w2a8(W, x).clone()
    assert torch.equal(a, cq.cq_matvec_w2a8(W, x))  # deterministic


# ------------------------------------------------------------- row gather

@pytest.mark.parametrize("bits", [1, 2, 3, 4, 5])
@pytest.mark.parametrize("rows,cols", [(8192, 512), (300, 1000), (17, 128), (5, 16384), (40, 77)])
@pytest.mark.parametrize("odt", [torch.float32, torch.bfloat16, torch.float16])
def test_gather_rows(bits, rows, cols, odt):
    # the embedding lookup of a tied CQ matrix: rows by id, repeated and
    # out-of-range ids included (NaN rows), against the oracle
    say("gather", bits, rows, cols, odt)
    W, blob = _random_cq(bits, rows, cols, 97)
    levels = _levels(bits)
    rng = np.random.default_rng(bits * 1000 + rows)
    ids = np.concatenate([rng.integers(0, rows, size=37), [0, rows - 1, rows - 1, -1, rows]])
    got = cq.cq_gather_rows(W, _to_dev(ids.astype(np.int64)), odt).float().cpu().numpy().astype(np.float64)
    ref = oracle.gather_rows(blob, bits, rows, cols, ids, levels)
    bad = (ids < 0) | (ids >= rows)
    assert np.all(np.isnan(got[bad])) and not np.any(np.isnan(got[~bad]))
    # fp32: the rounding of the level x norm products and of the butterfly's
    # sums, within 2^-16 of the group's L1 norm / sqrt(128); 16-bit outputs add
    # one rounding of the value (2^-8 bf16, 2^-11 fp16)
    packed, norms = oracle.split_blob(blob, bits, rows, cols)
    kpad = oracle.padded_cols(cols)
    vals = oracle.level_values(oracle.unpack_codes(packed[ids[~bad]], bits, kpad), bits, levels)
    l1 = np.abs(vals).reshape(-1, kpad // 128, 128).sum(-1) * norms[ids[~bad]].astype(np.float64)
    bound = 2.0 ** -16 * np.repeat(l1, 128, axis=1)[:, :cols] / np.sqrt(128)
    rel = {torch.float32: 0.0, torch.bfloat16: 2.0 ** -8, torch.float16: 2.0 ** -11}[odt]
    bound = bound + rel * np.abs(ref[~bad])
    assert np.all(np.abs(got[~bad] - ref[~bad]) <= bound + 1e-30)


def test_gather_rows_empty_and_consistent_with_the_product():
    W, blob = _random_cq(4, 64, 300, 98)
    assert cq.cq_gather_rows(W, torch.empty(0, dtype=torch.int64, device=DEV)).shape == (0, 300)
    ids = torch.arange(64, dtype=torch.int64, device=DEV)
    dense = cq.cq_gather_rows(W, ids)
    x = _to_dev(cq_inputs.activations(98, 0, 2, 300))
    # the gathered dense matrix reproduces the product of the packed one,
    # within the matvec's fp32-path bar (1e-4 * |w_hat_row| * |x|)
    y = cq.cq_matvec(W, cq.cq_rotate_acts(x))
    bound = 1e-4 * torch.outer(x.norm(dim=1), dense.norm(dim=1))
    assert torch.all((x @ dense.T - y).abs() <= bound)


def test_needle_decode_sweep_shapes():
    # the Needle-shaped decode workload at batch 1: 27 layers of Q 512x512,
    # K and V 256x512, gate and out 512x512 at CQ2 -- one rotated activation
    # feeds Q/K/V/gate, another feeds out -- and the tied 8192x512 logits at
    # CQ4; every product against the oracle
    say("needle decode sweep")
    cols = 512
    layer_mats = [("q", 512), ("k", 256), ("v", 256), ("gate", 512), ("out", 512)]
    for layer in range(27):
        x_in = cq_inputs.activations(2, 2 * layer, 1, cols)
        x_out = cq_inputs.activations(2, 2 * layer + 1, 1, cols)
        xr_in, xr_out = cq.cq_rotate_acts(_to_dev(x_in)), cq.cq_rotate_acts(_to_dev(x_out))
        for t, (name, rows) in enumerate(layer_mats):
            W, blob, levels, _ = _cq_from_oracle(2, rows, cols, 1000 + 8 * layer + t)
            x, xr = (x_out, xr_out) if name == "out" else (x_in, xr_in)
            y = cq.cq_matvec(W, xr).cpu().numpy()
            w_hat = np.linalg.norm(oracle.dequantize(blob, 2, rows, cols, levels), axis=1)
            _check_fp32_product(y, oracle.matvec(blob, 2, rows, cols, x, levels), w_hat,
                                np.linalg.norm(x.astype(np.float64), axis=1))
    W, blob, levels, _ = _cq_from_oracle(4, 8192, cols, 1999)
    x = cq_inputs.activations(2, 99, 1, cols)
    y = cq.cq_matvec(W, cq.cq_rotate_acts(_to_dev(x))).cpu().numpy()
    w_hat = np.linalg.norm(oracle.dequantize(blob, 4, 8192, cols, levels), axis=1)
    _check_fp32_product(y, oracle.matvec(blob, 4, 8192, cols, x, levels), w_hat,
                        np.linalg.norm(x.astype(np.float64), axis=1))


def test_needle_prefill_shapes():
    # the prefill workload: 2048 fp16 tokens x 512, rotated once to bf16,
    # through the 512x512 and 256x512 CQ2 and the 8192x512 CQ4 matrices
    say("needle prefill")
    cols, m = 512, 2048
    X = cq_inputs.activations(3, 0, m, cols, "f16")
    xr = cq.cq_rotate_acts(_to_dev(X, torch.float16), torch.bfloat16)
    xn = np.linalg.norm(X.astype(np.float64), axis=1)
    for t, (bits, rows) in enumerate(((2, 512), (2, 256), (4, 8192))):
        W, blob, levels, _ = _cq_from_oracle(bits, rows, cols, 3000 + t)
        got = cq.cq_gemm(W, xr).cpu().numpy().astype(np.float64)
        w_hat = np.linalg.norm(oracle.dequantize(blob, bits, rows, cols, levels), axis=1)
        _check_fp32_product(got, oracle.gemm(blob, bits, rows, cols, X, levels), w_hat, xn, tol=1e-2, min_cos=0.9999)
        # the bf16-operand variant: at 16.7 M outputs the tail includes the
        # few activations whose bf16 rounding differs between the GPU's fp32
        # rotation and the oracle's float64 one (one bf16 ulp, 2^-8), so the
        # tight bound is 2e-4 here rather than the 1e-4 of the small cases
        _check_fp32_product(got, oracle.gemm_bf16(blob, bits, rows, cols, X, levels), w_hat, xn,
                            tol=2e-4, min_cos=0.99999)


def test_matvec_step_replays_in_a_graph():
    # rotate + matvec captured once in a HIP graph (no memset nodes: every
    # node is a kernel); each replay, with eager work and synchronisation
    # between replays, must equal the eager result bit for bit
    for bits, batch, rows, cols in ((2, 1, 600, 16384), (4, 3, 700, 5000)):
        W, _, _, _ = _cq_from_oracle(bits, rows, cols, 70 + batch)
        x = _to_dev(cq_inputs.activations(70, bits, batch, cols))
        kpad = -(-cols // 128) * 128
        xr = torch.empty((batch, kpad), device=DEV)
        y = torch.empty((batch, rows), device=DEV)
        ws = torch.empty(max(cq.cq_workspace_bytes(cq.OP_MATVEC, W, batch), 16), dtype=torch.uint8, device=DEV)
        cq.cq_rotate_acts(x, out=xr)
        cq.cq_matvec(W, xr, out=y, workspace=ws)
        torch.cuda.synchronize()
        ref = y.clone()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            cq.cq_rotate_acts(x, out=xr)
            cq.cq_matvec(W, xr, out=y, workspace=ws)
        for i in range(4):
            y.fill_(float("nan"))
            xr.zero_()
            ws.fill_(0x7F)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(y, ref), (bits, batch, i)
        del g


# --------------------------------------------------------------------- GEMM

@pytest.mark.parametrize("bits", [1, 2, 3, 4, 5])
@pytest.mark.parametrize("m,rows,cols", [(1, 1, 128), (7, 100, 1000), (300, 200, 512), (130, 257, 640), (64, 129, 2048)])
def test_gemm(bits, m, rows, cols):
    say("gemm", bits, m, rows, cols)
    W, blob, levels, _ = _cq_from_oracle(bits, rows, cols, 40 + m)
    X = cq_inputs.activations(41, rows, m, cols, "f16")
    xr = cq.cq_rotate_acts(_to_dev(X, torch.float16), torch.bfloat16)
    C = cq.cq_gemm(W, xr)
    torch.cuda.synchronize()
    got = C.cpu().numpy().astype(np.float64)
    w_hat = np.linalg.norm(oracle.dequantize(blob, bits, rows, cols, levels), axis=1)
    xn = np.linalg.norm(X.astype(np.float64), axis=1)
    # the dense float64 product, to the bf16 bar
    _check_fp32_product(got, oracle.gemm(blob, bits, rows, cols, X, levels), w_hat, xn, tol=1e-2, min_cos=0.9999)
    # the same roundings as the matrix-core path (bf16 operands), much tighter
    _check_fp32_product(got, oracle.gemm_bf16(blob, bits, rows, cols, X, levels), w_hat, xn, tol=1e-4, min_cos=0.99999)


@pytest.mark.parametrize("bits", [4, 3])
def test_gemm_full_size_every_tile(bits):
    # M = 4096, N = K = 16384: C on a strided grid of 241 x 713 outputs (steps
    # 17 and 23, prime to the 256 x 256 tile, the 128 x 64 wave tile and the
    # 16 x 16 MFMA block, so every tile and every position class in them is
    # hit; every output runs through all K stages) against the oracle
    m, rows, cols = 4096, 16384, 16384
    say("gemm full size", bits)
    W, blob = _random_cq(bits, rows, cols, 61)
    levels = _levels(bits)
    X = cq_inputs.activations(61, bits, m, cols, "bf16")
    xr = cq.cq_rotate_acts(_to_dev(X, torch.bfloat16), torch.bfloat16)
    C = cq.cq_gemm(W, xr)
    mp = np.arange(0, m, 17)
    pick = np.arange(0, rows, 23)
    got = C[torch.from_numpy(mp).to(DEV)][:, torch.from_numpy(pick).to(DEV)].cpu().numpy().astype(np.float64)
    del C, W, xr
    torch.cuda.empty_cache()
    assert {(int(a) // 256, int(b) // 256) for a in mp for b in pick} == {(i, j) for i in range(16) for j in range(64)}
    sub = _row_subset(blob, bits, rows, cols, pick)
    w_hat = np.linalg.norm(oracle.dequantize(sub, bits, len(pick), cols, levels), axis=1)
    xn = np.linalg.norm(X[mp].astype(np.float64), axis=1)
    _check_fp32_product(got, oracle.gemm(sub, bits, len(pick), cols, X[mp], levels), w_hat, xn,
                        tol=1e-2, min_cos=0.9999)
    _check_fp32_product(got, oracle.gemm_bf16(sub, bits, len(pick), cols, X[mp], levels), w_hat, xn,
                        tol=1e-4, min_cos=0.99999)


@pytest.mark.parametrize("bits", [2, 4])
def test_gemm_large_tiles_ragged(bits):
    # 258 tiles of 256 x 256, so the large-tile kernel runs: N = 32900 leaves
    # a ragged last N-tile (132 of 256 rows), K = 640 five groups (ten stages)
    m, rows, cols = 512, 32900, 640
    say("gemm large tiles ragged", bits, m, rows, cols)
    W, blob, levels, _ = _cq_from_oracle(bits, rows, cols, 90 + bits)
    X = cq_inputs.activations(91, bits, m, cols, "f16")
    xr = cq.cq_rotate_acts(_to_dev(X, torch.float16), torch.bfloat16)
    got = cq.cq_gemm(W, xr).cpu().numpy().astype(np.float64)
    w_hat = np.linalg.norm(oracle.dequantize(blob, bits, rows, cols, levels), axis=1)
    xn = np.linalg.norm(X.astype(np.float64), axis=1)
    _check_fp32_product(got, oracle.gemm(blob, bits, rows, cols, X, levels), w_hat, xn, tol=1e-2, min_cos=0.9999)
    _check_fp32_product(got, oracle.gemm_bf16(blob, bits, rows, cols, X, levels), w_hat, xn, tol=1e-4, min_cos=0.99999)


def test_gemm_degenerate_shapes():
    levels = cq_inputs.codebook(4)
    W = cq.CQMatrix(4, 6, 0, torch.zeros(0, dtype=torch.uint8, device=DEV), levels)
    C = torch.full((3, 6), 5.0, device=DEV)
    cq.cq_gemm(W, torch.zeros((3, 0), dtype=torch.bfloat16, device=DEV), out=C)
    assert torch.all(C == 0)
    W1, _, _, _ = _cq_from_oracle(4, 4, 256, 42)
    assert cq.cq_gemm(W1, torch.zeros((0, 256), dtype=torch.bfloat16, device=DEV)).shape == (0, 4)


# ------------------------------------------------------------------ encoder

def _encoder_agreement(bits, w, blob_gpu, levels):
    rows, cols = w.shape
    codes_o, norms_o = oracle.encode(w, bits, levels)
    packed_g, norms_g = oracle.split_blob(blob_gpu, bits, rows, cols)
    codes_g = oracle.unpack_codes(packed_g, bits, codes_o.shape[1])
    same = codes_g == codes_o
    frac = np.mean(same)
    assert frac >= 0.9999, frac
    if not np.all(same):
        # every mismatch must sit within 1e-5 of a decision boundary
        kpad = codes_o.shape[1]
        wp = np.zeros((rows, kpad), np.float32)
        wp[:, :cols] = w
        r32 = oracle.rotate_fp32(wp.reshape(rows, -1, 128))
        n32 = np.sqrt(np.sum(r32.astype(np.float64) ** 2, axis=-1)).astype(np.float32)
        u = (r32 / np.maximum(n32, np.float32(1e-12))[..., None]).reshape(rows, kpad).astype(np.float64)
        lv = oracle.codebook_for(bits, levels).astype(np.float64)
        mids = (lv[:-1] + lv[1:]) / 2
        d = np.min(np.abs(u[~same][:, None] - mids[None, :]), axis=1)
        assert np.all(d <= 1e-5), np.max(d)
    assert np.array_equal(norms_g.view(np.uint16), norms_o.view(np.uint16))
    return frac


# binary (1) and ternary (5) levels are analytic: one code book kind each
@pytest.mark.parametrize("bits,kind", [(1, "empirical"), (5, "empirical")]
                         + [(b, k) for b in (2, 3, 4) for k in ("empirical", "gaussian")])
@pytest.mark.parametrize("rows,cols", [(512, 512), (37, 1000), (3, 16384), (1, 1)])
def test_quantize(bits, kind, rows, cols):
    say("quantize", bits, kind, rows, cols)
    levels = _levels(bits, kind)
    w = cq_inputs.master(50, bits, rows, cols)
    W = cq.cq_quantize(_to_dev(w), bits, levels)
    torch.cuda.synchronize()
    blob_g = W.blob.cpu().numpy()
    assert blob_g.size == oracle.blob_bytes(bits, 128, rows, cols)
    frac = _encoder_agreement(bits, w, blob_g, levels)
    say("  identical index fraction", frac)


@pytest.mark.parametrize("bits", [4, 3])
def test_quantize_full_size_all_rows(bits):
    # the 16384 x 16384 encode: every row of the blob against the oracle
    # encoder (in row chunks: rows are encoded independently)
    rows, cols = 16384, 16384
    say("quantize full size", bits)
    levels = _levels(bits)
    w = cq_inputs.master(63, bits, rows, cols)
    W = cq.cq_quantize(_to_dev(w), bits, levels)
    blob_g = W.blob.cpu().numpy()
    del W
    torch.cuda.empty_cache()
    fracs = _oracle_rows_parallel(
        lambda r0, r1: _encoder_agreement(bits, w[r0:r1], _row_subset(blob_g, bits, rows, cols, np.arange(r0, r1)),
                                          levels), rows)
    say("  identical index fraction", min(fracs))


def test_quantize_special_groups():
    # zero groups, a constant group (exact ties), a huge group (fp16 overflow), tiny values
    levels = np.array([-0.25, -0.125, 0.125, 0.25], np.float32)
    w = np.zeros((4, 256), np.float32)
    w[1, :128] = 0.03
    w[2, :128] = 1.0e4
    w[3, :] = 1e-30
    W = cq.cq_quantize(_to_dev(w), 2, levels)
    blob_g = W.blob.cpu().numpy()
    assert np.array_equal(blob_g, oracle.quantize(w, 2, levels))


def test_quantize_close_levels_count_the_midpoints():
    # a code book with two midpoints 1e-6 / sqrt(128) apart: too close for the
    # encoder's bucket lookup of the decision (one threshold per bucket), so
    # it counts the midpoints; the decisions are the oracle's either way
    say("quantize close levels")
    s = 1.0 / np.sqrt(128.0)
    levels = (np.array([-1.0, -0.5, -0.25, 0.0, 1e-6, 2e-6, 0.5, 1.0]) * s).astype(np.float32)
    w = cq_inputs.master(64, 3, 64, 512)
    W = cq.cq_quantize(_to_dev(w), 3, levels)
    _encoder_agreement(3, w, W.blob.cpu().numpy(), levels)


def test_concurrent_host_threads_on_their_own_streams():
    # the launchers' host-side caches are shared by every thread: calls from
    # several threads at once, each on its own stream, give the results of
    # the same calls made one by one (every kernel here is deterministic)
    import threading
    say("threads")
    mats = [_random_cq(bits, rows, 4096, 800 + i)[0] for i, (bits, rows) in enumerate([(2, 3000), (4, 700), (1, 5000), (3, 257)])]
    x = _to_dev(cq_inputs.activations(800, 0, 2, 4096))
    ref = [(cq.cq_rotate_matvec(W, x).clone(), cq.cq_matvec_w2a8(W, x[:1]).clone()) for W in mats]
    torch.cuda.synchronize()
    errors = []

    def worker(i):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                W = mats[i]
                for _ in range(20):
                    a = cq.cq_rotate_matvec(W, x)
                    b = cq.cq_matvec_w2a8(W, x[:1])
                s.synchronize()
                if not (torch.equal(a, ref[i][0]) and torch.equal(b, ref[i][1])):
                    errors.append(i)
        except Exception as e:  # reported below
            errors.append(repr(e))

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(mats))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
