"""HIP-graph capture of the calls a decode or prefill loop replays.

Each graph is captured once, after one eager call.  Before every replay new
inputs are written into the captured buffers, the same calls run eagerly on
them (the reference), the outputs are overwritten, and the replay must then
write the eager outputs again, bit for bit.  The library records no memset
nodes: every node is a kernel.
"""
import numpy as np
import pytest
import torch

import cq_inputs

pytestmark = pytest.mark.gpu

cq = pytest.importorskip("hadamard_rotated_codebook_amd")
DEV = torch.device("cuda:0")


def say(*a):
    print(*a, flush=True)


def _gen(seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    return g


def _encode(bits, rows, cols, seed):
    w = torch.randn((rows, cols), device=DEV, generator=_gen(seed)) * 0.02
    return cq.cq_quantize(w, bits, cq_inputs.codebook(bits))


def _check_replays(run, inputs, draw, outputs, state=(), replays=3):
    """run(): enqueue the calls; inputs: the tensors the calls read, refilled
    by draw(i) before replay i; outputs: the tensors they write; state:
    tensors the calls both read and write (restored before each replay to
    their contents before the eager call)."""
    run()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    torch.cuda.synchronize()
    for i in range(replays):
        for t, v in zip(inputs, draw(i)):
            t.copy_(v)
        saved = [s.clone() for s in state]
        run()
        torch.cuda.synchronize()
        want = [o.clone() for o in outputs] + [s.clone() for s in state]
        for o in outputs:
            o.fill_(float("nan")) if o.is_floating_point() else o.fill_(0x5A)
        for s, v in zip(state, saved):
            s.copy_(v)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = list(outputs) + list(state)
        for k, (a, b) in enumerate(zip(got, want)):
            assert torch.equal(a, b), f"replay {i}, tensor {k}"
    del g


def test_prefill_gemm_replays():
    # the prefill products of a 512-wide layer and the tied logits: 2048
    # rotated bf16 tokens through 512 x 512 CQ2 (128 x 128 tiles) and
    # 8192 x 512 CQ4 (256 x 256 tiles)
    say("graph: prefill gemm")
    Wq, Wl = _encode(2, 512, 512, 1), _encode(4, 8192, 512, 2)
    xr = torch.empty((2048, 512), dtype=torch.bfloat16, device=DEV)
    cq_, cl = torch.empty((2048, 512), device=DEV), torch.empty((2048, 8192), device=DEV)

    def run():
        cq.cq_gemm(Wq, xr, out=cq_)
        cq.cq_gemm(Wl, xr, out=cl)

    g = _gen(3)
    _check_replays(run, [xr], lambda i: [torch.randn(xr.shape, device=DEV, generator=g).to(torch.bfloat16)],
                   [cq_, cl])


@pytest.mark.parametrize("bits", [2, 4])
def test_kv_decode_step_replays(bits):
    # one decode step of a 256-token KV cache (8 query heads over 4 KV heads
    # of 64): append token t's key and value rows, then attend to t + 1 rows;
    # the replay has to rewrite row t of both caches
    say("graph: kv step", bits)
    rows, nq, nkv, hd, t = 256, 8, 4, 64, 200
    cols = nkv * hd
    mk = cq.CQMatrix(bits, rows, cols, torch.zeros(cq.cq_blob_bytes(bits, rows, cols), dtype=torch.uint8,
                                                    device=DEV), cq_inputs.codebook(bits))
    mv = cq.CQMatrix(bits, rows, cols, torch.zeros_like(mk.blob), cq_inputs.codebook(bits))
    g = _gen(10 + bits)
    cq.cq_kv_append(mk, mv, torch.randn((t, cols), device=DEV, generator=g),
                    torch.randn((t, cols), device=DEV, generator=g), 0)
    k, v = torch.empty((1, cols), device=DEV), torch.empty((1, cols), device=DEV)
    q, out = torch.empty((nq, hd), device=DEV), torch.empty((nq, hd), device=DEV)
    k.copy_(torch.randn(k.shape, device=DEV, generator=g))
    v.copy_(torch.randn(v.shape, device=DEV, generator=g))
    q.copy_(torch.randn(q.shape, device=DEV, generator=g))

    def run():
        cq.cq_kv_append(mk, mv, k, v, t)
        cq.cq_kv_attention(mk, mv, q, nkv, tokens=t + 1, out=out)

    _check_replays(run, [k, v, q],
                   lambda i: [torch.randn(k.shape, device=DEV, generator=g),
                              torch.randn(v.shape, device=DEV, generator=g),
                              torch.randn(q.shape, device=DEV, generator=g)],
                   [out], state=[mk.blob, mv.blob])


@pytest.mark.parametrize("bits,batch", [(2, 1), (4, 2), (1, 1)])
def test_w2a8_replays(bits, batch):
    say("graph: w2a8", bits, batch)
    W = _encode(bits, 4096, 4096, 20 + bits)
    x, y = torch.empty((batch, 4096), device=DEV), torch.empty((batch, 4096), device=DEV)
    ws = torch.empty(max(cq.cq_workspace_bytes(cq.OP_W2A8, W, batch), 16), dtype=torch.uint8, device=DEV)
    g = _gen(30 + bits)
    x.copy_(torch.randn(x.shape, device=DEV, generator=g))
    _check_replays(lambda: cq.cq_matvec_w2a8(W, x, out=y, workspace=ws), [x],
                   lambda i: [torch.randn(x.shape, device=DEV, generator=g)], [y])


@pytest.mark.parametrize("bits,batch", [(2, 1), (4, 3)])
def test_noalloc_replays(bits, batch):
    # the entry point for callers that cannot allocate, under capture; its
    # replays also equal the workspace call on the same inputs
    say("graph: noalloc", bits, batch)
    W = _encode(bits, 8192, 4096, 40 + bits)
    x, y = torch.empty((batch, 4096), device=DEV), torch.empty((batch, 8192), device=DEV)
    g = _gen(50 + bits)
    x.copy_(torch.randn(x.shape, device=DEV, generator=g))
    _check_replays(lambda: cq.cq_rotate_matvec_noalloc(W, x, y), [x],
                   lambda i: [torch.randn(x.shape, device=DEV, generator=g)], [y])
    ws = torch.empty(cq.cq_workspace_bytes(cq.OP_ROTATE_MATVEC, W, batch) + 16, dtype=torch.uint8, device=DEV)
    assert torch.equal(y, cq.cq_rotate_matvec(W, x, workspace=ws))
    assert np.isfinite(y.cpu().numpy()).all()
