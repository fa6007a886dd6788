"""GPU parity of the CQ-quantised KV cache calls against the oracle
(oracle/kv.py): appending rows to a cache (cq_quantize_rows), attention
scores (cq_kv_scores) and the value-side product (cq_matvec_t), then one
decode attention step over a 256-token window with the Needle 2 geometry
(8 query heads over 4 KV heads of 64)."""
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


def _levels(bits):
    return None if bits in (1, 5) else cq_inputs.codebook(bits)


def _empty(bits, rows, cols):
    n = cq.cq_blob_bytes(bits, rows, cols)
    return cq.CQMatrix(bits, rows, cols, torch.zeros(n, dtype=torch.uint8, device=DEV), _levels(bits))


def _codes_agree(blob, ref, bits, rows, cols):
    p, n = oracle.split_blob(blob, bits, rows, cols)
    pr, nr = oracle.split_blob(ref, bits, rows, cols)
    same = np.mean(oracle.unpack_codes(p, bits, cols) == oracle.unpack_codes(pr, bits, cols))
    return same, np.array_equal(n.view(np.uint16), nr.view(np.uint16))


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 1])
def test_quantize_rows_appends_like_whole_encoding(bits):
    tokens, kv = 256, 256
    say("kv append", bits)
    k = cq_inputs.master(70, bits, tokens, kv, sigma=1.0)
    kd = torch.from_numpy(k).to(DEV)
    whole = cq.cq_quantize(kd, bits, _levels(bits)).blob.cpu().numpy()
    cache = _empty(bits, tokens, kv)
    for a, b in [(0, 1), (1, 17), (17, 100), (100, 250), (250, 256)]:
        cq.cq_quantize_rows(cache, kd[a:b], a)
    torch.cuda.synchronize()
    assert np.array_equal(cache.blob.cpu().numpy(), whole)
    # and the oracle's encoder (indices: >= 99.99 % identical, norms equal)
    same, norms_equal = _codes_agree(whole, oracle.quantize(k, bits, _levels(bits)), bits, tokens, kv)
    assert same >= 0.9999 and norms_equal
    # ring order: the window wraps, later rows overwrite the oldest
    k2 = cq_inputs.master(71, bits, 8, kv, sigma=1.0)
    cq.cq_quantize_rows(cache, torch.from_numpy(k2[:5]).to(DEV), 251)
    cq.cq_quantize_rows(cache, torch.from_numpy(k2[5:]).to(DEV), 0)
    k3 = k.copy()
    k3[251:] = k2[:5]
    k3[:3] = k2[5:]
    torch.cuda.synchronize()
    want = cq.cq_quantize(torch.from_numpy(k3).to(DEV), bits, _levels(bits)).blob.cpu().numpy()
    assert np.array_equal(cache.blob.cpu().numpy(), want)


def _bar(y, ref, bound, what):
    y = np.asarray(y, dtype=np.float64)
    r = np.max(np.abs(y - ref) / np.maximum(bound, 1e-300))
    assert r <= 1.0, f"{what}: max err/bound {r:.3g}"


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 1])
@pytest.mark.parametrize("nq,nkv,hd,tokens", [(8, 4, 64, 256), (12, 2, 48, 200), (4, 1, 128, 1000), (8, 8, 64, 33)])
def test_kv_scores(bits, nq, nkv, hd, tokens):
    say("kv scores", bits, nq, nkv, hd, tokens)
    levels = _levels(bits)
    k = cq_inputs.master(72, bits, tokens, nkv * hd, sigma=1.0)
    blob = oracle.quantize(k, bits, levels)
    K = cq.CQMatrix(bits, tokens, nkv * hd, torch.from_numpy(blob).to(DEV), levels)
    k_hat = oracle.dequantize(blob, bits, tokens, nkv * hd, levels)
    # random queries, and queries equal to cached keys' head slices (every
    # term of a score of the same sign)
    qr = cq_inputs.activations(72, bits, nq, hd)
    qa = np.stack([k_hat[(37 * h) % tokens, oracle.kv_head_of(h, nq, nkv) * hd:][:hd] for h in range(nq)])
    for q in (qr, qa.astype(np.float32)):
        s = cq.cq_kv_scores(K, torch.from_numpy(np.ascontiguousarray(q)).to(DEV), nkv).cpu().numpy()
        ref = oracle.kv_scores(blob, bits, tokens, nkv, hd, q, levels)
        bound = 1e-4 * np.outer(np.linalg.norm(q.astype(np.float64), axis=1), np.linalg.norm(k_hat, axis=1))
        _bar(s, ref, bound, "cq_kv_scores")


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 1])
@pytest.mark.parametrize(
    "rows,cols,batch",
    # one row chunk of the kernel (up to 1024 rows), then 2 and 3 chunks (partial sums + combine)
    [(256, 256, 8), (1000, 384, 3), (64, 128, 1), (65, 200, 2), (300, 4096, 5), (1025, 128, 1), (2048, 256, 8), (2500, 384, 3)],
)
def test_matvec_t(bits, rows, cols, batch):
    say("matvec_t", bits, rows, cols, batch)
    levels = _levels(bits)
    w = cq_inputs.master(73, bits, rows, cols)
    blob = oracle.quantize(w, bits, levels)
    W = cq.CQMatrix(bits, rows, cols, torch.from_numpy(blob).to(DEV), levels)
    p = cq_inputs.activations(73, bits, batch, rows)
    out = cq.cq_matvec_t(W, torch.from_numpy(p).to(DEV)).cpu().numpy()
    ref = oracle.matvec_t(blob, bits, rows, cols, p, levels)
    col_norms = np.linalg.norm(oracle.dequantize(blob, bits, rows, cols, levels)[:, :cols], axis=0)
    bound = 1e-4 * np.outer(np.linalg.norm(p.astype(np.float64), axis=1), col_norms)
    _bar(out, ref, bound, "cq_matvec_t")


def test_matvec_t_degenerate():
    levels = _levels(2)
    W0 = _empty(2, 0, 256)  # no rows: the product is zero
    out = torch.full((2, 256), 5.0, device=DEV)
    cq.cq_matvec_t(W0, torch.zeros((2, 0), device=DEV), out=out)
    torch.cuda.synchronize()
    assert torch.all(out == 0)
    W = cq.CQMatrix(2, 3, 0, torch.zeros(0, dtype=torch.uint8, device=DEV), levels)
    assert cq.cq_matvec_t(W, torch.zeros((2, 3), device=DEV)).shape == (2, 0)


@pytest.mark.parametrize("kv_bits", [2, 3, 4])
def test_decode_attention_step(kv_bits):
    # Needle 2 geometry: 8 query heads over 4 KV heads of 64, a 256-token
    # window used as a ring; keys and values appended token by token in
    # blocks, then scores, softmax (outside the product), and the values
    say("attention step", kv_bits)
    nq, nkv, hd, window = 8, 4, 64, 256
    levels = _levels(kv_bits)
    K = _empty(kv_bits, window, nkv * hd)
    V = _empty(kv_bits, window, nkv * hd)
    keys = cq_inputs.master(74, kv_bits, 300, nkv * hd, sigma=1.0)
    vals = cq_inputs.master(75, kv_bits, 300, nkv * hd, sigma=1.0)
    pos = 0
    for step in (100, 100, 100):  # 300 tokens: the ring wraps
        for t0 in range(0, step, 60):
            n = min(60, step - t0)
            a = pos % window
            first = min(n, window - a)
            kk = torch.from_numpy(keys[pos:pos + n]).to(DEV)
            vv = torch.from_numpy(vals[pos:pos + n]).to(DEV)
            cq.cq_quantize_rows(K, kk[:first], a)
            cq.cq_quantize_rows(V, vv[:first], a)
            if first < n:
                cq.cq_quantize_rows(K, kk[first:], 0)
                cq.cq_quantize_rows(V, vv[first:], 0)
            pos += n
    # the ring now holds tokens 44..299: row r holds token r + 256 (r < 44) or r
    held = np.array([r + 256 if r < 44 else r for r in range(window)])
    kb = oracle.quantize(keys[held], kv_bits, levels)
    vb = oracle.quantize(vals[held], kv_bits, levels)
    same_k, _ = _codes_agree(K.blob.cpu().numpy(), kb, kv_bits, window, nkv * hd)
    assert same_k >= 0.9999
    q = cq_inputs.activations(76, kv_bits, nq, hd)
    s = cq.cq_kv_scores(K, torch.from_numpy(q).to(DEV), nkv)
    p = torch.softmax(s / 8.0, dim=1)  # 1/sqrt(64)
    o = cq.cq_matvec_t(V, p).cpu().numpy()
    # the oracle on the GPU's own blobs (the encoder is checked above)
    kblob, vblob = K.blob.cpu().numpy(), V.blob.cpu().numpy()
    sref = oracle.kv_scores(kblob, kv_bits, window, nkv, hd, q, levels) / 8.0
    pref = np.exp(sref - sref.max(axis=1, keepdims=True))
    pref /= pref.sum(axis=1, keepdims=True)
    oref = oracle.kv_weighted_values(vblob, kv_bits, window, nkv, hd, pref, levels)
    for h in range(nq):
        c0 = oracle.kv_head_of(h, nq, nkv) * hd
        got = o[h, c0:c0 + hd].astype(np.float64)
        assert np.max(np.abs(got - oref[h])) <= 1e-4 * np.max(np.abs(oref[h])) + 1e-6, h


@pytest.mark.parametrize("bits,rows,tokens,nq,nkv,hd", [
    (2, 256, 256, 8, 4, 64),      # Needle 2 geometry, ring full
    (3, 256, 256, 8, 4, 64),
    (4, 256, 256, 8, 4, 64),
    (5, 256, 100, 8, 4, 64),      # ternary, partly filled
    (1, 256, 256, 8, 4, 64),      # binary
    (4, 3000, 2500, 4, 2, 128),   # several token blocks per workgroup, one head per group
    (2, 640, 1, 16, 8, 32),       # one token; four heads per group
    (3, 1100, 1027, 6, 3, 16),    # ragged block tails, eight heads per group
])
def test_kv_attention_against_oracle(bits, rows, tokens, nq, nkv, hd):
    # the fused step (scores, softmax, values in one launch) against the
    # oracle's step on the same blobs, and against the composed calls
    say("kv attention", bits, rows, tokens, nq, nkv, hd)
    cols = nkv * hd
    lv = _levels(bits)
    K = cq.cq_quantize(torch.from_numpy(cq_inputs.master(80, bits, rows, cols, sigma=1.0)).to(DEV), bits, lv)
    V = cq.cq_quantize(torch.from_numpy(cq_inputs.master(81, bits, rows, cols, sigma=1.0)).to(DEV), bits, lv)
    q = cq_inputs.activations(82, bits, nq, hd)
    scale = 1.0 / np.sqrt(hd)
    got = cq.cq_kv_attention(K, V, torch.from_numpy(q).to(DEV), nkv, tokens=tokens, scale=scale).cpu().numpy()
    kb, vb = K.blob.cpu().numpy(), V.blob.cpu().numpy()
    ref = oracle.kv_attention(kb, vb, bits, rows, tokens, nkv, hd, q, scale, lv, lv)
    for h in range(nq):
        err = np.max(np.abs(got[h].astype(np.float64) - ref[h]))
        assert err <= 1e-4 * np.max(np.abs(ref[h])) + 1e-6, (h, err)
    # the composed path (cq_kv_scores, softmax, cq_matvec_t) agrees too
    s = cq.cq_kv_scores(K, torch.from_numpy(q).to(DEV), nkv)[:, :tokens]
    p = torch.zeros((nq, rows), device=DEV)
    p[:, :tokens] = torch.softmax(s * scale, dim=1)
    o = torch.cat([cq.cq_matvec_t(V, p[b:b + 8]) for b in range(0, nq, 8)]).cpu().numpy()  # batches of 8
    for h in range(nq):
        c0 = oracle.kv_head_of(h, nq, nkv) * hd
        assert np.max(np.abs(got[h] - o[h, c0:c0 + hd])) <= 2e-4 * np.max(np.abs(ref[h])) + 1e-6, h


def test_kv_attention_special_inputs():
    # a zero query weighs the rows equally (the mean of the value rows), and
    # a repeated call gives the same bytes
    bits, rows, nq, nkv, hd = 2, 512, 8, 4, 64
    lv = _levels(bits)
    K = cq.cq_quantize(torch.from_numpy(cq_inputs.master(83, bits, rows, nkv * hd, sigma=1.0)).to(DEV), bits, lv)
    V = cq.cq_quantize(torch.from_numpy(cq_inputs.master(84, bits, rows, nkv * hd, sigma=1.0)).to(DEV), bits, lv)
    z = torch.zeros((nq, hd), device=DEV)
    got = cq.cq_kv_attention(K, V, z, nkv, tokens=300).cpu().numpy()
    vd = oracle.dequantize(V.blob.cpu().numpy(), bits, rows, nkv * hd, lv)
    for h in range(nq):
        c0 = (h // 2) * hd
        mean = vd[:300, c0:c0 + hd].mean(axis=0)
        assert np.max(np.abs(got[h] - mean)) <= 1e-4 * np.max(np.abs(mean)) + 1e-6, h
    q = torch.from_numpy(cq_inputs.activations(85, bits, nq, hd)).to(DEV)
    a = cq.cq_kv_attention(K, V, q, nkv)
    b = cq.cq_kv_attention(K, V, q, nkv)
    assert torch.equal(a, b)


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 1])
def test_kv_append_equals_two_row_appends(bits):
    # the joint append (one launch) writes exactly what two cq_quantize_rows
    # calls write, across the ring's wrap; caches of different widths too
    say("kv joint append", bits)
    rows, kc, vc = 256, 256, 384
    lv = _levels(bits)
    K1, V1, K2, V2 = _empty(bits, rows, kc), _empty(bits, rows, vc), _empty(bits, rows, kc), _empty(bits, rows, vc)
    kk = torch.from_numpy(cq_inputs.master(86, bits, 300, kc, sigma=1.0)).to(DEV)
    vv = torch.from_numpy(cq_inputs.master(87, bits, 300, vc, sigma=1.0)).to(DEV)
    pos = 0
    for n in (1, 60, 3, 150, 86):  # 300 tokens
        a = pos % rows
        first = min(n, rows - a)
        cq.cq_kv_append(K1, V1, kk[pos:pos + first], vv[pos:pos + first], a)
        cq.cq_quantize_rows(K2, kk[pos:pos + first], a)
        cq.cq_quantize_rows(V2, vv[pos:pos + first], a)
        if first < n:
            cq.cq_kv_append(K1, V1, kk[pos + first:pos + n], vv[pos + first:pos + n], 0)
            cq.cq_quantize_rows(K2, kk[pos + first:pos + n], 0)
            cq.cq_quantize_rows(V2, vv[pos + first:pos + n], 0)
        pos += n
    torch.cuda.synchronize()
    assert torch.equal(K1.blob, K2.blob) and torch.equal(V1.blob, V2.blob)


def test_kv_append_with_two_code_books():
    # different levels for keys and values: one launch each, same bytes as
    # the row appends
    rows, cols = 64, 256
    lk = cq_inputs.codebook(2)
    lvv = (lk * np.float32(1.5)).astype(np.float32)
    K1 = cq.CQMatrix(2, rows, cols, torch.zeros(cq.cq_blob_bytes(2, rows, cols), dtype=torch.uint8, device=DEV), lk)
    V1 = cq.CQMatrix(2, rows, cols, torch.zeros(cq.cq_blob_bytes(2, rows, cols), dtype=torch.uint8, device=DEV), lvv)
    K2 = cq.CQMatrix(2, rows, cols, torch.zeros_like(K1.blob), lk)
    V2 = cq.CQMatrix(2, rows, cols, torch.zeros_like(V1.blob), lvv)
    kk = torch.from_numpy(cq_inputs.master(88, 2, 10, cols, sigma=1.0)).to(DEV)
    vv = torch.from_numpy(cq_inputs.master(89, 2, 10, cols, sigma=1.0)).to(DEV)
    cq.cq_kv_append(K1, V1, kk, vv, 7)
    cq.cq_quantize_rows(K2, kk, 7)
    cq.cq_quantize_rows(V2, vv, 7)
    torch.cuda.synchronize()
    assert torch.equal(K1.blob, K2.blob) and torch.equal(V1.blob, V2.blob)
