"""Pins of the KV-cache oracle (oracle/kv.py): attention scores and the
value-side product against a CQ-quantised cache, checked by explicit loops
over the Sylvester matrix, by the zero-padded-query identity the GPU path
uses, by the rotated-domain identity of the transposed product, and the
row independence of the encoder that appending rows relies on."""
import numpy as np
import pytest

import cq_inputs
import oracle


def _cache(cfg, bits, tokens, kv_dim, sigma=1.0):
    levels = None if bits in (1, 5) else cq_inputs.codebook(bits)
    k = cq_inputs.master(cfg, bits, tokens, kv_dim, sigma=sigma)
    return oracle.quantize(k, bits, levels), levels, k


def _dense_by_loops(blob, bits, rows, cols, levels):
    """w_hat[r, 128 g + k] = sum_j c[q[r, 128 g + j]] * n[r, g] * S[j, k] / sqrt(128)."""
    packed, norms = oracle.split_blob(blob, bits, rows, cols)
    kpad = oracle.padded_cols(cols)
    vals = oracle.level_values(oracle.unpack_codes(packed, bits, kpad), bits, levels)
    S = oracle.sylvester(128).astype(np.float64)
    out = np.zeros((rows, kpad))
    for r in range(rows):
        for g in range(kpad // 128):
            rot = vals[r, 128 * g:128 * (g + 1)] * float(np.float32(norms[r, g]))
            for k in range(128):
                out[r, 128 * g + k] = sum(rot[j] * S[j, k] for j in range(128)) / np.sqrt(128)
    return out[:, :cols]


def test_kv_head_of_grouped_queries():
    assert [oracle.kv_head_of(h, 8, 4) for h in range(8)] == [0, 0, 1, 1, 2, 2, 3, 3]
    assert [oracle.kv_head_of(h, 12, 2) for h in range(12)] == [0] * 6 + [1] * 6
    with pytest.raises(ValueError):
        oracle.kv_head_of(0, 6, 4)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_kv_scores_by_loops(bits):
    tokens, n_kv, hd, nq = 5, 4, 64, 8
    blob, levels, _ = _cache(60, bits, tokens, n_kv * hd)
    q = cq_inputs.activations(60, bits, nq, hd)
    got = oracle.kv_scores(blob, bits, tokens, n_kv, hd, q, levels)
    dense = _dense_by_loops(blob, bits, tokens, n_kv * hd, levels)
    for h in range(nq):
        kvh = h // 2
        for t in range(tokens):
            want = sum(float(q[h, d]) * dense[t, kvh * hd + d] for d in range(hd))
            assert abs(got[h, t] - want) <= 1e-12 * (1 + abs(want))


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_kv_scores_are_a_matvec_with_zero_padded_queries(bits):
    # the product the GPU path computes: each query head as a row of the
    # cache's width, zero outside its KV head's columns
    tokens, n_kv, hd, nq = 40, 4, 64, 8
    blob, levels, _ = _cache(61, bits, tokens, n_kv * hd)
    q = cq_inputs.activations(61, bits, nq, hd)
    xpad = np.zeros((nq, n_kv * hd), dtype=np.float32)
    for h in range(nq):
        c0 = oracle.kv_head_of(h, nq, n_kv) * hd
        xpad[h, c0:c0 + hd] = q[h]
    mv = oracle.matvec(blob, bits, tokens, n_kv * hd, xpad, levels)
    assert np.allclose(oracle.kv_scores(blob, bits, tokens, n_kv, hd, q, levels), mv, rtol=0, atol=1e-12)


@pytest.mark.parametrize("bits", [2, 4, 5])
def test_matvec_t_by_loops(bits):
    rows, cols = 6, 200
    blob, levels, _ = _cache(62, bits, rows, cols, sigma=0.02)
    p = cq_inputs.activations(62, bits, 3, rows)
    got = oracle.matvec_t(blob, bits, rows, cols, p, levels)
    dense = _dense_by_loops(blob, bits, rows, cols, levels)
    for b in range(3):
        for k in range(0, cols, 7):
            want = sum(float(p[b, r]) * dense[r, k] for r in range(rows))
            assert abs(got[b, k] - want) <= 1e-12 * (1 + abs(want))


def _butterfly(v):
    v = np.array(v, dtype=np.float64)
    h = 1
    while h < v.shape[-1]:
        for i in range(0, v.shape[-1], 2 * h):
            a = v[..., i:i + h].copy()
            b = v[..., i + h:i + 2 * h].copy()
            v[..., i:i + h] = a + b
            v[..., i + h:i + 2 * h] = a - b
        h *= 2
    return v / np.sqrt(v.shape[-1])


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 1])
def test_matvec_t_rotated_domain_identity(bits):
    # sum_r p_r w_hat[r, g] = (sum_r p_r n[r, g] c[q[r, g]]) . H: the weighted
    # sum can be taken on the codes and rotated back once per group
    rows, cols = 33, 384
    blob, levels, _ = _cache(63, bits, rows, cols, sigma=0.02)
    p = cq_inputs.activations(63, bits, 2, rows).astype(np.float64)
    packed, norms = oracle.split_blob(blob, bits, rows, cols)
    vals = oracle.level_values(oracle.unpack_codes(packed, bits, cols), bits, levels)
    rot = np.zeros((2, cols))
    for r in range(rows):
        n = np.repeat(norms[r].astype(np.float32).astype(np.float64), 128)
        rot += p[:, r:r + 1] * (vals[r] * n)[None, :]
    via_codes = _butterfly(rot.reshape(2, 3, 128)).reshape(2, cols)
    assert np.allclose(via_codes, oracle.matvec_t(blob, bits, rows, cols, p, levels), rtol=0, atol=1e-12)


def test_kv_weighted_values_pick_rows():
    tokens, n_kv, hd, nq = 7, 4, 64, 8
    blob, levels, _ = _cache(64, 2, tokens, n_kv * hd)
    dense = oracle.dequantize(blob, 2, tokens, n_kv * hd, levels)
    p = np.zeros((nq, tokens))
    for h in range(nq):
        p[h, (3 * h) % tokens] = 1.0
    o = oracle.kv_weighted_values(blob, 2, tokens, n_kv, hd, p, levels)
    for h in range(nq):
        c0 = (h // 2) * hd
        assert np.array_equal(o[h], dense[(3 * h) % tokens, c0:c0 + hd])
    # linear in p
    p2 = cq_inputs.activations(64, 1, nq, tokens).astype(np.float64)
    o2 = oracle.kv_weighted_values(blob, 2, tokens, n_kv, hd, p2, levels)
    o3 = oracle.kv_weighted_values(blob, 2, tokens, n_kv, hd, 2 * p + p2, levels)
    assert np.allclose(o3, 2 * o + o2, rtol=0, atol=1e-12)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_rows_encode_independently(bits):
    # appending rows to a cache encodes them on their own: the rows of a
    # block, encoded alone, equal the same rows of the whole matrix encoded
    rows, cols = 20, 256
    levels = cq_inputs.codebook(bits)
    k = cq_inputs.master(65, bits, rows, cols, sigma=1.0)
    whole = oracle.split_blob(oracle.quantize(k, bits, levels), bits, rows, cols)
    for a, b in [(0, 1), (3, 11), (19, 20)]:
        part = oracle.split_blob(oracle.quantize(k[a:b], bits, levels), bits, b - a, cols)
        assert np.array_equal(part[0], whole[0][a:b]) and np.array_equal(part[1], whole[1][a:b])


@pytest.mark.parametrize("bits", [2, 4])
def test_kv_attention_by_loops(bits):
    # the step written out: scaled scores from the loop-dequantised caches,
    # math.exp softmax over the first `tokens` rows only, weighted value rows
    import math
    rows, tokens, n_kv, hd, nq, scale = 9, 6, 4, 32, 8, 0.3
    kblob, levels, _ = _cache(66, bits, rows, n_kv * hd)
    vblob, _, _ = _cache(67, bits, rows, n_kv * hd)
    q = cq_inputs.activations(66, bits, nq, hd)
    kd = _dense_by_loops(kblob, bits, rows, n_kv * hd, levels)
    vd = _dense_by_loops(vblob, bits, rows, n_kv * hd, levels)
    got = oracle.kv_attention(kblob, vblob, bits, rows, tokens, n_kv, hd, q, scale, levels, levels)
    assert got.shape == (nq, hd)
    for h in range(nq):
        c0 = (h // (nq // n_kv)) * hd
        z = [scale * sum(float(q[h, d]) * kd[t, c0 + d] for d in range(hd)) for t in range(tokens)]
        zmax = max(z)
        e = [math.exp(v - zmax) for v in z]
        tot = sum(e)
        for d in range(hd):
            want = sum(e[t] / tot * vd[t, c0 + d] for t in range(tokens))
            assert abs(got[h, d] - want) <= 1e-12 * (1 + abs(want))


def test_kv_attention_special_cases():
    rows, n_kv, hd, nq = 12, 2, 64, 4
    kblob, levels, _ = _cache(68, 3, rows, n_kv * hd)
    vblob, _, _ = _cache(69, 3, rows, n_kv * hd)
    vd = oracle.dequantize(vblob, 3, rows, n_kv * hd, levels)
    q = cq_inputs.activations(68, 3, nq, hd)
    for tokens in (1, 5, rows):
        # a zero scale (or a zero query) weighs the first `tokens` rows equally
        flat = oracle.kv_attention(kblob, vblob, 3, rows, tokens, n_kv, hd, q, 0.0, levels, levels)
        zq = oracle.kv_attention(kblob, vblob, 3, rows, tokens, n_kv, hd, np.zeros_like(q), 1.0, levels, levels)
        for h in range(nq):
            c0 = (h // 2) * hd
            mean = vd[:tokens, c0:c0 + hd].mean(axis=0)
            assert np.allclose(flat[h], mean, rtol=0, atol=1e-12)
            assert np.allclose(zq[h], mean, rtol=0, atol=1e-12)
    # one token: its value row, whatever the query
    one = oracle.kv_attention(kblob, vblob, 3, rows, 1, n_kv, hd, q, 5.0, levels, levels)
    for h in range(nq):
        assert np.allclose(one[h], vd[0, (h // 2) * hd:(h // 2 + 1) * hd], rtol=0, atol=1e-12)
    # a scale large enough for a hard maximum picks the best-scoring row
    s = oracle.kv_scores(kblob, 3, rows, n_kv, hd, q, levels)
    hard = oracle.kv_attention(kblob, vblob, 3, rows, rows, n_kv, hd, q, 1e6, levels, levels)
    for h in range(nq):
        t = int(np.argmax(s[h]))
        assert np.allclose(hard[h], vd[t, (h // 2) * hd:(h // 2 + 1) * hd], rtol=0, atol=1e-9)
    with pytest.raises(ValueError):
        oracle.kv_attention(kblob, vblob, 3, rows, 0, n_kv, hd, q, 1.0, levels, levels)
