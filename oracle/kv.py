"""CQ-quantised KV cache oracle: rows appended to a cache matrix, attention
scores against it, and the probability-weighted sum of its value rows.

TEST INFRASTRUCTURE ONLY (see the package docstring).

[cact-format post, "Five regions"]: ``kv_bits`` is the KV-cache precision the
model was post-trained for -- 8 (int8), else 2, 3 or 4.  [cact-format post,
"How the kernel reads it"]: the same CQ path serves the KV cache at whatever
``kv_bits`` the header declares.  [OpenNeedle reference, numeric-paths
note]: below 8 bits the reference simulates the KV cache through CQ fake
quantisation (quantise, then use the dequantised values).

Readings (also listed in the design notes):
* R23 -- a cached key or value row is one token's whole KV vector,
  ``n_kv_heads * head_dim`` wide, quantised like a weight row: 128-groups
  along it, one fp16 norm per group, codes of the ``kv_bits`` code book.  A
  128-group may span several heads (Needle 2: four KV heads of 64, so each
  group holds two heads).  The cache is a CQ matrix [tokens, kv_dim].
* R24 -- grouped-query attention: query head h reads KV head
  h // (n_q_heads // n_kv_heads), consecutive query heads sharing one KV
  head [OpenNeedle reference, attention note: two query heads map to one
  KV head].
* R25 -- the score of query head h and token t is q_h . k_hat_t restricted to
  the KV head's ``head_dim`` columns (no 1/sqrt(head_dim) factor or mask:
  those belong to the attention around the product).
* R26 -- the value side is o_h = sum_t p[h, t] v_hat_t over the KV head's
  columns, p given.
* R27 -- one decode attention step over the first n cached rows (the rows
  filled so far; a full ring is every row): p[h] = softmax_t(scale *
  scores[h, t]) for t < n, no mask, then R26's sum with that p
  [OpenNeedle reference, attention note: softmax of the scaled scores of
  the cached keys, then the weighted values].
"""

import numpy as np

from .cq import dequantize

__all__ = ["kv_head_of", "kv_scores", "matvec_t", "kv_weighted_values", "kv_attention"]


def kv_head_of(h, n_q_heads, n_kv_heads):
    """KV head read by query head ``h`` (R24)."""
    if n_q_heads % n_kv_heads:
        raise ValueError("query heads must be a multiple of KV heads")
    return h // (n_q_heads // n_kv_heads)


def kv_scores(blob, bits, tokens, n_kv_heads, head_dim, q, levels=None):
    """scores[h, t] = sum_d q[h, d] * k_hat[t, kv(h) * head_dim + d], float64
    [n_q_heads, tokens], with k_hat the dense dequantisation of the cache
    (R23-R25).  ``q`` is [n_q_heads, head_dim]."""
    q = np.asarray(q, dtype=np.float64)
    cols = n_kv_heads * head_dim
    k_hat = dequantize(blob, bits, tokens, cols, levels)[:, :cols]
    out = np.empty((q.shape[0], tokens))
    for h in range(q.shape[0]):
        c0 = kv_head_of(h, q.shape[0], n_kv_heads) * head_dim
        out[h] = k_hat[:, c0:c0 + head_dim] @ q[h]
    return out


def matvec_t(blob, bits, rows, cols, p, levels=None):
    """out[b, k] = sum_r p[b, r] * w_hat[r, k] (k < cols), float64: the
    product with the transposed dequantised matrix."""
    p = np.asarray(p, dtype=np.float64)
    if p.ndim == 1:
        p = p[None, :]
    return p @ dequantize(blob, bits, rows, cols, levels)[:, :cols]


def kv_weighted_values(blob, bits, tokens, n_kv_heads, head_dim, p, levels=None):
    """o[h, d] = sum_t p[h, t] * v_hat[t, kv(h) * head_dim + d], float64
    [n_q_heads, head_dim] (R26).  ``p`` is [n_q_heads, tokens]."""
    p = np.asarray(p, dtype=np.float64)
    full = matvec_t(blob, bits, tokens, n_kv_heads * head_dim, p, levels)
    out = np.empty((p.shape[0], head_dim))
    for h in range(p.shape[0]):
        c0 = kv_head_of(h, p.shape[0], n_kv_heads) * head_dim
        out[h] = full[h, c0:c0 + head_dim]
    return out


def kv_attention(kblob, vblob, bits, rows, tokens, n_kv_heads, head_dim, q, scale, klevels=None, vlevels=None):
    """One decode attention step (R27), float64 [n_q_heads, head_dim]:
    o[h] = sum_{t < tokens} p[h, t] v_hat[t, kv(h) head columns] with p[h] the
    softmax over t < tokens of scale * scores[h, t].  Both caches are CQ
    matrices of ``rows`` rows (their capacity) and n_kv_heads * head_dim
    columns at the same width ``bits``; only their first ``tokens`` rows are
    read."""
    if not 1 <= tokens <= rows:
        raise ValueError("tokens must be in 1..rows")
    s = float(scale) * kv_scores(kblob, bits, rows, n_kv_heads, head_dim, q, klevels)[:, :tokens]
    p = np.exp(s - s.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    full = np.zeros((p.shape[0], rows))
    full[:, :tokens] = p
    return kv_weighted_values(vblob, bits, rows, n_kv_heads, head_dim, full, vlevels)
