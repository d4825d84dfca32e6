"""Attention of a decode step between the fused q/k/v projection and the
output projection (oracle).

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

The pages name the projections W_q, W_k, W_v and W_o [QeRL summary, §3.4
"Layer coverage"] but not the attention between them, which belongs to the
model.  This is standard scaled dot-product attention with grouped query
heads, in fp64:
    score[h, p] = q_h . k_{g(h), p} / sqrt(d),  g(h) = h // (n_q / n_kv)
    out_h       = sum_p softmax_p(score[h, :]) v_{g(h), p}
over the context positions p of one token row.  The stub on the decode
path has a context of one position: the row's own key and value.
"""
import numpy as np

from .formats import bf16_bits_to_f64


def split_qkv(qkv, n_q, n_kv, head_dim):
    """Rows of the fused projection output [m, (n_q + 2 n_kv) d] -> q [m,
    n_q, d], k [m, n_kv, d], v [m, n_kv, d] (q heads, then k, then v)."""
    qkv = np.asarray(qkv, dtype=np.float64)
    m = qkv.shape[0]
    q = qkv[:, :n_q * head_dim].reshape(m, n_q, head_dim)
    k = qkv[:, n_q * head_dim:(n_q + n_kv) * head_dim].reshape(m, n_kv, head_dim)
    v = qkv[:, (n_q + n_kv) * head_dim:].reshape(m, n_kv, head_dim)
    return q, k, v


def attend(q, keys, values, n_q, n_kv):
    """One token row: q [n_q, d]; keys, values [P, n_kv, d] over P context
    positions -> out [n_q, d]."""
    d = q.shape[-1]
    group = n_q // n_kv
    out = np.empty_like(q)
    for h in range(n_q):
        g = h // group
        s = keys[:, g, :] @ q[h] / np.sqrt(d)
        w = np.exp(s - s.max())
        w = w / w.sum()
        out[h] = w @ values[:, g, :]
    return out


def decode_attention(qkv_bits, n_q, n_kv, head_dim, past_k=None, past_v=None):
    """Attention of every row of the fused q/k/v output (bf16 bits [m, (n_q
    + 2 n_kv) d]) over its context: past keys/values [m, P, n_kv, d] (fp64,
    optional) followed by its own key and value.  Returns [m, n_q d]."""
    q, k, v = split_qkv(bf16_bits_to_f64(qkv_bits), n_q, n_kv, head_dim)
    m = q.shape[0]
    out = np.empty((m, n_q, head_dim))
    for i in range(m):
        keys, values = k[i][None], v[i][None]
        if past_k is not None:
            keys = np.concatenate([past_k[i], keys])
            values = np.concatenate([past_v[i], values])
        out[i] = attend(q[i], keys, values, n_q, n_kv)
    return out.reshape(m, n_q * head_dim)
