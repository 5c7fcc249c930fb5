"""Dense brute-force block-diagonal attention (numpy fp64), for tiny inputs only.

Builds the full T x T score matrix of every head, sets every pair of tokens from
different segments to -inf, and applies a row-wise stable softmax: the masked dense
form of the GigaPath-Flash page's naive_attention (section 4.1) combined with the
SparseAttn article's masked reference (section 4: masked scores set to -inf).  It is
a different formulation from the oracle's per-segment row loop, used to pin it.
"""
import numpy as np


def segment_ids(cu, T):
    cu = np.asarray(cu, dtype=np.int64)
    return np.searchsorted(cu[1:], np.arange(T), side="right")


def dense_block_diag(q, k, v, cu, scale):
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    T, H, _ = q.shape
    seg = segment_ids(cu, T)
    allowed = seg[:, None] == seg[None, :]
    out = np.empty((T, H, v.shape[2]))
    lse = np.empty((H, T))
    for h in range(H):
        s = scale * (q[:, h, :] @ k[:, h, :].T)
        s = np.where(allowed, s, -np.inf)
        mx = s.max(axis=1, keepdims=True)
        e = np.exp(s - mx)
        z = e.sum(axis=1, keepdims=True)
        out[:, h, :] = (e / z) @ v[:, h, :]
        lse[h] = mx[:, 0] + np.log(z[:, 0])
    return out, lse
