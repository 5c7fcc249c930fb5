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


def dense_block_rect(q, k, v, cu_q, cu_k, scale):
    """Rectangular variant: query token i of segment s may see key token j only when j
    lies in segment s of the key table.  A query whose key segment is empty has an
    all -inf row; it is given output 0 and LSE -inf explicitly (no softmax exists)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    Tq, H, _ = q.shape
    Tk = k.shape[0]
    sq = segment_ids(cu_q, Tq)
    sk = segment_ids(cu_k, Tk)
    allowed = sq[:, None] == sk[None, :]
    empty = ~allowed.any(axis=1)
    out = np.zeros((Tq, H, v.shape[2]))
    lse = np.full((H, Tq), -np.inf)
    for h in range(H):
        s = scale * (q[:, h, :] @ k[:, h, :].T)
        s = np.where(allowed, s, -np.inf)
        for i in np.nonzero(~empty)[0]:
            mx = s[i].max()
            e = np.exp(s[i] - mx)
            out[i, h, :] = (e / e.sum()) @ v[:, h, :]
            lse[h, i] = mx + np.log(e.sum())
    return out, lse
