"""Closed forms of exact attention with all queries zero (host side, fp64).

With q_i = 0 every visible score is 0, so query row i spreads its
probability evenly over its n_i visible keys: n_i = i + 1 under the causal
mask (queries and keys on one token axis), L_kv without it. Then
    O_i  = (1/n_i) sum_{j visible} v_j,            LSE_i = ln n_i,
    dV_j = sum_{i that see j} dO_i / n_i,          dK = 0,
and, as dS_ij = P_ij (dO_i . v_j - D_i) with P_ij = 1/n_i and
D_i = dO_i . O_i,
    dQ_i = (dO_i^T M_i - D_i s_i) / (sqrt(d_h) n_i),
    M_i  = sum_{j visible} v_j k_j^T,  s_i = sum_{j visible} k_j.
Running sums give every row in O(L d_h^2) per head.
"""
import numpy as np


def zero_query_attention(k, v, do, causal, Lq, block=256):
    """O, LSE, dQ and dV of one query head whose queries are all zero.

    k, v: [L_kv, d_h] fp64; do: [Lq, d_h] fp64 or None (forward only).
    Returns a dict of fp64 arrays: o [Lq, d_h], lse [Lq], and with do also
    dq [Lq, d_h] and dv [L_kv, d_h].
    """
    Lk, d = k.shape
    if causal:
        assert Lq == Lk, "the causal mask needs queries and keys on one token axis"
        n = np.arange(1, Lq + 1, dtype=np.float64)
        o = np.cumsum(v, axis=0) / n[:, None]
    else:
        n = np.full(Lq, float(Lk))
        o = np.broadcast_to(v.mean(axis=0), (Lq, d))
    out = {"o": o, "lse": np.log(n)}
    if do is None:
        return out
    D = np.sum(do * o, axis=1)
    if causal:
        s = np.cumsum(k, axis=0)
        acc = np.empty((Lq, d))
        M = np.zeros((d, d))
        for a in range(0, Lq, block):
            b = min(Lq, a + block)
            w = np.tril(do[a:b] @ v[a:b].T)      # dO_i . v_j for j <= i inside the block
            acc[a:b] = do[a:b] @ M + w @ k[a:b]
            M += v[a:b].T @ k[a:b]
        dv = np.cumsum((do / n[:, None])[::-1], axis=0)[::-1]
    else:
        s = np.broadcast_to(k.sum(axis=0), (Lq, d))
        acc = do @ (v.T @ k)
        dv = np.broadcast_to(do.sum(axis=0) / Lk, (Lk, d))
    out["dq"] = (acc - D[:, None] * s) / (np.sqrt(d) * n[:, None])
    out["dv"] = dv
    return out
