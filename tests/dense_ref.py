"""Independent dense brute force for tiny inputs (test helper, numpy fp64).

It builds the full n x n boolean mask of allowed (query, key) pairs with vectorised array
expressions, without enumerating key sets, and runs ordinary dense softmax attention with the
disallowed scores removed.  It is a second, structurally different statement of the same
definition the oracle implements, used to pin the oracle on tiny shapes.
"""

import numpy as np


def dense_mask(B, H, n, *, win_left, win_right, dilation=None, global_idx=None, key_pad=None,
               layout=None, block=0):
    """Boolean [B, H, n, n]: M[b, h, i, j] = key j is attended by query i."""
    I = np.arange(n)[:, None]
    J = np.arange(n)[None, :]
    D = J - I
    M = np.zeros((B, H, n, n), dtype=bool)
    for h in range(H):
        dil = 1 if dilation is None else int(dilation[h])
        if not (win_left == -1 and win_right == -1):
            band = (D % dil == 0) & (D >= -dil * win_left) & (D <= dil * win_right)
            M[:, h] |= band[None]
        if layout is not None:
            nb = n // block
            bm = np.zeros((nb, nb), dtype=bool)
            for qb in range(nb):
                for s in layout[h, qb]:
                    if s >= 0:
                        bm[qb, s] = True
            M[:, h] |= bm[I // block, J // block][None]
    if global_idx is not None and global_idx.shape[1] > 0:
        for b in range(B):
            isg = np.zeros(n, dtype=bool)
            isg[global_idx[b]] = True
            M[b] |= (isg[None, :] | isg[:, None])[None]
    if key_pad is not None:
        M &= ~(key_pad.astype(bool)[:, None, None, :])
    return M


def dense_attention(q, k, v, scale, M):
    """q, k, v: fp64 [B, H, n, d]; M: bool [B, H, n, n].  Returns (out, lse)."""
    S = np.einsum("bhid,bhjd->bhij", q, k) * scale
    S = np.where(M, S, -np.inf)
    m = S.max(axis=-1, keepdims=True)
    empty = ~M.any(axis=-1)
    m_safe = np.where(np.isfinite(m), m, 0.0)
    P = np.where(M, np.exp(S - m_safe), 0.0)
    l = P.sum(axis=-1)
    with np.errstate(invalid="ignore", divide="ignore"):
        out = np.einsum("bhij,bhjd->bhid", P, v) / l[..., None]
        lse = m_safe[..., 0] + np.log(l)
    out[empty] = 0.0
    lse[empty] = -np.inf
    return out, lse
