"""Brute-force MaxSim by materialising the similarity tensor.

This is the naive route the "Flash-MaxSim" paper describes in Sec. 3.1 (an
einsum that writes S[i, j, s, t], then max over t and sum over s). It shares no
code with the oracle: numpy forms S in one contraction and reduces it with
numpy's max/argmax (argmax returns the first maximum, i.e. the lowest index).
Only for tiny inputs.
"""

import numpy as np


def _np(x, dtype):
    if x is None:
        return None
    if hasattr(x, "detach"):
        x = x.detach().cpu()
        x = x.double().numpy() if dtype == np.float64 else x.numpy()
    return np.asarray(x, dtype=dtype)


def dense(Q, D, q_mask=None, d_mask=None, exact_int=False):
    """Returns (scores [Nq,Nd], argmax [Nq,Nd,Lq]) for Q [Nq,Lq,d], D [Nd,Ld,d]."""
    dt = np.int64 if exact_int else np.float64
    q = _np(Q, dt)
    d = _np(D, dt)
    Nq, Lq, _ = q.shape
    Nd, Ld, _ = d.shape
    S = np.einsum("isk,jtk->ijst", q, d).astype(np.float64)  # [Nq,Nd,Lq,Ld]
    if d_mask is not None:
        dm = _np(d_mask, np.uint8).astype(bool)
        S = np.where(dm[None, :, None, :], S, -np.inf)
    if Ld == 0:
        m = np.full((Nq, Nd, Lq), -np.inf)
        a = np.zeros((Nq, Nd, Lq), np.int64)
    else:
        m = S.max(axis=3)
        a = S.argmax(axis=3)
    keep = np.isfinite(m)
    if q_mask is not None:
        qm = _np(q_mask, np.uint8).astype(bool)
        keep &= qm[:, None, :]
    contrib = np.where(keep, m, 0.0)
    if exact_int:
        return contrib.astype(np.int64).sum(axis=2), a.astype(np.int32)
    return contrib.sum(axis=2), a.astype(np.int32)


def varlen(Q, cu_q, max_lq, D, cu_d):
    """Per-pair brute force over packed sequences; argmax [Nq,Nd,max_lq]."""
    q = _np(Q, np.float64)
    d = _np(D, np.float64)
    cq = _np(cu_q, np.int64)
    cd = _np(cu_d, np.int64)
    Nq, Nd = len(cq) - 1, len(cd) - 1
    scores = np.zeros((Nq, Nd))
    arg = np.zeros((Nq, Nd, max_lq), np.int32)
    for i in range(Nq):
        qi = q[cq[i]:cq[i + 1]]
        for j in range(Nd):
            dj = d[cd[j]:cd[j + 1]]
            if len(dj) == 0 or len(qi) == 0:
                continue
            S = qi @ dj.T
            scores[i, j] = S.max(axis=1).sum()
            arg[i, j, :len(qi)] = S.argmax(axis=1)
    return scores, arg


def chamfer(P, Q):
    """Chamfer distance by materialising the [B,N,M] squared-distance tensor
    (the naive form of Flash-MaxSim Sec. 4.2.4); numpy argmin returns the
    first minimum. Returns (dist1, idx1, dist2, idx2, loss)."""
    p = _np(P, np.float64)
    q = _np(Q, np.float64)
    S = ((p[:, :, None, :] - q[:, None, :, :]) ** 2).sum(-1)  # [B,N,M]
    d1, i1 = S.min(axis=2), S.argmin(axis=2)
    d2, i2 = S.min(axis=1), S.argmin(axis=1)
    loss = d1.mean(axis=1) + d2.mean(axis=1)
    return d1, i1.astype(np.int32), d2, i2.astype(np.int32), loss
