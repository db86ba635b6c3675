"""How GPU results are judged against the oracle -- TEST INFRASTRUCTURE ONLY.

* float scores and gradients: |got - ref| <= 1e-3 + 1e-4 * |ref| element by
  element;
* integer outputs (int8 score sums, int8 argmax, CSR maps): bit-exact;
* float argmax: several answers can be correct when two doc tokens are nearly
  tied, because the GPU accumulates each dot product in fp32 and the oracle in
  fp64. A GPU index t_g that differs from the oracle's t_o is accepted only if
  t_g is a valid (unmasked) token and
      v(t_o) - v(t_g) <= e(t_o) + e(t_g),
  with v the exact (fp64) dot product and e(t) = gamma * sum_k |q_k x_tk|,
  gamma = d*u / (1 - d*u), u = 2^-23, the textbook bound on an fp32 sum of d
  exact products in any order. Every other mismatch fails.
"""

from __future__ import annotations

import numpy as np

ATOL = 1e-3
RTOL = 1e-4
U32 = 2.0 ** -23


def gamma(d: int) -> float:
    return d * U32 / (1.0 - d * U32)


def close(got, ref, atol: float = ATOL, rtol: float = RTOL):
    """Returns (ok, worst_excess, index_of_worst)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    if got.size == 0:
        return True, 0.0, None
    excess = np.abs(got - ref) - (atol + rtol * np.abs(ref))
    k = int(np.argmax(excess))
    worst = float(excess.reshape(-1)[k])
    return bool(np.all(excess <= 0) and np.all(np.isfinite(got))), worst, np.unravel_index(k, got.shape)


def argmax_float(got, ref, q_rows, d_rows, valid=None):
    """Checks a float argmax with the near-tie rule.

    got, ref : int arrays of identical shape, entries are doc-token indices
    q_rows   : callable (entry index tuple) -> fp64 query row q (length d)
    d_rows   : callable (entry index tuple, t) -> fp64 doc row x_t
    valid    : callable (entry index tuple, t) -> bool, or None (all valid)
    Returns (n_mismatch, n_accepted, list of failing entries).
    """
    got = np.asarray(got)
    ref = np.asarray(ref)
    mism = np.argwhere(got != ref)
    bad = []
    acc = 0
    for e in mism:
        e = tuple(int(x) for x in e)
        tg, to = int(got[e]), int(ref[e])
        if valid is not None and not valid(e, tg):
            bad.append((e, tg, to, "masked or out-of-range token"))
            continue
        q = q_rows(e)
        xo = d_rows(e, to)
        xg = d_rows(e, tg)
        if xg is None:
            bad.append((e, tg, to, "out-of-range token"))
            continue
        vo, vg = float(q @ xo), float(q @ xg)
        eo = gamma(q.size) * float(np.abs(q * xo).sum())
        eg = gamma(q.size) * float(np.abs(q * xg).sum())
        if vo - vg <= eo + eg:
            acc += 1
        else:
            bad.append((e, tg, to, f"gap {vo - vg:.3e} > bound {eo + eg:.3e}"))
    return len(mism), acc, bad


def dense_argmax_float(got, ref, Q64, D64, d_mask=None, pairs=None):
    """argmax_float for the cross-product layout. got/ref are [Nq', Nd', Lq]
    over the query/doc index lists `pairs = (I, J)` (default: all)."""
    I, J = pairs if pairs is not None else (np.arange(Q64.shape[0]), np.arange(D64.shape[0]))
    Ld = D64.shape[1]
    dm = None if d_mask is None else np.asarray(d_mask).astype(bool)

    def qr(e):
        return Q64[I[e[0]], e[2]]

    def dr(e, t):
        if t < 0 or t >= Ld:
            return None
        return D64[J[e[1]], t]

    def ok(e, t):
        if t < 0 or t >= Ld:
            return False
        if dm is None:
            return True
        j = J[e[1]]
        if not dm[j].any():
            return False  # a doc with no valid token must report 0 exactly
        return bool(dm[j, t])

    return argmax_float(got, ref, qr, dr, ok)


def pair_argmax_float(got, ref, Q64, D64, d_mask, pair_q, pair_d):
    """argmax_float for a pair list; got/ref are [P, Lq] (pair p: query
    pair_q[p] against doc pair_d[p])."""
    Ld = D64.shape[1]
    dm = None if d_mask is None else np.asarray(d_mask).astype(bool)
    pq = np.asarray(pair_q)
    pd = np.asarray(pair_d)

    def qr(e):
        return Q64[pq[e[0]], e[1]]

    def dr(e, t):
        if t < 0 or t >= Ld:
            return None
        return D64[pd[e[0]], t]

    def ok(e, t):
        if t < 0 or t >= Ld:
            return False
        if dm is None:
            return True
        j = pd[e[0]]
        if not dm[j].any():
            return False  # a doc with no valid token must report 0 exactly
        return bool(dm[j, t])

    return argmax_float(got, ref, qr, dr, ok)


def varlen_argmax_float(got, ref, Q64, cu_q, D64, cu_d, q_index, d_index):
    """argmax_float for packed sequences; got/ref are [len(q_index), len(d_index), max_lq]."""
    cu_q = np.asarray(cu_q, dtype=np.int64)
    cu_d = np.asarray(cu_d, dtype=np.int64)

    def qr(e):
        i = q_index[e[0]]
        return Q64[cu_q[i] + e[2]]

    def dr(e, t):
        j = d_index[e[1]]
        if t < 0 or t >= cu_d[j + 1] - cu_d[j]:
            return None
        return D64[cu_d[j] + t]

    def ok(e, t):
        i, j = q_index[e[0]], d_index[e[1]]
        ld = cu_d[j + 1] - cu_d[j]
        if e[2] >= cu_q[i + 1] - cu_q[i]:
            return False  # rows past the query length must be 0 exactly
        return 0 <= t < ld

    return argmax_float(got, ref, qr, dr, ok)


def pairs_varlen_argmax_float(got, ref, Q64, cu_q, D64, cu_d, pair_q, pair_d):
    """argmax_float for a pair list over packed sequences; got/ref are
    [P, max_lq] (pair p: packed query pair_q[p] against packed doc pair_d[p])."""
    cu_q = np.asarray(cu_q, dtype=np.int64)
    cu_d = np.asarray(cu_d, dtype=np.int64)
    pq = np.asarray(pair_q)
    pd = np.asarray(pair_d)

    def qr(e):
        return Q64[cu_q[pq[e[0]]] + e[1]]

    def dr(e, t):
        j = pd[e[0]]
        if t < 0 or t >= cu_d[j + 1] - cu_d[j]:
            return None
        return D64[cu_d[j] + t]

    def ok(e, t):
        i, j = pq[e[0]], pd[e[0]]
        if e[1] >= cu_q[i + 1] - cu_q[i]:
            return False  # rows past the query length must be 0 exactly
        return 0 <= t < cu_d[j + 1] - cu_d[j]

    return argmax_float(got, ref, qr, dr, ok)


U24 = 2.0 ** -24


def int8_tok_argmax(got, ref, Q8, D8, d_scale, d_mask=None, pairs=None):
    """Argmax check for per-token INT8 scores. The GPU ranks doc tokens by the
    fp32 product fl(d_scale[t] * dot_t) of an exact integer dot product (one
    rounding, relative error <= 2^-24); the oracle by the exact product (the
    positive query scale does not change the order). A GPU index t_g != t_o
    is accepted only if t_g is valid and
        w(t_o) - w(t_g) <= 2^-24 * (|w(t_o)| + |w(t_g)|),  w(t) = d_scale[t] * dot_t.
    got/ref are [Nq', Nd', Lq] over the query/doc lists `pairs = (I, J)`."""
    Q8 = np.asarray(Q8, dtype=np.int64)
    D8 = np.asarray(D8, dtype=np.int64)
    ds = np.asarray(d_scale, dtype=np.float64)
    dm = None if d_mask is None else np.asarray(d_mask)
    I = np.arange(Q8.shape[0]) if pairs is None else np.asarray(pairs[0])
    J = np.arange(D8.shape[0]) if pairs is None else np.asarray(pairs[1])
    got = np.asarray(got)
    ref = np.asarray(ref)
    bad = []
    acc = 0
    mism = np.argwhere(got != ref)
    for e in mism:
        a, b, s = (int(x) for x in e)
        i, j = int(I[a]), int(J[b])
        tg, to = int(got[a, b, s]), int(ref[a, b, s])
        if not (0 <= tg < D8.shape[1]) or (dm is not None and not dm[j, tg]):
            bad.append(((a, b, s), tg, to, "masked or out-of-range token"))
            continue
        wo = ds[j, to] * float(Q8[i, s] @ D8[j, to])
        wg = ds[j, tg] * float(Q8[i, s] @ D8[j, tg])
        if wo - wg <= U24 * (abs(wo) + abs(wg)):
            acc += 1
        else:
            bad.append(((a, b, s), tg, to, f"gap {wo - wg:.3e}"))
    return len(mism), acc, bad


def chamfer_argmin(got, ref, A64, T64):
    """Nearest-neighbour indices of one Chamfer direction: got/ref [B, na]
    index into the targets T64 [B, nt, 3] for the sources A64 [B, na, 3]. A
    GPU index t_g differing from the oracle's t_o is accepted only if
    dist(t_g) - dist(t_o) <= e(t_o) + e(t_g), with dist the exact squared
    distance and e(t) the bound on an fp32 evaluation of the expanded form
    |s'|^2 + |t'|^2 - 2<s',t'> of coordinates taken relative to the batch's
    first target point c (s' = s - c, t' = t - c, each coordinate rounded
    once): gamma(10) * (|s'|^2 + |t'|^2 + 2 sum_k |s'_k t'_k|) for the norms'
    roundings, a 4-term dot product in any summation order and the final
    addition, plus 4u sum_k (|s'_k| + |t'_k|) |s_k - t_k| for the rounded
    differences. It also covers the direct form from coordinate differences.
    Returns (n_mismatch, n_accepted, failing entries)."""
    got = np.asarray(got)
    ref = np.asarray(ref)
    g10 = 10 * U32 / (1.0 - 10 * U32)
    bad, acc = [], 0
    for b, a in np.argwhere(got != ref):
        tg, to = int(got[b, a]), int(ref[b, a])
        if not 0 <= tg < T64.shape[1]:
            bad.append(((int(b), int(a)), tg, to, "index out of range"))
            continue
        s = A64[b, a]
        c = T64[b, 0]

        def dist_and_bound(t):
            tt = T64[b, t]
            sc, tc = s - c, tt - c
            e = g10 * float((sc * sc).sum() + (tc * tc).sum() + 2.0 * np.abs(sc * tc).sum())
            e += 4 * U32 * float(((np.abs(sc) + np.abs(tc)) * np.abs(s - tt)).sum())
            return float(((s - tt) ** 2).sum()), e

        dg, eg = dist_and_bound(tg)
        do, eo = dist_and_bound(to)
        if dg - do <= eg + eo:
            acc += 1
        else:
            bad.append(((int(b), int(a)), tg, to, f"gap {dg - do:.3e} > bound {eg + eo:.3e}"))
    return int((got != ref).sum()), acc, bad
