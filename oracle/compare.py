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
* Chamfer distances, indices and gradients (chamfer_*): bounds derived from an
  fp32 evaluation of the direct form sum_k (s_k - t_k)^2 and of the gradient
  sums, independent of how the GPU searches.
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
    """Nearest-neighbour indices of one Chamfer direction ("Flash-MaxSim"
    Sec. 4.2.4 defines the distance as the squared Euclidean distance and
    nothing about how it is evaluated): got/ref [B, na] index into the
    targets T64 [B, nt, 3] for the sources A64 [B, na, 3]. A GPU index t_g
    differing from the oracle's t_o is accepted only if
        dist(t_g) - dist(t_o) <= gamma(5) * (dist(t_g) + dist(t_o)),
    with dist the exact squared distance: an fp32 evaluation of the direct form
    sum_k (s_k - t_k)^2 (one rounding per difference, per square and per
    addition, in any order; every term >= 0) has relative error at most
    gamma(5), so either index could be its argmin. The bound does not depend on
    how the GPU searches. Returns (n_mismatch, n_accepted, failing entries)."""
    got = np.asarray(got)
    ref = np.asarray(ref)
    g5 = gamma(5)
    bad, acc = [], 0
    for b, a in np.argwhere(got != ref):
        tg, to = int(got[b, a]), int(ref[b, a])
        if not 0 <= tg < T64.shape[1]:
            bad.append(((int(b), int(a)), tg, to, "index out of range"))
            continue
        dg = float(((A64[b, a] - T64[b, tg]) ** 2).sum())
        do = float(((A64[b, a] - T64[b, to]) ** 2).sum())
        if dg - do <= g5 * (dg + do):
            acc += 1
        else:
            bad.append(((int(b), int(a)), tg, to, f"gap {dg - do:.3e} > bound {g5 * (dg + do):.3e}"))
    return int((got != ref).sum()), acc, bad


def chamfer_dist(got, ref):
    """Nearest-neighbour distances of one Chamfer direction, element by
    element: |got - ref| <= 3.01 * gamma(5) * ref. If the GPU's index obeys
    chamfer_argmin and its distance is a direct-form fp32 evaluation at that
    index (relative error <= gamma(5)), then got lies in
    [(1 - gamma(5)) ref, (1 + gamma(5))^2 / (1 - gamma(5)) ref]. No absolute
    term: a zero distance (coincident points) must come out exactly 0.
    Returns (ok, worst excess, index of the worst)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    if got.size == 0:
        return True, 0.0, None
    excess = np.abs(got - ref) - 3.01 * gamma(5) * np.abs(ref)
    k = int(np.argmax(excess))
    return (bool(np.all(excess <= 0) and np.all(np.isfinite(got))), float(excess.reshape(-1)[k]),
            np.unravel_index(k, got.shape))


def chamfer_dist_at_index(got_dist, got_idx, A64, T64):
    """The distance written for each source is a direct-form fp32 evaluation
    at the index written next to it: |got - exact(idx)| <= gamma(5) * exact(idx).
    Returns (ok, worst excess)."""
    got_idx = np.asarray(got_idx, dtype=np.int64)
    b = np.arange(A64.shape[0])[:, None]
    ex = ((A64 - T64[b, got_idx]) ** 2).sum(-1)
    excess = np.abs(np.asarray(got_dist, dtype=np.float64) - ex) - gamma(5) * ex
    return bool(np.all(excess <= 0)), float(excess.max()) if excess.size else 0.0


def chamfer_loss_tol(depth: int) -> float:
    """Relative tolerance of a Chamfer loss (1/N) sum dist1 + (1/M) sum dist2:
    each distance within 3.01 gamma(5) (chamfer_dist), an fp32 sum of positive
    terms whose rounding depth (the additions any one term passes through) is
    at most `depth`, the rounding of N (or M) to fp32, one division and one
    addition."""
    return 3.01 * gamma(5) + gamma(depth + 3) + gamma(5) * gamma(depth + 3)


def chamfer_grad_bounds(A64, T64, idx_a, idx_t, g_a, g_t):
    """Per point and coordinate of the gradient with respect to the sources A
    (dA[b,p] = 2 g_a[b,p] (A[b,p] - T[b,idx_a[b,p]]) + sum over the targets q
    with idx_t[b,q] = p of 2 g_t[b,q] (A[b,p] - T[b,q])): the sum of the
    terms' magnitudes S and their number n. An fp32 sum of those terms, each
    formed with two roundings (the difference and the product by g; the factor
    2 is exact), in any order, is within gamma(n + 2) * S of the exact sum."""
    B, na, _ = A64.shape
    nt = T64.shape[1]
    b_a = np.broadcast_to(np.arange(B)[:, None], (B, na))
    b_t = np.broadcast_to(np.arange(B)[:, None], (B, nt))
    S = 2 * np.abs(g_a)[..., None] * np.abs(A64 - T64[b_a, idx_a])
    terms = 2 * np.abs(g_t)[..., None] * np.abs(T64 - A64[b_t, idx_t])
    np.add.at(S, (b_t.reshape(-1), np.asarray(idx_t).reshape(-1)), terms.reshape(-1, 3))
    n = np.ones((B, na), np.int64)
    np.add.at(n, (b_t.reshape(-1), np.asarray(idx_t).reshape(-1)), 1)
    return S, n


def chamfer_grad(got, ref, S, n):
    """|got - ref| <= gamma(n + 2) * S element by element (chamfer_grad_bounds).
    Returns (ok, worst excess, index of the worst)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    nn = np.asarray(n, dtype=np.float64)[..., None] + 2
    tol = nn * U32 / (1.0 - nn * U32) * S
    excess = np.abs(got - ref) - tol
    if got.size == 0:
        return True, 0.0, None
    k = int(np.argmax(excess))
    return (bool(np.all(excess <= 0) and np.all(np.isfinite(got))), float(excess.reshape(-1)[k]),
            np.unravel_index(k, got.shape))
