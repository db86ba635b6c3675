"""Python front end of the CPU oracle -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline leg
may import this module. It loads ``liboracle.so`` (built from
``maxsim_oracle.c`` with gcc, never with the HIP toolchain) and passes it
inputs widened exactly to float64 (fp16/bf16/fp32 -> double is exact) or int8.

Functions follow "Flash-MaxSim" Eq. (1), Sec. 4.2.1-4.2.2, Sec. 4.3 and the
"late-interaction-kernels design notes" Forward / Backward / Varlen passages;
the C source lists each reading taken where the pages leave a step open.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "maxsim_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (plain C11 + pthreads)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB)
        i64, i32, dbl, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_double, ctypes.c_void_p
        lib.oracle_fwd_f64.argtypes = [vp, vp, i64, i64, i64, i64, i64, vp, vp, vp, vp, i32]
        lib.oracle_fwd_varlen_f64.argtypes = [vp, vp, i64, i64, vp, vp, i64, i64, vp, vp, i32]
        lib.oracle_fwd_i8.argtypes = [vp, dbl, vp, dbl, i64, i64, i64, i64, i64, vp, vp, vp, vp,
                                      vp, i32]
        lib.oracle_bwd_f64.argtypes = [vp, vp, i64, i64, i64, i64, i64, vp, vp, vp, vp, vp, vp,
                                       vp, vp, i32]
        lib.oracle_fwd_i8_tok.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i64, vp, vp, vp,
                                          vp, i32]
        lib.oracle_topk.argtypes = [vp, i64, i64, i64, vp, vp, i32]
        lib.oracle_fwd_pairs_f64.argtypes = [vp, vp, i64, i64, i64, i64, i64, vp, vp, vp, vp,
                                             i64, vp, vp, i32]
        lib.oracle_bwd_varlen_f64.argtypes = [vp, vp, i64, i64, vp, vp, i64, i64, vp, vp, vp,
                                              vp, vp, vp, i32]
        lib.oracle_fwd_pairs_varlen_f64.argtypes = [vp, vp, i64, i64, vp, vp, i64, i64, vp, vp,
                                                    i64, vp, vp, i32]
        lib.oracle_chamfer_fwd.argtypes = [vp, vp, i64, i64, i64, vp, vp, vp, vp, vp, i32]
        lib.oracle_chamfer_bwd.argtypes = [vp, vp, i64, i64, i64, vp, vp, vp, vp, vp, vp, vp, vp,
                                           vp, vp]
        lib.oracle_chamfer_fwd.restype = ctypes.c_int
        lib.oracle_chamfer_bwd.restype = ctypes.c_int
        for f in (lib.oracle_fwd_f64, lib.oracle_fwd_varlen_f64, lib.oracle_fwd_i8,
                  lib.oracle_bwd_f64, lib.oracle_fwd_i8_tok, lib.oracle_topk,
                  lib.oracle_fwd_pairs_f64, lib.oracle_bwd_varlen_f64,
                  lib.oracle_fwd_pairs_varlen_f64):
            f.restype = ctypes.c_int
        _lib = lib
    return _lib


def default_threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _f64(x) -> np.ndarray:
    """Exact widening to a C-contiguous float64 array (torch or numpy input)."""
    if x is None:
        return None
    if hasattr(x, "detach"):
        x = x.detach().cpu().double().contiguous().numpy()
    return np.ascontiguousarray(x, dtype=np.float64)


def _arr(x, dtype) -> Optional[np.ndarray]:
    if x is None:
        return None
    if hasattr(x, "detach"):
        x = x.detach().cpu().contiguous().numpy()
    return np.ascontiguousarray(x, dtype=dtype)


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise ValueError(f"oracle {what}: input breaks a precondition (code {rc})")


def fwd(Q, D, q_mask=None, d_mask=None, want_argmax=True, threads=None):
    """Cross-product forward. Returns (scores float64 [Nq,Nd], argmax int32
    [Nq,Nd,Lq] or None)."""
    q = _f64(Q)
    dd = _f64(D)
    Nq, Lq, d = q.shape
    Nd, Ld, d2 = dd.shape
    assert d == d2
    qm = _arr(q_mask, np.uint8)
    dm = _arr(d_mask, np.uint8)
    scores = np.zeros((Nq, Nd), np.float64)
    arg = np.zeros((Nq, Nd, Lq), np.int32) if want_argmax else None
    assert np.isfinite(q).all() and np.isfinite(dd).all()
    rc = _load().oracle_fwd_f64(_p(q), _p(dd), Nq, Nd, Lq, Ld, d, _p(qm), _p(dm), _p(scores),
                                _p(arg), threads or default_threads())
    _check(rc, "fwd")
    return scores, arg


def fwd_varlen(Q, cu_q, max_lq, D, cu_d, want_argmax=True, threads=None):
    """Padding-free forward. Returns (scores [Nq,Nd], argmax [Nq,Nd,max_lq] or None)."""
    q = _f64(Q)
    dd = _f64(D)
    cq = _arr(cu_q, np.int32)
    cd = _arr(cu_d, np.int32)
    Nq, Nd = len(cq) - 1, len(cd) - 1
    d = q.shape[1] if q.ndim == 2 else dd.shape[1]
    scores = np.zeros((Nq, Nd), np.float64)
    arg = np.zeros((Nq, Nd, max_lq), np.int32) if want_argmax else None
    rc = _load().oracle_fwd_varlen_f64(_p(q), _p(cq), Nq, max_lq, _p(dd), _p(cd), Nd, d,
                                       _p(scores), _p(arg), threads or default_threads())
    _check(rc, "fwd_varlen")
    return scores, arg


def fwd_i8(Q, q_scale, D, d_scale, q_mask=None, d_mask=None, want_argmax=True, threads=None):
    """INT8 forward. Returns (score_int int64 [Nq,Nd], score float64 [Nq,Nd],
    argmax int32 [Nq,Nd,Lq] or None)."""
    q = _arr(Q, np.int8)
    dd = _arr(D, np.int8)
    Nq, Lq, d = q.shape
    Nd, Ld, _ = dd.shape
    qm = _arr(q_mask, np.uint8)
    dm = _arr(d_mask, np.uint8)
    si = np.zeros((Nq, Nd), np.int64)
    sf = np.zeros((Nq, Nd), np.float64)
    arg = np.zeros((Nq, Nd, Lq), np.int32) if want_argmax else None
    rc = _load().oracle_fwd_i8(_p(q), float(q_scale), _p(dd), float(d_scale), Nq, Nd, Lq, Ld, d,
                               _p(qm), _p(dm), _p(si), _p(sf), _p(arg),
                               threads or default_threads())
    _check(rc, "fwd_i8")
    return si, sf, arg


def bwd(Q, D, argmax, grad_scores, q_mask=None, d_mask=None, threads=None):
    """Backward through a saved argmax. Returns (dQ float64 [Nq,Lq,d],
    dD float64 [Nd,Ld,d], row_ptr int32 [Nd*Ld+1], col_idx int32 [Nq*Nd*Lq])."""
    q = _f64(Q)
    dd = _f64(D)
    Nq, Lq, d = q.shape
    Nd, Ld, _ = dd.shape
    a = _arr(argmax, np.int32)
    g = _f64(grad_scores)
    qm = _arr(q_mask, np.uint8)
    dm = _arr(d_mask, np.uint8)
    dQ = np.zeros((Nq, Lq, d), np.float64)
    dD = np.zeros((Nd, Ld, d), np.float64)
    rp = np.zeros(Nd * Ld + 1, np.int32)
    ci = np.zeros(Nq * Nd * Lq, np.int32)
    rc = _load().oracle_bwd_f64(_p(q), _p(dd), Nq, Nd, Lq, Ld, d, _p(qm), _p(dm), _p(a), _p(g),
                                _p(dQ), _p(dD), _p(rp), _p(ci), threads or default_threads())
    _check(rc, "bwd")
    return dQ, dD, rp, ci


def fwd_i8_tok(Q, q_scale, D, d_scale, q_mask=None, d_mask=None, want_argmax=True, threads=None):
    """INT8 forward with per-token scales q_scale [Nq,Lq], d_scale [Nd,Ld].
    Returns (score float64 [Nq,Nd], argmax int32 [Nq,Nd,Lq] or None)."""
    q = _arr(Q, np.int8)
    dd = _arr(D, np.int8)
    Nq, Lq, d = q.shape
    Nd, Ld, _ = dd.shape
    qs = _f64(q_scale).reshape(Nq, Lq)
    ds = _f64(d_scale).reshape(Nd, Ld)
    qm = _arr(q_mask, np.uint8)
    dm = _arr(d_mask, np.uint8)
    sf = np.zeros((Nq, Nd), np.float64)
    arg = np.zeros((Nq, Nd, Lq), np.int32) if want_argmax else None
    rc = _load().oracle_fwd_i8_tok(_p(q), _p(qs), _p(dd), _p(ds), Nq, Nd, Lq, Ld, d, _p(qm),
                                   _p(dm), _p(sf), _p(arg), threads or default_threads())
    _check(rc, "fwd_i8_tok")
    return sf, arg


def topk(scores, k, threads=None):
    """Per-row top-k of scores [Nq,Nd]: (idx int32 [Nq,k], val float64 [Nq,k]),
    values decreasing, equal values in increasing index order."""
    v = _f64(scores)
    Nq, Nd = v.shape
    idx = np.zeros((Nq, k), np.int32)
    val = np.zeros((Nq, k), np.float64)
    rc = _load().oracle_topk(_p(v), Nq, Nd, k, _p(idx), _p(val), threads or default_threads())
    _check(rc, "topk")
    return idx, val


def fwd_pairs(Q, D, pair_q, pair_d, q_mask=None, d_mask=None, want_argmax=True, threads=None):
    """Scores of the listed (query, doc) pairs of dense Q [Nq,Lq,d], D [Nd,Ld,d].
    Returns (scores float64 [P], argmax int32 [P,Lq] or None)."""
    q = _f64(Q)
    dd = _f64(D)
    Nq, Lq, d = q.shape
    Nd, Ld, _ = dd.shape
    pq = _arr(pair_q, np.int32)
    pd = _arr(pair_d, np.int32)
    P = len(pq)
    qm = _arr(q_mask, np.uint8)
    dm = _arr(d_mask, np.uint8)
    sc = np.zeros(P, np.float64)
    arg = np.zeros((P, Lq), np.int32) if want_argmax else None
    rc = _load().oracle_fwd_pairs_f64(_p(q), _p(dd), Nq, Nd, Lq, Ld, d, _p(qm), _p(dm), _p(pq),
                                      _p(pd), P, _p(sc), _p(arg), threads or default_threads())
    _check(rc, "fwd_pairs")
    return sc, arg


def bwd_varlen(Q, cu_q, max_lq, D, cu_d, argmax, grad_scores, threads=None):
    """Padding-free backward through the saved [Nq, Nd, max_lq] argmax.
    Returns (dQ float64 [Tq,d], dD float64 [Td,d], row_ptr int32 [Td+1],
    col_idx int32 [nnz]) with nnz = Tq * (number of docs with a token)."""
    q = _f64(Q)
    dd = _f64(D)
    cq = _arr(cu_q, np.int32)
    cd = _arr(cu_d, np.int32)
    Nq, Nd = len(cq) - 1, len(cd) - 1
    d = q.shape[1] if q.ndim == 2 else dd.shape[1]
    Tq, Td = int(cq[-1]), int(cd[-1])
    a = _arr(argmax, np.int32)
    g = _f64(grad_scores)
    live = int(np.count_nonzero(np.diff(cd.astype(np.int64)) > 0))
    dQ = np.zeros((Tq, d), np.float64)
    dD = np.zeros((Td, d), np.float64)
    rp = np.zeros(Td + 1, np.int32)
    ci = np.zeros(max(Tq * live, 1), np.int32)
    rc = _load().oracle_bwd_varlen_f64(_p(q), _p(cq), Nq, max_lq, _p(dd), _p(cd), Nd, d, _p(a),
                                       _p(g), _p(dQ), _p(dD), _p(rp), _p(ci),
                                       threads or default_threads())
    _check(rc, "bwd_varlen")
    return dQ, dD, rp, ci[:Tq * live]


def fwd_pairs_varlen(Q, cu_q, max_lq, D, cu_d, pair_q, pair_d, want_argmax=True, threads=None):
    """Scores of listed (query, doc) pairs of packed batches. Returns
    (scores float64 [P], argmax int32 [P, max_lq] or None)."""
    q = _f64(Q)
    dd = _f64(D)
    cq = _arr(cu_q, np.int32)
    cd = _arr(cu_d, np.int32)
    Nq, Nd = len(cq) - 1, len(cd) - 1
    d = q.shape[1] if q.ndim == 2 else dd.shape[1]
    pq = _arr(pair_q, np.int32)
    pd = _arr(pair_d, np.int32)
    P = len(pq)
    scores = np.zeros(P, np.float64)
    arg = np.zeros((P, max_lq), np.int32) if want_argmax else None
    rc = _load().oracle_fwd_pairs_varlen_f64(_p(q), _p(cq), Nq, max_lq, _p(dd), _p(cd), Nd, d,
                                             _p(pq), _p(pd), P, _p(scores), _p(arg),
                                             threads or default_threads())
    _check(rc, "fwd_pairs_varlen")
    return scores, arg


def chamfer_fwd(P, Q, threads=None):
    """Chamfer distance of point-set batches P [B,N,3], Q [B,M,3]. Returns
    (dist1 [B,N], idx1 int32 [B,N], dist2 [B,M], idx2 int32 [B,M], loss [B])."""
    p = _f64(P)
    q = _f64(Q)
    B, N, _ = p.shape
    M = q.shape[1]
    d1 = np.zeros((B, N))
    i1 = np.zeros((B, N), np.int32)
    d2 = np.zeros((B, M))
    i2 = np.zeros((B, M), np.int32)
    loss = np.zeros(B)
    rc = _load().oracle_chamfer_fwd(_p(p), _p(q), B, N, M, _p(d1), _p(i1), _p(d2), _p(i2),
                                    _p(loss), threads or default_threads())
    _check(rc, "chamfer_fwd")
    return d1, i1, d2, i2, loss


def chamfer_bwd(P, Q, idx1, idx2, grad_dist1, grad_dist2):
    """Gradients of sum(g1*dist1) + sum(g2*dist2) at the saved argmins.
    Returns (dP [B,N,3], dQ [B,M,3], row_ptr1 [B*M+1], col_idx1 [B*N],
    row_ptr2 [B*N+1], col_idx2 [B*M])."""
    p = _f64(P)
    q = _f64(Q)
    B, N, _ = p.shape
    M = q.shape[1]
    i1 = _arr(idx1, np.int32)
    i2 = _arr(idx2, np.int32)
    g1 = _f64(grad_dist1)
    g2 = _f64(grad_dist2)
    dP = np.zeros((B, N, 3))
    dQ = np.zeros((B, M, 3))
    rp1 = np.zeros(B * M + 1, np.int32)
    ci1 = np.zeros(max(B * N, 1), np.int32)
    rp2 = np.zeros(B * N + 1, np.int32)
    ci2 = np.zeros(max(B * M, 1), np.int32)
    rc = _load().oracle_chamfer_bwd(_p(p), _p(q), B, N, M, _p(i1), _p(i2), _p(g1), _p(g2), _p(dP),
                                    _p(dQ), _p(rp1), _p(ci1), _p(rp2), _p(ci2))
    _check(rc, "chamfer_bwd")
    return dP, dQ, rp1, ci1[:B * N], rp2, ci2[:B * M]
