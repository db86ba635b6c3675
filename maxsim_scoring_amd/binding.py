"""Python binding of the C ABI in include/maxsim.h (argument marshalling only).

Every function takes torch tensors that live on the GPU, checks that they have
the layout the ABI documents, allocates missing outputs with torch (device
memory is PyTorch's job here) and calls the C entry point of the same name on
the current HIP stream. All arithmetic runs in the HIP kernels; there is no
CPU path. When the library is missing, or a tensor is not on the GPU, the call
raises.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmaxsim_amd.so")

MAXSIM_F16 = 0
MAXSIM_BF16 = 1
D_MODEL = 128

_lib = None


class MaxSimError(RuntimeError):
    """A non-zero status from the library."""

    def __init__(self, fn: str, status: int):
        msg = lib().maxsim_status_string(status).decode()
        super().__init__(f"{fn}: status {status} ({msg})")
        self.status = status


def lib() -> ctypes.CDLL:
    """The loaded C library (loaded once)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"HIP library {LIB_PATH} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, i32, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float
        ci = ctypes.c_int
        L.maxsim_fwd.argtypes = [ci, vp, vp, i64, i64, i64, i64, i64, vp, vp, vp, vp, vp]
        L.maxsim_fwd_varlen.argtypes = [ci, vp, vp, i64, i32, vp, vp, i64, i64, vp, vp, vp]
        L.maxsim_fwd_i8.argtypes = [vp, f32, vp, f32, i64, i64, i64, i64, i64, vp, vp, vp, vp, vp, vp]
        L.maxsim_bwd.argtypes = [ci, vp, vp, i64, i64, i64, i64, i64, vp, vp, vp, vp, vp, vp, vp,
                                 vp, vp]
        L.maxsim_fwd_i8_tok.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i64, vp, vp, vp, vp, vp]
        L.maxsim_fwd_pairs.argtypes = [ci, vp, vp, i64, i64, i64, i64, i64, vp, vp, vp, vp, i64, vp,
                                       vp, vp]
        L.maxsim_topk.argtypes = [vp, i64, i64, i64, vp, vp, vp, vp, vp]
        L.maxsim_fwd_pairs_varlen.argtypes = [ci, vp, vp, i64, i32, vp, vp, i64, i64, vp, vp, i64,
                                              vp, vp, vp]
        L.maxsim_bwd_varlen.argtypes = [ci, vp, vp, i64, i64, i32, vp, vp, i64, i64, i64, vp, vp,
                                        vp, vp, vp, vp, vp]
        L.maxsim_chamfer_fwd.argtypes = [vp, vp, i64, i64, i64, vp, vp, vp, vp, vp, vp]
        L.maxsim_chamfer_bwd.argtypes = [vp, vp, i64, i64, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                         vp, vp]
        for f in (L.maxsim_fwd, L.maxsim_fwd_varlen, L.maxsim_fwd_i8, L.maxsim_bwd,
                  L.maxsim_fwd_i8_tok, L.maxsim_fwd_pairs, L.maxsim_topk,
                  L.maxsim_fwd_pairs_varlen, L.maxsim_bwd_varlen, L.maxsim_chamfer_fwd,
                  L.maxsim_chamfer_bwd):
            f.restype = ci
        L.maxsim_status_string.argtypes = [ci]
        L.maxsim_status_string.restype = ctypes.c_char_p
        L.maxsim_abi_version.argtypes = []
        L.maxsim_abi_version.restype = ci
        _lib = L
    return _lib


def _p(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(name: str, t: Optional[torch.Tensor], dtype=None) -> None:
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")


def _out(name: str, t: Optional[torch.Tensor], dtype, shape) -> None:
    """An output the caller passed in: on the GPU, contiguous, of `dtype` and
    exactly the documented `shape` (the kernels write every element of it)."""
    if t is None:
        return
    _dev(name, t, dtype)
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {list(shape)}, got {list(t.shape)}")


def _out_flat(name: str, t: torch.Tensor, dtype, n: int) -> None:
    """A flat output of n elements; with n == 0 a placeholder of at most one
    element is accepted (the default allocation keeps one)."""
    _dev(name, t, dtype)
    if t.dim() != 1 or (t.numel() != n if n > 0 else t.numel() > 1):
        raise ValueError(f"{name} must have shape [{n}], got {list(t.shape)}")


def _mask(name: str, t: Optional[torch.Tensor], shape) -> None:
    _dev(name, t, torch.uint8)
    if t is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {list(shape)}, got {list(t.shape)}")


def _stream(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float16:
        return MAXSIM_F16
    if t.dtype == torch.bfloat16:
        return MAXSIM_BF16
    raise ValueError(f"embeddings must be float16 or bfloat16, got {t.dtype}")


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise MaxSimError(fn, status)


def maxsim_fwd(Q: torch.Tensor, D: torch.Tensor, q_mask: Optional[torch.Tensor] = None,
               d_mask: Optional[torch.Tensor] = None, want_argmax: bool = False,
               scores: Optional[torch.Tensor] = None, argmax: Optional[torch.Tensor] = None,
               stream=None):
    """Cross-product forward. Q [Nq,Lq,d], D [Nd,Ld,d] fp16/bf16; masks uint8.
    Returns (scores float32 [Nq,Nd], argmax int32 [Nq,Nd,Lq] or None)."""
    Nq, Lq, d = Q.shape
    Nd, Ld, d2 = D.shape
    if d2 != d or D.dtype != Q.dtype:
        raise ValueError("Q and D must share d and dtype")
    _dev("Q", Q)
    _dev("D", D)
    _mask("q_mask", q_mask, (Nq, Lq))
    _mask("d_mask", d_mask, (Nd, Ld))
    if scores is None:
        scores = torch.empty((Nq, Nd), dtype=torch.float32, device=Q.device)
    if argmax is None and want_argmax:
        argmax = torch.empty((Nq, Nd, Lq), dtype=torch.int32, device=Q.device)
    _out("scores", scores, torch.float32, (Nq, Nd))
    _out("argmax", argmax, torch.int32, (Nq, Nd, Lq))
    st = lib().maxsim_fwd(_dtype_code(Q), _p(Q), _p(D), Nq, Nd, Lq, Ld, d, _p(q_mask), _p(d_mask),
                          _p(scores), _p(argmax), _stream(stream))
    _check("maxsim_fwd", st)
    return scores, argmax


def maxsim_fwd_varlen(Q: torch.Tensor, cu_q: torch.Tensor, max_lq: int, D: torch.Tensor,
                      cu_d: torch.Tensor, want_argmax: bool = False,
                      scores: Optional[torch.Tensor] = None,
                      argmax: Optional[torch.Tensor] = None, stream=None):
    """Padding-free forward. Q [Tq,d], D [Td,d] packed; cu_* int32 [N+1].
    Returns (scores [Nq,Nd], argmax [Nq,Nd,max_lq] or None)."""
    if Q.dim() != 2 or D.dim() != 2 or Q.shape[1] != D.shape[1] or Q.dtype != D.dtype:
        raise ValueError("Q and D must be packed [tokens, d] of one dtype")
    d = Q.shape[1]
    for n, t in (("Q", Q), ("D", D)):
        _dev(n, t)
    _dev("cu_q", cu_q, torch.int32)
    _dev("cu_d", cu_d, torch.int32)
    if cu_q.dim() != 1 or cu_d.dim() != 1:
        raise ValueError("cu_q and cu_d must be [N+1]")
    Nq, Nd = cu_q.numel() - 1, cu_d.numel() - 1
    if scores is None:
        scores = torch.empty((Nq, Nd), dtype=torch.float32, device=Q.device)
    if argmax is None and want_argmax:
        argmax = torch.empty((Nq, Nd, max_lq), dtype=torch.int32, device=Q.device)
    _out("scores", scores, torch.float32, (Nq, Nd))
    _out("argmax", argmax, torch.int32, (Nq, Nd, max_lq))
    st = lib().maxsim_fwd_varlen(_dtype_code(Q), _p(Q), _p(cu_q), Nq, int(max_lq), _p(D),
                                 _p(cu_d), Nd, d, _p(scores), _p(argmax), _stream(stream))
    _check("maxsim_fwd_varlen", st)
    return scores, argmax


def maxsim_fwd_i8(Q: torch.Tensor, q_scale: float, D: torch.Tensor, d_scale: float,
                  q_mask: Optional[torch.Tensor] = None, d_mask: Optional[torch.Tensor] = None,
                  want_argmax: bool = False, want_int: bool = True, want_float: bool = True,
                  scores_i32: Optional[torch.Tensor] = None, scores: Optional[torch.Tensor] = None,
                  argmax: Optional[torch.Tensor] = None, stream=None):
    """INT8 forward with per-tensor scales. Returns (scores_i32, scores, argmax)."""
    Nq, Lq, d = Q.shape
    Nd, Ld, d2 = D.shape
    if d2 != d:
        raise ValueError("Q and D must share d")
    _dev("Q", Q, torch.int8)
    _dev("D", D, torch.int8)
    _mask("q_mask", q_mask, (Nq, Lq))
    _mask("d_mask", d_mask, (Nd, Ld))
    dev = Q.device
    if scores_i32 is None and want_int:
        scores_i32 = torch.empty((Nq, Nd), dtype=torch.int32, device=dev)
    if scores is None and want_float:
        scores = torch.empty((Nq, Nd), dtype=torch.float32, device=dev)
    if argmax is None and want_argmax:
        argmax = torch.empty((Nq, Nd, Lq), dtype=torch.int32, device=dev)
    _out("scores_i32", scores_i32, torch.int32, (Nq, Nd))
    _out("scores", scores, torch.float32, (Nq, Nd))
    _out("argmax", argmax, torch.int32, (Nq, Nd, Lq))
    st = lib().maxsim_fwd_i8(_p(Q), float(q_scale), _p(D), float(d_scale), Nq, Nd, Lq, Ld, d,
                             _p(q_mask), _p(d_mask), _p(scores_i32), _p(scores), _p(argmax),
                             _stream(stream))
    _check("maxsim_fwd_i8", st)
    return scores_i32, scores, argmax


def maxsim_bwd(Q: torch.Tensor, D: torch.Tensor, argmax: torch.Tensor, grad_scores: torch.Tensor,
               q_mask: Optional[torch.Tensor] = None, d_mask: Optional[torch.Tensor] = None,
               dQ: Optional[torch.Tensor] = None, dD: Optional[torch.Tensor] = None,
               csr_row_ptr: Optional[torch.Tensor] = None,
               csr_col_idx: Optional[torch.Tensor] = None, stream=None):
    """Backward through a saved argmax. Returns (dQ, dD, csr_row_ptr, csr_col_idx)."""
    Nq, Lq, d = Q.shape
    Nd, Ld, d2 = D.shape
    if d2 != d or D.dtype != Q.dtype:
        raise ValueError("Q and D must share d and dtype")
    _dev("Q", Q)
    _dev("D", D)
    _dev("argmax", argmax, torch.int32)
    _dev("grad_scores", grad_scores, torch.float32)
    _mask("q_mask", q_mask, (Nq, Lq))
    _mask("d_mask", d_mask, (Nd, Ld))
    if tuple(argmax.shape) != (Nq, Nd, Lq) or tuple(grad_scores.shape) != (Nq, Nd):
        raise ValueError("argmax must be [Nq,Nd,Lq] and grad_scores [Nq,Nd]")
    dev = Q.device
    if dQ is None:
        dQ = torch.empty((Nq, Lq, d), dtype=torch.float32, device=dev)
    if dD is None:
        dD = torch.empty((Nd, Ld, d), dtype=torch.float32, device=dev)
    if csr_row_ptr is None:
        csr_row_ptr = torch.empty((Nd * Ld + 1,), dtype=torch.int32, device=dev)
    if csr_col_idx is None:
        csr_col_idx = torch.empty((max(1, Nq * Nd * Lq),), dtype=torch.int32, device=dev)
    _out("dQ", dQ, torch.float32, (Nq, Lq, d))
    _out("dD", dD, torch.float32, (Nd, Ld, d))
    _out("csr_row_ptr", csr_row_ptr, torch.int32, (Nd * Ld + 1,))
    _out_flat("csr_col_idx", csr_col_idx, torch.int32, Nq * Nd * Lq)
    st = lib().maxsim_bwd(_dtype_code(Q), _p(Q), _p(D), Nq, Nd, Lq, Ld, d, _p(q_mask), _p(d_mask),
                          _p(argmax), _p(grad_scores), _p(dQ), _p(dD), _p(csr_row_ptr),
                          _p(csr_col_idx), _stream(stream))
    _check("maxsim_bwd", st)
    return dQ, dD, csr_row_ptr, csr_col_idx[:Nq * Nd * Lq]


def maxsim_fwd_pairs_varlen(Q: torch.Tensor, cu_q: torch.Tensor, max_lq: int, D: torch.Tensor,
                            cu_d: torch.Tensor, pair_q: torch.Tensor, pair_d: torch.Tensor,
                            want_argmax: bool = False, scores: Optional[torch.Tensor] = None,
                            argmax: Optional[torch.Tensor] = None, stream=None):
    """Scores of listed (query, doc) pairs of packed batches. Q [Tq,d], D [Td,d]
    packed; pair_q, pair_d int32 [P]. Returns (scores [P], argmax [P,max_lq] or None)."""
    if Q.dim() != 2 or D.dim() != 2 or Q.shape[1] != D.shape[1] or Q.dtype != D.dtype:
        raise ValueError("Q and D must be packed [tokens, d] of one dtype")
    d = Q.shape[1]
    for n, t in (("Q", Q), ("D", D)):
        _dev(n, t)
    for n, t in (("cu_q", cu_q), ("cu_d", cu_d), ("pair_q", pair_q), ("pair_d", pair_d)):
        _dev(n, t, torch.int32)
    if pair_q.shape != pair_d.shape or pair_q.dim() != 1:
        raise ValueError("pair_q and pair_d must be [P]")
    Nq, Nd, P = cu_q.numel() - 1, cu_d.numel() - 1, pair_q.numel()
    if scores is None:
        scores = torch.empty((P,), dtype=torch.float32, device=Q.device)
    if argmax is None and want_argmax:
        argmax = torch.empty((P, max_lq), dtype=torch.int32, device=Q.device)
    _out("scores", scores, torch.float32, (P,))
    _out("argmax", argmax, torch.int32, (P, max_lq))
    st = lib().maxsim_fwd_pairs_varlen(_dtype_code(Q), _p(Q), _p(cu_q), Nq, int(max_lq), _p(D),
                                       _p(cu_d), Nd, d, _p(pair_q), _p(pair_d), P, _p(scores),
                                       _p(argmax), _stream(stream))
    _check("maxsim_fwd_pairs_varlen", st)
    return scores, argmax


def maxsim_bwd_varlen(Q: torch.Tensor, cu_q: torch.Tensor, max_lq: int, D: torch.Tensor,
                      cu_d: torch.Tensor, argmax: torch.Tensor, grad_scores: torch.Tensor,
                      dQ: Optional[torch.Tensor] = None, dD: Optional[torch.Tensor] = None,
                      csr_row_ptr: Optional[torch.Tensor] = None,
                      csr_col_idx: Optional[torch.Tensor] = None, stream=None):
    """Padding-free backward through the saved [Nq,Nd,max_lq] argmax. Q [Tq,d],
    D [Td,d] packed. Returns (dQ [Tq,d], dD [Td,d], csr_row_ptr [Td+1],
    csr_col_idx [Tq*Nd]: the first Tq*(docs with a token) entries are the CSR)."""
    if Q.dim() != 2 or D.dim() != 2 or Q.shape[1] != D.shape[1] or Q.dtype != D.dtype:
        raise ValueError("Q and D must be packed [tokens, d] of one dtype")
    Tq, d = Q.shape
    Td = D.shape[0]
    for n, t in (("Q", Q), ("D", D)):
        _dev(n, t)
    _dev("cu_q", cu_q, torch.int32)
    _dev("cu_d", cu_d, torch.int32)
    _dev("argmax", argmax, torch.int32)
    _dev("grad_scores", grad_scores, torch.float32)
    Nq, Nd = cu_q.numel() - 1, cu_d.numel() - 1
    if tuple(argmax.shape) != (Nq, Nd, max_lq) or tuple(grad_scores.shape) != (Nq, Nd):
        raise ValueError("argmax must be [Nq,Nd,max_lq] and grad_scores [Nq,Nd]")
    dev = Q.device
    if dQ is None:
        dQ = torch.empty((Tq, d), dtype=torch.float32, device=dev)
    if dD is None:
        dD = torch.empty((Td, d), dtype=torch.float32, device=dev)
    if csr_row_ptr is None:
        csr_row_ptr = torch.empty((Td + 1,), dtype=torch.int32, device=dev)
    if csr_col_idx is None:
        csr_col_idx = torch.empty((max(1, Tq * Nd),), dtype=torch.int32, device=dev)
    _out("dQ", dQ, torch.float32, (Tq, d))
    _out("dD", dD, torch.float32, (Td, d))
    _out("csr_row_ptr", csr_row_ptr, torch.int32, (Td + 1,))
    _out_flat("csr_col_idx", csr_col_idx, torch.int32, Tq * Nd)
    st = lib().maxsim_bwd_varlen(_dtype_code(Q), _p(Q), _p(cu_q), Nq, Tq, int(max_lq), _p(D),
                                 _p(cu_d), Nd, Td, d, _p(argmax), _p(grad_scores), _p(dQ), _p(dD),
                                 _p(csr_row_ptr), _p(csr_col_idx), _stream(stream))
    _check("maxsim_bwd_varlen", st)
    return dQ, dD, csr_row_ptr, csr_col_idx


def maxsim_chamfer_fwd(P: torch.Tensor, Q: torch.Tensor, want_loss: bool = True,
                       dist1: Optional[torch.Tensor] = None, idx1: Optional[torch.Tensor] = None,
                       dist2: Optional[torch.Tensor] = None, idx2: Optional[torch.Tensor] = None,
                       loss: Optional[torch.Tensor] = None, stream=None):
    """Chamfer distance of point-set batches P [B,N,3], Q [B,M,3] float32.
    Returns (dist1 [B,N], idx1 [B,N], dist2 [B,M], idx2 [B,M], loss [B] or None)."""
    if P.dim() != 3 or Q.dim() != 3 or P.shape[2] != 3 or Q.shape[2] != 3 or P.shape[0] != Q.shape[0]:
        raise ValueError("P and Q must be [B,N,3] and [B,M,3]")
    _dev("P", P, torch.float32)
    _dev("Q", Q, torch.float32)
    B, N, _ = P.shape
    M = Q.shape[1]
    dev = P.device
    if dist1 is None:
        dist1 = torch.empty((B, N), dtype=torch.float32, device=dev)
    if idx1 is None:
        idx1 = torch.empty((B, N), dtype=torch.int32, device=dev)
    if dist2 is None:
        dist2 = torch.empty((B, M), dtype=torch.float32, device=dev)
    if idx2 is None:
        idx2 = torch.empty((B, M), dtype=torch.int32, device=dev)
    if loss is None and want_loss:
        loss = torch.empty((B,), dtype=torch.float32, device=dev)
    _out("dist1", dist1, torch.float32, (B, N))
    _out("idx1", idx1, torch.int32, (B, N))
    _out("dist2", dist2, torch.float32, (B, M))
    _out("idx2", idx2, torch.int32, (B, M))
    _out("loss", loss, torch.float32, (B,))
    st = lib().maxsim_chamfer_fwd(_p(P), _p(Q), B, N, M, _p(dist1), _p(idx1), _p(dist2), _p(idx2),
                                  _p(loss), _stream(stream))
    _check("maxsim_chamfer_fwd", st)
    return dist1, idx1, dist2, idx2, loss


def maxsim_chamfer_bwd(P: torch.Tensor, Q: torch.Tensor, idx1: torch.Tensor, idx2: torch.Tensor,
                       grad_dist1: torch.Tensor, grad_dist2: torch.Tensor,
                       dP: Optional[torch.Tensor] = None, dQ: Optional[torch.Tensor] = None,
                       csr_row_ptr1: Optional[torch.Tensor] = None,
                       csr_col_idx1: Optional[torch.Tensor] = None,
                       csr_row_ptr2: Optional[torch.Tensor] = None,
                       csr_col_idx2: Optional[torch.Tensor] = None, stream=None):
    """Chamfer backward through the saved indices. Returns (dP [B,N,3],
    dQ [B,M,3], row_ptr1 [B*M+1], col_idx1 [B*N], row_ptr2 [B*N+1], col_idx2 [B*M])."""
    B, N, _ = P.shape
    M = Q.shape[1]
    _dev("P", P, torch.float32)
    _dev("Q", Q, torch.float32)
    for n, t, shp in (("idx1", idx1, (B, N)), ("idx2", idx2, (B, M))):
        _dev(n, t, torch.int32)
        if tuple(t.shape) != shp:
            raise ValueError(f"{n} must be {list(shp)}")
    for n, t, shp in (("grad_dist1", grad_dist1, (B, N)), ("grad_dist2", grad_dist2, (B, M))):
        _dev(n, t, torch.float32)
        if tuple(t.shape) != shp:
            raise ValueError(f"{n} must be {list(shp)}")
    dev = P.device
    if dP is None:
        dP = torch.empty((B, N, 3), dtype=torch.float32, device=dev)
    if dQ is None:
        dQ = torch.empty((B, M, 3), dtype=torch.float32, device=dev)
    if csr_row_ptr1 is None:
        csr_row_ptr1 = torch.empty((B * M + 1,), dtype=torch.int32, device=dev)
    if csr_col_idx1 is None:
        csr_col_idx1 = torch.empty((max(1, B * N),), dtype=torch.int32, device=dev)
    if csr_row_ptr2 is None:
        csr_row_ptr2 = torch.empty((B * N + 1,), dtype=torch.int32, device=dev)
    if csr_col_idx2 is None:
        csr_col_idx2 = torch.empty((max(1, B * M),), dtype=torch.int32, device=dev)
    _out("dP", dP, torch.float32, (B, N, 3))
    _out("dQ", dQ, torch.float32, (B, M, 3))
    _out("csr_row_ptr1", csr_row_ptr1, torch.int32, (B * M + 1,))
    _out_flat("csr_col_idx1", csr_col_idx1, torch.int32, B * N)
    _out("csr_row_ptr2", csr_row_ptr2, torch.int32, (B * N + 1,))
    _out_flat("csr_col_idx2", csr_col_idx2, torch.int32, B * M)
    st = lib().maxsim_chamfer_bwd(_p(P), _p(Q), B, N, M, _p(idx1), _p(idx2), _p(grad_dist1),
                                  _p(grad_dist2), _p(dP), _p(dQ), _p(csr_row_ptr1), _p(csr_col_idx1),
                                  _p(csr_row_ptr2), _p(csr_col_idx2), _stream(stream))
    _check("maxsim_chamfer_bwd", st)
    return dP, dQ, csr_row_ptr1, csr_col_idx1[:B * N], csr_row_ptr2, csr_col_idx2[:B * M]


def maxsim_status_string(status: int) -> str:
    return lib().maxsim_status_string(status).decode()


def maxsim_abi_version() -> int:
    return lib().maxsim_abi_version()


def maxsim_fwd_i8_tok(Q: torch.Tensor, q_scale: torch.Tensor, D: torch.Tensor,
                      d_scale: torch.Tensor, q_mask: Optional[torch.Tensor] = None,
                      d_mask: Optional[torch.Tensor] = None, want_argmax: bool = False,
                      scores: Optional[torch.Tensor] = None,
                      argmax: Optional[torch.Tensor] = None, stream=None):
    """INT8 forward with per-token scales q_scale [Nq,Lq], d_scale [Nd,Ld]
    (float32, positive). Returns (scores float32 [Nq,Nd], argmax or None)."""
    Nq, Lq, d = Q.shape
    Nd, Ld, d2 = D.shape
    if d2 != d or Q.dtype != torch.int8 or D.dtype != torch.int8:
        raise ValueError("Q and D must be int8 with the same d")
    for n, t in (("Q", Q), ("D", D)):
        _dev(n, t)
    _dev("q_scale", q_scale, torch.float32)
    _dev("d_scale", d_scale, torch.float32)
    if tuple(q_scale.shape) != (Nq, Lq) or tuple(d_scale.shape) != (Nd, Ld):
        raise ValueError("scales must be [Nq, Lq] and [Nd, Ld]")
    _mask("q_mask", q_mask, (Nq, Lq))
    _mask("d_mask", d_mask, (Nd, Ld))
    if scores is None:
        scores = torch.empty((Nq, Nd), dtype=torch.float32, device=Q.device)
    if argmax is None and want_argmax:
        argmax = torch.empty((Nq, Nd, Lq), dtype=torch.int32, device=Q.device)
    _out("scores", scores, torch.float32, (Nq, Nd))
    _out("argmax", argmax, torch.int32, (Nq, Nd, Lq))
    st = lib().maxsim_fwd_i8_tok(_p(Q), _p(q_scale), _p(D), _p(d_scale), Nq, Nd, Lq, Ld, d,
                                 _p(q_mask), _p(d_mask), _p(scores), _p(argmax), _stream(stream))
    _check("maxsim_fwd_i8_tok", st)
    return scores, argmax


def maxsim_fwd_pairs(Q: torch.Tensor, D: torch.Tensor, pair_q: torch.Tensor,
                     pair_d: torch.Tensor, q_mask: Optional[torch.Tensor] = None,
                     d_mask: Optional[torch.Tensor] = None, want_argmax: bool = False,
                     scores: Optional[torch.Tensor] = None,
                     argmax: Optional[torch.Tensor] = None, stream=None):
    """Scores of the listed (query, doc) pairs of dense Q, D (fp16/bf16).
    pair_q, pair_d int32 [P]. Returns (scores [P], argmax [P,Lq] or None)."""
    Nq, Lq, d = Q.shape
    Nd, Ld, d2 = D.shape
    if d2 != d or D.dtype != Q.dtype:
        raise ValueError("Q and D must share d and dtype")
    for n, t in (("Q", Q), ("D", D)):
        _dev(n, t)
    _dev("pair_q", pair_q, torch.int32)
    _dev("pair_d", pair_d, torch.int32)
    P = pair_q.numel()
    if pair_d.numel() != P:
        raise ValueError("pair_q and pair_d must have the same length")
    _mask("q_mask", q_mask, (Nq, Lq))
    _mask("d_mask", d_mask, (Nd, Ld))
    if scores is None:
        scores = torch.empty((P,), dtype=torch.float32, device=Q.device)
    if argmax is None and want_argmax:
        argmax = torch.empty((P, Lq), dtype=torch.int32, device=Q.device)
    _out("scores", scores, torch.float32, (P,))
    _out("argmax", argmax, torch.int32, (P, Lq))
    st = lib().maxsim_fwd_pairs(_dtype_code(Q), _p(Q), _p(D), Nq, Nd, Lq, Ld, d, _p(q_mask),
                                _p(d_mask), _p(pair_q), _p(pair_d), P, _p(scores), _p(argmax),
                                _stream(stream))
    _check("maxsim_fwd_pairs", st)
    return scores, argmax


def maxsim_topk(scores: torch.Tensor, k: int, ids: Optional[torch.Tensor] = None,
                want_rows: bool = False, idx: Optional[torch.Tensor] = None,
                val: Optional[torch.Tensor] = None, rows: Optional[torch.Tensor] = None,
                stream=None):
    """Per-row top-k of scores [Nq,Nd] float32: (idx int32 [Nq,k], val float32
    [Nq,k], rows int32 [Nq,k] or None), values decreasing, equal values in
    increasing column order. With ``ids`` [Nq,Nd] int32, idx reports
    ids[row, column] instead of the column; ``rows`` holds each entry's row."""
    if scores.dim() != 2:
        raise ValueError("scores must be [Nq, Nd]")
    _dev("scores", scores, torch.float32)
    Nq, Nd = scores.shape
    _dev("ids", ids, torch.int32)
    if ids is not None and tuple(ids.shape) != (Nq, Nd):
        raise ValueError("ids must have the shape of scores")
    if idx is None:
        idx = torch.empty((Nq, k), dtype=torch.int32, device=scores.device)
    if val is None:
        val = torch.empty((Nq, k), dtype=torch.float32, device=scores.device)
    if rows is None and want_rows:
        rows = torch.empty((Nq, k), dtype=torch.int32, device=scores.device)
    _out("idx", idx, torch.int32, (Nq, k))
    _out("val", val, torch.float32, (Nq, k))
    _out("rows", rows, torch.int32, (Nq, k))
    st = lib().maxsim_topk(_p(scores), Nq, Nd, k, _p(ids), _p(idx), _p(val), _p(rows),
                           _stream(stream))
    _check("maxsim_topk", st)
    return idx, val, rows


def two_stage_topk(Qi8: torch.Tensor, q_scale: torch.Tensor, Di8: torch.Tensor,
                   d_scale: torch.Tensor, Qf: torch.Tensor, Df: torch.Tensor, k: int,
                   candidates: int, q_mask: Optional[torch.Tensor] = None,
                   d_mask: Optional[torch.Tensor] = None, stream=None):
    """The INT8 -> FP16 top-K scan ("Flash-MaxSim" Sec. 4.1.4): per-token INT8
    scores of every doc, the `candidates` best docs per query, exact fp16/bf16
    scores of those (query, doc) pairs, and the top-k of the rescored
    candidates. Four library calls. Returns (doc idx int32 [Nq,k], exact
    scores float32 [Nq,k], int8-stage scores [Nq,Nd])."""
    Nq = Qi8.shape[0]
    s8, _ = maxsim_fwd_i8_tok(Qi8, q_scale, Di8, d_scale, q_mask, d_mask, stream=stream)
    cand, _, cand_q = maxsim_topk(s8, candidates, want_rows=True, stream=stream)
    exact, _ = maxsim_fwd_pairs(Qf, Df, cand_q.view(-1), cand.view(-1), q_mask, d_mask,
                                stream=stream)
    doc, val, _ = maxsim_topk(exact.view(Nq, candidates), k, ids=cand, stream=stream)
    return doc, val, s8
