"""Seeded synthetic inputs for the MaxSim workloads.

This module only draws data: token embeddings, sequence lengths, masks, saved
argmax maps and upstream gradients, and it quantises embeddings to int8 for the
INT8 workload. It holds no part of the scoring arithmetic. Both the HIP path and
the CPU oracle are fed from here, so the two always see identical bytes.

Recipe (the same for every workload):
  * an embedding row is d i.i.d. standard normal float32 draws (d = 128 unless a
    workload names another width) divided by
    the row's l2 norm (computed in float32), then rounded to nearest-even into
    the workload dtype (fp16 via numpy, bf16 via torch's CPU cast);
  * rows are produced in chunks of ``CHUNK_ROWS``; chunk ``c`` of stream ``s``
    under seed ``seed`` comes from ``numpy.random.default_rng([seed, s, c])``
    (PCG64), so the result does not depend on the number of worker threads;
  * integers (lengths, mask prefixes, argmax draws) come from
    ``default_rng([seed, s])`` streams of their own.

The shapes and distributions follow the pages' workloads: ColBERT reranking
(one 32-token query against passages of 50-300 tokens, packed without
padding), ColPali in-batch contrastive scoring (128 queries of 128 tokens
against 128 pages of 1024 patches with prefix masks), long-query INT8
scoring with per-tensor symmetric scales, and the embedding-width sweep (one
32-token query against 10,000 docs of 128 tokens at widths 64 to 768).
"""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

D_MODEL = 128
CHUNK_ROWS = 1 << 15

# stream ids inside one seed
_S_LEN, _S_Q, _S_D, _S_QMASK, _S_DMASK, _S_G, _S_ARG, _S_MISC = range(8)


def _workers() -> int:
    n = os.cpu_count() or 1
    return max(1, min(16, n))


def _unit_rows_f32_chunk(seed: int, stream: int, chunk: int, rows: int, d: int) -> np.ndarray:
    rng = np.random.default_rng([seed, stream, chunk])
    x = rng.standard_normal((rows, d), dtype=np.float32)
    x /= np.sqrt(np.einsum("ij,ij->i", x, x))[:, None]
    return x


def unit_rows(seed: int, stream: int, n_rows: int, d: int = D_MODEL,
              dtype: torch.dtype = torch.float16) -> torch.Tensor:
    """``n_rows`` l2-normalised Gaussian rows as a CPU tensor of ``dtype``.

    ``dtype`` is one of float16, bfloat16, float32.
    """
    out = torch.empty((n_rows, d), dtype=dtype)
    nchunks = (n_rows + CHUNK_ROWS - 1) // CHUNK_ROWS

    def fill(c: int) -> None:
        lo = c * CHUNK_ROWS
        hi = min(n_rows, lo + CHUNK_ROWS)
        x = _unit_rows_f32_chunk(seed, stream, c, hi - lo, d)
        out[lo:hi] = torch.from_numpy(x).to(dtype)

    if nchunks <= 1:
        for c in range(nchunks):
            fill(c)
    else:
        with ThreadPoolExecutor(_workers()) as ex:
            list(ex.map(fill, range(nchunks)))
    return out


def quantise_per_tensor(x: torch.Tensor) -> tuple[torch.Tensor, float]:
    """Symmetric per-tensor int8: s = max|x|/127 (float32),
    q = clamp(round_half_even(x/s), -127, 127)."""
    xf = x.float()
    amax = float(xf.abs().max()) if xf.numel() else 1.0
    s = np.float32(amax / 127.0) if amax > 0 else np.float32(1.0)
    q = torch.empty(x.shape, dtype=torch.int8)
    flat_in = xf.reshape(-1)
    flat_out = q.reshape(-1)
    step = 1 << 24

    def fill(c: int) -> None:
        lo = c * step
        hi = min(flat_in.numel(), lo + step)
        v = np.rint(flat_in[lo:hi].numpy() / s)
        flat_out[lo:hi] = torch.from_numpy(np.clip(v, -127, 127).astype(np.int8))

    n = (flat_in.numel() + step - 1) // step
    with ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(fill, range(n)))
    return q, float(s)


def quantise_per_token(x: torch.Tensor) -> tuple[torch.Tensor, torch.Tensor]:
    """Symmetric int8 with one scale per row (token) of x [..., d]:
    s = max|row|/127 (float32; 1 for an all-zero row),
    q = clamp(round_half_even(row/s), -127, 127). Returns (q int8, s float32 [...])."""
    xf = x.float().reshape(-1, x.shape[-1])
    q = torch.empty(xf.shape, dtype=torch.int8)
    s = torch.empty(xf.shape[0], dtype=torch.float32)
    step = 1 << 16

    def fill(c: int) -> None:
        lo = c * step
        hi = min(xf.shape[0], lo + step)
        rows = xf[lo:hi].numpy()
        amax = np.abs(rows).max(axis=1) if rows.shape[1] else np.zeros(rows.shape[0], np.float32)
        sc = np.where(amax > 0, amax / np.float32(127.0), np.float32(1.0)).astype(np.float32)
        v = np.rint(rows / sc[:, None])
        q[lo:hi] = torch.from_numpy(np.clip(v, -127, 127).astype(np.int8))
        s[lo:hi] = torch.from_numpy(sc)

    n = (xf.shape[0] + step - 1) // step
    with ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(fill, range(n)))
    return q.view(x.shape), s.view(x.shape[:-1])


def prefix_mask(lengths: np.ndarray, width: int) -> torch.Tensor:
    """uint8 [len(lengths), width] with the first lengths[r] entries of row r set."""
    ar = np.arange(width)[None, :]
    return torch.from_numpy((ar < np.asarray(lengths)[:, None]).astype(np.uint8))


def cu_seqlens(lengths: np.ndarray) -> torch.Tensor:
    """int32 [N+1] offsets, FlashAttention convention."""
    cu = np.zeros(len(lengths) + 1, dtype=np.int64)
    np.cumsum(lengths, out=cu[1:])
    if cu[-1] >= 2**31:
        raise ValueError("packed token count does not fit int32 offsets")
    return torch.from_numpy(cu.astype(np.int32))


@dataclass
class Dense:
    """Cross-product workload: Q [Nq,Lq,d], D [Nd,Ld,d] with optional masks."""
    name: str
    Q: torch.Tensor
    D: torch.Tensor
    q_mask: Optional[torch.Tensor] = None
    d_mask: Optional[torch.Tensor] = None
    want_argmax: bool = True
    seed: int = 0
    meta: dict = field(default_factory=dict)


@dataclass
class Varlen:
    """Padding-free workload: packed Q [cu_q[-1],d], D [cu_d[-1],d]."""
    name: str
    Q: torch.Tensor
    cu_q: torch.Tensor
    max_lq: int
    D: torch.Tensor
    cu_d: torch.Tensor
    want_argmax: bool = False
    seed: int = 0
    meta: dict = field(default_factory=dict)


@dataclass
class Int8:
    """INT8 cross-product workload with per-tensor scales."""
    name: str
    Q: torch.Tensor
    q_scale: float
    D: torch.Tensor
    d_scale: float
    q_mask: Optional[torch.Tensor] = None
    d_mask: Optional[torch.Tensor] = None
    want_argmax: bool = False
    seed: int = 0
    meta: dict = field(default_factory=dict)


@dataclass
class Int8Tok:
    """INT8 cross-product workload with one scale per token, plus (optionally)
    the float rows the int8 values were quantised from, for rescoring."""
    name: str
    Q: torch.Tensor
    q_scale: torch.Tensor  # [Nq, Lq] float32
    D: torch.Tensor
    d_scale: torch.Tensor  # [Nd, Ld] float32
    q_mask: Optional[torch.Tensor] = None
    d_mask: Optional[torch.Tensor] = None
    Qf: Optional[torch.Tensor] = None  # fp16/bf16 copies for the rescoring stage
    Df: Optional[torch.Tensor] = None
    seed: int = 0


@dataclass
class Backward:
    """Backward workload: forward tensors plus a saved argmax and dL/dscore."""
    name: str
    fwd: Dense
    argmax: torch.Tensor
    grad_scores: torch.Tensor
    seed: int = 0


# --------------------------------------------------------------------------
# The five workloads of the pages, at full size.
# --------------------------------------------------------------------------

def tiny_fp16(seed: int = 1) -> Dense:
    """4 queries x 32 docs, Lq=32, Ld=180, fp16, no masks, argmax on."""
    Nq, Nd, Lq, Ld = 4, 32, 32, 180
    Q = unit_rows(seed, _S_Q, Nq * Lq).view(Nq, Lq, D_MODEL)
    D = unit_rows(seed, _S_D, Nd * Ld).view(Nd, Ld, D_MODEL)
    return Dense("tiny_fp16_4x32_lq32_ld180", Q, D, None, None, True, seed)


def rerank_lengths(seed: int, n_docs: int, lo: int = 50, hi: int = 300) -> np.ndarray:
    return np.random.default_rng([seed, _S_LEN]).integers(lo, hi + 1, size=n_docs)


def rerank_varlen_fp16(seed: int = 2, n_docs: int = 100_000, lq: int = 32) -> Varlen:
    """One 32-token query against n_docs packed passages of 50-300 tokens."""
    lengths = rerank_lengths(seed, n_docs)
    cu_d = cu_seqlens(lengths)
    T = int(cu_d[-1])
    Q = unit_rows(seed, _S_Q, lq)
    D = unit_rows(seed, _S_D, T)
    cu_q = torch.tensor([0, lq], dtype=torch.int32)
    return Varlen(f"rerank_varlen_fp16_1x{n_docs}_lq{lq}_ld50-300", Q, cu_q, lq, D, cu_d,
                  False, seed, {"tokens": T})


def colpali_bf16(seed: int = 3, Nq: int = 128, Nd: int = 128, Lq: int = 128,
                 Ld: int = 1024) -> Dense:
    """In-batch contrastive cross-product with prefix masks, bf16, argmax on.

    q_mask keeps the first k ~ U{16..Lq} tokens, d_mask the first
    m ~ U{768..Ld} patches (bounds scaled when Lq, Ld are reduced).
    """
    Q = unit_rows(seed, _S_Q, Nq * Lq, dtype=torch.bfloat16).view(Nq, Lq, D_MODEL)
    D = unit_rows(seed, _S_D, Nd * Ld, dtype=torch.bfloat16).view(Nd, Ld, D_MODEL)
    k = np.random.default_rng([seed, _S_QMASK]).integers(min(16, Lq), Lq + 1, size=Nq)
    m = np.random.default_rng([seed, _S_DMASK]).integers((3 * Ld) // 4, Ld + 1, size=Nd)
    return Dense(f"colpali_bf16_{Nq}x{Nd}_lq{Lq}_ld{Ld}_masked", Q, D,
                 prefix_mask(k, Lq), prefix_mask(m, Ld), True, seed,
                 {"k": k, "m": m})


def dim_scaling_fp16(d: int, seed: int = 6, Nd: int = 10_000, Lq: int = 32, Ld: int = 128) -> Dense:
    """The embedding-width sweep: one 32-token query against Nd uniform docs
    of 128 tokens, fp16, rows of width d, no masks."""
    Q = unit_rows(seed, _S_Q, Lq, d).view(1, Lq, d)
    D = unit_rows(seed, _S_D, Nd * Ld, d).view(Nd, Ld, d)
    return Dense(f"dim_fp16_1x{Nd}_lq{Lq}_ld{Ld}_d{d}", Q, D, None, None, False, seed)


def int8_long_query(seed: int = 4, Nd: int = 10_000, Lq: int = 1024, Ld: int = 1024) -> Int8:
    """One 1024-token query against Nd docs of 1024 tokens, int8 per-tensor."""
    Qf = unit_rows(seed, _S_Q, Lq, dtype=torch.float32).view(1, Lq, D_MODEL)
    Df = unit_rows(seed, _S_D, Nd * Ld, dtype=torch.float32).view(Nd, Ld, D_MODEL)
    Q, qs = quantise_per_tensor(Qf)
    del Qf
    D, ds = quantise_per_tensor(Df)
    del Df
    return Int8(f"int8_1x{Nd}_lq{Lq}_ld{Ld}", Q, qs, D, ds, None, None, False, seed)


def two_stage_long_query(seed: int = 4, Nd: int = 10_000, Lq: int = 1024, Ld: int = 1024,
                         float_dtype: torch.dtype = torch.float16) -> Int8Tok:
    """The long-query INT8 corpus with per-token scales (the rows of
    ``int8_long_query``), with fp16 copies of the same unit rows for the
    rescoring stage of the INT8 -> FP16 top-K scan."""
    Qf = unit_rows(seed, _S_Q, Lq, dtype=torch.float32).view(1, Lq, D_MODEL)
    Q, qs = quantise_per_token(Qf)
    Qh = Qf.to(float_dtype)
    del Qf
    Df = unit_rows(seed, _S_D, Nd * Ld, dtype=torch.float32).view(Nd, Ld, D_MODEL)
    D, ds = quantise_per_token(Df)
    Dh = Df.to(float_dtype)
    del Df
    return Int8Tok(f"int8tok_1x{Nd}_lq{Lq}_ld{Ld}", Q, qs, D, ds, None, None, Qh, Dh, seed)


def colpali_backward(seed: int = 5, fwd: Optional[Dense] = None,
                     argmax: Optional[torch.Tensor] = None) -> Backward:
    """Backward at the ColPali shapes: g ~ N(0,1) [Nq,Nd] float32.

    ``argmax`` is the saved forward argmax when the caller has one; otherwise it
    is drawn uniformly over each doc's valid (unmasked) tokens, which is the
    distribution Gaussian embeddings give.
    """
    if fwd is None:
        fwd = colpali_bf16()
    Nq, Lq = fwd.Q.shape[0], fwd.Q.shape[1]
    Nd, Ld = fwd.D.shape[0], fwd.D.shape[1]
    g = torch.from_numpy(np.random.default_rng(seed).standard_normal((Nq, Nd)).astype(np.float32))
    if argmax is None:
        argmax = draw_argmax(seed, Nq, Nd, Lq, Ld, fwd.d_mask)
    return Backward(f"backward_{fwd.name}", fwd, argmax, g, seed)


def draw_argmax(seed: int, Nq: int, Nd: int, Lq: int, Ld: int,
                d_mask: Optional[torch.Tensor] = None, hub_frac: float = 0.0) -> torch.Tensor:
    """int32 [Nq,Nd,Lq] indices uniform over each doc's valid prefix.

    With ``hub_frac`` > 0 that fraction of entries points at token 0 of the
    doc, a stand-in for the frequent tokens real corpora have.
    """
    rng = np.random.default_rng([seed, _S_ARG])
    if Ld == 0:
        return torch.zeros((Nq, Nd, Lq), dtype=torch.int32)
    if d_mask is None:
        hi = np.full(Nd, Ld)
    else:
        dm = d_mask.numpy().astype(bool)
        # index one past the last valid token (masks here are prefixes)
        hi = np.where(dm.any(1), Ld - np.argmax(dm[:, ::-1], axis=1), 1)
    u = rng.random((Nq, Nd, Lq))
    a = np.floor(u * hi[None, :, None]).astype(np.int64)
    a = np.minimum(a, hi[None, :, None] - 1)
    if hub_frac > 0:
        hub = rng.random((Nq, Nd, Lq)) < hub_frac
        a[hub] = 0
    return torch.from_numpy(a.astype(np.int32))


def draw_argmax_varlen(seed: int, cu_q, cu_d, max_lq: int, hub_frac: float = 0.0) -> torch.Tensor:
    """int32 [Nq,Nd,max_lq] doc-relative indices uniform over each packed doc's
    tokens for the real rows of each query; rows past a query's length and
    every row of an empty doc are 0 (the packed forward's layout). With
    ``hub_frac`` > 0 that fraction of real entries points at token 0."""
    cq = np.asarray(cu_q, dtype=np.int64)
    cd = np.asarray(cu_d, dtype=np.int64)
    lq, ld = np.diff(cq), np.diff(cd)
    rng = np.random.default_rng([seed, _S_ARG])
    Nq, Nd = len(lq), len(ld)
    u = rng.random((Nq, Nd, max_lq))
    a = np.floor(u * np.maximum(ld, 1)[None, :, None]).astype(np.int64)
    a = np.minimum(a, np.maximum(ld, 1)[None, :, None] - 1)
    if hub_frac > 0:
        a[rng.random((Nq, Nd, max_lq)) < hub_frac] = 0
    real = (np.arange(max_lq)[None, None, :] < lq[:, None, None]) & (ld[None, :, None] > 0)
    return torch.from_numpy(np.where(real, a, 0).astype(np.int32))


# --------------------------------------------------------------------------
# Small and stress inputs for parity (not timed).
# --------------------------------------------------------------------------

def random_dense(seed: int, Nq: int, Nd: int, Lq: int, Ld: int,
                 dtype: torch.dtype = torch.float16, q_mask_p: float = 0.0,
                 d_mask_p: float = 0.0, dup_tokens: bool = False,
                 dead_docs: int = 0, dead_queries: int = 0,
                 want_argmax: bool = True, d: int = D_MODEL) -> Dense:
    """Random masks (Bernoulli keep-probabilities 1-p), optionally duplicated
    doc tokens (exact ties), fully masked docs and fully masked queries."""
    Q = unit_rows(seed, _S_Q, Nq * Lq, d, dtype=dtype).view(Nq, Lq, d)
    D = unit_rows(seed, _S_D, Nd * Ld, d, dtype=dtype).view(Nd, Ld, d).clone()
    rng = np.random.default_rng([seed, _S_MISC])
    if dup_tokens and Ld >= 2:
        for j in range(Nd):
            src = rng.integers(0, Ld, size=max(1, Ld // 4))
            dst = rng.integers(0, Ld, size=src.size)
            D[j, dst] = D[j, src]
    qm = dm = None
    if q_mask_p > 0 or dead_queries > 0:
        qm = torch.from_numpy((rng.random((Nq, Lq)) >= q_mask_p).astype(np.uint8))
        qm[:min(dead_queries, Nq)] = 0
    if d_mask_p > 0 or dead_docs > 0:
        dm = torch.from_numpy((rng.random((Nd, Ld)) >= d_mask_p).astype(np.uint8))
        dm[Nd - min(dead_docs, Nd):] = 0
    return Dense(f"random_{Nq}x{Nd}_lq{Lq}_ld{Ld}", Q, D, qm, dm, want_argmax, seed)


def random_varlen(seed: int, q_lengths, d_lengths, dtype: torch.dtype = torch.float16,
                  max_lq: Optional[int] = None, want_argmax: bool = True,
                  d: int = D_MODEL) -> Varlen:
    q_lengths = np.asarray(q_lengths, dtype=np.int64)
    d_lengths = np.asarray(d_lengths, dtype=np.int64)
    cu_q = cu_seqlens(q_lengths)
    cu_d = cu_seqlens(d_lengths)
    Q = unit_rows(seed, _S_Q, int(cu_q[-1]), d, dtype=dtype)
    D = unit_rows(seed, _S_D, int(cu_d[-1]), d, dtype=dtype)
    mlq = int(q_lengths.max()) if max_lq is None and len(q_lengths) else (max_lq or 0)
    return Varlen(f"varlen_{len(q_lengths)}x{len(d_lengths)}", Q, cu_q, mlq, D, cu_d,
                  want_argmax, seed)


def random_int8(seed: int, Nq: int, Nd: int, Lq: int, Ld: int, ternary: bool = False,
                extreme: bool = False, d_mask_p: float = 0.0, q_mask_p: float = 0.0,
                want_argmax: bool = True, d: int = D_MODEL) -> Int8:
    """Quantised unit rows; ``ternary`` draws values in {-1,0,1} (many exact
    ties); ``extreme`` fills everything with +-127 (largest int32 sums)."""
    rng = np.random.default_rng([seed, _S_MISC])
    if ternary or extreme:
        if extreme:
            Q = torch.full((Nq, Lq, d), 127, dtype=torch.int8)
            D = torch.from_numpy(np.where(rng.random((Nd, Ld, d)) < 0.9, 127, -127)
                                 .astype(np.int8))
        else:
            Q = torch.from_numpy(rng.integers(-1, 2, size=(Nq, Lq, d)).astype(np.int8))
            D = torch.from_numpy(rng.integers(-1, 2, size=(Nd, Ld, d)).astype(np.int8))
        qs, ds = 0.0078125, 0.015625
    else:
        Qf = unit_rows(seed, _S_Q, Nq * Lq, d, dtype=torch.float32).view(Nq, Lq, d)
        Df = unit_rows(seed, _S_D, Nd * Ld, d, dtype=torch.float32).view(Nd, Ld, d)
        Q, qs = quantise_per_tensor(Qf)
        D, ds = quantise_per_tensor(Df)
    qm = dm = None
    if q_mask_p > 0:
        qm = torch.from_numpy((rng.random((Nq, Lq)) >= q_mask_p).astype(np.uint8))
    if d_mask_p > 0:
        dm = torch.from_numpy((rng.random((Nd, Ld)) >= d_mask_p).astype(np.uint8))
    return Int8(f"int8_{Nq}x{Nd}_lq{Lq}_ld{Ld}", Q, qs, D, ds, qm, dm, want_argmax, seed)


def hub_docs(dense: Dense) -> Dense:
    """Copy of ``dense`` where token 0 of every doc is the normalised mean of
    all query rows, so most query tokens pick it (a hot destination row)."""
    q = dense.Q.double().reshape(-1, dense.Q.shape[-1]).mean(0)
    q = q / q.norm()
    D = dense.D.clone()
    D[:, 0] = q.to(D.dtype)
    return Dense(dense.name + "_hub", dense.Q, D, dense.q_mask, dense.d_mask,
                 dense.want_argmax, dense.seed)


def upstream_grad(seed: int, Nq: int, Nd: int) -> torch.Tensor:
    return torch.from_numpy(np.random.default_rng([seed, _S_G]).standard_normal((Nq, Nd))
                            .astype(np.float32))


def random_int8_tok(seed: int, Nq: int, Nd: int, Lq: int, Ld: int, q_mask_p: float = 0.0,
                    d_mask_p: float = 0.0, dead_docs: int = 0, pow2_scales: bool = False,
                    float_dtype: Optional[torch.dtype] = None, d: int = D_MODEL) -> Int8Tok:
    """Per-token quantised unit rows. ``pow2_scales`` replaces the scales by
    powers of two in [2^-9, 2^-5] (every product is then exact in float64)."""
    rng = np.random.default_rng([seed, _S_MISC])
    Qf = unit_rows(seed, _S_Q, Nq * Lq, d, dtype=torch.float32).view(Nq, Lq, d)
    Df = unit_rows(seed, _S_D, Nd * Ld, d, dtype=torch.float32).view(Nd, Ld, d)
    Q, qs = quantise_per_token(Qf)
    D, ds = quantise_per_token(Df)
    if pow2_scales:
        qs = torch.from_numpy(np.ldexp(1.0, rng.integers(-9, -4, size=(Nq, Lq))).astype(np.float32))
        ds = torch.from_numpy(np.ldexp(1.0, rng.integers(-9, -4, size=(Nd, Ld))).astype(np.float32))
    qm = dm = None
    if q_mask_p > 0:
        qm = torch.from_numpy((rng.random((Nq, Lq)) >= q_mask_p).astype(np.uint8))
    if d_mask_p > 0 or dead_docs:
        dm = torch.from_numpy((rng.random((Nd, Ld)) >= d_mask_p).astype(np.uint8))
        for j in range(min(dead_docs, Nd)):
            dm[Nd - 1 - j] = 0
    Qh = Qf.to(float_dtype) if float_dtype is not None else None
    Dh = Df.to(float_dtype) if float_dtype is not None else None
    return Int8Tok(f"int8tok_{Nq}x{Nd}_lq{Lq}_ld{Ld}", Q, qs, D, ds, qm, dm, Qh, Dh, seed)


def random_scores(seed: int, Nq: int, Nd: int, ties: bool = False) -> torch.Tensor:
    """Scores [Nq, Nd] float32 for the top-k step; ``ties`` rounds them to a
    coarse grid so that many values repeat."""
    v = np.random.default_rng([seed, _S_MISC]).standard_normal((Nq, Nd)).astype(np.float32)
    if ties:
        v = np.round(v * 4.0).astype(np.float32) / np.float32(4.0)
    return torch.from_numpy(v)


def random_pairs(seed: int, Nq: int, Nd: int, P: int) -> tuple[torch.Tensor, torch.Tensor]:
    """P (query, doc) index pairs, int32, drawn uniformly (repeats allowed)."""
    rng = np.random.default_rng([seed, _S_ARG])
    return (torch.from_numpy(rng.integers(0, Nq, size=P).astype(np.int32)),
            torch.from_numpy(rng.integers(0, Nd, size=P).astype(np.int32)))


# -------------------------------------------------------------------------- Chamfer

_S_PTS = 8  # stream of point-cloud draws


def point_clouds(seed: int, B: int, N: int, M: int) -> tuple[torch.Tensor, torch.Tensor]:
    """Batches of 3-D point sets P [B,N,3] and Q [B,M,3], float32, coordinates
    i.i.d. N(0,1) (a stand-in for shape-matching point clouds)."""
    rng = np.random.default_rng([seed, _S_PTS])
    P = rng.standard_normal((B, N, 3)).astype(np.float32)
    Q = rng.standard_normal((B, M, 3)).astype(np.float32)
    return torch.from_numpy(P), torch.from_numpy(Q)


def chamfer_grads(seed: int, B: int, N: int, M: int) -> tuple[torch.Tensor, torch.Tensor]:
    """Upstream gradients of the per-point distances, [B,N] and [B,M] float32."""
    rng = np.random.default_rng([seed, _S_G])
    return (torch.from_numpy(rng.standard_normal((B, N)).astype(np.float32)),
            torch.from_numpy(rng.standard_normal((B, M)).astype(np.float32)))
