"""Algorithmic byte and operation counts for MaxSim scoring.

The byte model is the IO argument of the pages: a fused kernel reads every
operand once and writes only its outputs (TileMaxSim v1, Sec. 2.3 Eqs. (3)-(5)
and Sec. 3.4 Theorem 1; Flash-MaxSim Sec. 4.1.2). The naive path additionally
writes and re-reads the fp32 similarity tensor. These counts are what the
benchmark divides by a measured kernel time; they never include cache effects.
"""

from __future__ import annotations


# --- the pages' own model (pinned by a worked example in the tests) ---------

def flops_naive_model(nq_tokens: int, nd_tokens: int, d: int, B: int) -> int:
    """Eq. (3) of TileMaxSim v1: B*Nq*Nd*(2d + 1) (dot products plus one max compare)."""
    return B * nq_tokens * nd_tokens * (2 * d + 1)


def io_naive_model(nq_tokens: int, nd_tokens: int, d: int, B: int, elem: int = 2) -> int:
    """Eq. (4): read Q and D once, write and read back an fp32 S."""
    return nq_tokens * d * elem + B * nd_tokens * d * elem + 2 * B * nq_tokens * nd_tokens * 4


def io_fused_model(nq_tokens: int, nd_tokens: int, d: int, B: int, elem: int = 2) -> int:
    """Eq. (5): read Q and D once, write B*Nq fp32 values."""
    return nq_tokens * d * elem + B * nd_tokens * d * elem + B * nq_tokens * 4


def similarity_tensor_bytes(n_pairs: int, lq: int, ld: int, elem: int) -> int:
    """Size of the materialised S for n_pairs (query, doc) pairs."""
    return n_pairs * lq * ld * elem


def argmax_bytes(nq: int, nd: int, lq: int) -> int:
    """The saved int32 argmax, [Nq*Nd, Lq]."""
    return nq * nd * lq * 4


# --- per-entry-point algorithmic counts used by the benchmark ----------------

def dense_fwd_bytes(nq: int, nd: int, lq: int, ld: int, d: int, elem: int,
                    q_mask: bool, d_mask: bool, argmax: bool, int_scores: bool = False) -> int:
    """Operands read once, outputs written once."""
    b = nq * lq * d * elem + nd * ld * d * elem + nq * nd * 4
    if q_mask:
        b += nq * lq
    if d_mask:
        b += nd * ld
    if argmax:
        b += nq * nd * lq * 4
    if int_scores:
        b += nq * nd * 4
    return b


def dense_fwd_flops(nq: int, lq: int, d: int, valid_doc_tokens: int) -> int:
    """2*d per (query token, valid doc token, query) product; every query row
    counts because its argmax is produced even when it is masked."""
    return 2 * d * lq * nq * valid_doc_tokens


def varlen_fwd_bytes(tq: int, nq: int, td: int, nd: int, d: int, elem: int,
                     argmax_max_lq: int = 0) -> int:
    """Packed Q and D read once, both offset arrays read once, scores written once."""
    b = (tq + td) * d * elem + (nq + 1) * 4 + (nd + 1) * 4 + nq * nd * 4
    if argmax_max_lq:
        b += nq * nd * argmax_max_lq * 4
    return b


def varlen_fwd_flops(q_lengths, td: int, d: int) -> int:
    return 2 * d * int(sum(q_lengths)) * td


def bwd_compulsory_bytes(nq: int, nd: int, lq: int, ld: int, d: int, elem: int,
                         q_mask: bool, d_mask: bool) -> int:
    """argmax, g, Q, D and masks read once; dQ, dD fp32 written once; the CSR
    (row_ptr, col_idx) written once and read back once."""
    nsrc = nq * nd * lq
    nrows = nd * ld
    b = nsrc * 4 + nq * nd * 4 + nq * lq * d * elem + nd * ld * d * elem
    if q_mask:
        b += nq * lq
    if d_mask:
        b += nd * ld
    b += nq * lq * d * 4 + nd * ld * d * 4
    b += 2 * ((nrows + 1) * 4 + nsrc * 4)
    return b


def bwd_varlen_compulsory_bytes(nq: int, nd: int, max_lq: int, tq: int, td: int, live_docs: int,
                                d: int, elem: int) -> int:
    """Padding-free backward: argmax [Nq,Nd,max_lq], g, packed Q and D and both
    offset arrays read once; dQ, dD fp32 written once; the CSR (row_ptr [Td+1],
    col_idx of Tq per doc with a token) written once and read back once."""
    nnz = tq * live_docs
    b = nq * nd * max_lq * 4 + nq * nd * 4 + (tq + td) * d * elem + (nq + 1 + nd + 1) * 4
    b += (tq + td) * d * 4
    b += 2 * ((td + 1) * 4 + nnz * 4)
    return b


def pairs_varlen_fwd_bytes(q_rows: int, d_rows_per_pair, d: int, elem: int) -> int:
    """Listed packed pairs: the queries read once (they are shared by many
    pairs), each pair's doc rows read once (a doc listed twice is read twice),
    both pair indices read, one score written per pair."""
    n = len(d_rows_per_pair)
    return (int(q_rows) + int(sum(d_rows_per_pair))) * d * elem + n * (4 + 4 + 4)
