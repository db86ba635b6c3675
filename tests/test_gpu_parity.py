"""GPU parity: every entry point of the HIP library against the CPU oracle.

All calls go through the C ABI (via the ctypes binding). Inputs come from the
seeded generators; expected values come only from the oracle (run here, or
stored by a script under tests/golden that calls only the oracle). Rules (see
oracle/compare.py): float scores/gradients within 1e-3 + 1e-4*|ref|; int8
sums, int8 argmax and CSR maps bit-exact; float argmax exact except for
certified near-ties; Chamfer distances, indices and gradients within bounds
derived from an fp32 direct-form evaluation.
"""

import hashlib
import json
import os

import numpy as np
import pytest
import torch

from maxsim_scoring_amd import synth
from oracle import compare

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _say(msg):
    print(f"[case] {msg}", flush=True)


@pytest.fixture(scope="module")
def ms():
    import maxsim_scoring_amd as m
    m.binding.lib()
    assert torch.cuda.is_available()
    return m


def _g(t):
    return None if t is None else t.to(DEV)


def _assert_close(name, got, ref):
    ok, worst, where = compare.close(got, ref)
    assert ok, f"{name}: worst excess {worst:.3e} at {where}"


def _assert_float_argmax(name, got, ref, w, pairs=None):
    n, acc, bad = compare.dense_argmax_float(got, ref, w.Q.double().numpy(), w.D.double().numpy(),
                                             None if w.d_mask is None else w.d_mask.numpy(), pairs)
    assert not bad, f"{name}: {len(bad)} argmax mismatches outside the near-tie bound: {bad[:5]}"
    return n, acc


def _run_dense(ms, w, want_argmax=True):
    s, a = ms.maxsim_fwd(_g(w.Q), _g(w.D), _g(w.q_mask), _g(w.d_mask), want_argmax=want_argmax)
    torch.cuda.synchronize()
    return s.cpu(), (None if a is None else a.cpu())


# --------------------------------------------------------------------- dense

DENSE_CASES = [
    # (Nq, Nd, Lq, Ld, dtype, q_mask_p, d_mask_p, dead_docs, dead_queries, dup)
    (4, 32, 32, 180, torch.float16, 0.0, 0.0, 0, 0, False),    # the tiny workload's shape
    (3, 5, 45, 200, torch.bfloat16, 0.3, 0.3, 1, 1, False),    # ragged tiles, masks, dead rows
    (9, 4, 32, 64, torch.float16, 0.0, 0.1, 0, 0, False),      # 8 queries per workgroup + 1
    (2, 3, 300, 130, torch.bfloat16, 0.2, 0.0, 0, 0, False),   # long query: two passes
    (2, 2, 1, 1, torch.float16, 0.0, 0.0, 0, 0, False),        # Lq = Ld = 1
    (1, 3, 7, 70, torch.float16, 0.0, 0.0, 0, 0, True),        # duplicated doc tokens
    (5, 7, 128, 96, torch.bfloat16, 0.5, 0.5, 2, 1, False),
    (2, 2, 33, 65, torch.float16, 0.0, 0.0, 0, 0, False),      # one past a tile edge
]


@pytest.mark.parametrize("case", DENSE_CASES, ids=lambda c: f"{c[0]}x{c[1]}_lq{c[2]}_ld{c[3]}_{str(c[4])[6:]}")
def test_dense_small(ms, case, oracle_mod):
    Nq, Nd, Lq, Ld, dt, qp, dp, dd, dq, dup = case
    _say(f"dense {case}")
    w = synth.random_dense(100 + Lq + Ld, Nq, Nd, Lq, Ld, dtype=dt, q_mask_p=qp, d_mask_p=dp,
                           dead_docs=dd, dead_queries=dq, dup_tokens=dup)
    s, a = _run_dense(ms, w)
    rs, ra = oracle_mod.fwd(w.Q, w.D, w.q_mask, w.d_mask)
    _assert_close("scores", s.numpy(), rs)
    _assert_float_argmax("argmax", a.numpy(), ra, w)
    # no-argmax variant gives the same scores
    s2, _ = _run_dense(ms, w, want_argmax=False)
    _assert_close("scores (no argmax)", s2.numpy(), rs)


EXACT_TIE_CASES = [
    # (Nq, Nd, Lq, Ld, dtype, largest |k|, seed)
    (3, 4, 40, 150, torch.float16, 2, 3),
    (3, 4, 40, 150, torch.bfloat16, 2, 3),
    (2, 3, 64, 300, torch.bfloat16, 1, 5),    # ternary: the max recurs in many rows
    (4, 2, 100, 520, torch.float16, 1, 6),    # several 128-token tiles per doc
]


@pytest.mark.parametrize("case", EXACT_TIE_CASES, ids=lambda c: f"{c[0]}x{c[1]}_lq{c[2]}_ld{c[3]}_{str(c[4])[6:]}_k{c[5]}")
def test_dense_exact_ties(ms, oracle_mod, case):
    """Values k/8: every dot product is exact in fp32 too, so argmax must match
    the oracle exactly, including lowest-index tie-breaking: within a lane's
    rows of one 32-row block, across blocks and tiles, and across the two
    lane halves."""
    Nq, Nd, Lq, Ld, dt, kmax, seed = case
    _say(f"dense exact ties {case}")
    rng = np.random.default_rng(seed)
    Q = torch.from_numpy(rng.integers(-kmax, kmax + 1, size=(Nq, Lq, 128)) / 8.0).to(dt)
    D = torch.from_numpy(rng.integers(-kmax, kmax + 1, size=(Nd, Ld, 128)) / 8.0).to(dt)
    D[:, 100:140] = D[:, 10:50]
    D[Nd - 2] = D[Nd - 2, 0]
    dm = torch.from_numpy((rng.random((Nd, Ld)) > 0.1).astype(np.uint8))
    w = synth.Dense("ties", Q, D, None, dm)
    s, a = _run_dense(ms, w)
    rs, ra = oracle_mod.fwd(Q, D, None, dm)
    assert np.array_equal(s.numpy().astype(np.float64), rs)
    assert np.array_equal(a.numpy(), ra)


def test_dense_fp16_subnormals(ms, oracle_mod):
    """fp16 subnormal inputs must not be flushed by the MFMA path."""
    _say("dense fp16 subnormals")
    rng = np.random.default_rng(4)
    Q = torch.from_numpy(rng.standard_normal((2, 32, 128))).to(torch.float16)
    sub = torch.from_numpy(rng.integers(1, 1024, size=(3, 64, 128)).astype(np.int16))
    D = sub.view(torch.float16)  # positive subnormals (exponent field 0)
    D = torch.where(torch.from_numpy(rng.random((3, 64, 128)) < 0.5), D, -D)
    w = synth.Dense("subnormal", Q, D.contiguous())
    s, a = _run_dense(ms, w)
    rs, ra = oracle_mod.fwd(w.Q, w.D)
    assert np.abs(rs).max() > 1e-3  # the inputs really carry signal
    _assert_close("scores", s.numpy() * 1e3, rs * 1e3)  # tolerance scaled to the values' size
    _assert_float_argmax("argmax", a.numpy(), ra, w)


def test_dense_empty_and_degenerate(ms):
    _say("dense empty sizes")
    Q = torch.zeros((2, 0, 128), dtype=torch.float16, device=DEV)
    D = torch.randn((3, 5, 128), device=DEV).half()
    s, a = ms.maxsim_fwd(Q, D, want_argmax=True)
    torch.cuda.synchronize()
    assert torch.all(s == 0)
    D0 = torch.zeros((3, 0, 128), dtype=torch.float16, device=DEV)
    Q1 = torch.randn((2, 4, 128), device=DEV).half()
    s, a = ms.maxsim_fwd(Q1, D0, want_argmax=True)
    torch.cuda.synchronize()
    assert torch.all(s == 0) and torch.all(a == 0)
    s, a = ms.maxsim_fwd(Q1[:0], D, want_argmax=True)
    assert s.numel() == 0


def test_colpali_full_size(ms, oracle_mod):
    """The ColPali cross-product (128 x 128 pairs, Lq = 128, Ld = 1024, bf16,
    prefix masks) in the launch configuration the benchmark times: every
    score and every argmax entry of the 16,384 pairs against the oracle
    (argmax under the near-tie rule), then a second run bit for bit."""
    _say("colpali full size")
    w = synth.colpali_bf16()
    s, a = _run_dense(ms, w)
    rs, ra = oracle_mod.fwd(w.Q, w.D, w.q_mask, w.d_mask)
    _assert_close("scores", s.numpy(), rs)
    n, acc = _assert_float_argmax("argmax", a.numpy(), ra, w)
    print(f"argmax near-tie deviations: {n} of {ra.size}")
    s2, a2 = _run_dense(ms, w)
    assert torch.equal(s, s2) and torch.equal(a, a2)
    # the timed configuration without argmax gives the same scores
    s3, _ = _run_dense(ms, w, want_argmax=False)
    _assert_close("scores (no argmax)", s3.numpy(), rs)


# --------------------------------------------------------------------- varlen

def _run_varlen(ms, w, want_argmax):
    s, a = ms.maxsim_fwd_varlen(_g(w.Q), _g(w.cu_q), w.max_lq, _g(w.D), _g(w.cu_d),
                                want_argmax=want_argmax)
    torch.cuda.synchronize()
    return s.cpu(), (None if a is None else a.cpu())


VARLEN_CASES = [
    ([32], [50, 0, 1, 17, 300, 0, 0, 64, 16, 15]),          # empty docs, tile edges
    ([5, 0, 32, 31], list(range(0, 120, 7))),               # several queries, an empty one
    ([60, 17], [40] * 30 + [0] * 5),                        # 4 N-tiles, trailing empty docs
    ([130], [33, 80, 1, 0, 200]),                           # multi-pass query
    ([3], [0, 0, 0]),                                       # only empty docs
]


@pytest.mark.parametrize("case", VARLEN_CASES, ids=lambda c: f"q{len(c[0])}_d{len(c[1])}")
@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16], ids=["f16", "bf16"])
def test_varlen_small(ms, oracle_mod, case, dtype):
    ql, dl = case
    _say(f"varlen {ql} {dl} {dtype}")
    w = synth.random_varlen(200 + len(dl), ql, dl, dtype=dtype)
    s, a = _run_varlen(ms, w, True)
    rs, ra = oracle_mod.fwd_varlen(w.Q, w.cu_q, w.max_lq, w.D, w.cu_d)
    _assert_close("scores", s.numpy(), rs)
    Nq, Nd = len(ql), len(dl)
    n, acc, bad = compare.varlen_argmax_float(a.numpy(), ra, w.Q.double().numpy(), w.cu_q.numpy(),
                                              w.D.double().numpy(), w.cu_d.numpy(),
                                              np.arange(Nq), np.arange(Nd))
    assert not bad, bad[:5]
    s2, _ = _run_varlen(ms, w, False)
    _assert_close("scores (no argmax)", s2.numpy(), rs)


def test_varlen_many_docs(ms, oracle_mod):
    """Enough docs that many streaming units split the range."""
    _say("varlen 20000 docs")
    lens = synth.rerank_lengths(9, 20000, 1, 120)
    w = synth.random_varlen(9, [32], lens)
    s, _ = _run_varlen(ms, w, False)
    rs, _ = oracle_mod.fwd_varlen(w.Q, w.cu_q, w.max_lq, w.D, w.cu_d, want_argmax=False)
    _assert_close("scores", s.numpy(), rs)
    s2, _ = _run_varlen(ms, w, False)
    assert torch.equal(s, s2)


def _repack(w, docs):
    cu = w.cu_d.numpy().astype(np.int64)
    parts = [w.D[cu[j]:cu[j + 1]] for j in docs]
    lens = np.array([cu[j + 1] - cu[j] for j in docs])
    return torch.cat(parts), synth.cu_seqlens(lens)


def test_rerank_full_size(ms, oracle_mod):
    """One 32-token query against 100,000 packed docs of 50-300 tokens (about
    17.5M tokens, 4.5 GB fp16) in the benchmark's launch configuration: every
    score against the oracle, and with argmax on, every argmax entry (near-tie
    rule) and the same scores bit for bit."""
    _say("rerank varlen full size")
    w = synth.rerank_varlen_fp16()
    s, _ = _run_varlen(ms, w, False)
    rs, ra = oracle_mod.fwd_varlen(w.Q, w.cu_q, w.max_lq, w.D, w.cu_d)
    _assert_close("scores", s.numpy(), rs)
    s_a, a = _run_varlen(ms, w, True)
    assert torch.equal(s_a, s)
    n, acc, bad = compare.varlen_argmax_float(a.numpy(), ra, w.Q.double().numpy(), w.cu_q.numpy(),
                                              w.D.double().numpy(), w.cu_d.numpy(), np.arange(1),
                                              np.arange(100_000))
    assert not bad, bad[:5]
    print(f"argmax near-tie deviations: {n} of {ra.size}")


# --------------------------------------------------------------------- int8

def _run_i8(ms, w, want_argmax):
    si, sf, a = ms.maxsim_fwd_i8(_g(w.Q), w.q_scale, _g(w.D), w.d_scale, _g(w.q_mask),
                                 _g(w.d_mask), want_argmax=want_argmax)
    torch.cuda.synchronize()
    return si.cpu(), sf.cpu(), (None if a is None else a.cpu())


INT8_CASES = [
    (2, 5, 9, 13, "ternary", 0.2, 0.2),
    (3, 4, 100, 130, "quantised", 0.0, 0.3),
    (1, 3, 1024, 70, "quantised", 0.1, 0.0),     # 32 N-tiles: one pass of 8 waves x 4
    (1, 2, 1040, 40, "quantised", 0.0, 0.0),     # past one workgroup: two passes
    (2, 3, 128, 64, "extreme", 0.0, 0.0),        # largest sums
    (4, 3, 32, 200, "ternary", 0.0, 0.0),
    (2, 3, 64, 600, "ternary", 0.0, 0.1),        # argmax ties across 256-token tiles
]


@pytest.mark.parametrize("case", INT8_CASES, ids=lambda c: f"{c[0]}x{c[1]}_lq{c[2]}_ld{c[3]}_{c[4]}")
def test_int8_small(ms, oracle_mod, case):
    Nq, Nd, Lq, Ld, kind, qp, dp = case
    _say(f"int8 {case}")
    w = synth.random_int8(300 + Lq, Nq, Nd, Lq, Ld, ternary=kind == "ternary",
                          extreme=kind == "extreme", d_mask_p=dp, q_mask_p=qp)
    si, sf, a = _run_i8(ms, w, True)
    ri, rf, ra = oracle_mod.fwd_i8(w.Q, w.q_scale, w.D, w.d_scale, w.q_mask, w.d_mask)
    assert np.array_equal(si.numpy().astype(np.int64), ri)
    _assert_close("scores", sf.numpy(), rf)
    assert np.array_equal(sf.numpy(), rf.astype(np.float32))  # same double rounding
    assert np.array_equal(a.numpy(), ra)
    si2, sf2, _ = _run_i8(ms, w, False)
    assert torch.equal(si2, si) and torch.equal(sf2, sf)


def _block_digests(argmax, block):
    a = np.ascontiguousarray(np.asarray(argmax, dtype="<i4"))
    return [hashlib.sha256(a[0, j:j + block].tobytes()).hexdigest()[:16]
            for j in range(0, a.shape[1], block)]


def test_int8_full_size(ms, oracle_mod):
    """One 1024-token query against 10,000 docs of 1024 tokens, int8 with
    per-tensor scales, in the benchmark's launch configuration (argmax off)
    and with argmax on: every doc's exact int32 sum, fp32 score and argmax row
    bit for bit against the oracle's, stored by
    tests/golden/make_int8_long_query.py (the oracle takes minutes here)."""
    _say("int8 full size")
    with open(os.path.join(GOLDEN, "int8_long_query_expected.json")) as f:
        exp = json.load(f)
    w = synth.int8_long_query()
    h = exp["inputs_sha256"]
    assert hashlib.sha256(w.D.numpy().tobytes()).hexdigest() == h["D"], "inputs differ from the stored run"
    assert hashlib.sha256(w.Q.numpy().tobytes()).hexdigest() == h["Q"], "inputs differ from the stored run"
    ri = np.array(exp["scores_i32"], dtype=np.int64)
    rf = np.frombuffer(bytes.fromhex(exp["scores_f32_hex"]), dtype="<f4")
    si, sf, _ = _run_i8(ms, w, False)
    assert np.array_equal(si.numpy()[0].astype(np.int64), ri), "int32 sums (argmax off)"
    assert np.array_equal(sf.numpy()[0], rf), "fp32 scores (argmax off)"
    si2, sf2, a = _run_i8(ms, w, True)
    assert torch.equal(si2, si) and torch.equal(sf2, sf)
    blk = exp["argmax_block"]
    got = _block_digests(a.numpy(), blk)
    bad = [b for b, (x, y) in enumerate(zip(got, exp["argmax_block_digests"])) if x != y]
    if bad:
        # name the first differing entries from the oracle on the first differing block
        docs = np.arange(bad[0] * blk, min(10_000, (bad[0] + 1) * blk))
        _, _, ra = oracle_mod.fwd_i8(w.Q, w.q_scale, w.D[docs], w.d_scale, want_argmax=True)
        diff = np.argwhere(a.numpy()[0, docs] != ra[0])[:8]
        raise AssertionError(f"argmax differs in {len(bad)} blocks of {blk} docs; (doc, row, got, oracle): "
                             f"{[(int(docs[k]), int(s), int(a[0, docs[k], s]), int(ra[0, k, s])) for k, s in diff]}")


# --------------------------------------------------------------------- backward

def _run_bwd(ms, w, argmax, g):
    out = ms.maxsim_bwd(_g(w.Q), _g(w.D), _g(argmax), _g(g), _g(w.q_mask), _g(w.d_mask))
    torch.cuda.synchronize()
    return [t.cpu() for t in out]


def _check_bwd(ms, oracle_mod, w, argmax, g):
    dQ, dD, rp, ci = _run_bwd(ms, w, argmax, g)
    rdQ, rdD, rrp, rci = oracle_mod.bwd(w.Q, w.D, argmax, g, w.q_mask, w.d_mask)
    assert np.array_equal(rp.numpy(), rrp), "row_ptr"
    assert np.array_equal(ci.numpy(), rci), "col_idx"
    _assert_close("dQ", dQ.numpy(), rdQ)
    _assert_close("dD", dD.numpy(), rdD)
    again = _run_bwd(ms, w, argmax, g)
    assert all(torch.equal(x, y) for x, y in zip(again, (dQ, dD, rp, ci))), "not deterministic"


BWD_CASES = [
    (3, 4, 9, 14, torch.float16, 0.3, 0.2, 1, 0.0),
    (5, 6, 70, 130, torch.bfloat16, 0.2, 0.1, 1, 0.0),
    (4, 3, 64, 64, torch.bfloat16, 0.0, 0.0, 0, 0.7),   # hub token: 70% of sources in one row
    (2, 2, 1, 5000, torch.float16, 0.0, 0.0, 0, 0.0),   # CSR bins in two rounds
    (130, 2, 3, 10, torch.float16, 0.0, 0.0, 0, 0.0),   # many queries per doc
    (130, 2, 128, 10, torch.float16, 0.2, 0.0, 0, 0.0),  # > 16384 sources per doc: two CSR chunks,
                                                         # weights read per source
    (6, 3, 40, 700, torch.bfloat16, 0.1, 0.2, 1, 0.0),   # a doc's bins split over workgroups
    (1, 513, 2, 1030, torch.float16, 0.0, 0.0, 0, 0.0),  # one bin range per doc, two rounds
    (3, 2, 5, 1, torch.float16, 0.0, 0.0, 0, 0.0),       # one row per doc: a row range with no rows
    (64, 3, 256, 96, torch.bfloat16, 0.1, 0.1, 1, 0.0),  # exactly 16384 sources per doc
    (8, 3, 100, 300, torch.float16, 0.0, 0.0, 0, 1.0),   # every source of a doc in one row:
                                                         # groups of 64 equal keys per step
    (4, 130, 40, 60, torch.bfloat16, 0.3, 0.2, 2, 0.0),  # dQ over three rounds of staged docs
    (3, 200, 64, 33, torch.float16, 0.0, 0.3, 1, 0.0),   # rounds of 64 + 64 + 64 + 8 docs
    (40, 128, 80, 20, torch.float16, 0.2, 0.0, 0, 0.0),  # more query rows than doc rows
]


@pytest.mark.parametrize("case", BWD_CASES, ids=lambda c: f"{c[0]}x{c[1]}_lq{c[2]}_ld{c[3]}_hub{c[8]}")
def test_bwd_small(ms, oracle_mod, case):
    Nq, Nd, Lq, Ld, dt, qp, dp, dead, hub = case
    _say(f"bwd {case}")
    w = synth.random_dense(400 + Lq, Nq, Nd, Lq, Ld, dtype=dt, q_mask_p=qp, d_mask_p=dp,
                           dead_docs=dead)
    if hub > 0:
        argmax = synth.draw_argmax(400 + Lq, Nq, Nd, Lq, Ld, None, hub_frac=hub)
    else:
        _, ra = oracle_mod.fwd(w.Q, w.D, w.q_mask, w.d_mask)  # the oracle's forward argmax
        argmax = torch.from_numpy(ra)
    g = synth.upstream_grad(400 + Lq, Nq, Nd)
    _check_bwd(ms, oracle_mod, w, argmax, g)


@pytest.mark.parametrize("dt", [torch.float16, torch.bfloat16], ids=["f16", "bf16"])
def test_bwd_zero_weights(ms, oracle_mod, dt):
    """Upstream gradients that are zero for most (query, doc) pairs, with
    masked query tokens and a dead doc: every term of zero weight is skipped
    by the gathers, which must leave dQ and dD as the oracle's (rows whose
    terms are all zero come out exactly 0)."""
    _say(f"bwd zero weights {dt}")
    Nq, Nd, Lq, Ld = 6, 5, 48, 90
    w = synth.random_dense(470, Nq, Nd, Lq, Ld, dtype=dt, q_mask_p=0.4, d_mask_p=0.2, dead_docs=1)
    _, ra = oracle_mod.fwd(w.Q, w.D, w.q_mask, w.d_mask)
    g = synth.upstream_grad(470, Nq, Nd)
    keep = torch.from_numpy(np.random.default_rng(471).random((Nq, Nd)) < 0.3)
    g = torch.where(keep, g, torch.zeros_like(g))
    g[0] = 0.0  # a query with no gradient at all
    _check_bwd(ms, oracle_mod, w, torch.from_numpy(ra), g)
    dQ, dD, _, _ = _run_bwd(ms, w, torch.from_numpy(ra), g)
    assert torch.all(dQ[0] == 0), "a query whose gradients are all zero"
    rdQ, rdD, _, _ = oracle_mod.bwd(w.Q, w.D, torch.from_numpy(ra), g, w.q_mask, w.d_mask)
    zero_rows = np.all(rdD == 0, axis=-1)  # destinations with no term of nonzero weight
    assert zero_rows.any() and torch.all(dD[torch.from_numpy(zero_rows)] == 0)


def test_bwd_full_size(ms, oracle_mod):
    """Backward at the ColPali shapes (dQ [128,128,128], dD [128,1024,128]) as
    the benchmark times it: through the argmax saved by the GPU forward (its
    hub tokens skew the CSR rows), with the upstream gradient of the workload;
    the CSR bit for bit and every gradient element against the oracle, which
    takes the same argmax."""
    _say("bwd full size, forward argmax")
    w = synth.colpali_bf16()
    _, a = _run_dense(ms, w)
    g = synth.upstream_grad(5, 128, 128)
    _check_bwd(ms, oracle_mod, w, a, g)


def test_bwd_full_size_uniform_argmax(ms, oracle_mod):
    """The same shapes with an argmax drawn uniformly over each doc's valid
    prefix (every CSR row about equally long)."""
    _say("bwd full size, uniform argmax")
    w = synth.colpali_bf16()
    b = synth.colpali_backward(fwd=w)
    _check_bwd(ms, oracle_mod, w, b.argmax, b.grad_scores)


# ------------------------------------------------ per-token INT8, top-k, pairs

INT8_TOK_CASES = [
    # (Nq, Nd, Lq, Ld, q_mask_p, d_mask_p, dead_docs)
    (2, 5, 9, 13, 0.2, 0.2, 1),
    (3, 4, 100, 130, 0.0, 0.3, 0),
    (1, 3, 1024, 70, 0.1, 0.0, 0),     # 32 N-tiles: one pass of 8 waves x 4
    (1, 2, 1100, 40, 0.0, 0.0, 0),     # past one workgroup: two passes (no int32 sum limit)
    (4, 3, 32, 200, 0.0, 0.0, 0),
]


@pytest.mark.parametrize("case", INT8_TOK_CASES, ids=lambda c: f"{c[0]}x{c[1]}_lq{c[2]}_ld{c[3]}")
def test_int8_tok_small(ms, oracle_mod, case):
    Nq, Nd, Lq, Ld, qp, dp, dead = case
    _say(f"int8 per-token {case}")
    w = synth.random_int8_tok(700 + Lq, Nq, Nd, Lq, Ld, q_mask_p=qp, d_mask_p=dp, dead_docs=dead)
    s, a = ms.maxsim_fwd_i8_tok(_g(w.Q), _g(w.q_scale), _g(w.D), _g(w.d_scale), _g(w.q_mask),
                                _g(w.d_mask), want_argmax=True)
    s2, _ = ms.maxsim_fwd_i8_tok(_g(w.Q), _g(w.q_scale), _g(w.D), _g(w.d_scale), _g(w.q_mask),
                                 _g(w.d_mask))
    torch.cuda.synchronize()
    rs, ra = oracle_mod.fwd_i8_tok(w.Q, w.q_scale, w.D, w.d_scale, w.q_mask, w.d_mask)
    _assert_close("scores", s.cpu().numpy(), rs)
    _assert_close("scores (no argmax)", s2.cpu().numpy(), rs)
    n, acc, bad = compare.int8_tok_argmax(a.cpu().numpy(), ra, w.Q.numpy(), w.D.numpy(),
                                          w.d_scale.numpy(),
                                          None if w.d_mask is None else w.d_mask.numpy())
    assert not bad, f"argmax mismatches outside the rounding bound: {bad[:5]}"


def test_int8_tok_full_size_sampled(ms, oracle_mod):
    """One 1024-token query against 10,000 docs of 1024 tokens with per-token
    scales; the oracle scores 16 docs."""
    _say("int8 per-token full size")
    w = synth.two_stage_long_query()
    s, _ = ms.maxsim_fwd_i8_tok(_g(w.Q), _g(w.q_scale), _g(w.D), _g(w.d_scale))
    torch.cuda.synchronize()
    rng = np.random.default_rng(3)
    docs = np.sort(np.concatenate([[0, 9999], rng.choice(np.arange(1, 9999), 14, replace=False)]))
    rs, _ = oracle_mod.fwd_i8_tok(w.Q, w.q_scale, w.D[docs], w.d_scale[docs], want_argmax=False)
    _assert_close("scores", s.cpu().numpy()[:, docs], rs)


PAIR_CASES = [
    # (Nq, Nd, Lq, Ld, dtype, P)
    (3, 5, 40, 150, torch.bfloat16, 40),
    (2, 7, 300, 130, torch.float16, 9),      # a query longer than one workgroup
    (1, 4, 1024, 100, torch.bfloat16, 6),
    (4, 3, 1, 1, torch.float16, 5),
]


@pytest.mark.parametrize("case", PAIR_CASES, ids=lambda c: f"{c[0]}x{c[1]}_lq{c[2]}_ld{c[3]}_p{c[5]}")
def test_pairs(ms, oracle_mod, case):
    Nq, Nd, Lq, Ld, dt, P = case
    _say(f"pairs {case}")
    w = synth.random_dense(800 + Lq, Nq, Nd, Lq, Ld, dtype=dt, q_mask_p=0.2, d_mask_p=0.2,
                           dead_docs=1)
    pq, pd = synth.random_pairs(800 + Lq, Nq, Nd, P)
    s, a = ms.maxsim_fwd_pairs(_g(w.Q), _g(w.D), _g(pq), _g(pd), _g(w.q_mask), _g(w.d_mask),
                               want_argmax=True)
    torch.cuda.synchronize()
    rs, ra = oracle_mod.fwd_pairs(w.Q, w.D, pq, pd, w.q_mask, w.d_mask)
    _assert_close("scores", s.cpu().numpy(), rs)
    n, acc, bad = compare.pair_argmax_float(a.cpu().numpy(), ra, w.Q.double().numpy(),
                                            w.D.double().numpy(),
                                            None if w.d_mask is None else w.d_mask.numpy(),
                                            pq.numpy(), pd.numpy())
    assert not bad, f"argmax mismatches outside the near-tie bound: {bad[:5]}"


TOPK_CASES = [
    # (Nq, Nd, k, ties)
    (3, 1, 1, False),
    (5, 300, 7, True),
    (2, 5000, 100, False),
    (4, 2048, 1024, True),      # the largest k
    (1, 100000, 100, False),    # a reranking-size row
    (6, 1000, 1000, False),     # k = Nd: a full sort
    (2, 20000, 50, True),       # row 1 constant: too many candidates, exact radix path
]


@pytest.mark.parametrize("case", TOPK_CASES, ids=lambda c: f"{c[0]}x{c[1]}_k{c[2]}_ties{int(c[3])}")
def test_topk(ms, oracle_mod, case):
    Nq, Nd, k, ties = case
    _say(f"topk {case}")
    v = synth.random_scores(900 + k, Nq, Nd, ties=ties)
    if Nd > 2:
        v[0, 1] = -0.0   # -0 and +0 are equal and ordered by column
        v[0, 2] = 0.0
    if Nq > 1 and Nd >= 20000:
        v[1, :] = 1.0    # every column ties
    idx, val, rows = ms.maxsim_topk(_g(v), k, want_rows=True)
    ids = torch.arange(Nq * Nd, dtype=torch.int32).view(Nq, Nd) * 3 + 1
    idx2, _, _ = ms.maxsim_topk(_g(v), k, ids=_g(ids))
    torch.cuda.synchronize()
    ri, rv = oracle_mod.topk(v, k)
    assert np.array_equal(idx.cpu().numpy(), ri)
    assert np.array_equal(val.cpu().numpy().view(np.int32), rv.astype(np.float32).view(np.int32))
    assert np.array_equal(rows.cpu().numpy(), np.repeat(np.arange(Nq), k).reshape(Nq, k))
    assert np.array_equal(idx2.cpu().numpy(), np.take_along_axis(ids.numpy(), ri.astype(np.int64), 1))


def test_two_stage_scan(ms, oracle_mod):
    """INT8 per-token scan of every doc, the best 12 docs as candidates, their
    exact bf16 scores, the final top 5. With every doc a candidate the result
    is the exact top 5; the oracle's gaps between consecutive scores of the top
    6 are checked to be far above the fp32 rounding of these sums (about 1e-5)
    before the order is compared."""
    _say("two-stage scan")
    Nq, Nd, Lq, Ld = 2, 12, 64, 150
    w = synth.random_int8_tok(950, Nq, Nd, Lq, Ld, d_mask_p=0.1, float_dtype=torch.bfloat16)
    doc, val, s8 = ms.two_stage_topk(_g(w.Q), _g(w.q_scale), _g(w.D), _g(w.d_scale), _g(w.Qf),
                                     _g(w.Df), 5, Nd, None, _g(w.d_mask))
    torch.cuda.synchronize()
    rs, _ = oracle_mod.fwd(w.Qf, w.Df, None, w.d_mask, want_argmax=False)
    ri, rv = oracle_mod.topk(rs, 6)
    assert np.all(np.abs(np.diff(rv, axis=1)) > 1e-4), "seed gives near-ties; pick another"
    assert np.array_equal(doc.cpu().numpy(), ri[:, :5])
    _assert_close("scores", val.cpu().numpy(), rv[:, :5])
    r8, _ = oracle_mod.fwd_i8_tok(w.Q, w.q_scale, w.D, w.d_scale, None, w.d_mask, want_argmax=False)
    _assert_close("int8 stage scores", s8.cpu().numpy(), r8)


# ------------------------------------------- padding-free backward, packed pairs

VARBWD_CASES = [
    # (query lengths, doc lengths, dtype, hub fraction, argmax from the forward)
    ([5, 12, 3], [7, 0, 19, 3, 1], torch.float16, 0.0, True),     # an empty doc
    ([32] * 4, list(range(50, 300, 13)), torch.bfloat16, 0.0, True),
    ([64] * 4, [64] * 3, torch.bfloat16, 0.7, False),             # hub token
    ([2], [5000, 7], torch.float16, 0.0, False),                  # CSR bins in several rounds
    ([128] * 130, [10, 0, 20], torch.float16, 0.0, False),        # > 16384 sources: two chunks
    ([0, 3, 0], [4, 0, 4], torch.bfloat16, 0.0, True),            # empty queries
    ([3], [0, 0], torch.float16, 0.0, True),                      # no doc token at all
    ([0], [5, 3], torch.float16, 0.0, True),                      # no query row at all
    ([128] * 128, [100, 1024, 1], torch.bfloat16, 1.0, False),    # 16384 rows, docs of up to 1024
                                                                   # rows, every source in one row
]


def _run_bwd_varlen(ms, w, argmax, g):
    out = ms.maxsim_bwd_varlen(_g(w.Q), _g(w.cu_q), w.max_lq, _g(w.D), _g(w.cu_d), _g(argmax), _g(g))
    torch.cuda.synchronize()
    return tuple(x.cpu() for x in out)


@pytest.mark.parametrize("case", VARBWD_CASES, ids=lambda c: f"q{len(c[0])}_d{len(c[1])}_hub{c[3]}")
def test_bwd_varlen(ms, oracle_mod, case):
    ql, dl, dt, hub, from_fwd = case
    _say(f"bwd varlen {case[0][:4]} {case[1][:6]} {dt} hub {hub}")
    seed = 900 + len(ql) + len(dl)
    w = synth.random_varlen(seed, ql, dl, dtype=dt, max_lq=max(max(ql), 1))
    if from_fwd:
        _, ra = oracle_mod.fwd_varlen(w.Q, w.cu_q, w.max_lq, w.D, w.cu_d)
        argmax = torch.from_numpy(ra)
    else:
        argmax = synth.draw_argmax_varlen(seed, w.cu_q, w.cu_d, w.max_lq, hub_frac=hub)
    g = synth.upstream_grad(seed, len(ql), len(dl))
    dQ, dD, rp, ci = _run_bwd_varlen(ms, w, argmax, g)
    rdQ, rdD, rrp, rci = oracle_mod.bwd_varlen(w.Q, w.cu_q, w.max_lq, w.D, w.cu_d, argmax, g)
    assert np.array_equal(rp.numpy(), rrp), "row_ptr"
    assert np.array_equal(ci.numpy()[:len(rci)], rci), "col_idx"
    _assert_close("dQ", dQ.numpy(), rdQ)
    _assert_close("dD", dD.numpy(), rdD)
    again = _run_bwd_varlen(ms, w, argmax, g)
    n = len(rci)
    assert all(torch.equal(x, y) for x, y in zip(again[:3], (dQ, dD, rp))), "not deterministic"
    assert torch.equal(again[3][:n], ci[:n]), "not deterministic"


def test_bwd_varlen_colpali_packed(ms, oracle_mod):
    """The ColPali training shapes packed without padding: 128 queries of
    16-128 tokens against 128 docs of 768-1024 patches (the masked prefixes
    of the cross-product workload), argmax from the GPU forward; every output
    compared."""
    _say("bwd varlen colpali packed")
    rng = np.random.default_rng(3)
    ql = rng.integers(16, 129, 128)
    dl = rng.integers(768, 1025, 128)
    w = synth.random_varlen(31, ql, dl, dtype=torch.bfloat16, max_lq=128)
    _, a = ms.maxsim_fwd_varlen(_g(w.Q), _g(w.cu_q), w.max_lq, _g(w.D), _g(w.cu_d), want_argmax=True)
    argmax = a.cpu()
    g = synth.upstream_grad(31, 128, 128)
    dQ, dD, rp, ci = _run_bwd_varlen(ms, w, argmax, g)
    rdQ, rdD, rrp, rci = oracle_mod.bwd_varlen(w.Q, w.cu_q, w.max_lq, w.D, w.cu_d, argmax, g)
    assert np.array_equal(rp.numpy(), rrp), "row_ptr"
    assert np.array_equal(ci.numpy()[:len(rci)], rci), "col_idx"
    _assert_close("dQ", dQ.numpy(), rdQ)
    _assert_close("dD", dD.numpy(), rdD)


PAIRS_VARLEN_CASES = [
    # (query lengths, doc lengths, dtype, P)
    ([32, 5, 0, 17], [50, 0, 1, 300, 64, 16], torch.float16, 40),
    ([130, 8], [33, 80, 0, 200], torch.bfloat16, 11),     # multi-pass query
    ([32], synth.rerank_lengths(5, 3000, 50, 300).tolist(), torch.float16, 2000),
]


@pytest.mark.parametrize("case", PAIRS_VARLEN_CASES, ids=lambda c: f"q{len(c[0])}_d{len(c[1])}_p{c[3]}")
def test_pairs_varlen(ms, oracle_mod, case):
    ql, dl, dt, P = case
    _say(f"pairs varlen q{len(ql)} d{len(dl)} P{P}")
    w = synth.random_varlen(950 + P, ql, dl, dtype=dt)
    pq, pd = synth.random_pairs(950 + P, len(ql), len(dl), P)
    s, a = ms.maxsim_fwd_pairs_varlen(_g(w.Q), _g(w.cu_q), w.max_lq, _g(w.D), _g(w.cu_d), _g(pq),
                                      _g(pd), want_argmax=True)
    torch.cuda.synchronize()
    rs, ra = oracle_mod.fwd_pairs_varlen(w.Q, w.cu_q, w.max_lq, w.D, w.cu_d, pq, pd)
    _assert_close("scores", s.cpu().numpy(), rs)
    n, acc, bad = compare.pairs_varlen_argmax_float(a.cpu().numpy(), ra, w.Q.double().numpy(),
                                                    w.cu_q.numpy(), w.D.double().numpy(),
                                                    w.cu_d.numpy(), pq.numpy(), pd.numpy())
    assert not bad, f"argmax mismatches outside the near-tie bound: {bad[:5]}"
    s2, _ = ms.maxsim_fwd_pairs_varlen(_g(w.Q), _g(w.cu_q), w.max_lq, _g(w.D), _g(w.cu_d), _g(pq),
                                       _g(pd))
    torch.cuda.synchronize()
    _assert_close("scores (no argmax)", s2.cpu().numpy(), rs)


# ------------------------------------------------------------------ Chamfer distance

# the last two give the forward more 16-point source blocks than resident
# waves: runs of several blocks per wave that cross (batch, direction)
# segment ends, and (256 batches) more blocks than the waves can hold at once
CHAMFER_CASES = [(1, 1, 1), (2, 5, 7), (3, 1000, 1500), (2, 3000, 2500), (1, 20000, 20000),
                 (64, 1024, 1000), (256, 600, 520)]


def _chamfer_gpu(ms, P, Q):
    out = ms.maxsim_chamfer_fwd(_g(P), _g(Q))
    torch.cuda.synchronize()
    return tuple(x.cpu() for x in out)


def _loss_depth(n):
    """Rounding depth of the loss kernel's sum of n distances: each of
    1024 x 16 partial sums takes ceil(n / 16384) terms, 15 additions join a
    thread's 16 partials, and a 10-level tree joins the 1024 threads."""
    return -(-n // 16384) + 15 + 10


def _check_chamfer_fwd(oracle_mod, P, Q, got):
    d1, i1, d2, i2, loss = got
    r1, j1, r2, j2, rl = oracle_mod.chamfer_fwd(P, Q)
    P64, Q64 = P.double().numpy(), Q.double().numpy()
    for name, dg, ig, rd, ri, A, T in (("1", d1, i1, r1, j1, P64, Q64), ("2", d2, i2, r2, j2, Q64, P64)):
        n, acc, bad = compare.chamfer_argmin(ig.numpy(), ri, A, T)
        assert not bad, f"idx{name}: {len(bad)} mismatches outside the direct-form bound: {bad[:5]}"
        ok, worst, where = compare.chamfer_dist(dg.numpy(), rd)
        assert ok, f"dist{name}: worst excess {worst:.3e} at {where}"
        ok, worst = compare.chamfer_dist_at_index(dg.numpy(), ig.numpy(), A, T)
        assert ok, f"dist{name} is not the direct-form distance of idx{name}: worst excess {worst:.3e}"
    tol = compare.chamfer_loss_tol(_loss_depth(max(P.shape[1], Q.shape[1])))
    err = np.abs(loss.numpy().astype(np.float64) - rl)
    assert np.all(err <= tol * np.abs(rl)), f"loss: {err.max():.3e} > {tol:.3e} relative"


def _check_chamfer_bwd(P, Q, i1, i2, g1, g2, dP, dQ, rdP, rdQ):
    P64, Q64 = P.double().numpy(), Q.double().numpy()
    i1, i2 = i1.numpy(), i2.numpy()
    g1, g2 = g1.double().numpy(), g2.double().numpy()
    for name, got, ref, bounds in (("dP", dP, rdP, (P64, Q64, i1, i2, g1, g2)),
                                   ("dQ", dQ, rdQ, (Q64, P64, i2, i1, g2, g1))):
        S, n = compare.chamfer_grad_bounds(*bounds)
        ok, worst, where = compare.chamfer_grad(got.numpy(), ref, S, n)
        assert ok, f"{name}: worst excess {worst:.3e} at {where}"


@pytest.mark.parametrize("shape", CHAMFER_CASES, ids=lambda c: f"{c[0]}x{c[1]}x{c[2]}")
def test_chamfer(ms, oracle_mod, shape):
    B, N, M = shape
    _say(f"chamfer {shape}")
    P, Q = synth.point_clouds(700 + N, B, N, M)
    got = _chamfer_gpu(ms, P, Q)
    _check_chamfer_fwd(oracle_mod, P, Q, got)
    # backward through the GPU's own indices
    g1, g2 = synth.chamfer_grads(700 + N, B, N, M)
    _, i1, _, i2, _ = got
    out = ms.maxsim_chamfer_bwd(_g(P), _g(Q), _g(i1), _g(i2), _g(g1), _g(g2))
    torch.cuda.synchronize()
    dP, dQ, rp1, ci1, rp2, ci2 = (x.cpu() for x in out)
    rdP, rdQ, rrp1, rci1, rrp2, rci2 = oracle_mod.chamfer_bwd(P, Q, i1, i2, g1, g2)
    for name, x, y in (("row_ptr1", rp1, rrp1), ("col_idx1", ci1, rci1), ("row_ptr2", rp2, rrp2),
                       ("col_idx2", ci2, rci2)):
        assert np.array_equal(x.numpy(), y), name
    _check_chamfer_bwd(P, Q, i1, i2, g1, g2, dP, dQ, rdP, rdQ)
    again = ms.maxsim_chamfer_bwd(_g(P), _g(Q), _g(i1), _g(i2), _g(g1), _g(g2))
    torch.cuda.synchronize()
    assert torch.equal(again[0].cpu(), dP) and torch.equal(again[1].cpu(), dQ), "not deterministic"


def test_chamfer_exact_ties(ms, oracle_mod):
    """Duplicated target points: every tie goes to the lowest index."""
    _say("chamfer ties")
    P, Q = synth.point_clouds(781, 2, 300, 100)
    Q = torch.cat([Q, Q, Q[:, :50]], dim=1)  # each target appears two or three times
    got = _chamfer_gpu(ms, P, Q)
    _, i1, _, _, _ = got
    assert int(i1.max()) < 100  # the first copy always wins
    _check_chamfer_fwd(oracle_mod, P, Q, got)


def test_chamfer_tie_across_many_tiles(ms, oracle_mod):
    """A source whose nearest distance is tied by targets in six different
    256-point tiles, more than the search keeps per source, so its answer
    comes from the direct-form scan of the whole set: the lowest index wins."""
    _say("chamfer tie across tiles")
    rng = np.random.default_rng(791)
    M = 2000
    Q = rng.standard_normal((1, M, 3)).astype(np.float32)
    Q /= np.linalg.norm(Q, axis=2, keepdims=True)
    Q *= 10.0  # every other target at distance 10 from the origin
    axes = np.array([[1, 0, 0], [0, 1, 0], [0, 0, 1], [-1, 0, 0], [0, -1, 0], [0, 0, -1]], np.float32)
    where = [5, 300, 700, 1100, 1500, 1900]  # six different tiles
    for k, j in enumerate(where):
        Q[0, j] = axes[k]
    P = np.zeros((1, 3, 3), np.float32)
    P[0, 1] = [0.5, 0.0, 0.0]   # nearest (1, 0, 0) alone, squared distance 0.25
    P[0, 2] = [0.0, 0.0, -3.0]  # nearest (0, 0, -1), squared distance 4
    P, Q = torch.from_numpy(P), torch.from_numpy(Q)
    got = _chamfer_gpu(ms, P, Q)
    d1, i1 = got[0], got[1]
    assert i1[0].tolist() == [5, 5, 1900]
    assert d1[0].tolist() == [1.0, 0.25, 4.0]
    _check_chamfer_fwd(oracle_mod, P, Q, got)


def test_chamfer_offset_clouds(ms, oracle_mod):
    """Point clouds far from the origin (unit spread around (100, -50, 200)):
    distances and indices still meet the tolerance and the near-tie bound,
    which the expanded form's rounding would not at this offset without
    taking the coordinates relative to a point of the set."""
    _say("chamfer offset clouds")
    P, Q = synth.point_clouds(783, 2, 3000, 2500)
    off = torch.tensor([100.0, -50.0, 200.0])
    P, Q = P + off, Q + off
    got = _chamfer_gpu(ms, P, Q)
    _check_chamfer_fwd(oracle_mod, P, Q, got)


def test_chamfer_100k_points(ms, oracle_mod):
    """Two 100,000-point clouds (the size the pages report the naive form
    cannot hold): every distance, index and the loss of the forward, then the
    backward (both CSRs and every gradient), all against the oracle."""
    _say("chamfer 100k")
    P, Q = synth.point_clouds(782, 1, 100_000, 100_000)
    got = _chamfer_gpu(ms, P, Q)
    _check_chamfer_fwd(oracle_mod, P, Q, got)
    _, i1, _, i2, _ = got
    g1, g2 = synth.chamfer_grads(782, 1, 100_000, 100_000)
    out = ms.maxsim_chamfer_bwd(_g(P), _g(Q), _g(i1), _g(i2), _g(g1), _g(g2))
    torch.cuda.synchronize()
    dP, dQ, rp1, ci1, rp2, ci2 = (x.cpu() for x in out)
    rdP, rdQ, rrp1, rci1, rrp2, rci2 = oracle_mod.chamfer_bwd(P, Q, i1, i2, g1, g2)
    for name, x, y in (("row_ptr1", rp1, rrp1), ("col_idx1", ci1, rci1), ("row_ptr2", rp2, rrp2),
                       ("col_idx2", ci2, rci2)):
        assert np.array_equal(x.numpy(), y), name
    _check_chamfer_bwd(P, Q, i1, i2, g1, g2, dP, dQ, rdP, rdQ)


def test_chamfer_many_near_ties(ms, oracle_mod):
    """Sources with many targets at almost the same distance: each source sits
    at the centre of a ring of 24 targets whose radii differ by a few ulps, so
    the matrix-core pass cannot order them and more than two target tiles lie
    inside its rounding window (the exhaustive direct-form pass decides), and
    a cloud of 20,000 random targets around them."""
    _say("chamfer ring near-ties")
    rng = np.random.default_rng(784)
    ns = 256
    src = rng.standard_normal((ns, 3)).astype(np.float32)
    ring = []
    for k in range(24):
        v = rng.standard_normal((ns, 3))
        v /= np.linalg.norm(v, axis=1, keepdims=True)
        ring.append((src + 0.05 * (1 + k * 2.0 ** -22) * v).astype(np.float32))
    far = (3.0 * rng.standard_normal((20_000, 3))).astype(np.float32)
    T = np.concatenate([far[:7000]] + ring[:12] + [far[7000:14000]] + ring[12:] + [far[14000:]])
    P = torch.from_numpy(src[None].copy())
    Q = torch.from_numpy(T[None].copy())
    got = _chamfer_gpu(ms, P, Q)
    _check_chamfer_fwd(oracle_mod, P, Q, got)


def test_chamfer_near_ties_many_batches(ms, oracle_mod):
    """Overflowed sources of several batches and both directions inside one
    fix workgroup (its 1,024 sources span many batch segments): 12 batches of
    40 sources, each source at the centre of a ring of 10 targets whose radii
    differ by a few ulps, spread over the batch's 3,000 random targets."""
    _say("chamfer ring near-ties, many batches")
    rng = np.random.default_rng(786)
    B, ns, nfar, nring = 12, 40, 3000, 10
    P = rng.standard_normal((B, ns, 3)).astype(np.float32)
    Q = []
    for b in range(B):
        ring = []
        for k in range(nring):
            v = rng.standard_normal((ns, 3))
            v /= np.linalg.norm(v, axis=1, keepdims=True)
            ring.append((P[b] + 0.05 * (1 + k * 2.0 ** -22) * v).astype(np.float32))
        far = (3.0 * rng.standard_normal((nfar, 3))).astype(np.float32)
        parts = [far[:700]] + ring[:5] + [far[700:1900]] + ring[5:] + [far[1900:]]
        Q.append(np.concatenate(parts))
    P = torch.from_numpy(P)
    Q = torch.from_numpy(np.stack(Q))
    got = _chamfer_gpu(ms, P, Q)
    _check_chamfer_fwd(oracle_mod, P, Q, got)


# ------------------------------------------------------------------ streams

def test_concurrent_streams(ms, oracle_mod):
    """Calls on two streams at once (the ABI allows it; the library's shared
    state is per-process launch caches): each stream's results equal the
    oracle's and the single-stream results, bit for bit."""
    _say("two streams at once")
    w1 = synth.random_varlen(61, [32], synth.rerank_lengths(61, 4000, 50, 300).tolist())
    w2 = synth.random_dense(62, 3, 40, 64, 200, dtype=torch.bfloat16, q_mask_p=0.2, d_mask_p=0.2, d=96)
    a1 = [_g(t) for t in (w1.Q, w1.cu_q, w1.D, w1.cu_d)]
    a2 = [_g(t) for t in (w2.Q, w2.D, w2.q_mask, w2.d_mask)]
    ref1, _ = ms.maxsim_fwd_varlen(a1[0], a1[1], w1.max_lq, a1[2], a1[3])
    ref2, ref2a = ms.maxsim_fwd(*a2, want_argmax=True)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    for _ in range(3):
        with torch.cuda.stream(s1):
            o1, _ = ms.maxsim_fwd_varlen(a1[0], a1[1], w1.max_lq, a1[2], a1[3], stream=s1)
        with torch.cuda.stream(s2):
            o2, o2a = ms.maxsim_fwd(*a2, want_argmax=True, stream=s2)
        outs.append((o1, o2, o2a))
    torch.cuda.synchronize()
    for o1, o2, o2a in outs:
        assert torch.equal(o1, ref1) and torch.equal(o2, ref2) and torch.equal(o2a, ref2a)
    rs1, _ = oracle_mod.fwd_varlen(w1.Q, w1.cu_q, w1.max_lq, w1.D, w1.cu_d, want_argmax=False)
    rs2, _ = oracle_mod.fwd(w2.Q, w2.D, w2.q_mask, w2.d_mask, want_argmax=False)
    _assert_close("stream 1 scores", ref1.cpu().numpy(), rs1)
    _assert_close("stream 2 scores", ref2.cpu().numpy(), rs2)
