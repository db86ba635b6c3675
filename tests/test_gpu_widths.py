"""GPU parity of the forwards and backwards at embedding widths other than 128.

Every fp16/bf16 entry point accepts 1 <= d <= 1024; forwards at widths other
than 128 run the general-width kernel (TileMaxSim Sec. 3 dimension tiling, Sec. 6
Table 9 width sweep). The cases cover one-chunk widths whose query stays in
registers (d <= 128), several chunks with a query staged in LDS (d > 128), a
partial last chunk and K-step, rows whose byte length is not a multiple of 16
(gathered element by element), masks, dead docs, empty sequences, multi-pass
queries and pair lists; the backwards gather rows in 128-wide chunks with a
partial or unaligned tail; int8 rows (per-tensor scales: exact int32 sums and
argmax; per-token scales: float compare inside the max) take the same kernel.
Expected values come only from the oracle; tolerances and the argmax rule are
those of oracle/compare.py.
"""

import numpy as np
import pytest
import torch

from maxsim_scoring_amd import synth
from oracle import compare

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


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


DENSE_CASES = [
    # (Nq, Nd, Lq, Ld, dtype, d, mask_p, dead_docs)
    (2, 5, 45, 200, torch.bfloat16, 64, 0.3, 1),
    (3, 4, 32, 130, torch.float16, 96, 0.0, 0),
    (2, 3, 70, 90, torch.float16, 100, 0.2, 1),     # 200-byte rows: element gathers
    (2, 3, 33, 40, torch.bfloat16, 1, 0.0, 0),
    (2, 3, 20, 50, torch.float16, 8, 0.1, 0),
    (2, 4, 40, 77, torch.bfloat16, 200, 0.2, 1),    # two chunks, partial K-step
    (1, 3, 32, 128, torch.float16, 256, 0.0, 0),
    (3, 3, 64, 60, torch.float16, 384, 0.3, 1),
    (1, 2, 32, 70, torch.bfloat16, 768, 0.0, 0),
    (2, 2, 16, 33, torch.float16, 1000, 0.0, 0),    # eight chunks, partial last
    (1, 2, 5, 9, torch.float16, 1021, 0.0, 0),      # eight chunks, unaligned rows
    (2, 3, 300, 50, torch.bfloat16, 64, 0.2, 0),    # ten passes over the docs
    (2, 2, 1, 1, torch.float16, 32, 0.0, 0),
]


@pytest.mark.parametrize("case", DENSE_CASES,
                         ids=lambda c: f"{c[0]}x{c[1]}_lq{c[2]}_ld{c[3]}_{str(c[4])[6:]}_d{c[5]}")
def test_dense_widths(ms, oracle_mod, case):
    Nq, Nd, Lq, Ld, dt, d, p, dead = case
    _say(f"dense width {case}")
    w = synth.random_dense(1200 + d + Lq, Nq, Nd, Lq, Ld, dtype=dt, q_mask_p=p, d_mask_p=p,
                           dead_docs=dead, d=d)
    s, a = ms.maxsim_fwd(_g(w.Q), _g(w.D), _g(w.q_mask), _g(w.d_mask), want_argmax=True)
    torch.cuda.synchronize()
    rs, ra = oracle_mod.fwd(w.Q, w.D, w.q_mask, w.d_mask)
    _assert_close("scores", s.cpu().numpy(), rs)
    n, acc, bad = compare.dense_argmax_float(a.cpu().numpy(), ra, w.Q.double().numpy(),
                                             w.D.double().numpy(),
                                             None if w.d_mask is None else w.d_mask.numpy())
    assert not bad, f"argmax mismatches outside the near-tie bound: {bad[:5]}"
    s2, _ = ms.maxsim_fwd(_g(w.Q), _g(w.D), _g(w.q_mask), _g(w.d_mask))
    torch.cuda.synchronize()
    _assert_close("scores (no argmax)", s2.cpu().numpy(), rs)


@pytest.mark.parametrize("d", [64, 300])
def test_split_docs_across_waves(ms, oracle_mod, d):
    """A workgroup's rows are split among its waves: long docs continue across
    several waves (their partial maxima handed over to the owner), empty docs
    sit on wave boundaries, and duplicated rows put exact ties on both sides of
    a boundary (the lowest row must win)."""
    _say(f"split docs across waves d={d}")
    rng = np.random.default_rng(90 + d)
    lens = [0, 0, 1000, 0, 3, 0, 37, 0, 700, 16, 0]
    w = synth.random_varlen(2100 + d, [32, 20], lens, dtype=torch.float16, d=d)
    Dk = (torch.from_numpy(rng.integers(-2, 3, size=(int(w.cu_d[-1]), d)) / 8.0)).to(torch.float16)
    Qk = (torch.from_numpy(rng.integers(-2, 3, size=(int(w.cu_q[-1]), d)) / 8.0)).to(torch.float16)
    c = w.cu_d.numpy()
    Dk[c[2] + 600:c[2] + 700] = Dk[c[2] + 10:c[2] + 110]  # ties far apart in the long doc
    Dk[c[8] + 500:c[8] + 560] = Dk[c[8]:c[8] + 60]
    s, a = ms.maxsim_fwd_varlen(_g(Qk), _g(w.cu_q), w.max_lq, _g(Dk), _g(w.cu_d), want_argmax=True)
    torch.cuda.synchronize()
    rs, ra = oracle_mod.fwd_varlen(Qk, w.cu_q, w.max_lq, Dk, w.cu_d)
    assert np.array_equal(s.cpu().numpy().astype(np.float64), rs)  # k/8 values: exact in fp32
    assert np.array_equal(a.cpu().numpy(), ra)


@pytest.mark.parametrize("d", [64, 100, 300])
def test_dense_widths_exact_ties(ms, oracle_mod, d):
    """Values k/8 make every dot product exact in fp32, so scores and argmax
    (lowest index on ties) must equal the oracle's exactly."""
    _say(f"dense width exact ties d={d}")
    rng = np.random.default_rng(70 + d)
    Nq, Nd, Lq, Ld = 3, 4, 40, 150
    Q = torch.from_numpy(rng.integers(-2, 3, size=(Nq, Lq, d)) / 8.0).to(torch.float16)
    D = torch.from_numpy(rng.integers(-2, 3, size=(Nd, Ld, d)) / 8.0).to(torch.float16)
    D[:, 100:140] = D[:, 10:50]
    D[2] = D[2, 0]
    dm = torch.from_numpy((rng.random((Nd, Ld)) > 0.1).astype(np.uint8))
    s, a = ms.maxsim_fwd(_g(Q), _g(D), None, _g(dm), want_argmax=True)
    torch.cuda.synchronize()
    rs, ra = oracle_mod.fwd(Q, D, None, dm)
    assert np.array_equal(s.cpu().numpy().astype(np.float64), rs)
    assert np.array_equal(a.cpu().numpy(), ra)


def test_dense_widths_empty(ms):
    _say("dense width empty sizes")
    Q = torch.zeros((2, 0, 64), dtype=torch.float16, device=DEV)
    D = torch.randn((3, 5, 64), device=DEV).half()
    s, a = ms.maxsim_fwd(Q, D, want_argmax=True)
    torch.cuda.synchronize()
    assert torch.all(s == 0)
    D0 = torch.zeros((3, 0, 300), dtype=torch.bfloat16, device=DEV)
    Q1 = torch.randn((2, 4, 300), device=DEV).bfloat16()
    s, a = ms.maxsim_fwd(Q1, D0, want_argmax=True)
    torch.cuda.synchronize()
    assert torch.all(s == 0) and torch.all(a == 0)


VARLEN_CASES = [
    # (query lengths, doc lengths, dtype, d)
    ([32], [50, 0, 1, 17, 300, 0, 0, 64, 16, 15], torch.float16, 64),
    ([5, 0, 32, 31], list(range(0, 120, 7)), torch.bfloat16, 100),
    ([60, 17], [40] * 30 + [0] * 5, torch.float16, 384),
    ([130], [33, 80, 1, 0, 200], torch.bfloat16, 96),
    ([3], [0, 0, 0], torch.float16, 200),
    ([32], synth.rerank_lengths(71, 3000, 1, 120).tolist(), torch.float16, 64),
]


@pytest.mark.parametrize("case", VARLEN_CASES, ids=lambda c: f"q{len(c[0])}_d{len(c[1])}_w{c[3]}")
def test_varlen_widths(ms, oracle_mod, case):
    ql, dl, dt, d = case
    _say(f"varlen width q{ql[:4]} docs{len(dl)} d={d}")
    w = synth.random_varlen(1300 + d + len(dl), ql, dl, dtype=dt, d=d)
    s, a = ms.maxsim_fwd_varlen(_g(w.Q), _g(w.cu_q), w.max_lq, _g(w.D), _g(w.cu_d), want_argmax=True)
    torch.cuda.synchronize()
    rs, ra = oracle_mod.fwd_varlen(w.Q, w.cu_q, w.max_lq, w.D, w.cu_d)
    _assert_close("scores", s.cpu().numpy(), rs)
    n, acc, bad = compare.varlen_argmax_float(a.cpu().numpy(), ra, w.Q.double().numpy(),
                                              w.cu_q.numpy(), w.D.double().numpy(), w.cu_d.numpy(),
                                              np.arange(len(ql)), np.arange(len(dl)))
    assert not bad, bad[:5]
    s2, _ = ms.maxsim_fwd_varlen(_g(w.Q), _g(w.cu_q), w.max_lq, _g(w.D), _g(w.cu_d))
    torch.cuda.synchronize()
    _assert_close("scores (no argmax)", s2.cpu().numpy(), rs)


@pytest.mark.parametrize("d", [64, 300])
def test_pairs_widths(ms, oracle_mod, d):
    _say(f"pairs width d={d}")
    Nq, Nd, Lq, Ld, P = 3, 5, 40, 150, 40
    w = synth.random_dense(1400 + d, Nq, Nd, Lq, Ld, dtype=torch.bfloat16, q_mask_p=0.2,
                           d_mask_p=0.2, dead_docs=1, d=d)
    pq, pd = synth.random_pairs(1400 + d, Nq, Nd, P)
    s, a = ms.maxsim_fwd_pairs(_g(w.Q), _g(w.D), _g(pq), _g(pd), _g(w.q_mask), _g(w.d_mask),
                               want_argmax=True)
    torch.cuda.synchronize()
    rs, ra = oracle_mod.fwd_pairs(w.Q, w.D, pq, pd, w.q_mask, w.d_mask)
    _assert_close("scores", s.cpu().numpy(), rs)
    n, acc, bad = compare.pair_argmax_float(a.cpu().numpy(), ra, w.Q.double().numpy(),
                                            w.D.double().numpy(), w.d_mask.numpy(),
                                            pq.numpy(), pd.numpy())
    assert not bad, f"argmax mismatches outside the near-tie bound: {bad[:5]}"


@pytest.mark.parametrize("d", [96, 520])
def test_pairs_varlen_widths(ms, oracle_mod, d):
    _say(f"pairs varlen width d={d}")
    ql, dl, P = [32, 5, 0, 70], [50, 0, 1, 300, 64, 16], 40
    w = synth.random_varlen(1500 + d, ql, dl, dtype=torch.float16, d=d)
    pq, pd = synth.random_pairs(1500 + d, len(ql), len(dl), P)
    s, a = ms.maxsim_fwd_pairs_varlen(_g(w.Q), _g(w.cu_q), w.max_lq, _g(w.D), _g(w.cu_d), _g(pq),
                                      _g(pd), want_argmax=True)
    torch.cuda.synchronize()
    rs, ra = oracle_mod.fwd_pairs_varlen(w.Q, w.cu_q, w.max_lq, w.D, w.cu_d, pq, pd)
    _assert_close("scores", s.cpu().numpy(), rs)
    n, acc, bad = compare.pairs_varlen_argmax_float(a.cpu().numpy(), ra, w.Q.double().numpy(),
                                                    w.cu_q.numpy(), w.D.double().numpy(),
                                                    w.cu_d.numpy(), pq.numpy(), pd.numpy())
    assert not bad, f"argmax mismatches outside the near-tie bound: {bad[:5]}"


@pytest.mark.parametrize("d", [64, 200])
def test_dense_widths_many_queries(ms, oracle_mod, d):
    """More queries than the grid's query axis holds (65,535): workgroups loop
    over queries, with the staged-query barriers when d > 128."""
    _say(f"dense width many queries d={d}")
    Nq, Nd, Lq, Ld = 70_000, 3, 2, 7
    w = synth.random_dense(2000 + d, Nq, Nd, Lq, Ld, dtype=torch.float16, d_mask_p=0.2, d=d)
    s, a = ms.maxsim_fwd(_g(w.Q), _g(w.D), None, _g(w.d_mask), want_argmax=True)
    torch.cuda.synchronize()
    rs, ra = oracle_mod.fwd(w.Q, w.D, None, w.d_mask)
    _assert_close("scores", s.cpu().numpy(), rs)
    n, acc, bad = compare.dense_argmax_float(a.cpu().numpy(), ra, w.Q.double().numpy(),
                                             w.D.double().numpy(), w.d_mask.numpy())
    assert not bad, f"argmax mismatches outside the near-tie bound: {bad[:5]}"


@pytest.mark.parametrize("d", [64, 100, 256, 768])
def test_dim_sweep_full_size_sampled(ms, oracle_mod, d):
    """The width sweep at full size (one 32-token query against 10,000 docs of
    128 tokens, fp16) in the benchmark's launch configuration; the oracle
    scores 400 docs including both ends."""
    _say(f"width sweep full size d={d}")
    w = synth.dim_scaling_fp16(d)
    s, _ = ms.maxsim_fwd(_g(w.Q), _g(w.D))
    torch.cuda.synchronize()
    rng = np.random.default_rng(d)
    docs = np.unique(np.concatenate([np.arange(100), np.arange(9900, 10000),
                                     rng.choice(10000, 200, replace=False)]))
    rs, _ = oracle_mod.fwd(w.Q, w.D[docs], want_argmax=False)
    _assert_close("scores", s.cpu().numpy()[:, docs], rs)


BWD_CASES = [
    # (Nq, Nd, Lq, Ld, dtype, d, mask_p, hub)
    (3, 4, 9, 14, torch.float16, 64, 0.3, 0.0),
    (5, 6, 70, 130, torch.bfloat16, 100, 0.2, 0.0),    # 200-byte rows: element gathers
    (4, 3, 64, 64, torch.bfloat16, 300, 0.0, 0.7),     # three chunks, hub token
    (2, 3, 33, 50, torch.float16, 768, 0.1, 0.0),
    (2, 2, 5, 9, torch.float16, 1021, 0.0, 0.0),
    (2, 2, 4, 6, torch.bfloat16, 3, 0.0, 0.0),
]


@pytest.mark.parametrize("case", BWD_CASES,
                         ids=lambda c: f"{c[0]}x{c[1]}_lq{c[2]}_ld{c[3]}_{str(c[4])[6:]}_d{c[5]}")
def test_bwd_widths(ms, oracle_mod, case):
    Nq, Nd, Lq, Ld, dt, d, p, hub = case
    _say(f"bwd width {case}")
    w = synth.random_dense(1600 + d + Lq, Nq, Nd, Lq, Ld, dtype=dt, q_mask_p=p, d_mask_p=p,
                           dead_docs=1 if p > 0 else 0, d=d)
    if hub > 0:
        argmax = synth.draw_argmax(1600 + d, Nq, Nd, Lq, Ld, None, hub_frac=hub)
    else:
        _, ra = oracle_mod.fwd(w.Q, w.D, w.q_mask, w.d_mask)
        argmax = torch.from_numpy(ra)
    g = synth.upstream_grad(1600 + d, Nq, Nd)

    def run():
        out = ms.maxsim_bwd(_g(w.Q), _g(w.D), _g(argmax), _g(g), _g(w.q_mask), _g(w.d_mask))
        torch.cuda.synchronize()
        return [t.cpu() for t in out]

    dQ, dD, rp, ci = run()
    rdQ, rdD, rrp, rci = oracle_mod.bwd(w.Q, w.D, argmax, g, w.q_mask, w.d_mask)
    assert np.array_equal(rp.numpy(), rrp), "row_ptr"
    assert np.array_equal(ci.numpy(), rci), "col_idx"
    _assert_close("dQ", dQ.numpy(), rdQ)
    _assert_close("dD", dD.numpy(), rdD)
    again = run()
    assert all(torch.equal(x, y) for x, y in zip(again, (dQ, dD, rp, ci))), "not deterministic"


VARBWD_CASES = [
    # (query lengths, doc lengths, dtype, d)
    ([5, 12, 3], [7, 0, 19, 3, 1], torch.float16, 64),
    ([32] * 4, list(range(50, 300, 13)), torch.bfloat16, 100),
    ([0, 3, 40], [4, 0, 60], torch.bfloat16, 384),
    ([7], [9, 2], torch.float16, 1000),
]


@pytest.mark.parametrize("case", VARBWD_CASES, ids=lambda c: f"q{len(c[0])}_d{len(c[1])}_w{c[3]}")
def test_bwd_varlen_widths(ms, oracle_mod, case):
    ql, dl, dt, d = case
    _say(f"bwd varlen width {ql[:4]} {dl[:6]} d={d}")
    seed = 1700 + d + len(dl)
    w = synth.random_varlen(seed, ql, dl, dtype=dt, max_lq=max(max(ql), 1), d=d)
    _, ra = oracle_mod.fwd_varlen(w.Q, w.cu_q, w.max_lq, w.D, w.cu_d)
    argmax = torch.from_numpy(ra)
    g = synth.upstream_grad(seed, len(ql), len(dl))

    def run():
        out = ms.maxsim_bwd_varlen(_g(w.Q), _g(w.cu_q), w.max_lq, _g(w.D), _g(w.cu_d), _g(argmax), _g(g))
        torch.cuda.synchronize()
        return tuple(x.cpu() for x in out)

    dQ, dD, rp, ci = run()
    rdQ, rdD, rrp, rci = oracle_mod.bwd_varlen(w.Q, w.cu_q, w.max_lq, w.D, w.cu_d, argmax, g)
    assert np.array_equal(rp.numpy(), rrp), "row_ptr"
    assert np.array_equal(ci.numpy()[:len(rci)], rci), "col_idx"
    _assert_close("dQ", dQ.numpy(), rdQ)
    _assert_close("dD", dD.numpy(), rdD)
    again = run()
    assert all(torch.equal(x, y) for x, y in zip(again[:3], (dQ, dD, rp))), "not deterministic"


INT8_CASES = [
    # (Nq, Nd, Lq, Ld, kind, d, q_mask_p, d_mask_p)
    (2, 5, 9, 13, "ternary", 64, 0.2, 0.2),
    (3, 4, 100, 130, "quantised", 100, 0.0, 0.3),    # 100-byte rows: byte gathers
    (2, 3, 128, 64, "extreme", 300, 0.0, 0.0),       # largest sums, two chunks
    (1, 3, 64, 70, "quantised", 1000, 0.1, 0.0),     # four chunks, partial K-step
    (2, 3, 40, 50, "ternary", 256, 0.0, 0.1),        # exactly one chunk
    (1, 2, 100, 40, "quantised", 48, 0.0, 0.0),      # four passes
    (2, 2, 3, 5, "ternary", 7, 0.0, 0.0),
]


@pytest.mark.parametrize("case", INT8_CASES, ids=lambda c: f"{c[0]}x{c[1]}_lq{c[2]}_ld{c[3]}_{c[4]}_d{c[5]}")
def test_int8_widths(ms, oracle_mod, case):
    Nq, Nd, Lq, Ld, kind, d, qp, dp = case
    _say(f"int8 width {case}")
    w = synth.random_int8(1800 + d + Lq, Nq, Nd, Lq, Ld, ternary=kind == "ternary",
                          extreme=kind == "extreme", d_mask_p=dp, q_mask_p=qp, d=d)

    def run(want_argmax, both=True):
        si = torch.empty((Nq, Nd), dtype=torch.int32, device=DEV) if both else None
        out = ms.maxsim_fwd_i8(_g(w.Q), w.q_scale, _g(w.D), w.d_scale, _g(w.q_mask), _g(w.d_mask),
                               want_argmax=want_argmax, scores_i32=si)
        torch.cuda.synchronize()
        return [None if t is None else t.cpu() for t in out]

    si, sf, a = run(True)
    ri, rf, ra = oracle_mod.fwd_i8(w.Q, w.q_scale, w.D, w.d_scale, w.q_mask, w.d_mask)
    assert np.array_equal(si.numpy().astype(np.int64), ri)
    assert np.array_equal(sf.numpy(), rf.astype(np.float32))  # same double rounding
    assert np.array_equal(a.numpy(), ra)
    si2, sf2, _ = run(False)
    assert torch.equal(si2, si) and torch.equal(sf2, sf)
    # float scores alone: the running int32 sum is kept in the float output's bits
    _, sf3, _ = ms.maxsim_fwd_i8(_g(w.Q), w.q_scale, _g(w.D), w.d_scale, _g(w.q_mask), _g(w.d_mask),
                                 want_int=False)
    torch.cuda.synchronize()
    assert torch.equal(sf3.cpu(), sf)


@pytest.mark.parametrize("d", [64, 100, 384])
def test_int8_tok_widths(ms, oracle_mod, d):
    _say(f"int8 per-token width d={d}")
    Nq, Nd, Lq, Ld = 3, 5, 70, 90
    w = synth.random_int8_tok(1900 + d, Nq, Nd, Lq, Ld, q_mask_p=0.2, d_mask_p=0.2, dead_docs=1, d=d)
    s, a = ms.maxsim_fwd_i8_tok(_g(w.Q), _g(w.q_scale), _g(w.D), _g(w.d_scale), _g(w.q_mask),
                                _g(w.d_mask), want_argmax=True)
    s2, _ = ms.maxsim_fwd_i8_tok(_g(w.Q), _g(w.q_scale), _g(w.D), _g(w.d_scale), _g(w.q_mask),
                                 _g(w.d_mask))
    torch.cuda.synchronize()
    rs, ra = oracle_mod.fwd_i8_tok(w.Q, w.q_scale, w.D, w.d_scale, w.q_mask, w.d_mask)
    _assert_close("scores", s.cpu().numpy(), rs)
    _assert_close("scores (no argmax)", s2.cpu().numpy(), rs)
    n, acc, bad = compare.int8_tok_argmax(a.cpu().numpy(), ra, w.Q.numpy(), w.D.numpy(),
                                          w.d_scale.numpy(), w.d_mask.numpy())
    assert not bad, f"argmax mismatches outside the rounding bound: {bad[:5]}"
