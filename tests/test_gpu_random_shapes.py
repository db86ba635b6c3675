"""GPU parity on a seeded sweep of irregular shapes: the dense forward (with
masks, dead rows and widths other than 128), its backward through the
oracle's argmax, the packed forward with empty and ragged sequences, the
int8 forwards (per-tensor and per-token scales), the packed backward, the
pair-list scorers, top-k, and Chamfer on clouds of any size, offset and
scale, each against the CPU oracle under the same rules as
tests/test_gpu_parity.py.
The shapes are drawn once from a fixed seed, so every run checks the same
cases; they sit off the tile sizes the kernels use (16, 32, 64, 128, 256)."""

import numpy as np
import pytest
import torch

from maxsim_scoring_amd import synth
from oracle import compare
from test_gpu_parity import (_assert_close, _assert_float_argmax, _chamfer_gpu, _check_bwd,  # noqa: F401
                             _check_chamfer_bwd, _check_chamfer_fwd, _g, _run_bwd_varlen, _say, ms)

pytestmark = pytest.mark.gpu

_rng = np.random.default_rng(2027)
DTYPES = (torch.float16, torch.bfloat16)
WIDTHS = (128, 128, 128, 64, 96, 200, 256)


def _dense_case(k):
    return dict(seed=900 + k, Nq=int(_rng.integers(1, 7)), Nd=int(_rng.integers(1, 25)),
                Lq=int(_rng.integers(1, 261)), Ld=int(_rng.integers(1, 301)),
                dtype=DTYPES[int(_rng.integers(0, 2))], d=int(WIDTHS[int(_rng.integers(0, len(WIDTHS)))]),
                q_mask_p=float(_rng.choice([0.0, 0.2, 0.5])), d_mask_p=float(_rng.choice([0.0, 0.2, 0.5])),
                dead_docs=int(_rng.integers(0, 2)), dead_queries=int(_rng.integers(0, 2)))


DENSE = [_dense_case(k) for k in range(16)]
for c in DENSE:
    c["dead_docs"] = min(c["dead_docs"], c["Nd"])
    c["dead_queries"] = min(c["dead_queries"], c["Nq"])


def _varlen_case(k):
    nq, nd = int(_rng.integers(1, 4)), int(_rng.integers(1, 31))
    ql = [int(x) for x in _rng.integers(0, 101, nq)]
    ql[0] = max(ql[0], 1)
    dl = [int(x) if _rng.random() > 0.15 else 0 for x in _rng.integers(1, 301, nd)]
    return dict(seed=950 + k, ql=ql, dl=dl, dtype=DTYPES[int(_rng.integers(0, 2))],
                d=int((128, 128, 64, 192)[int(_rng.integers(0, 4))]))


VARLEN = [_varlen_case(k) for k in range(8)]


def _dense_id(c):
    return f"{c['Nq']}x{c['Nd']}_lq{c['Lq']}_ld{c['Ld']}_d{c['d']}_{str(c['dtype'])[6:]}"


@pytest.mark.parametrize("case", DENSE, ids=_dense_id)
def test_random_dense_fwd_bwd(ms, oracle_mod, case):
    c = case
    _say(f"random dense {_dense_id(c)}")
    w = synth.random_dense(c["seed"], c["Nq"], c["Nd"], c["Lq"], c["Ld"], dtype=c["dtype"],
                           q_mask_p=c["q_mask_p"], d_mask_p=c["d_mask_p"], dead_docs=c["dead_docs"],
                           dead_queries=c["dead_queries"], d=c["d"])
    s, a = ms.maxsim_fwd(_g(w.Q), _g(w.D), _g(w.q_mask), _g(w.d_mask), want_argmax=True)
    torch.cuda.synchronize()
    rs, ra = oracle_mod.fwd(w.Q, w.D, w.q_mask, w.d_mask)
    _assert_close("scores", s.cpu().numpy(), rs)
    _assert_float_argmax("argmax", a.cpu().numpy(), ra, w)
    # the backward through the oracle's argmax
    g = synth.upstream_grad(c["seed"], c["Nq"], c["Nd"])
    _check_bwd(ms, oracle_mod, w, torch.from_numpy(ra), g)


@pytest.mark.parametrize("case", VARLEN, ids=lambda c: f"q{len(c['ql'])}_d{len(c['dl'])}_w{c['d']}")
def test_random_varlen_fwd(ms, oracle_mod, case):
    c = case
    _say(f"random varlen {c['ql']} {c['dl']} d{c['d']}")
    w = synth.random_varlen(c["seed"], c["ql"], c["dl"], dtype=c["dtype"], d=c["d"])
    s, a = ms.maxsim_fwd_varlen(_g(w.Q), _g(w.cu_q), w.max_lq, _g(w.D), _g(w.cu_d), want_argmax=True)
    torch.cuda.synchronize()
    rs, ra = oracle_mod.fwd_varlen(w.Q, w.cu_q, w.max_lq, w.D, w.cu_d)
    _assert_close("scores", s.cpu().numpy(), rs)
    n, acc, bad = compare.varlen_argmax_float(a.cpu().numpy(), ra, w.Q.double().numpy(), w.cu_q.numpy(),
                                              w.D.double().numpy(), w.cu_d.numpy(),
                                              np.arange(len(c["ql"])), np.arange(len(c["dl"])))
    assert not bad, bad[:5]


def _int8_case(k):
    return dict(seed=980 + k, Nq=int(_rng.integers(1, 5)), Nd=int(_rng.integers(1, 20)),
                Lq=int(_rng.integers(1, 300)), Ld=int(_rng.integers(1, 300)),
                d=int((128, 128, 64, 192, 256)[int(_rng.integers(0, 5))]),
                q_mask_p=float(_rng.choice([0.0, 0.3])), d_mask_p=float(_rng.choice([0.0, 0.3])),
                ternary=bool(_rng.random() < 0.3))


INT8 = [_int8_case(k) for k in range(8)]


def _int8_id(c):
    return f"{c['Nq']}x{c['Nd']}_lq{c['Lq']}_ld{c['Ld']}_d{c['d']}" + ("_ternary" if c["ternary"] else "")


@pytest.mark.parametrize("case", INT8, ids=_int8_id)
def test_random_int8_fwd(ms, oracle_mod, case):
    """Per-tensor scales: exact int32 sums and argmax, the same fp32 scores;
    per-token scales on the same shapes: scores within tolerance, argmax
    within the scale-product rounding bound."""
    c = case
    _say(f"random int8 {_int8_id(c)}")
    w = synth.random_int8(c["seed"], c["Nq"], c["Nd"], c["Lq"], c["Ld"], ternary=c["ternary"],
                          q_mask_p=c["q_mask_p"], d_mask_p=c["d_mask_p"], d=c["d"])
    si, sf, a = ms.maxsim_fwd_i8(_g(w.Q), w.q_scale, _g(w.D), w.d_scale, _g(w.q_mask), _g(w.d_mask),
                                 want_argmax=True)
    torch.cuda.synchronize()
    ri, rf, ra = oracle_mod.fwd_i8(w.Q, w.q_scale, w.D, w.d_scale, w.q_mask, w.d_mask)
    assert np.array_equal(si.cpu().numpy().astype(np.int64), ri)
    assert np.array_equal(sf.cpu().numpy(), rf.astype(np.float32))
    assert np.array_equal(a.cpu().numpy(), ra)
    t = synth.random_int8_tok(c["seed"], c["Nq"], c["Nd"], c["Lq"], c["Ld"], q_mask_p=c["q_mask_p"],
                              d_mask_p=c["d_mask_p"], d=c["d"])
    s, a = ms.maxsim_fwd_i8_tok(_g(t.Q), _g(t.q_scale), _g(t.D), _g(t.d_scale), _g(t.q_mask),
                                _g(t.d_mask), want_argmax=True)
    torch.cuda.synchronize()
    rs, ra = oracle_mod.fwd_i8_tok(t.Q, t.q_scale, t.D, t.d_scale, t.q_mask, t.d_mask)
    _assert_close("scores (per-token)", s.cpu().numpy(), rs)
    n, acc, bad = compare.int8_tok_argmax(a.cpu().numpy(), ra, t.Q.numpy(), t.D.numpy(), t.d_scale.numpy(),
                                          None if t.d_mask is None else t.d_mask.numpy())
    assert not bad, f"argmax mismatches outside the rounding bound: {bad[:5]}"


def _chamfer_case(k):
    return dict(seed=1100 + k, B=int(_rng.integers(1, 7)), N=int(_rng.integers(1, 3001)),
                M=int(_rng.integers(1, 3001)), scale=float(_rng.choice([0.01, 1.0, 100.0])),
                offset=float(_rng.choice([0.0, 1000.0])), dup=bool(_rng.random() < 0.4))


CHAMFER = [_chamfer_case(k) for k in range(8)] + [
    dict(seed=1190, B=3, N=1, M=1, scale=1.0, offset=0.0, dup=False),
    dict(seed=1191, B=2, N=1, M=2500, scale=1.0, offset=5.0, dup=True),
]


def _chamfer_id(c):
    return f"{c['B']}x{c['N']}x{c['M']}_s{c['scale']}_o{c['offset']}" + ("_dup" if c["dup"] else "")


@pytest.mark.parametrize("case", CHAMFER, ids=_chamfer_id)
def test_random_chamfer(ms, oracle_mod, case):
    """Forward under the direct-form rules, then the backward through the
    GPU's indices: both CSRs bit for bit and the gradients within their
    rounding bound. Clouds are scaled and moved far from the origin; with
    `dup` a random half of the targets is repeated (exact ties)."""
    c = case
    _say(f"random chamfer {_chamfer_id(c)}")
    rng = np.random.default_rng(c["seed"])
    P = (rng.standard_normal((c["B"], c["N"], 3)) * c["scale"] + c["offset"]).astype(np.float32)
    Q = (rng.standard_normal((c["B"], c["M"], 3)) * c["scale"] + c["offset"]).astype(np.float32)
    if c["dup"] and c["M"] > 1:
        pick = rng.choice(c["M"], c["M"] // 2, replace=False)
        Q[:, pick[1:]] = Q[:, pick[:-1]]
    P, Q = torch.from_numpy(P), torch.from_numpy(Q)
    got = _chamfer_gpu(ms, P, Q)
    _check_chamfer_fwd(oracle_mod, P, Q, got)
    _, i1, _, i2, _ = got
    g1, g2 = synth.chamfer_grads(c["seed"], c["B"], c["N"], c["M"])
    out = ms.maxsim_chamfer_bwd(_g(P), _g(Q), _g(i1), _g(i2), _g(g1), _g(g2))
    torch.cuda.synchronize()
    dP, dQ, rp1, ci1, rp2, ci2 = (x.cpu() for x in out)
    rdP, rdQ, rrp1, rci1, rrp2, rci2 = oracle_mod.chamfer_bwd(P, Q, i1, i2, g1, g2)
    for name, x, y in (("row_ptr1", rp1, rrp1), ("col_idx1", ci1, rci1), ("row_ptr2", rp2, rrp2),
                       ("col_idx2", ci2, rci2)):
        assert np.array_equal(x.numpy(), y), name
    _check_chamfer_bwd(P, Q, i1, i2, g1, g2, dP, dQ, rdP, rdQ)


def _varbwd_case(k):
    nq, nd = int(_rng.integers(1, 9)), int(_rng.integers(1, 12))
    ql = [int(x) if _rng.random() > 0.15 else 0 for x in _rng.integers(1, 140, nq)]
    dl = [int(x) if _rng.random() > 0.15 else 0 for x in _rng.integers(1, 1200, nd)]
    return dict(seed=1200 + k, ql=ql, dl=dl, dtype=DTYPES[int(_rng.integers(0, 2))],
                d=int((128, 128, 64, 200)[int(_rng.integers(0, 4))]), from_fwd=bool(_rng.random() < 0.5),
                hub=float(_rng.choice([0.0, 0.0, 0.6])))


VARBWD = [_varbwd_case(k) for k in range(8)]


@pytest.mark.parametrize("case", VARBWD, ids=lambda c: f"q{len(c['ql'])}_d{len(c['dl'])}_w{c['d']}_hub{c['hub']}")
def test_random_bwd_varlen(ms, oracle_mod, case):
    c = case
    _say(f"random bwd varlen {c['ql']} {c['dl']} d{c['d']}")
    w = synth.random_varlen(c["seed"], c["ql"], c["dl"], dtype=c["dtype"], d=c["d"],
                            max_lq=max(max(c["ql"]), 1))
    if c["from_fwd"] or c["hub"] == 0.0:
        _, ra = oracle_mod.fwd_varlen(w.Q, w.cu_q, w.max_lq, w.D, w.cu_d)
        argmax = torch.from_numpy(ra)
    else:
        argmax = synth.draw_argmax_varlen(c["seed"], w.cu_q, w.cu_d, w.max_lq, hub_frac=c["hub"])
    g = synth.upstream_grad(c["seed"], len(c["ql"]), len(c["dl"]))
    dQ, dD, rp, ci = _run_bwd_varlen(ms, w, argmax, g)
    rdQ, rdD, rrp, rci = oracle_mod.bwd_varlen(w.Q, w.cu_q, w.max_lq, w.D, w.cu_d, argmax, g)
    assert np.array_equal(rp.numpy(), rrp), "row_ptr"
    assert np.array_equal(ci.numpy()[:len(rci)], rci), "col_idx"
    _assert_close("dQ", dQ.numpy(), rdQ)
    _assert_close("dD", dD.numpy(), rdD)


def _pairs_case(k):
    return dict(seed=1300 + k, Nq=int(_rng.integers(1, 6)), Nd=int(_rng.integers(1, 9)),
                Lq=int(_rng.integers(1, 300)), Ld=int(_rng.integers(1, 400)), P=int(_rng.integers(1, 60)),
                dtype=DTYPES[int(_rng.integers(0, 2))], d=int((128, 128, 96)[int(_rng.integers(0, 3))]))


PAIRS = [_pairs_case(k) for k in range(6)]


@pytest.mark.parametrize("case", PAIRS, ids=lambda c: f"{c['Nq']}x{c['Nd']}_lq{c['Lq']}_ld{c['Ld']}_p{c['P']}_d{c['d']}")
def test_random_pairs(ms, oracle_mod, case):
    """Dense pair lists with masks, and the same pairs over the packed layout
    of the same rows (every query and doc its full length)."""
    c = case
    _say(f"random pairs {c}")
    w = synth.random_dense(c["seed"], c["Nq"], c["Nd"], c["Lq"], c["Ld"], dtype=c["dtype"], q_mask_p=0.2,
                           d_mask_p=0.2, d=c["d"])
    pq, pd = synth.random_pairs(c["seed"], c["Nq"], c["Nd"], c["P"])
    s, a = ms.maxsim_fwd_pairs(_g(w.Q), _g(w.D), _g(pq), _g(pd), _g(w.q_mask), _g(w.d_mask), want_argmax=True)
    torch.cuda.synchronize()
    rs, ra = oracle_mod.fwd_pairs(w.Q, w.D, pq, pd, w.q_mask, w.d_mask)
    _assert_close("scores", s.cpu().numpy(), rs)
    n, acc, bad = compare.pair_argmax_float(a.cpu().numpy(), ra, w.Q.double().numpy(), w.D.double().numpy(),
                                            None if w.d_mask is None else w.d_mask.numpy(), pq.numpy(),
                                            pd.numpy())
    assert not bad, bad[:5]
    Qp = w.Q.reshape(-1, c["d"]).contiguous()
    Dp = w.D.reshape(-1, c["d"]).contiguous()
    cu_q = synth.cu_seqlens(np.full(c["Nq"], c["Lq"]))
    cu_d = synth.cu_seqlens(np.full(c["Nd"], c["Ld"]))
    s2, a2 = ms.maxsim_fwd_pairs_varlen(_g(Qp), _g(cu_q), c["Lq"], _g(Dp), _g(cu_d), _g(pq), _g(pd),
                                        want_argmax=True)
    torch.cuda.synchronize()
    rs2, ra2 = oracle_mod.fwd_pairs_varlen(Qp, cu_q, c["Lq"], Dp, cu_d, pq, pd)
    _assert_close("packed scores", s2.cpu().numpy(), rs2)
    n, acc, bad = compare.pairs_varlen_argmax_float(a2.cpu().numpy(), ra2, Qp.double().numpy(), cu_q.numpy(),
                                                    Dp.double().numpy(), cu_d.numpy(), pq.numpy(), pd.numpy())
    assert not bad, bad[:5]


def _topk_case(k):
    nd = int(_rng.integers(1, 30000))
    return dict(seed=1400 + k, Nq=int(_rng.integers(1, 5)), Nd=nd, k=int(_rng.integers(0, min(nd, 1024) + 1)),
                ties=bool(_rng.random() < 0.5))


TOPK = [_topk_case(k) for k in range(8)]


@pytest.mark.parametrize("case", TOPK, ids=lambda c: f"{c['Nq']}x{c['Nd']}_k{c['k']}_ties{int(c['ties'])}")
def test_random_topk(ms, oracle_mod, case):
    c = case
    _say(f"random topk {c}")
    v = synth.random_scores(c["seed"], c["Nq"], c["Nd"], ties=c["ties"])
    idx, val, _ = ms.maxsim_topk(_g(v), c["k"])
    torch.cuda.synchronize()
    ri, rv = oracle_mod.topk(v, c["k"])
    assert np.array_equal(idx.cpu().numpy(), ri)
    assert np.array_equal(val.cpu().numpy().view(np.int32), rv.astype(np.float32).view(np.int32))
