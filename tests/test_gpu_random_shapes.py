"""GPU parity on a seeded sweep of irregular shapes: the dense forward (with
masks, dead rows and widths other than 128), its backward through the
oracle's argmax, the packed forward with empty and ragged sequences, and the
int8 forwards (per-tensor and per-token scales), each against the CPU oracle
under the same rules as tests/test_gpu_parity.py.
The shapes are drawn once from a fixed seed, so every run checks the same
cases; they sit off the tile sizes the kernels use (16, 32, 64, 128, 256)."""

import numpy as np
import pytest
import torch

from maxsim_scoring_amd import synth
from oracle import compare
from test_gpu_parity import _assert_close, _assert_float_argmax, _check_bwd, _g, _say, ms  # noqa: F401

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
