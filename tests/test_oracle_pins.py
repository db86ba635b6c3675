"""Pins for the CPU oracle: it is checked against things other than itself.

* a worked example computed by hand (tests/golden/hand_example.json);
* brute force by materialising S (tests/brute_force.py) on tiny inputs, with
  masks, dead docs/queries, exact ties and empty varlen sequences;
* closed forms and invariants the pages state or imply: self-score, chunked
  sums (late-interaction-kernels design notes, "Long-query chunking"),
  fully-masked doc -> 0, permutation invariance, power-of-two scaling,
  padding-free == padded (Flash-MaxSim Sec. 5.5), int8 == scaled float;
* special cases that reduce to a library routine (Ld = 1, Lq = 1);
* backward: finite differences, the Euler identity of a bilinear form at a
  fixed argmax, and the CSR against numpy's bincount/cumsum/stable argsort
  (the construction Flash-MaxSim Sec. 4.2.2 names).
"""

import json
import os

import numpy as np
import pytest
import torch

import brute_force as bf
from maxsim_scoring_amd import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _exact_grid(rng, shape, scale=8):
    """Values k/scale with small integer k: every dot product is exact."""
    return rng.integers(-scale, scale + 1, size=shape).astype(np.float64) / scale


# ----------------------------------------------------------------- worked example

def test_hand_example_forward(oracle_mod):
    g = _gold("hand_example.json")
    Q = np.array(g["Q"], np.float64)
    D = np.array(g["D"], np.float64)
    dm = np.array(g["d_mask"], np.uint8)
    s, a = oracle_mod.fwd(Q, D, None, dm)
    assert np.array_equal(s, np.array(g["scores"], np.float64))
    assert np.array_equal(a, np.array(g["argmax"], np.int32))
    v = g["q_mask_variant"]
    s, a = oracle_mod.fwd(Q, D, np.array(v["q_mask"], np.uint8), dm)
    assert np.array_equal(s, np.array(v["scores"], np.float64))
    assert np.array_equal(a, np.array(v["argmax"], np.int32))


def test_hand_example_backward(oracle_mod):
    g = _gold("hand_example.json")
    b = g["backward"]
    Q = np.array(g["Q"], np.float64)
    D = np.array(g["D"], np.float64)
    dm = np.array(g["d_mask"], np.uint8)
    arg = np.array(g["argmax"], np.int32)
    dQ, dD, rp, ci = oracle_mod.bwd(Q, D, arg, np.array(b["grad_scores"], np.float64),
                                    np.array(b["q_mask"], np.uint8), dm)
    assert np.array_equal(dQ, np.array(b["dQ"], np.float64))
    assert np.array_equal(dD, np.array(b["dD"], np.float64))
    assert np.array_equal(rp, np.array(b["row_ptr"], np.int32))
    assert np.array_equal(ci, np.array(b["col_idx"], np.int32))


def test_hand_example_int8(oracle_mod):
    g = _gold("hand_example.json")
    t = g["int8"]
    Q = np.array(g["Q"], np.int8)
    D = np.array(g["D"], np.int8)
    dm = np.array(g["d_mask"], np.uint8)
    si, sf, a = oracle_mod.fwd_i8(Q, t["q_scale"], D, t["d_scale"], None, dm)
    assert np.array_equal(si, np.array(t["score_int"], np.int64))
    assert np.array_equal(sf, np.array(t["score"], np.float64))
    assert np.array_equal(a, np.array(g["argmax"], np.int32))


# ----------------------------------------------------------------- brute force

@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
@pytest.mark.parametrize("shape", [(2, 3, 5, 7), (3, 4, 33, 70), (1, 5, 1, 1), (2, 2, 8, 0)])
def test_brute_force_random(oracle_mod, dtype, shape):
    Nq, Nd, Lq, Ld = shape
    w = synth.random_dense(11 + Lq, Nq, Nd, Lq, Ld, dtype=dtype, q_mask_p=0.3, d_mask_p=0.3,
                           dead_docs=1, dead_queries=1)
    s, a = oracle_mod.fwd(w.Q, w.D, w.q_mask, w.d_mask)
    sb, ab = bf.dense(w.Q, w.D, w.q_mask, w.d_mask)
    np.testing.assert_allclose(s, sb, rtol=0, atol=1e-12)
    assert np.array_equal(a, ab)
    # a dead doc contributes exactly 0 and keeps argmax 0
    assert np.all(s[:, -1] == 0.0)
    if Lq:
        assert np.all(a[:, -1, :] == 0)


def test_brute_force_exact_ties(oracle_mod):
    rng = np.random.default_rng(5)
    Nq, Nd, Lq, Ld, d = 3, 4, 6, 9, 16
    Q = _exact_grid(rng, (Nq, Lq, d))
    D = _exact_grid(rng, (Nd, Ld, d))
    D[:, 5] = D[:, 2]           # duplicated tokens: exact ties, lowest index must win
    D[:, 8] = D[:, 2]
    D[1, :] = D[1, 0]           # a doc whose tokens are all identical
    dm = (rng.random((Nd, Ld)) > 0.2).astype(np.uint8)
    dm[:, 2] = 1
    s, a = oracle_mod.fwd(Q, D, None, dm)
    sb, ab = bf.dense(Q, D, None, dm)
    assert np.array_equal(s, sb)
    assert np.array_equal(a, ab)
    assert not np.any(a == 5) and not np.any(a == 8)


def test_brute_force_varlen_with_empty(oracle_mod):
    w = synth.random_varlen(21, [3, 0, 17, 1], [5, 0, 1, 40, 0, 2])
    s, a = oracle_mod.fwd_varlen(w.Q, w.cu_q, w.max_lq, w.D, w.cu_d)
    sb, ab = bf.varlen(w.Q, w.cu_q, w.max_lq, w.D, w.cu_d)
    np.testing.assert_allclose(s, sb, rtol=0, atol=1e-12)
    assert np.array_equal(a, ab)
    assert np.all(s[1, :] == 0) and np.all(s[:, 1] == 0) and np.all(s[:, 4] == 0)


@pytest.mark.parametrize("kind", ["ternary", "quantised", "extreme"])
def test_brute_force_int8(oracle_mod, kind):
    w = synth.random_int8(31, 2, 5, 9, 13, ternary=kind == "ternary", extreme=kind == "extreme",
                          d_mask_p=0.2, q_mask_p=0.2)
    si, sf, a = oracle_mod.fwd_i8(w.Q, w.q_scale, w.D, w.d_scale, w.q_mask, w.d_mask)
    sb, ab = bf.dense(w.Q, w.D, w.q_mask, w.d_mask, exact_int=True)
    assert np.array_equal(si, sb)
    assert np.array_equal(a, ab)
    np.testing.assert_allclose(sf, sb * w.q_scale * w.d_scale, rtol=1e-15, atol=0)


# ----------------------------------------------------------------- closed forms

def test_self_score_is_sum_of_squared_norms(oracle_mod):
    """Cauchy-Schwarz: each unit query row scores 1 against itself and less
    against any other distinct row, so score(Q, Q) = Lq and argmax = identity."""
    rng = np.random.default_rng(7)
    Lq, d = 64, 128
    x = rng.standard_normal((1, Lq, d))
    x /= np.linalg.norm(x, axis=-1, keepdims=True)
    s, a = oracle_mod.fwd(x, x)
    assert abs(s[0, 0] - Lq) < 1e-12
    assert np.array_equal(a[0, 0], np.arange(Lq))
    # fp16-rounded rows: score = sum of squared norms of the rounded rows
    q16 = synth.unit_rows(3, 1, Lq).view(1, Lq, d)
    s16, a16 = oracle_mod.fwd(q16, q16)
    ref = float((q16.double() ** 2).sum())
    assert abs(s16[0, 0] - ref) < 1e-12
    assert abs(s16[0, 0] - Lq) < Lq * 2.0 ** -10
    assert np.array_equal(a16[0, 0], np.arange(Lq))


def test_ld_one_is_a_dot_product(oracle_mod):
    rng = np.random.default_rng(8)
    Q = rng.standard_normal((3, 10, 128))
    D = rng.standard_normal((4, 1, 128))
    s, a = oracle_mod.fwd(Q, D)
    ref = Q.sum(axis=1) @ D[:, 0, :].T
    np.testing.assert_allclose(s, ref, rtol=1e-12, atol=1e-12)
    assert np.all(a == 0)


def test_lq_one_is_max_of_gemv(oracle_mod):
    rng = np.random.default_rng(9)
    Q = rng.standard_normal((2, 1, 128))
    D = rng.standard_normal((3, 50, 128))
    s, a = oracle_mod.fwd(Q, D)
    for i in range(2):
        for j in range(3):
            v = D[j] @ Q[i, 0]
            assert abs(s[i, j] - v.max()) < 1e-12
            assert a[i, j, 0] == int(np.argmax(v))


# ----------------------------------------------------------------- invariants

def test_chunked_query_sum_equals_full(oracle_mod):
    """Design notes, "Long-query chunking": scoring 128-token chunks as separate
    queries and summing per query is exact."""
    w = synth.random_dense(41, 2, 3, 300, 50, dtype=torch.bfloat16, q_mask_p=0.2)
    s, a = oracle_mod.fwd(w.Q, w.D, w.q_mask, w.d_mask)
    parts, args = [], []
    for c0 in range(0, 300, 128):
        sl = slice(c0, min(300, c0 + 128))
        sc, ac = oracle_mod.fwd(w.Q[:, sl], w.D, w.q_mask[:, sl], w.d_mask)
        parts.append(sc)
        args.append(ac)
    np.testing.assert_allclose(sum(parts), s, rtol=1e-12, atol=1e-12)
    assert np.array_equal(np.concatenate(args, axis=2), a)
    # int8: exact
    wi = synth.random_int8(42, 1, 3, 300, 40)
    si, _, _ = oracle_mod.fwd_i8(wi.Q, wi.q_scale, wi.D, wi.d_scale)
    tot = sum(oracle_mod.fwd_i8(wi.Q[:, c:c + 128], wi.q_scale, wi.D, wi.d_scale)[0]
              for c in range(0, 300, 128))
    assert np.array_equal(tot, si)


def test_masked_query_rows_drop_out(oracle_mod):
    w = synth.random_dense(43, 2, 3, 20, 30, q_mask_p=0.5)
    s, a = oracle_mod.fwd(w.Q, w.D, w.q_mask, None)
    for i in range(2):
        keep = w.q_mask[i].bool()
        si, ai = oracle_mod.fwd(w.Q[i:i + 1, keep], w.D)
        np.testing.assert_allclose(s[i], si[0], rtol=1e-12, atol=1e-12)
    s_all, a_all = oracle_mod.fwd(w.Q, w.D)
    assert np.array_equal(a, a_all)  # masked rows keep their real argmax


def test_permutation_invariance(oracle_mod):
    w = synth.random_dense(44, 2, 3, 16, 40, dtype=torch.float16)
    s, a = oracle_mod.fwd(w.Q, w.D)
    rng = np.random.default_rng(0)
    pt = rng.permutation(40)
    s2, a2 = oracle_mod.fwd(w.Q, w.D[:, pt])
    np.testing.assert_allclose(s2, s, rtol=0, atol=1e-12)
    assert np.array_equal(pt[a2], a)
    ps = rng.permutation(16)
    s3, a3 = oracle_mod.fwd(w.Q[:, ps], w.D)
    np.testing.assert_allclose(s3, s, rtol=0, atol=1e-12)
    assert np.array_equal(a3, a[:, :, ps])


def test_power_of_two_scaling(oracle_mod):
    w = synth.random_dense(45, 2, 2, 8, 25, d_mask_p=0.3)
    s, a = oracle_mod.fwd(w.Q, w.D, None, w.d_mask)
    s2, a2 = oracle_mod.fwd(w.Q, w.D.double() * 2.0, None, w.d_mask)
    assert np.array_equal(s2, 2.0 * s)
    assert np.array_equal(a2, a)


def test_padding_free_equals_padded(oracle_mod):
    """Flash-MaxSim Sec. 5.5: the cu_seqlens path gives the padded scores."""
    lens_q = [5, 12]
    lens_d = [7, 1, 19, 3]
    w = synth.random_varlen(46, lens_q, lens_d)
    s, a = oracle_mod.fwd_varlen(w.Q, w.cu_q, w.max_lq, w.D, w.cu_d)
    Lq, Ld = max(lens_q), max(lens_d)
    Qp = torch.zeros(2, Lq, 128, dtype=w.Q.dtype)
    Dp = torch.zeros(4, Ld, 128, dtype=w.D.dtype)
    cq, cd = w.cu_q.tolist(), w.cu_d.tolist()
    for i in range(2):
        Qp[i, :lens_q[i]] = w.Q[cq[i]:cq[i + 1]]
    for j in range(4):
        Dp[j, :lens_d[j]] = w.D[cd[j]:cd[j + 1]]
    qm = synth.prefix_mask(np.array(lens_q), Lq)
    dm = synth.prefix_mask(np.array(lens_d), Ld)
    sp, ap = oracle_mod.fwd(Qp, Dp, qm, dm)
    assert np.array_equal(s, sp)
    for i in range(2):
        assert np.array_equal(a[i, :, :lens_q[i]], ap[i, :, :lens_q[i]])
        assert np.all(a[i, :, lens_q[i]:] == 0)


def test_int8_equals_scaled_float(oracle_mod):
    w = synth.random_int8(47, 2, 3, 20, 30)
    si, sf, a = oracle_mod.fwd_i8(w.Q, w.q_scale, w.D, w.d_scale)
    s, af = oracle_mod.fwd(w.Q.double() * w.q_scale, w.D.double() * w.d_scale)
    np.testing.assert_allclose(sf, s, rtol=1e-12, atol=1e-12)
    assert np.array_equal(a, af)


# ----------------------------------------------------------------- backward

def _loss(oracle_mod, Q, D, g, qm, dm):
    s, _ = oracle_mod.fwd(Q, D, qm, dm, want_argmax=False)
    return float((g * s).sum())


def test_backward_finite_differences(oracle_mod):
    """Central differences of L = sum g*score in fp64 on inputs whose top-2
    gaps are far larger than the step, so the argmax is fixed."""
    rng = np.random.default_rng(12)
    Nq, Nd, Lq, Ld, d = 2, 3, 3, 4, 5
    for _ in range(100):
        Q = rng.standard_normal((Nq, Lq, d))
        D = rng.standard_normal((Nd, Ld, d))
        S = np.einsum("isk,jtk->ijst", Q, D)
        srt = np.sort(S, axis=-1)
        if (srt[..., -1] - srt[..., -2]).min() > 1e-3:
            break
    qm = np.array([[1, 0, 1], [1, 1, 1]], np.uint8)
    dm = np.array([[1, 1, 1, 1], [0, 0, 0, 0], [1, 1, 1, 1]], np.uint8)
    g = rng.standard_normal((Nq, Nd))
    _, arg = oracle_mod.fwd(Q, D, qm, dm)
    dQ, dD, _, _ = oracle_mod.bwd(Q, D, arg, g, qm, dm)
    h = 1e-6
    fdQ = np.zeros_like(Q)
    for idx in np.ndindex(Q.shape):
        Qp, Qm = Q.copy(), Q.copy()
        Qp[idx] += h
        Qm[idx] -= h
        fdQ[idx] = (_loss(oracle_mod, Qp, D, g, qm, dm) - _loss(oracle_mod, Qm, D, g, qm, dm)) / (2 * h)
    fdD = np.zeros_like(D)
    for idx in np.ndindex(D.shape):
        Dp, Dm = D.copy(), D.copy()
        Dp[idx] += h
        Dm[idx] -= h
        fdD[idx] = (_loss(oracle_mod, Q, Dp, g, qm, dm) - _loss(oracle_mod, Q, Dm, g, qm, dm)) / (2 * h)
    np.testing.assert_allclose(dQ, fdQ, rtol=0, atol=1e-7)
    np.testing.assert_allclose(dD, fdD, rtol=0, atol=1e-7)
    assert np.all(dQ[0, 1] == 0) and np.all(dD[1] == 0)


def test_backward_euler_identity(oracle_mod):
    """score is bilinear in (Q, D) at a fixed argmax: sum g*score equals
    <dQ, Q> and <dD, D>."""
    w = synth.random_dense(51, 4, 5, 12, 30, dtype=torch.bfloat16, q_mask_p=0.3, d_mask_p=0.2,
                           dead_docs=1)
    g = synth.upstream_grad(51, 4, 5).double().numpy()
    s, a = oracle_mod.fwd(w.Q, w.D, w.q_mask, w.d_mask)
    dQ, dD, _, _ = oracle_mod.bwd(w.Q, w.D, a, g, w.q_mask, w.d_mask)
    lhs = float((g * s).sum())
    np.testing.assert_allclose(float((dQ * w.Q.double().numpy()).sum()), lhs, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(float((dD * w.D.double().numpy()).sum()), lhs, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("hub", [0.0, 0.7])
def test_csr_matches_stable_argsort(oracle_mod, hub):
    Nq, Nd, Lq, Ld = 3, 4, 10, 16
    arg = synth.draw_argmax(61, Nq, Nd, Lq, Ld, None, hub_frac=hub).numpy()
    Q = np.zeros((Nq, Lq, 2))
    D = np.zeros((Nd, Ld, 2))
    g = np.ones((Nq, Nd))
    _, _, rp, ci = oracle_mod.bwd(Q, D, arg, g)
    src = np.arange(Nq * Nd * Lq)
    j = (src // Lq) % Nd
    dest = j * Ld + arg.reshape(-1)
    cnt = np.bincount(dest, minlength=Nd * Ld)
    assert np.array_equal(rp, np.concatenate([[0], np.cumsum(cnt)]).astype(np.int32))
    assert np.array_equal(ci, np.argsort(dest, kind="stable").astype(np.int32))
    # the invariants that pin the CSR uniquely
    assert rp[0] == 0 and rp[-1] == Nq * Nd * Lq and np.all(np.diff(rp) >= 0)
    assert np.array_equal(np.sort(ci), src)
    rows = np.repeat(np.arange(Nd * Ld), np.diff(rp))
    assert np.array_equal(dest[ci], rows)
    for r in range(Nd * Ld):
        seg = ci[rp[r]:rp[r + 1]]
        assert np.all(np.diff(seg) > 0)


def test_backward_gradients_match_scatter_reference(oracle_mod):
    """dD checked against numpy's unbuffered scatter-add of the per-source
    contributions, dQ against a gather with numpy fancy indexing."""
    w = synth.random_dense(71, 3, 4, 9, 14, q_mask_p=0.3, d_mask_p=0.2, dead_docs=1)
    g = synth.upstream_grad(71, 3, 4).double().numpy()
    _, a = oracle_mod.fwd(w.Q, w.D, w.q_mask, w.d_mask)
    dQ, dD, _, _ = oracle_mod.bwd(w.Q, w.D, a, g, w.q_mask, w.d_mask)
    Q = w.Q.double().numpy()
    D = w.D.double().numpy()
    live = w.d_mask.numpy().any(axis=1)
    wgt = g[:, :, None] * w.q_mask.numpy()[:, None, :] * live[None, :, None]  # [Nq,Nd,Lq]
    Nq, Nd, Lq = a.shape
    jj = np.broadcast_to(np.arange(Nd)[None, :, None], a.shape)
    gathered = D[jj, a]                                   # [Nq,Nd,Lq,d]
    refQ = (wgt[..., None] * gathered).sum(axis=1)
    np.testing.assert_allclose(dQ, refQ, rtol=1e-12, atol=1e-12)
    refD = np.zeros_like(D)
    ii = np.broadcast_to(np.arange(Nq)[:, None, None], a.shape)
    ss = np.broadcast_to(np.arange(Lq)[None, None, :], a.shape)
    np.add.at(refD, (jj.ravel(), a.ravel()), wgt.ravel()[:, None] * Q[ii.ravel(), ss.ravel()])
    np.testing.assert_allclose(dD, refD, rtol=1e-12, atol=1e-12)


# ----------------------------------------------------------------- byte model

def test_io_model_worked_example():
    from maxsim_scoring_amd import workload as wl
    g = _gold("io_model.json")
    p = g["params"]
    naive = wl.io_naive_model(p["nq_tokens"], p["nd_tokens"], p["d"], p["B"], p["elem_bytes"])
    fused = wl.io_fused_model(p["nq_tokens"], p["nd_tokens"], p["d"], p["B"], p["elem_bytes"])
    assert naive == g["io_naive_bytes"]
    assert fused == g["io_fused_bytes"]
    fl = wl.flops_naive_model(p["nq_tokens"], p["nd_tokens"], p["d"], p["B"])
    assert abs(fl / naive - g["ai_naive_flop_per_byte"]) < g["ai_rounding"]
    assert abs(fl / fused - g["ai_fused_flop_per_byte"]) < g["ai_rounding"]


def test_size_examples():
    from maxsim_scoring_amd import workload as wl
    g = _gold("sizes.json")
    for it in g["items"]:
        b = wl.similarity_tensor_bytes(it["n_pairs"], it["lq"], it["ld"], it["elem"])
        assert abs(b / 1e9 - it["approx_gb"]) <= it["rel_tol"] * it["approx_gb"]
    am = g["argmax"]
    b = wl.argmax_bytes(am["nq"], am["nd"], am["lq"])
    assert abs(b / 2**20 - am["approx_mb"]) <= am["rel_tol"] * am["approx_mb"]


# ------------------------------------------- per-token INT8, top-k, pair lists

def test_hand_example_int8_per_token(oracle_mod):
    g = _gold("hand_example.json")
    t = g["int8_per_token"]
    Q = np.array(g["Q"], np.int8)
    D = np.array(g["D"], np.int8)
    dm = np.array(g["d_mask"], np.uint8)
    s, a = oracle_mod.fwd_i8_tok(Q, np.array(t["q_scale"]), D, np.array(t["d_scale"]), None, dm)
    assert np.array_equal(s, np.array(t["score"], np.float64))
    assert np.array_equal(a, np.array(t["argmax"], np.int32))


def test_int8_tok_uniform_scales_is_per_tensor(oracle_mod):
    """One scale for every token reduces to the per-tensor form."""
    w = synth.random_int8(31, 3, 4, 40, 70, d_mask_p=0.2, q_mask_p=0.2)
    qs = np.full(w.Q.shape[:2], w.q_scale)
    ds = np.full(w.D.shape[:2], w.d_scale)
    s, a = oracle_mod.fwd_i8_tok(w.Q, qs, w.D, ds, w.q_mask, w.d_mask)
    _, sf, ar = oracle_mod.fwd_i8(w.Q, w.q_scale, w.D, w.d_scale, w.q_mask, w.d_mask)
    np.testing.assert_allclose(s, sf, rtol=1e-13, atol=1e-13)
    assert np.array_equal(a, ar)


@pytest.mark.parametrize("shape", [(2, 3, 9, 20), (1, 4, 33, 65), (3, 2, 1, 1)])
def test_int8_tok_brute_force(oracle_mod, shape):
    """Power-of-two scales make every product exact, so the brute force over
    dequantised rows must agree exactly, argmax included."""
    Nq, Nd, Lq, Ld = shape
    w = synth.random_int8_tok(40 + Lq, Nq, Nd, Lq, Ld, q_mask_p=0.2, d_mask_p=0.2, dead_docs=1,
                              pow2_scales=True)
    s, a = oracle_mod.fwd_i8_tok(w.Q, w.q_scale, w.D, w.d_scale, w.q_mask, w.d_mask)
    Qd = w.Q.double() * w.q_scale.double()[..., None]
    Dd = w.D.double() * w.d_scale.double()[..., None]
    sb, ab = bf.dense(Qd, Dd, w.q_mask, w.d_mask)
    assert np.array_equal(s, sb)
    assert np.array_equal(a, ab)


def test_hand_example_topk(oracle_mod):
    for c in _gold("hand_example.json")["topk"]["cases"]:
        idx, val = oracle_mod.topk(np.array(c["scores"], np.float64), c["k"])
        assert np.array_equal(idx, np.array(c["idx"], np.int32).reshape(idx.shape))
        assert np.array_equal(val, np.array(c["val"], np.float64).reshape(val.shape))


@pytest.mark.parametrize("ties", [False, True])
@pytest.mark.parametrize("k", [1, 7, 100, 300])
def test_topk_matches_lexsort(oracle_mod, ties, k):
    v = synth.random_scores(50 + k, 5, 300, ties=ties).numpy()
    idx, val = oracle_mod.topk(v, k)
    for i in range(v.shape[0]):
        order = np.lexsort((np.arange(v.shape[1]), -v[i].astype(np.float64)))[:k]
        assert np.array_equal(idx[i], order)
        assert np.array_equal(val[i], v[i, order].astype(np.float64))
        assert np.all(np.diff(val[i]) <= 0)


def test_hand_example_pairs(oracle_mod):
    g = _gold("hand_example.json")
    t = g["pairs"]
    Q = np.array(g["Q"], np.float64)
    D = np.array(g["D"], np.float64)
    dm = np.array(g["d_mask"], np.uint8)
    s, a = oracle_mod.fwd_pairs(Q, D, np.array(t["pair_q"]), np.array(t["pair_d"]), None, dm)
    assert np.array_equal(s, np.array(t["score"], np.float64))
    assert np.array_equal(a, np.array(t["argmax"], np.int32))


def test_pairs_brute_force(oracle_mod):
    w = synth.random_dense(61, 4, 6, 20, 45, dtype=torch.bfloat16, q_mask_p=0.2, d_mask_p=0.2,
                           dead_docs=1)
    pq, pd = synth.random_pairs(61, 4, 6, 30)
    s, a = oracle_mod.fwd_pairs(w.Q, w.D, pq, pd, w.q_mask, w.d_mask)
    for p in range(30):
        i, j = int(pq[p]), int(pd[p])
        sb, ab = bf.dense(w.Q[i:i + 1], w.D[j:j + 1],
                          None if w.q_mask is None else w.q_mask[i:i + 1],
                          None if w.d_mask is None else w.d_mask[j:j + 1])
        np.testing.assert_allclose(s[p], sb[0, 0], rtol=0, atol=1e-12)
        assert np.array_equal(a[p], ab[0, 0])


# ----------------------------------------------------- padding-free backward, pairs

def _pad(w, lens_q, lens_d):
    """The packed inputs of `w` laid out padded with prefix masks."""
    Nq, Nd = len(lens_q), len(lens_d)
    Lq, Ld = max(lens_q), max(max(lens_d), 1)
    Qp = torch.zeros(Nq, Lq, 128, dtype=w.Q.dtype)
    Dp = torch.zeros(Nd, Ld, 128, dtype=w.D.dtype)
    cq, cd = w.cu_q.tolist(), w.cu_d.tolist()
    for i in range(Nq):
        Qp[i, :lens_q[i]] = w.Q[cq[i]:cq[i + 1]]
    for j in range(Nd):
        Dp[j, :lens_d[j]] = w.D[cd[j]:cd[j + 1]]
    return Qp, Dp, synth.prefix_mask(np.array(lens_q), Lq), synth.prefix_mask(np.array(lens_d), Ld)


def test_backward_padding_free_equals_padded(oracle_mod):
    """The packed backward gives the padded backward's gradients on the real
    rows, and its CSR is the padded CSR without the sources of padded query
    rows and of empty docs, rows renumbered to packed doc tokens (Flash-MaxSim
    Sec. 4.2.1-4.2.2 on the cu_seqlens layout of Sec. 4.3.2)."""
    lens_q = [5, 12, 3]
    lens_d = [7, 0, 19, 3, 1]
    w = synth.random_varlen(47, lens_q, lens_d)
    Nq, Nd, Lq = len(lens_q), len(lens_d), w.max_lq
    g = synth.upstream_grad(47, Nq, Nd).double().numpy()
    _, a = oracle_mod.fwd_varlen(w.Q, w.cu_q, w.max_lq, w.D, w.cu_d)
    dQ, dD, rp, ci = oracle_mod.bwd_varlen(w.Q, w.cu_q, w.max_lq, w.D, w.cu_d, a, g)
    Qp, Dp, qm, dm = _pad(w, lens_q, lens_d)
    assert Qp.shape[1] == Lq
    _, ap = oracle_mod.fwd(Qp, Dp, qm, dm)
    dQp, dDp, rpp, cip = oracle_mod.bwd(Qp, Dp, ap, g, qm, dm)
    cq, cd = w.cu_q.tolist(), w.cu_d.tolist()
    for i in range(Nq):
        assert np.array_equal(dQ[cq[i]:cq[i + 1]], dQp[i, :lens_q[i]])
    for j in range(Nd):
        assert np.array_equal(dD[cd[j]:cd[j + 1]], dDp[j, :lens_d[j]])
    # the padded CSR restricted to real sources, in the same order
    Ldp = Dp.shape[1]
    rows = []
    for j in range(Nd):
        for t in range(lens_d[j]):
            seg = cip[rpp[j * Ldp + t]:rpp[j * Ldp + t + 1]]
            s = seg % Lq
            i = seg // Lq // Nd
            rows.append(seg[s < np.array(lens_q)[i]])
    assert np.array_equal(rp, np.concatenate([[0], np.cumsum([len(r) for r in rows])]).astype(np.int32))
    assert np.array_equal(ci, np.concatenate(rows).astype(np.int32))
    assert rp[-1] == sum(lens_q) * sum(1 for l in lens_d if l > 0)


def test_backward_padding_free_euler_identity(oracle_mod):
    lens_q = [4, 9]
    lens_d = [6, 0, 11, 2]
    w = synth.random_varlen(48, lens_q, lens_d)
    g = synth.upstream_grad(48, 2, 4).double().numpy()
    s, a = oracle_mod.fwd_varlen(w.Q, w.cu_q, w.max_lq, w.D, w.cu_d)
    dQ, dD, _, _ = oracle_mod.bwd_varlen(w.Q, w.cu_q, w.max_lq, w.D, w.cu_d, a, g)
    lhs = float((g * s).sum())
    np.testing.assert_allclose(float((dQ * w.Q.double().numpy()).sum()), lhs, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(float((dD * w.D.double().numpy()).sum()), lhs, rtol=1e-12, atol=1e-12)


def test_backward_padding_free_finite_differences(oracle_mod):
    """Central differences of sum(g * score) in fp64 on a tiny packed batch
    whose top-2 gaps are far larger than the step."""
    rng = np.random.default_rng(49)
    cq = np.array([0, 2, 5], np.int32)
    cd = np.array([0, 3, 3, 7], np.int32)
    Q = _exact_grid(rng, (5, 3))
    D = _exact_grid(rng, (7, 3)) * 3.0
    g = rng.standard_normal((2, 3))
    s, a = oracle_mod.fwd_varlen(Q, cq, 3, D, cd)
    dQ, dD, _, _ = oracle_mod.bwd_varlen(Q, cq, 3, D, cd, a, g)
    h = 1e-6

    def f(Qx, Dx):
        sc, ax = oracle_mod.fwd_varlen(Qx, cq, 3, Dx, cd)
        assert np.array_equal(ax, a)  # the step does not move any argmax
        return float((g * sc).sum())

    for (X, grad) in ((Q, dQ), (D, dD)):
        for idx in np.ndindex(X.shape):
            Xp, Xm = X.copy(), X.copy()
            Xp[idx] += h
            Xm[idx] -= h
            num = (f(Xp, D) - f(Xm, D)) / (2 * h) if X is Q else (f(Q, Xp) - f(Q, Xm)) / (2 * h)
            assert abs(num - grad[idx]) < 1e-6


def test_pairs_varlen_equals_cross_product(oracle_mod):
    """Scores of listed packed pairs are the packed cross-product's entries
    (brute force by materialising S), repeats and empty sequences included."""
    lens_q = [5, 0, 9]
    lens_d = [7, 0, 12, 3]
    w = synth.random_varlen(50, lens_q, lens_d)
    pq = np.array([0, 2, 2, 1, 0, 2], np.int32)
    pd = np.array([3, 0, 2, 2, 1, 2], np.int32)
    ps, pa = oracle_mod.fwd_pairs_varlen(w.Q, w.cu_q, w.max_lq, w.D, w.cu_d, pq, pd)
    rs, ra = bf.varlen(w.Q, w.cu_q, w.max_lq, w.D, w.cu_d)
    np.testing.assert_allclose(ps, rs[pq, pd], rtol=0, atol=1e-12)
    assert np.array_equal(pa, ra[pq, pd])


# ------------------------------------------------------------------ embedding widths

@pytest.mark.parametrize("d", [1, 8, 100, 200, 768])
def test_brute_force_widths(oracle_mod, d):
    """Any embedding width (TileMaxSim Sec. 6, Table 9 sweeps d from 64 to
    768): cross product with masks and a dead doc, and packed sequences with
    empty ones, against brute force."""
    w = synth.random_dense(40 + d, 2, 3, 9, 21, dtype=torch.bfloat16, q_mask_p=0.2, d_mask_p=0.2,
                           dead_docs=1, d=d)
    s, a = oracle_mod.fwd(w.Q, w.D, w.q_mask, w.d_mask)
    sb, ab = bf.dense(w.Q, w.D, w.q_mask, w.d_mask)
    np.testing.assert_allclose(s, sb, rtol=0, atol=1e-12)
    assert np.array_equal(a, ab)
    v = synth.random_varlen(41 + d, [3, 0, 17], [5, 0, 1, 40], d=d)
    s, a = oracle_mod.fwd_varlen(v.Q, v.cu_q, v.max_lq, v.D, v.cu_d)
    sb, ab = bf.varlen(v.Q, v.cu_q, v.max_lq, v.D, v.cu_d)
    np.testing.assert_allclose(s, sb, rtol=0, atol=1e-12)
    assert np.array_equal(a, ab)


def test_zero_padded_width_is_identical(oracle_mod):
    """Widening the rows with zero lanes changes no score and no argmax (the
    TileMaxSim README's embedding-dimension dispatch: padded lanes read as
    zero and add nothing)."""
    rng = np.random.default_rng(61)
    Q = rng.standard_normal((2, 11, 100))
    D = rng.standard_normal((3, 30, 100))
    dm = (rng.random((3, 30)) > 0.2).astype(np.uint8)
    s, a = oracle_mod.fwd(Q, D, None, dm)
    for width in (128, 256):
        Qp = np.zeros((2, 11, width))
        Dp = np.zeros((3, 30, width))
        Qp[..., :100] = Q
        Dp[..., :100] = D
        sp, ap = oracle_mod.fwd(Qp, Dp, None, dm)
        assert np.array_equal(s, sp) and np.array_equal(a, ap)


def test_width_chunks_sum_to_full_dot(oracle_mod):
    """Dimension tiling (TileMaxSim Sec. 3): cutting d = 300 into 128-wide
    chunks and summing the chunks' partial similarity tiles before the max
    gives the oracle's scores; taking the max per chunk first does not."""
    rng = np.random.default_rng(62)
    Q = rng.standard_normal((2, 7, 300))
    D = rng.standard_normal((3, 19, 300))
    s, _ = oracle_mod.fwd(Q, D)
    S = sum(np.einsum("isk,jtk->ijst", Q[..., c:c + 128], D[..., c:c + 128]) for c in range(0, 300, 128))
    np.testing.assert_allclose(s, S.max(axis=3).sum(axis=2), rtol=0, atol=1e-10)
    wrong = sum(np.einsum("isk,jtk->ijst", Q[..., c:c + 128], D[..., c:c + 128]).max(axis=3).sum(axis=2)
                for c in range(0, 300, 128))
    assert np.abs(wrong - s).max() > 1e-3


@pytest.mark.parametrize("d", [5, 100, 300])
def test_brute_force_int8_widths(oracle_mod, d):
    """INT8 sums and argmax at widths other than 128 against integer brute
    force; per-token scales against the float brute force of the scaled dots."""
    w = synth.random_int8(32 + d, 2, 4, 9, 13, ternary=True, d_mask_p=0.2, q_mask_p=0.2, d=d)
    si, sf, a = oracle_mod.fwd_i8(w.Q, w.q_scale, w.D, w.d_scale, w.q_mask, w.d_mask)
    sb, ab = bf.dense(w.Q, w.D, w.q_mask, w.d_mask, exact_int=True)
    assert np.array_equal(si, sb)
    assert np.array_equal(a, ab)
    t = synth.random_int8_tok(33 + d, 2, 3, 7, 11, pow2_scales=True, d=d)
    s, a = oracle_mod.fwd_i8_tok(t.Q, t.q_scale, t.D, t.d_scale)
    Qs = t.Q.double() * t.q_scale.double()[..., None]
    Ds = t.D.double() * t.d_scale.double()[..., None]
    sb, ab = bf.dense(Qs, Ds)
    np.testing.assert_allclose(s, sb, rtol=0, atol=1e-12)
    assert np.array_equal(a, ab)


@pytest.mark.parametrize("d", [7, 300])
def test_backward_euler_identity_widths(oracle_mod, d):
    """The bilinear Euler identity of the backward (sum g*score = <dQ, Q> =
    <dD, D> at a fixed argmax) at widths other than 128, padded and packed."""
    w = synth.random_dense(52 + d, 3, 4, 10, 25, dtype=torch.bfloat16, q_mask_p=0.3, d_mask_p=0.2,
                           dead_docs=1, d=d)
    g = synth.upstream_grad(52 + d, 3, 4).double().numpy()
    s, a = oracle_mod.fwd(w.Q, w.D, w.q_mask, w.d_mask)
    dQ, dD, _, _ = oracle_mod.bwd(w.Q, w.D, a, g, w.q_mask, w.d_mask)
    lhs = float((g * s).sum())
    np.testing.assert_allclose(float((dQ * w.Q.double().numpy()).sum()), lhs, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(float((dD * w.D.double().numpy()).sum()), lhs, rtol=1e-12, atol=1e-12)
    v = synth.random_varlen(53 + d, [4, 0, 9], [6, 0, 11, 2], d=d)
    g = synth.upstream_grad(53 + d, 3, 4).double().numpy()
    s, a = oracle_mod.fwd_varlen(v.Q, v.cu_q, v.max_lq, v.D, v.cu_d)
    dQ, dD, _, _ = oracle_mod.bwd_varlen(v.Q, v.cu_q, v.max_lq, v.D, v.cu_d, a, g)
    lhs = float((g * s).sum())
    np.testing.assert_allclose(float((dQ * v.Q.double().numpy()).sum()), lhs, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(float((dD * v.D.double().numpy()).sum()), lhs, rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------------ Chamfer distance

@pytest.mark.parametrize("shape", [(1, 1, 1), (2, 5, 7), (3, 40, 13), (1, 64, 64)])
def test_chamfer_brute_force(oracle_mod, shape):
    B, N, M = shape
    P, Q = synth.point_clouds(71, B, N, M)
    d1, i1, d2, i2, loss = oracle_mod.chamfer_fwd(P, Q)
    r1, j1, r2, j2, rl = bf.chamfer(P, Q)
    np.testing.assert_allclose(d1, r1, rtol=1e-13, atol=0)
    np.testing.assert_allclose(d2, r2, rtol=1e-13, atol=0)
    assert np.array_equal(i1, j1) and np.array_equal(i2, j2)
    np.testing.assert_allclose(loss, rl, rtol=1e-13, atol=0)


def test_chamfer_closed_forms(oracle_mod):
    rng = np.random.default_rng(72)
    P = torch.from_numpy(rng.standard_normal((2, 20, 3)).astype(np.float32))
    # a set against itself: distance 0, each point its own nearest neighbour
    d1, i1, d2, i2, loss = oracle_mod.chamfer_fwd(P, P)
    assert np.all(d1 == 0) and np.all(d2 == 0) and np.all(loss == 0)
    assert np.array_equal(i1, np.tile(np.arange(20), (2, 1))) and np.array_equal(i1, i2)
    # one point each: both terms are the squared distance
    a = torch.tensor([[[1.0, 2.0, 3.0]]])
    b = torch.tensor([[[0.5, -1.0, 4.0]]])
    _, _, _, _, loss = oracle_mod.chamfer_fwd(a, b)
    assert loss[0] == 2 * (0.25 + 9.0 + 1.0)
    # exact ties go to the lowest index: two equidistant targets
    a = torch.tensor([[[0.0, 0.0, 0.0]]])
    b = torch.tensor([[[1.0, 0.0, 0.0], [0.0, -1.0, 0.0], [0.0, 0.0, 1.0]]])
    d1, i1, d2, i2, _ = oracle_mod.chamfer_fwd(a, b)
    assert i1[0, 0] == 0 and d1[0, 0] == 1.0 and np.all(i2 == 0)
    # translating both sets together changes nothing (dyadic shift: exact)
    P, Q = synth.point_clouds(73, 2, 15, 9)
    s = oracle_mod.chamfer_fwd(P, Q)
    t = oracle_mod.chamfer_fwd(P + 0.5, Q + 0.5)
    for x, y in zip(s, t):
        np.testing.assert_allclose(x, y, rtol=1e-6, atol=1e-6)


def test_chamfer_backward_identities(oracle_mod):
    """At fixed argmins sum(g1*dist1) + sum(g2*dist2) is translation invariant
    (gradients sum to zero over all points) and homogeneous of degree 2
    (<dP,P> + <dQ,Q> = 2 * sum(g*dist))."""
    P, Q = synth.point_clouds(74, 3, 30, 17)
    g1, g2 = synth.chamfer_grads(74, 3, 30, 17)
    d1, i1, d2, i2, _ = oracle_mod.chamfer_fwd(P, Q)
    dP, dQ, *_ = oracle_mod.chamfer_bwd(P, Q, i1, i2, g1, g2)
    np.testing.assert_allclose(dP.sum(axis=1) + dQ.sum(axis=1), 0.0, atol=1e-10)
    lhs = float((dP * P.double().numpy()).sum() + (dQ * Q.double().numpy()).sum())
    rhs = 2 * float((g1.double().numpy() * d1).sum() + (g2.double().numpy() * d2).sum())
    np.testing.assert_allclose(lhs, rhs, rtol=1e-12)


def test_chamfer_backward_finite_differences(oracle_mod):
    P, Q = synth.point_clouds(75, 2, 6, 5)
    P, Q = P.double(), Q.double()
    g1, g2 = synth.chamfer_grads(75, 2, 6, 5)
    g1, g2 = g1.double().numpy(), g2.double().numpy()
    d1, i1, d2, i2, _ = oracle_mod.chamfer_fwd(P, Q)
    dP, dQ, *_ = oracle_mod.chamfer_bwd(P, Q, i1, i2, g1, g2)
    h = 1e-6

    def f(Pn, Qn):
        e1, j1, e2, j2, _ = oracle_mod.chamfer_fwd(Pn, Qn)
        assert np.array_equal(j1, i1) and np.array_equal(j2, i2)
        return float((g1 * e1).sum() + (g2 * e2).sum())

    Pn, Qn = P.numpy(), Q.numpy()
    for X, G, is_p in ((Pn, dP, True), (Qn, dQ, False)):
        for idx in np.ndindex(X.shape):
            Xp, Xm = X.copy(), X.copy()
            Xp[idx] += h
            Xm[idx] -= h
            if is_p:
                num = (f(Xp, Qn) - f(Xm, Qn)) / (2 * h)
            else:
                num = (f(Pn, Xp) - f(Pn, Xm)) / (2 * h)
            assert abs(num - G[idx]) < 1e-6


def test_chamfer_csr_matches_stable_argsort(oracle_mod):
    B, N, M = 3, 50, 8
    P, Q = synth.point_clouds(76, B, N, M)
    _, i1, _, i2, _ = oracle_mod.chamfer_fwd(P, Q)
    g1, g2 = synth.chamfer_grads(76, B, N, M)
    _, _, rp1, ci1, rp2, ci2 = oracle_mod.chamfer_bwd(P, Q, i1, i2, g1, g2)
    for idx, ns, nr, rp, ci in ((i1, N, M, rp1, ci1), (i2, M, N, rp2, ci2)):
        k = np.arange(B * ns)
        dest = (k // ns) * nr + idx.reshape(-1)
        cnt = np.bincount(dest, minlength=B * nr)
        assert np.array_equal(rp, np.concatenate([[0], np.cumsum(cnt)]).astype(np.int32))
        assert np.array_equal(ci, np.argsort(dest, kind="stable").astype(np.int32))


def test_chamfer_argmin_comparator():
    """The near-tie rule for Chamfer indices accepts a swap only inside the
    direct form's fp32 rounding bound: two targets whose exact squared
    distances differ by far less than the bound may swap, a clearly farther
    target may not, and an index out of range never passes."""
    from oracle import compare
    s = np.array([[[0.5, -0.25, 1.0]]])                     # one source
    T = np.array([[[0.5, -0.25, 1.0 + 1e-3],                # dist 1e-6
                   [0.5, -0.25 + 1e-3 * (1 + 1e-9), 1.0],   # dist 1e-6 (1 + 2e-9): a near tie
                   [0.5, -0.25 + 1e-3 * (1 + 1e-5), 1.0],   # dist 1e-6 (1 + 2e-5): outside the bound
                   [0.6, -0.25, 1.0]]])                     # dist 1e-2: clearly farther
    ref = np.array([[0]])
    assert compare.chamfer_argmin(np.array([[1]]), ref, s, T)[2] == []
    assert len(compare.chamfer_argmin(np.array([[2]]), ref, s, T)[2]) == 1
    assert len(compare.chamfer_argmin(np.array([[3]]), ref, s, T)[2]) == 1
    assert len(compare.chamfer_argmin(np.array([[4]]), ref, s, T)[2]) == 1
    assert compare.chamfer_argmin(ref, ref, s, T)[:2] == (0, 0)


def _fp32_direct_nn(A, T):
    """Nearest neighbours with every operation in fp32, direct form, in the
    order (dx*dx + dy*dy) + dz*dz: the evaluation the comparator's bounds are
    derived for (any order or fusion is covered)."""
    A32, T32 = A.astype(np.float32), T.astype(np.float32)
    diff = A32[:, :, None, :] - T32[:, None, :, :]
    sq = diff * diff
    v = (sq[..., 0] + sq[..., 1]) + sq[..., 2]
    idx = np.argmin(v, axis=2)
    return np.take_along_axis(v, idx[..., None], 2)[..., 0], idx


def test_chamfer_comparator_accepts_fp32_direct_form(oracle_mod):
    """An fp32 direct-form evaluation passes every Chamfer rule against the
    fp64 oracle, on clouds with near ties (targets duplicated with one-ulp
    moves) and far from the origin; a 1 % distance error, a loss 1 % off and
    a gradient 1 % off fail."""
    from oracle import compare
    rng = np.random.default_rng(785)
    P = (rng.standard_normal((2, 300, 3)) * 0.3 + [40.0, -7.0, 3.0]).astype(np.float32)
    base = (rng.standard_normal((2, 200, 3)) * 0.3 + [40.0, -7.0, 3.0]).astype(np.float32)
    nudged = np.nextafter(base, np.float32(np.inf))
    Q = np.concatenate([base, nudged], axis=1)
    d1, i1, d2, i2, loss = oracle_mod.chamfer_fwd(P, Q)
    P64, Q64 = P.astype(np.float64), Q.astype(np.float64)
    for A, T, rd, ri in ((P64, Q64, d1, i1), (Q64, P64, d2, i2)):
        gd, gi = _fp32_direct_nn(A, T)
        assert compare.chamfer_argmin(gi, ri, A, T)[2] == []
        assert compare.chamfer_dist(gd, rd)[0]
        assert compare.chamfer_dist_at_index(gd, gi, A, T)[0]
        assert not compare.chamfer_dist(gd * 1.01, rd)[0]
        assert not compare.chamfer_dist_at_index(gd * 1.01, gi, A, T)[0]
    # exact coincidence must come out exactly 0
    assert not compare.chamfer_dist(np.array([[1e-30]]), np.array([[0.0]]))[0]
    # loss: the fp32 sum of fp32 distances meets the tolerance, 1 % off does not
    gd1, _ = _fp32_direct_nn(P64, Q64)
    gd2, _ = _fp32_direct_nn(Q64, P64)
    l32 = gd1.sum(1, dtype=np.float32) / np.float32(300) + gd2.sum(1, dtype=np.float32) / np.float32(400)
    tol = compare.chamfer_loss_tol(400)  # a sequential fp32 sum of up to 400 terms
    assert np.all(np.abs(l32 - loss) <= tol * loss)
    assert not np.all(np.abs(1.01 * l32 - loss) <= tol * loss)
    # gradients: fp32 terms summed in fp32 pass; a 1 % error fails
    g1 = rng.standard_normal((2, 300))
    g2 = rng.standard_normal((2, 400))
    dP, dQ, *_ = oracle_mod.chamfer_bwd(P, Q, i1, i2, g1, g2)
    S, n = compare.chamfer_grad_bounds(P64, Q64, i1, i2, g1, g2)
    assert compare.chamfer_grad(dP, dP, S, n)[0]
    P32, Q32, g132, g232 = P, Q, g1.astype(np.float32), g2.astype(np.float32)
    b = np.arange(2)[:, None]
    dP32 = np.float32(2) * g132[..., None] * (P32 - Q32[b, i1])
    for bb in range(2):
        for q in range(400):
            p = i2[bb, q]
            dP32[bb, p] += np.float32(2) * g232[bb, q] * (P32[bb, p] - Q32[bb, q])
    g1r = g132.astype(np.float64)
    g2r = g232.astype(np.float64)
    dPr, _, *_ = oracle_mod.chamfer_bwd(P, Q, i1, i2, g1r, g2r)
    S, n = compare.chamfer_grad_bounds(P64, Q64, i1, i2, g1r, g2r)
    assert compare.chamfer_grad(dP32, dPr, S, n)[0]
    assert not compare.chamfer_grad(dP32 * 1.01, dPr, S, n)[0]


@pytest.mark.slow
def test_int8_long_query_expectation_is_the_oracles(oracle_mod):
    """The stored expectation of the long-query INT8 workload
    (tests/golden/make_int8_long_query.py) still describes the generated
    inputs, and its first argmax block, scores and fp32 scores of those docs
    are the oracle's."""
    import hashlib
    import json
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                        "int8_long_query_expected.json")
    with open(path) as f:
        exp = json.load(f)
    w = synth.int8_long_query()
    assert hashlib.sha256(w.D.numpy().tobytes()).hexdigest() == exp["inputs_sha256"]["D"]
    assert hashlib.sha256(w.Q.numpy().tobytes()).hexdigest() == exp["inputs_sha256"]["Q"]
    blk = exp["argmax_block"]
    si, sf, a = oracle_mod.fwd_i8(w.Q, w.q_scale, w.D[:blk], w.d_scale, want_argmax=True)
    assert list(si[0]) == exp["scores_i32"][:blk]
    rf = np.frombuffer(bytes.fromhex(exp["scores_f32_hex"]), dtype="<f4")
    assert np.array_equal(sf[0].astype(np.float32), rf[:blk])
    d = hashlib.sha256(np.ascontiguousarray(a, dtype="<i4")[0].tobytes()).hexdigest()[:16]
    assert d == exp["argmax_block_digests"][0]
