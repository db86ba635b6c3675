"""The Chamfer search's candidate window, checked on the CPU.

The forward kernel (csrc/chamfer.hip) finds nearest-neighbour candidates from
a bf16 matrix-core evaluation of the bracket |t'|^2 - 2 <s', t'> with
coordinates taken relative to a centring point c and split into bf16 hi/lo
parts, and keeps every target tile whose min lies inside
thr(b) = b + tau (2 |s'|^2 + b) of the running min b. Its correctness rests
on one inequality, that the computed |s'|^2 + bracket is within
2^-14 (|s'|^2 + D) of the exact squared distance D, and on its consequence,
that the exact nearest point's bracket is always inside thr(b). Both are
checked here by emulating that arithmetic in numpy: fp32 centring
differences and squared norm, bf16 round-to-nearest-even parts, the 11
products (exact in fp64) summed in fp32 in several orders ("Flash-MaxSim"
Sec. 4.2.4 defines the distance; how the search evaluates it is the kernel's
own). No GPU and no oracle code is involved.
"""

import numpy as np
import pytest

TAU = np.float32(float.fromhex("0x1.03p-13"))  # the kernel's window constant
KTAUK = np.float32(1.0) + TAU


def bf16(x):
    """fp32 -> bf16 (round to nearest even), returned as fp32 values."""
    u = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return r.astype(np.uint32).view(np.float32)


def split(v):
    """v = hi + lo + e with hi = bf16(v), lo = bf16(v - hi) (v - hi exact in fp32)."""
    v = np.asarray(v, np.float32)
    hi = bf16(v)
    lo = bf16((v - hi).astype(np.float32))
    return hi, lo


def f32_fma(a, b, c):
    return (np.float64(a) * np.float64(b) + np.float64(c)).astype(np.float32)


def sq_norm_f32(x, y, z):
    """fma(z, z, fma(y, y, x * x)) in fp32, as the kernel computes |t'|^2 and |s'|^2."""
    return f32_fma(z, z, f32_fma(y, y, (x * x).astype(np.float32)))


def brackets(S, T, c, order):
    """The search's bracket for every (source, target) pair: [ns, nt] fp32,
    its 11 exact products summed in fp32 in the given order of the terms."""
    a = (S - c).astype(np.float32)  # centred sources, fp32
    b = (T - c).astype(np.float32)  # centred targets
    n = sq_norm_f32(b[:, 0], b[:, 1], b[:, 2])
    nh, nl = split(n)
    th, tl = split(b)
    mh, ml = split((np.float32(-2.0) * a).astype(np.float32))
    f = np.float64
    terms = []
    for k in range(3):
        terms.append(f(th[None, :, k]) * f(mh[:, None, k]))  # hi x hi
    for k in range(3):
        terms.append(f(tl[None, :, k]) * f(mh[:, None, k]))  # lo x hi
    for k in range(3):
        terms.append(f(th[None, :, k]) * f(ml[:, None, k]))  # hi x lo
    terms.append(np.broadcast_to(f(nh)[None, :], terms[0].shape))
    terms.append(np.broadcast_to(f(nl)[None, :], terms[0].shape))
    acc = np.zeros(terms[0].shape, np.float32)
    for i in order:  # each product is exact; each addition rounds to fp32
        acc = (acc.astype(np.float64) + terms[i]).astype(np.float32)
    return acc, a


def clouds(rng, ns, nt, scale, offset, dup):
    S = (rng.standard_normal((ns, 3)) * scale + offset).astype(np.float32)
    T = (rng.standard_normal((nt, 3)) * scale + offset).astype(np.float32)
    if dup:  # near-duplicates of some sources among the targets
        k = ns // 4
        T[:k] = (S[:k] + rng.standard_normal((k, 3)) * scale * 1e-6).astype(np.float32)
    return S, T


CASES = [(1.0, 0.0, False), (1e-3, 0.0, True), (1e3, 0.0, False), (1.0, 1e4, True),
         (0.01, 1000.0, False), (100.0, -50.0, True)]


@pytest.mark.parametrize("scale,offset,dup", CASES)
def test_bracket_error_bound(scale, offset, dup):
    """|(|s'|^2 + bracket) - D| <= 2^-14 (|s'|^2 + D) for every pair."""
    rng = np.random.default_rng(int(scale * 7919 + abs(offset) + dup))
    S, T = clouds(rng, 300, 400, scale, offset, dup)
    c = T[:64].mean(axis=0, dtype=np.float32)
    D = ((S[:, None, :].astype(np.float64) - T[None, :, :].astype(np.float64)) ** 2).sum(axis=2)
    for order in (list(range(11)), list(range(10, -1, -1)), list(rng.permutation(11))):
        br, a = brackets(S, T, c, order)
        na = (a.astype(np.float64) ** 2).sum(axis=1)[:, None]
        err = np.abs(na + br.astype(np.float64) - D)
        bound = 2.0 ** -14 * (na + D)
        assert np.all(err <= bound), float((err / bound).max())


@pytest.mark.parametrize("scale,offset,dup", CASES)
def test_nearest_point_inside_window(scale, offset, dup):
    """The exact nearest target's bracket is at most thr(b), b the smallest
    computed bracket, with thr computed in fp32 as the kernel does."""
    rng = np.random.default_rng(int(scale * 104729 + abs(offset) + 3 * dup))
    S, T = clouds(rng, 300, 2000, scale, offset, dup)
    c = T[:64].mean(axis=0, dtype=np.float32)
    D = ((S[:, None, :].astype(np.float64) - T[None, :, :].astype(np.float64)) ** 2).sum(axis=2)
    star = D.argmin(axis=1)
    for order in (list(range(11)), list(rng.permutation(11))):
        br, a = brackets(S, T, c, order)
        b = br.min(axis=1)
        na32 = sq_norm_f32(a[:, 0], a[:, 1], a[:, 2])
        tau0 = (np.float32(2.0) * TAU * na32).astype(np.float32)
        thr = f32_fma(b, KTAUK, tau0)
        got = br[np.arange(len(S)), star]
        assert np.all(got <= thr)


def test_window_excludes_far_points():
    """The window is not vacuous: on an N(0,1) cloud most targets lie outside
    it, so the search keeps few candidates per source."""
    rng = np.random.default_rng(5)
    S, T = clouds(rng, 200, 2000, 1.0, 0.0, False)
    c = T[:64].mean(axis=0, dtype=np.float32)
    br, a = brackets(S, T, c, list(range(11)))
    b = br.min(axis=1)
    na32 = sq_norm_f32(a[:, 0], a[:, 1], a[:, 2])
    thr = f32_fma(b, KTAUK, (np.float32(2.0) * TAU * na32).astype(np.float32))
    inside = (br <= thr[:, None]).sum(axis=1)
    assert inside.mean() < 3.0
