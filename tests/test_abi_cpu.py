"""The C-ABI library on a machine without a GPU: it loads, exports every entry
point include/maxsim.h declares, and rejects bad arguments on the host before
touching a device (every call here returns from host-side validation)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "maxsim.h")

OK, ERR_NULL, ERR_SHAPE, ERR_UNSUPPORTED, ERR_OVERFLOW, ERR_LAUNCH = range(6)
FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first
MIS8 = ctypes.c_void_p(0x1008)  # 8- but not 16-byte aligned
MIS2 = ctypes.c_void_p(0x1002)  # 2- but not 4-byte aligned


def _declared():
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:maxsim_status_t|const char\*|int)\s+(maxsim_\w+)\s*\(",
                                 txt, re.M)))


@pytest.fixture(scope="module")
def L():
    from maxsim_scoring_amd import binding
    if not os.path.exists(binding.LIB_PATH):
        from maxsim_scoring_amd import build
        build.build()
    return binding.lib()


def test_exports_every_declared_symbol(L):
    names = _declared()
    assert set(names) == {"maxsim_fwd", "maxsim_fwd_varlen", "maxsim_fwd_i8", "maxsim_bwd",
                          "maxsim_fwd_i8_tok", "maxsim_fwd_pairs", "maxsim_topk",
                          "maxsim_fwd_pairs_varlen", "maxsim_bwd_varlen",
                          "maxsim_chamfer_fwd", "maxsim_chamfer_bwd",
                          "maxsim_status_string", "maxsim_abi_version"}
    for n in names:
        assert hasattr(L, n), n


def test_version_and_status_strings(L):
    txt = open(HEADER).read()
    ver = int(re.search(r"#define MAXSIM_ABI_VERSION (\d+)", txt).group(1))
    assert L.maxsim_abi_version() == ver
    for s in range(6):
        assert L.maxsim_status_string(s)
    assert L.maxsim_status_string(99) == b"unknown status"


def fwd(L, dtype=0, Q=FAKE, D=FAKE, Nq=2, Nd=3, Lq=4, Ld=5, d=128, qm=None, dm=None, sc=FAKE,
        am=None):
    return L.maxsim_fwd(dtype, Q, D, Nq, Nd, Lq, Ld, d, qm, dm, sc, am, None)


def test_fwd_validation(L):
    assert fwd(L, Nq=-1) == ERR_SHAPE
    assert fwd(L, Ld=-5) == ERR_SHAPE
    assert fwd(L, d=0) == ERR_UNSUPPORTED         # widths 1 .. 1024
    assert fwd(L, d=1025) == ERR_UNSUPPORTED
    assert fwd(L, d=64, Nd=1 << 16, Ld=1 << 15) == ERR_OVERFLOW  # other widths: Nd*Ld < 2^31
    assert fwd(L, dtype=7) == ERR_UNSUPPORTED
    assert fwd(L, sc=None) == ERR_NULL
    assert fwd(L, Q=None) == ERR_NULL
    assert fwd(L, D=None) == ERR_NULL
    assert fwd(L, Nq=0) == OK            # nothing to do, nothing enqueued
    assert fwd(L, Nd=0, sc=None) == OK
    assert fwd(L, Nq=1 << 16, Nd=1 << 15, Lq=2, am=FAKE) == ERR_OVERFLOW
    assert fwd(L, Nq=1 << 20, Nd=1 << 12) == ERR_OVERFLOW
    # row tensors need 16-byte alignment, outputs their element alignment
    assert fwd(L, Q=MIS8) == ERR_UNSUPPORTED
    assert fwd(L, D=MIS8) == ERR_UNSUPPORTED
    assert fwd(L, sc=MIS2) == ERR_UNSUPPORTED
    assert fwd(L, am=MIS2) == ERR_UNSUPPORTED


def test_varlen_validation(L):
    f = L.maxsim_fwd_varlen
    assert f(0, FAKE, FAKE, 1, -1, FAKE, FAKE, 2, 128, FAKE, None, None) == ERR_SHAPE
    assert f(0, FAKE, FAKE, 1, 32, FAKE, FAKE, 2, 0, FAKE, None, None) == ERR_UNSUPPORTED
    assert f(0, FAKE, FAKE, 1, 32, FAKE, FAKE, 2, 2048, FAKE, None, None) == ERR_UNSUPPORTED
    assert f(1, FAKE, None, 1, 32, FAKE, FAKE, 2, 128, FAKE, None, None) == ERR_NULL
    assert f(1, FAKE, FAKE, 1, 32, FAKE, None, 2, 128, FAKE, None, None) == ERR_NULL
    assert f(1, FAKE, FAKE, 1, 32, FAKE, FAKE, 2, 128, None, None, None) == ERR_NULL
    assert f(1, FAKE, FAKE, 0, 32, FAKE, FAKE, 2, 128, None, None, None) == OK
    assert f(0, FAKE, FAKE, 1 << 10, 1 << 12, FAKE, FAKE, 1 << 10, 128, FAKE, FAKE, None) == ERR_OVERFLOW
    assert f(0, MIS8, FAKE, 1, 32, FAKE, FAKE, 2, 128, FAKE, None, None) == ERR_UNSUPPORTED
    assert f(0, FAKE, MIS2, 1, 32, FAKE, FAKE, 2, 128, FAKE, None, None) == ERR_UNSUPPORTED
    assert f(0, FAKE, FAKE, 1, 32, MIS8, FAKE, 2, 128, FAKE, None, None) == ERR_UNSUPPORTED


def test_i8_validation(L):
    f = L.maxsim_fwd_i8
    args = dict(Q=FAKE, qs=1.0, D=FAKE, ds=1.0, Nq=1, Nd=2, Lq=8, Ld=8, d=128, qm=None, dm=None,
                si=FAKE, sf=FAKE, am=None)

    def call(**kw):
        a = dict(args, **kw)
        return f(a["Q"], a["qs"], a["D"], a["ds"], a["Nq"], a["Nd"], a["Lq"], a["Ld"], a["d"],
                 a["qm"], a["dm"], a["si"], a["sf"], a["am"], None)

    assert call(si=None, sf=None) == ERR_NULL
    assert call(d=0) == ERR_UNSUPPORTED
    assert call(d=1025) == ERR_UNSUPPORTED
    assert call(Lq=-1) == ERR_SHAPE
    # Lq*d*127^2 must stay below 2^31: 1041 rows * 128 * 16129 overflow, 1040 do not
    assert call(Lq=1041) == ERR_OVERFLOW
    assert call(Lq=1040, Q=None) == ERR_NULL
    assert call(Nq=0) == OK
    assert call(D=MIS8) == ERR_UNSUPPORTED
    assert call(si=MIS2) == ERR_UNSUPPORTED


def test_bwd_validation(L):
    f = L.maxsim_bwd

    def call(dtype=0, Nq=2, Nd=3, Lq=4, Ld=5, d=128, Q=FAKE, D=FAKE, am=FAKE, g=FAKE, dQ=FAKE,
             dD=FAKE, rp=FAKE, ci=FAKE):
        return f(dtype, Q, D, Nq, Nd, Lq, Ld, d, None, None, am, g, dQ, dD, rp, ci, None)

    assert call(Nq=-2) == ERR_SHAPE
    assert call(d=0) == ERR_UNSUPPORTED
    assert call(d=1025) == ERR_UNSUPPORTED
    assert call(Ld=0) == ERR_SHAPE            # sources with no destination
    assert call(am=None) == ERR_NULL
    assert call(rp=None) == ERR_NULL
    assert call(ci=None) == ERR_NULL
    assert call(dQ=None) == ERR_NULL
    assert call(dD=None) == ERR_NULL
    assert call(Nq=1 << 11, Nd=1 << 10, Lq=1 << 10) == ERR_OVERFLOW
    assert call(Nd=1 << 16, Ld=1 << 15) == ERR_OVERFLOW
    assert call(Q=MIS8) == ERR_UNSUPPORTED
    assert call(dQ=MIS8) == ERR_UNSUPPORTED
    assert call(dD=MIS8) == ERR_UNSUPPORTED
    assert call(ci=MIS2) == ERR_UNSUPPORTED
    assert call(Nq=0, Nd=0, Lq=0, Ld=0, Q=None, D=None, am=None, g=None, dQ=None, dD=None,
                rp=None, ci=None) == OK


def test_i8_tok_validation(L):
    f = L.maxsim_fwd_i8_tok

    def call(Q=FAKE, qs=FAKE, D=FAKE, ds=FAKE, Nq=2, Nd=3, Lq=4, Ld=5, d=128, sc=FAKE, am=None):
        return f(Q, qs, D, ds, Nq, Nd, Lq, Ld, d, None, None, sc, am, None)

    assert call(Lq=-1) == ERR_SHAPE
    assert call(d=0) == ERR_UNSUPPORTED
    assert call(d=2000) == ERR_UNSUPPORTED
    assert call(sc=None) == ERR_NULL
    assert call(qs=None) == ERR_NULL
    assert call(ds=None) == ERR_NULL
    assert call(D=MIS8) == ERR_UNSUPPORTED
    assert call(qs=MIS2) == ERR_UNSUPPORTED
    assert call(Nd=0, sc=None) == OK
    assert call(Nq=1 << 16, Nd=1 << 15, Lq=2, am=FAKE) == ERR_OVERFLOW


def test_pairs_validation(L):
    f = L.maxsim_fwd_pairs

    def call(dtype=0, Q=FAKE, D=FAKE, Nq=2, Nd=3, Lq=4, Ld=5, d=128, pq=FAKE, pd=FAKE, P=7,
             sc=FAKE, am=None):
        return f(dtype, Q, D, Nq, Nd, Lq, Ld, d, None, None, pq, pd, P, sc, am, None)

    assert call(P=-1) == ERR_SHAPE
    assert call(Nd=0) == ERR_SHAPE          # a pair needs a doc
    assert call(P=0, Nd=0, pq=None) == OK   # nothing to score
    assert call(dtype=5) == ERR_UNSUPPORTED
    assert call(d=1100) == ERR_UNSUPPORTED
    assert call(d=96, Nd=1 << 16, Ld=1 << 15) == ERR_OVERFLOW
    assert call(pq=None) == ERR_NULL
    assert call(sc=None) == ERR_NULL
    assert call(pd=MIS2) == ERR_UNSUPPORTED
    assert call(Q=MIS8) == ERR_UNSUPPORTED
    assert call(P=1 << 22, Lq=1 << 10, am=FAKE) == ERR_OVERFLOW


def test_pairs_varlen_validation(L):
    def f(dtype=0, Q=FAKE, cq=FAKE, Nq=2, mlq=8, D=FAKE, cd=FAKE, Nd=3, d=128, pq=FAKE, pd=FAKE,
          P=4, sc=FAKE, am=None):
        return L.maxsim_fwd_pairs_varlen(dtype, Q, cq, Nq, mlq, D, cd, Nd, d, pq, pd, P, sc, am,
                                         None)
    assert f(P=-1) == ERR_SHAPE
    assert f(mlq=-1) == ERR_SHAPE
    assert f(Nq=0) == ERR_SHAPE                # a pair needs a query
    assert f(d=0) == ERR_UNSUPPORTED
    assert f(d=1025) == ERR_UNSUPPORTED
    assert f(dtype=3) == ERR_UNSUPPORTED
    assert f(pq=None) == ERR_NULL
    assert f(cd=None) == ERR_NULL
    assert f(sc=None) == ERR_NULL
    assert f(P=0, sc=None) == OK                # nothing to do, nothing enqueued
    assert f(pd=MIS2) == ERR_UNSUPPORTED
    assert f(Q=MIS8) == ERR_UNSUPPORTED
    assert f(P=1 << 28, mlq=16, am=FAKE) == ERR_OVERFLOW


def test_bwd_varlen_validation(L):
    def f(dtype=1, Q=FAKE, cq=FAKE, Nq=2, Tq=40, mlq=32, D=FAKE, cd=FAKE, Nd=3, Td=500, d=128,
          am=FAKE, g=FAKE, dQ=FAKE, dD=FAKE, rp=FAKE, ci=FAKE):
        return L.maxsim_bwd_varlen(dtype, Q, cq, Nq, Tq, mlq, D, cd, Nd, Td, d, am, g, dQ, dD, rp,
                                   ci, None)
    assert f(Tq=-1) == ERR_SHAPE
    assert f(Nd=-2) == ERR_SHAPE
    assert f(Nq=0) == ERR_SHAPE                 # packed query rows without a query
    assert f(Nd=0) == ERR_SHAPE                 # packed doc rows without a doc
    assert f(mlq=0) == ERR_SHAPE                # query rows need a max_lq slot
    assert f(d=0) == ERR_UNSUPPORTED
    assert f(d=4096) == ERR_UNSUPPORTED
    assert f(dtype=2) == ERR_UNSUPPORTED
    assert f(cq=None) == ERR_NULL
    assert f(rp=None) == ERR_NULL
    assert f(ci=None) == ERR_NULL
    assert f(dQ=None) == ERR_NULL
    assert f(am=None) == ERR_NULL
    assert f(Nq=1 << 16, Nd=1 << 10, mlq=32) == ERR_OVERFLOW   # flat source index
    assert f(Tq=1 << 22, Nd=1 << 10, mlq=1 << 12) == ERR_OVERFLOW  # CSR entries
    assert f(Td=1 << 31) == ERR_OVERFLOW
    assert f(dD=MIS8) == ERR_UNSUPPORTED
    assert f(rp=MIS2) == ERR_UNSUPPORTED


def test_chamfer_validation(L):
    def fw(P=FAKE, Q=FAKE, B=2, N=100, M=50, d1=FAKE, i1=FAKE, d2=FAKE, i2=FAKE, loss=None):
        return L.maxsim_chamfer_fwd(P, Q, B, N, M, d1, i1, d2, i2, loss, None)
    assert fw(N=-1) == ERR_SHAPE
    assert fw(M=0) == ERR_SHAPE                # a min over an empty set
    assert fw(B=0, P=None) == OK               # nothing to do, nothing enqueued
    assert fw(P=None) == ERR_NULL
    assert fw(i2=None) == ERR_NULL
    assert fw(d1=MIS2) == ERR_UNSUPPORTED
    assert fw(B=1 << 20, N=1 << 12) == ERR_OVERFLOW

    def bw(B=2, N=100, M=50, **kw):
        args = dict(P=FAKE, Q=FAKE, i1=FAKE, i2=FAKE, g1=FAKE, g2=FAKE, dP=FAKE, dQ=FAKE,
                    rp1=FAKE, ci1=FAKE, rp2=FAKE, ci2=FAKE)
        args.update(kw)
        return L.maxsim_chamfer_bwd(args["P"], args["Q"], B, N, M, args["i1"], args["i2"],
                                    args["g1"], args["g2"], args["dP"], args["dQ"], args["rp1"],
                                    args["ci1"], args["rp2"], args["ci2"], None)
    assert bw(B=-1) == ERR_SHAPE
    assert bw(N=0) == ERR_SHAPE
    assert bw(B=0) == OK
    assert bw(rp2=None) == ERR_NULL
    assert bw(g1=None) == ERR_NULL
    assert bw(ci1=MIS2) == ERR_UNSUPPORTED
    assert bw(B=1 << 16, M=1 << 15) == ERR_OVERFLOW


def test_topk_validation(L):
    f = L.maxsim_topk

    def call(sc=FAKE, Nq=2, Nd=10, K=3, ids=None, idx=FAKE, val=FAKE, rows=None):
        return f(sc, Nq, Nd, K, ids, idx, val, rows, None)

    assert call(K=11) == ERR_SHAPE           # k > Nd
    assert call(K=-1) == ERR_SHAPE
    assert call(Nd=5000, K=1025) == ERR_UNSUPPORTED
    assert call(K=0, idx=None, val=None) == OK
    assert call(Nq=0) == OK
    assert call(idx=None) == ERR_NULL
    assert call(val=MIS2) == ERR_UNSUPPORTED
    assert call(rows=MIS2) == ERR_UNSUPPORTED
    assert call(Nq=1 << 31, Nd=1 << 31) == ERR_OVERFLOW


def test_binding_refuses_cpu_tensors():
    import torch
    import maxsim_scoring_amd as ms
    Q = torch.zeros((1, 4, 128), dtype=torch.float16)
    with pytest.raises(ValueError, match="GPU tensor"):
        ms.maxsim_fwd(Q, Q)


class _FakeGpuTensor:
    """Stands in for a contiguous GPU tensor on a machine without a GPU: the
    binding's layout checks read only these attributes, and every case below
    fails a check before the library is called."""

    def __init__(self, shape, dtype):
        self.shape = tuple(shape)
        self.dtype = dtype
        self.is_cuda = True
        self.device = "cuda:0"

    def is_contiguous(self):
        return True

    def dim(self):
        return len(self.shape)

    def numel(self):
        n = 1
        for s in self.shape:
            n *= s
        return n


def test_binding_rejects_outputs_and_masks_of_the_wrong_shape():
    """Every output a caller passes in must have exactly the documented shape,
    and every mask must be [N, L]: an undersized buffer would let the kernels
    write past it."""
    import torch
    from maxsim_scoring_amd import binding as b

    def T(*shape, dtype=torch.float32):
        return _FakeGpuTensor(shape, dtype)

    bf, i32, u8, i8 = torch.bfloat16, torch.int32, torch.uint8, torch.int8
    Q, D = T(2, 4, 128, dtype=bf), T(3, 5, 128, dtype=bf)
    am, g = T(2, 3, 4, dtype=i32), T(2, 3)
    cases = [
        lambda: b.maxsim_fwd(Q, D, scores=T(2, 2)),
        lambda: b.maxsim_fwd(Q, D, scores=T(2, 3), argmax=T(2, 3, 3, dtype=i32)),
        lambda: b.maxsim_fwd(Q, D, q_mask=T(2, 5, dtype=u8), scores=T(2, 3)),
        lambda: b.maxsim_bwd(Q, D, am, g, dQ=T(2, 4, 127), dD=T(3, 5, 128), csr_row_ptr=T(16, dtype=i32),
                             csr_col_idx=T(24, dtype=i32)),
        lambda: b.maxsim_bwd(Q, D, am, g, dQ=T(2, 4, 128), dD=T(3, 4, 128), csr_row_ptr=T(16, dtype=i32),
                             csr_col_idx=T(24, dtype=i32)),
        lambda: b.maxsim_bwd(Q, D, am, g, dQ=T(2, 4, 128), dD=T(3, 5, 128), csr_row_ptr=T(15, dtype=i32),
                             csr_col_idx=T(24, dtype=i32)),
        lambda: b.maxsim_bwd(Q, D, am, g, dQ=T(2, 4, 128), dD=T(3, 5, 128), csr_row_ptr=T(16, dtype=i32),
                             csr_col_idx=T(23, dtype=i32)),
        lambda: b.maxsim_bwd(Q, D, am, g, q_mask=T(2, 3, dtype=u8), dQ=T(2, 4, 128), dD=T(3, 5, 128),
                             csr_row_ptr=T(16, dtype=i32), csr_col_idx=T(24, dtype=i32)),
        lambda: b.maxsim_bwd(Q, D, am, g, d_mask=T(3, 6, dtype=u8), dQ=T(2, 4, 128), dD=T(3, 5, 128),
                             csr_row_ptr=T(16, dtype=i32), csr_col_idx=T(24, dtype=i32)),
        lambda: b.maxsim_fwd_i8(T(2, 4, 128, dtype=i8), 1.0, T(3, 5, 128, dtype=i8), 1.0,
                                q_mask=T(4, 2, dtype=u8), scores_i32=T(2, 3, dtype=i32), scores=T(2, 3)),
        lambda: b.maxsim_fwd_i8(T(2, 4, 128, dtype=i8), 1.0, T(3, 5, 128, dtype=i8), 1.0,
                                scores_i32=T(1, 3, dtype=i32), scores=T(2, 3)),
        lambda: b.maxsim_fwd_i8_tok(T(2, 4, 128, dtype=i8), T(2, 4), T(3, 5, 128, dtype=i8), T(3, 5),
                                    d_mask=T(3, 4, dtype=u8), scores=T(2, 3)),
        lambda: b.maxsim_fwd_varlen(T(8, 128, dtype=bf), T(3, dtype=i32), 4, T(9, 128, dtype=bf),
                                    T(4, dtype=i32), scores=T(2, 2)),
        lambda: b.maxsim_fwd_varlen(T(8, 128, dtype=bf), T(3, dtype=i32), 4, T(9, 128, dtype=bf),
                                    T(4, dtype=i32), scores=T(2, 3), argmax=T(2, 3, 3, dtype=i32)),
        lambda: b.maxsim_bwd_varlen(T(8, 128, dtype=bf), T(3, dtype=i32), 4, T(9, 128, dtype=bf),
                                    T(4, dtype=i32), T(2, 3, 4, dtype=i32), T(2, 3), dQ=T(8, 128),
                                    dD=T(8, 128), csr_row_ptr=T(10, dtype=i32), csr_col_idx=T(24, dtype=i32)),
        lambda: b.maxsim_fwd_pairs(Q, D, T(6, dtype=i32), T(6, dtype=i32), scores=T(5)),
        lambda: b.maxsim_fwd_pairs_varlen(T(8, 128, dtype=bf), T(3, dtype=i32), 4, T(9, 128, dtype=bf),
                                          T(4, dtype=i32), T(6, dtype=i32), T(6, dtype=i32), scores=T(6),
                                          argmax=T(6, 3, dtype=i32)),
        lambda: b.maxsim_topk(T(2, 50), 10, idx=T(2, 9, dtype=i32), val=T(2, 10)),
        lambda: b.maxsim_topk(T(2, 50), 10, idx=T(2, 10, dtype=i32), val=T(2, 10), rows=T(10, dtype=i32)),
    ]
    for k, call in enumerate(cases):
        with pytest.raises(ValueError):
            call()
