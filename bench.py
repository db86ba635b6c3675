"""Benchmark of the MaxSim HIP path on one MI355X.

A step is one pass of the hot path over one batch of synthetic input: for the
headline workload, one padding-free reranking forward of a 32-token query
against 100,000 packed docs of 50-300 tokens (fp16, d = 128), i.e. one call of
maxsim_fwd_varlen. The value is docs scored per second with the inputs already
resident in HBM. The other workloads of the pages (tiny cross-product,
ColPali cross-product, INT8 long query, backward at ColPali shapes) are timed
in the same run and reported under "per_config".

Each workload runs in a child process of its own (a kernel fault poisons only
that process's context); the parent never touches the GPU. Every timing
starts after the W warm-up launches and, beyond them, at least --min-warmup-s
seconds of launches, so the part's clocks have settled before the timed
region.

The oracle (the plain CPU implementation) is timed on a bounded sample of the
headline workload on this host's cores and reported as "cpu_baseline"; the
tiny, ColPali, INT8 and backward workloads report their own oracle samples.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--only NAME]
       python bench.py --child NAME ...   (one workload in this process)
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
INT8_PEAK_TOPS = 5000.0
FP32_PEAK_TFLOPS = 157.3
# values a three-operand VALU min folds per second: 1,024 SIMDs x 16 lanes per
# clock x 2 values x 2.4 GHz (the Chamfer search's bound)
VALU_MIN_PEAK_T = 1024 * 16 * 2 * 2.4e9 / 1e12
METRIC = ("docs/sec + achieved HBM GB/s or MFMA TFLOP/s as % of MI355X peak, per config")
HEADLINE = "rerank"
COUNTERS_FILE = os.path.join(ROOT, "profiles", "hbm_counters.json")


def _log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# the files each measured kernel is built from (its source, the shared
# headers and the build script that holds the compiler flags)
KERNEL_SOURCES = {
    "fwd_varlen_kernel": ["csrc/fwd_varlen.hip", "csrc/common.hpp", "csrc/kernels.hpp", "build.py"],
    "fwd_dense_kernel": ["csrc/fwd_dense.hip", "csrc/common.hpp", "csrc/kernels.hpp", "build.py"],
}


def kernel_source_digest(kernel: str) -> str:
    """Hash of one kernel's sources; counter readings are valid only for it."""
    h = hashlib.sha256()
    pkg = os.path.join(ROOT, "maxsim_scoring_amd")
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(pkg, name), "rb") as f:
            h.update(name.encode())
            h.update(f.read())
    return h.hexdigest()[:16]


MIN_WARMUP_S = 1.0  # set from --min-warmup-s
WARMUP_LOG = []      # (launches, seconds) of each warm-up in this process


def warm_up(torch, fn, warmup: int) -> None:
    """W launches, then more until at least MIN_WARMUP_S seconds of launches
    have run (the clocks ramp up under load), all outside any timed region."""
    t0 = time.perf_counter()
    n = 0
    for _ in range(warmup):
        fn()
        n += 1
    torch.cuda.synchronize()
    while time.perf_counter() - t0 < MIN_WARMUP_S:
        for _ in range(16):
            fn()
        n += 16
        torch.cuda.synchronize()
    WARMUP_LOG.append((n, round(time.perf_counter() - t0, 3)))


FLUSH_BYTES = 512 << 20
FLUSH_PREWRITES = 32
_FLUSH = []  # the process's cache-flush buffer, once written


def flush_buffer(torch):
    """The process's 512 MiB cache-flush buffer (twice the last-level cache).
    It is allocated once and written FLUSH_PREWRITES times before any timed
    region: while a freshly allocated buffer of this size had been written
    only a few times, the kernels launched between its writes ran slower (the
    ColPali kernel took 427-478 us per launch in the kernel trace, against
    398 us for the same launches once the buffer had been written about 20
    times), which would charge a one-time cost of the process to the kernel."""
    if not _FLUSH:
        buf = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
        for _ in range(FLUSH_PREWRITES):
            buf.fill_(1.0)
        torch.cuda.synchronize()
        _FLUSH.append(buf)
    return _FLUSH[0]


def time_steps(torch, fn, steps: int, warmup: int, flush_bytes: int = 0):
    """Times `fn` (one launch per call) with HIP events on torch's current
    stream, which is the stream the library launches on. Without a flush the
    K launches run back to back between one pair of events; with a flush, a
    buffer larger than the 256 MiB last-level cache is rewritten before every
    launch, outside the events, and each launch is timed by its own pair."""
    warm_up(torch, fn, warmup)
    if not flush_bytes:
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        total = e0.elapsed_time(e1)
        return total, [total / steps]
    assert flush_bytes == FLUSH_BYTES
    scratch = flush_buffer(torch)
    times = []
    for _ in range(steps):
        scratch.fill_(1.0)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    return sum(times), times


def per_launch(torch, fn, steps: int):
    """Each of `steps` back-to-back launches timed by its own event pair (for
    the spread; the value comes from the back-to-back total)."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for e0, e1 in evs:
        e0.record()
        fn()
        e1.record()
    torch.cuda.synchronize()
    return [e0.elapsed_time(e1) for e0, e1 in evs]


def spread(times) -> dict:
    """Minimum and 90th percentile of per-launch times (ms), beside the median."""
    ts = sorted(times)
    return {"ms_min": round(ts[0], 5), "ms_p90": round(ts[min(len(ts) - 1, (9 * len(ts)) // 10)], 5)}


def roofline(bound: str, achieved: float, peak: float, unit: str, traffic=None) -> dict:
    return {"bound": bound, "achieved": round(achieved, 3), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4), "traffic": traffic}


def load_traffic(kernel: str, workload: str):
    """HBM bytes per dispatch from the committed counter runs, scaled by the
    copy-kernel calibration, or None when absent or taken on other sources."""
    try:
        with open(COUNTERS_FILE) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return None
    e = c.get("kernels", {}).get(kernel, {}).get(workload)
    if not e or e.get("source_digest") != kernel_source_digest(kernel):
        return None
    return e.get("hbm_bytes_per_dispatch")


# ------------------------------------------------------------------ workloads

def bench_rerank(torch, ms, synth, wl, steps, warmup):
    w = synth.rerank_varlen_fp16()
    T = int(w.cu_d[-1])
    Q, cu_q, D, cu_d = (t.cuda() for t in (w.Q, w.cu_q, w.D, w.cu_d))
    scores = torch.empty((1, 100_000), dtype=torch.float32, device="cuda")

    def step():
        ms.maxsim_fwd_varlen(Q, cu_q, w.max_lq, D, cu_d, scores=scores)

    total_ms, _ = time_steps(torch, step, steps, warmup)
    ms_per = total_ms / steps
    launches = per_launch(torch, step, steps)
    nbytes = wl.varlen_fwd_bytes(32, 1, T, 100_000, 128, 2)
    gbs = nbytes / (ms_per * 1e-3) / 1e9
    out = {
        "workload": w.name, "ms": ms_per, "docs_per_s": 100_000 / (ms_per * 1e-3),
        "per_launch_ms": {"median": round(statistics.median(launches), 5), **spread(launches)},
        "algorithmic_bytes": nbytes, "tokens": T,
        "roofline": roofline("hbm", gbs, HBM_PEAK_GBS, "GB/s",
                             load_traffic("fwd_varlen_kernel", w.name)),
        "kernel": "fwd_varlen_kernel",
    }
    return out, w


KEEP = {}  # inputs a workload leaves for its oracle sample (child process only)


def bench_tiny(torch, ms, synth, wl, steps, warmup):
    w = synth.tiny_fp16()
    KEEP["tiny"] = w
    Q, D = w.Q.cuda(), w.D.cuda()
    scores = torch.empty((4, 32), dtype=torch.float32, device="cuda")
    argmax = torch.empty((4, 32, 32), dtype=torch.int32, device="cuda")

    def step():
        ms.maxsim_fwd(Q, D, scores=scores, argmax=argmax)

    total, times = time_steps(torch, step, steps, warmup, flush_bytes=FLUSH_BYTES)
    t = statistics.median(times)
    nbytes = wl.dense_fwd_bytes(4, 32, 32, 180, 128, 2, False, False, True)
    return {"workload": w.name, "ms": t, **spread(times), "pairs_per_s": 128 / (t * 1e-3),
            "roofline": roofline("hbm", nbytes / (t * 1e-3) / 1e9, HBM_PEAK_GBS, "GB/s"),
            "note": "launch-bound: 1.5 MB of operands", "kernel": "fwd_dense_kernel"}


def bench_colpali(torch, ms, synth, wl, steps, warmup):
    w = synth.colpali_bf16()
    KEEP["colpali"] = w
    Q, D, qm, dm = (t.cuda() for t in (w.Q, w.D, w.q_mask, w.d_mask))
    scores = torch.empty((128, 128), dtype=torch.float32, device="cuda")
    argmax = torch.empty((128, 128, 128), dtype=torch.int32, device="cuda")

    def step():
        ms.maxsim_fwd(Q, D, qm, dm, scores=scores, argmax=argmax)

    total, times = time_steps(torch, step, steps, warmup, flush_bytes=FLUSH_BYTES)
    t = statistics.median(times)
    valid = int(w.d_mask.sum())
    flops = wl.dense_fwd_flops(128, 128, 128, valid)
    return {"workload": w.name, "ms": t, **spread(times), "pairs_per_s": 128 * 128 / (t * 1e-3),
            "algorithmic_flops": flops, "dense_flops": 2 * 128 * 128 * 128 * 128 * 1024,
            "roofline": roofline("mfma", flops / (t * 1e-3) / 1e12, BF16_PEAK_TFLOPS, "TFLOP/s",
                                 load_traffic("fwd_dense_kernel", w.name)),
            "kernel": "fwd_dense_kernel"}


def bench_int8(torch, ms, synth, wl, steps, warmup):
    w = synth.int8_long_query()
    KEEP["int8"] = w
    Q, D = w.Q.cuda(), w.D.cuda()
    si = torch.empty((1, 10_000), dtype=torch.int32, device="cuda")
    sf = torch.empty((1, 10_000), dtype=torch.float32, device="cuda")

    def step():
        ms.maxsim_fwd_i8(Q, w.q_scale, D, w.d_scale, scores_i32=si, scores=sf)

    total, _ = time_steps(torch, step, steps, warmup)
    t = total / steps
    ops = 2 * 128 * 1024 * 1024 * 10_000
    nbytes = wl.dense_fwd_bytes(1, 10_000, 1024, 1024, 128, 1, False, False, False, True)
    return {"workload": w.name, "ms": t, "docs_per_s": 10_000 / (t * 1e-3),
            "algorithmic_ops": ops, "algorithmic_bytes": nbytes,
            "roofline": roofline("mfma", ops / (t * 1e-3) / 1e12, INT8_PEAK_TOPS, "TOP/s",
                                 load_traffic("fwd_dense_kernel", w.name)),
            "kernel": "fwd_dense_kernel"}


DIM_SWEEP = (64, 96, 128, 256, 384, 768)


def bench_dim_sweep(torch, ms, synth, wl, steps, warmup):
    """The embedding-width sweep: one 32-token fp16 query against 10,000 docs
    of 128 tokens at each width, no masks, no argmax; every launch follows a
    cache flush because the smaller widths' D fits in the last-level cache."""
    rows = {}
    for d in DIM_SWEEP:
        w = synth.dim_scaling_fp16(d)
        Q, D = w.Q.cuda(), w.D.cuda()
        scores = torch.empty((1, 10_000), dtype=torch.float32, device="cuda")

        def step():
            ms.maxsim_fwd(Q, D, scores=scores)

        total, times = time_steps(torch, step, min(steps, 10), min(warmup, 5), flush_bytes=FLUSH_BYTES)
        t = statistics.median(times)
        nbytes = wl.dense_fwd_bytes(1, 10_000, 32, 128, d, 2, False, False, False)
        rows[f"d{d}"] = {"workload": w.name, "ms": t, **spread(times), "docs_per_s": 10_000 / (t * 1e-3),
                         "algorithmic_bytes": nbytes,
                         "roofline": roofline("hbm", nbytes / (t * 1e-3) / 1e9, HBM_PEAK_GBS, "GB/s")}
        del Q, D, w
        torch.cuda.empty_cache()
    best = max(rows.values(), key=lambda r: r["roofline"]["frac"])
    return {"workload": "dim_sweep_fp16_1x10000_lq32_ld128", "ms": rows["d768"]["ms"],
            "widths": rows, "roofline": rows["d768"]["roofline"], "best_width": best["workload"],
            "kernel": "fwd_dim_kernel"}


BATCHES = (1_000, 10_000, 100_000, 200_000)


def bench_batch_sweep(torch, ms, synth, wl, steps, warmup):
    """Batch scaling ([TMS] Sec. 6, Table 8): one 32-token fp16 query against
    B docs of 128 tokens (d = 128, no masks), B = 1,000 ... 200,000, the first
    B docs of one 200,000-doc corpus. Launches whose D fits the 256 MiB
    last-level cache (B <= 10,000) are timed one by one after a cache flush,
    the others back to back. Not in the default run."""
    w = synth.dim_scaling_fp16(128, seed=8, Nd=max(BATCHES))
    Q, Dall = w.Q.cuda(), w.D.cuda()
    del w
    rows = {}
    for B in BATCHES:
        D = Dall[:B]
        scores = torch.empty((1, B), dtype=torch.float32, device="cuda")

        def step():
            ms.maxsim_fwd(Q, D, scores=scores)

        flush = FLUSH_BYTES if B * 128 * 256 < (256 << 20) else 0
        total, times = time_steps(torch, step, steps, warmup, flush_bytes=flush)
        t = statistics.median(times) if flush else total / steps
        nbytes = wl.dense_fwd_bytes(1, B, 32, 128, 128, 2, False, False, False)
        rows[f"B{B}"] = {"docs": B, "ms": t, **(spread(times) if flush else {}),
                         "docs_per_s": B / (t * 1e-3), "algorithmic_bytes": nbytes,
                         "roofline": roofline("hbm", nbytes / (t * 1e-3) / 1e9, HBM_PEAK_GBS, "GB/s")}
    return {"workload": "batch_sweep_fp16_1xB_lq32_ld128", "ms": rows["B200000"]["ms"], "batches": rows,
            "roofline": rows["B200000"]["roofline"], "kernel": "fwd_dim_kernel (one short query)"}


def bench_backward(torch, ms, synth, wl, steps, warmup):
    fw = synth.colpali_bf16()
    Q, D, qm, dm = (t.cuda() for t in (fw.Q, fw.D, fw.q_mask, fw.d_mask))
    _, argmax = ms.maxsim_fwd(Q, D, qm, dm, want_argmax=True)  # the saved forward argmax
    g = synth.upstream_grad(5, 128, 128).cuda()
    KEEP["backward"] = (fw, argmax.cpu(), g.cpu())
    dQ = torch.empty((128, 128, 128), dtype=torch.float32, device="cuda")
    dD = torch.empty((128, 1024, 128), dtype=torch.float32, device="cuda")
    rp = torch.empty((128 * 1024 + 1,), dtype=torch.int32, device="cuda")
    ci = torch.empty((128 * 128 * 128,), dtype=torch.int32, device="cuda")

    def step():
        ms.maxsim_bwd(Q, D, argmax, g, qm, dm, dQ=dQ, dD=dD, csr_row_ptr=rp, csr_col_idx=ci)

    total, times = time_steps(torch, step, steps, warmup, flush_bytes=FLUSH_BYTES)
    t = statistics.median(times)
    nbytes = wl.bwd_compulsory_bytes(128, 128, 128, 1024, 128, 2, True, True)
    # the row gathers the two passes make beyond the compulsory bytes (served
    # from L2 and the last-level cache): one 256-byte D row per doc and
    # unmasked query row for dQ, and one Q row per CSR entry of nonzero weight
    # g[i,j] q_mask[i,s] live(j) for dD (every g here is nonzero and every doc
    # live, so both count the unmasked query rows times the docs)
    gathered = 2 * int(fw.q_mask.sum()) * 128 * 128 * 2
    return {"workload": "backward_colpali_bf16_128x128_lq128_ld1024", "ms": t, **spread(times),
            "pairs_per_s": 128 * 128 / (t * 1e-3), "compulsory_bytes": nbytes,
            "gathered_bytes": gathered,
            "gathered_GBps": round(gathered / (t * 1e-3) / 1e9, 1),
            "roofline": roofline("hbm", nbytes / (t * 1e-3) / 1e9, HBM_PEAK_GBS, "GB/s"),
            "kernels": ["csr_dq_kernel", "dd_kernel"]}


def bench_backward_varlen(torch, ms, synth, wl, steps, warmup):
    """Padding-free backward at the ColPali training shapes without padding:
    128 queries of 16-128 tokens and 128 docs of 768-1024 patches (the valid
    prefixes of the cross-product workload), bf16, argmax from the GPU forward."""
    import numpy as np
    rng = np.random.default_rng(3)
    ql, dl = rng.integers(16, 129, 128), rng.integers(768, 1025, 128)
    w = synth.random_varlen(31, ql, dl, dtype=torch.bfloat16, max_lq=128)
    Q, cu_q, D, cu_d = (t.cuda() for t in (w.Q, w.cu_q, w.D, w.cu_d))
    _, argmax = ms.maxsim_fwd_varlen(Q, cu_q, 128, D, cu_d, want_argmax=True)
    g = synth.upstream_grad(5, 128, 128).cuda()
    Tq, Td = int(cu_q[-1]), int(cu_d[-1])
    dQ = torch.empty((Tq, 128), dtype=torch.float32, device="cuda")
    dD = torch.empty((Td, 128), dtype=torch.float32, device="cuda")
    rp = torch.empty((Td + 1,), dtype=torch.int32, device="cuda")
    ci = torch.empty((Tq * 128,), dtype=torch.int32, device="cuda")

    def step():
        ms.maxsim_bwd_varlen(Q, cu_q, 128, D, cu_d, argmax, g, dQ=dQ, dD=dD, csr_row_ptr=rp,
                             csr_col_idx=ci)

    total, times = time_steps(torch, step, steps, warmup, flush_bytes=FLUSH_BYTES)
    t = statistics.median(times)
    nbytes = wl.bwd_varlen_compulsory_bytes(128, 128, 128, Tq, Td, 128, 128, 2)
    gathered = 2 * Tq * 128 * 128 * 2  # a D row per (query row, doc) for dQ, a Q row per CSR entry for dD
    return {"workload": f"backward_varlen_bf16_128x128_lq16-128_ld768-1024_packed_{Tq}x{Td}", "ms": t, **spread(times),
            "pairs_per_s": 128 * 128 / (t * 1e-3), "compulsory_bytes": nbytes,
            "gathered_bytes": gathered,
            "gathered_GBps": round(gathered / (t * 1e-3) / 1e9, 1),
            "roofline": roofline("hbm", nbytes / (t * 1e-3) / 1e9, HBM_PEAK_GBS, "GB/s"),
            "kernels": ["vbwd_prep_kernel", "vbwd_csr_dq_kernel", "vbwd_dd_kernel"]}


def bench_pairs_varlen(torch, ms, synth, wl, steps, warmup):
    """Reranker scheduling on the packed corpus: 32 queries of 32 tokens, each
    with 1,000 candidate docs drawn from the 100,000-passage corpus (50-300
    tokens), scored as one list of 32,000 (query, doc) pairs."""
    import numpy as np
    lens = synth.rerank_lengths(2, 100_000)
    w = synth.random_varlen(12, [32] * 32, lens)
    pq, pd = synth.random_pairs(12, 32, 100_000, 32_000)
    Q, cu_q, D, cu_d, pq_d, pd_d = (t.cuda() for t in (w.Q, w.cu_q, w.D, w.cu_d, pq, pd))
    scores = torch.empty((32_000,), dtype=torch.float32, device="cuda")

    def step():
        ms.maxsim_fwd_pairs_varlen(Q, cu_q, 32, D, cu_d, pq_d, pd_d, scores=scores)

    total, _ = time_steps(torch, step, steps, warmup)
    t = total / steps
    nbytes = wl.pairs_varlen_fwd_bytes(32 * 32, lens[pd.numpy()], 128, 2)
    return {"workload": "pairs_varlen_fp16_32q_lq32_32000pairs_ld50-300", "ms": t,
            "pairs_per_s": 32_000 / (t * 1e-3), "algorithmic_bytes": nbytes,
            "roofline": roofline("hbm", nbytes / (t * 1e-3) / 1e9, HBM_PEAK_GBS, "GB/s"),
            "kernel": "fwd_varlen_kernel (pair list)"}


def bench_chamfer(torch, ms, synth, wl, steps, warmup):
    """Chamfer distance between two 100,000-point clouds (N(0,1) coordinates,
    fp32): the forward (both nearest-neighbour directions and the loss) and the
    backward through the saved indices. The forward's distance tiles are bf16
    matrix-core contractions of the coordinates' hi/lo parts, and each
    (point, point) pair and direction then costs one min on the VALU, which
    bounds the search: the roofline counts those values against the VALU's
    rate for them (a three-operand min folds 2 values per lane and
    instruction: 1,024 SIMDs x 16 lanes per clock x 2 x 2.4 GHz). The fp32
    contraction of the definition (8 operations per pair and direction) is
    reported beside it against the fp32 peak."""
    P, Q = synth.point_clouds(782, 1, 100_000, 100_000)
    P, Q = P.cuda(), Q.cuda()
    g1, g2 = (t.cuda() for t in synth.chamfer_grads(782, 1, 100_000, 100_000))
    n = 100_000
    f32, i32 = torch.float32, torch.int32
    fo = dict(dist1=torch.empty((1, n), dtype=f32, device="cuda"), idx1=torch.empty((1, n), dtype=i32, device="cuda"),
              dist2=torch.empty((1, n), dtype=f32, device="cuda"), idx2=torch.empty((1, n), dtype=i32, device="cuda"),
              loss=torch.empty((1,), dtype=f32, device="cuda"))
    bo = dict(dP=torch.empty((1, n, 3), dtype=f32, device="cuda"), dQ=torch.empty((1, n, 3), dtype=f32, device="cuda"),
              csr_row_ptr1=torch.empty((n + 1,), dtype=i32, device="cuda"),
              csr_col_idx1=torch.empty((n,), dtype=i32, device="cuda"),
              csr_row_ptr2=torch.empty((n + 1,), dtype=i32, device="cuda"),
              csr_col_idx2=torch.empty((n,), dtype=i32, device="cuda"))

    def fwd():
        ms.maxsim_chamfer_fwd(P, Q, **fo)

    total, _ = time_steps(torch, fwd, steps, warmup)
    t_f = total / steps
    i1, i2 = fo["idx1"], fo["idx2"]

    def bwd():
        ms.maxsim_chamfer_bwd(P, Q, i1, i2, g1, g2, **bo)

    total, _ = time_steps(torch, bwd, steps, warmup)
    t_b = total / steps
    flops = 8 * 2 * 100_000 * 100_000
    values = 2 * 100_000 * 100_000  # one min per (point, point) pair and direction
    return {"workload": "chamfer_fp32_1x100000x100000", "ms": t_f, "backward_ms": t_b,
            "pairs_per_s": values / (t_f * 1e-3), "algorithmic_flops": flops,
            "fp32_equivalent": roofline("mfma", flops / (t_f * 1e-3) / 1e12, FP32_PEAK_TFLOPS, "TFLOP/s"),
            "roofline": roofline("alu", values / (t_f * 1e-3) / 1e12, VALU_MIN_PEAK_T, "T values/s"),
            "kernels": ["chamfer_nn_kernel", "chamfer_fix_kernel", "chamfer_loss_kernel", "cham_part_kernel",
                        "cham_part_scan_kernel", "cham_bucket_kernel", "cham_grad_kernel"]}


def bench_two_stage(torch, ms, synth, wl, steps, warmup):
    """The INT8 -> FP16 top-K scan on the long-query corpus (1 query of 1024
    tokens, 10,000 docs of 1024 tokens): per-token INT8 scores of every doc,
    100 candidates, their exact fp16 scores, the final top 10. Reports the
    per-token INT8 scan alone (MFMA roofline) and the whole scan."""
    w = synth.two_stage_long_query()
    Q8, qs, D8, ds = (t.cuda() for t in (w.Q, w.q_scale, w.D, w.d_scale))
    Qf, Df = w.Qf.cuda(), w.Df.cuda()
    del w
    s8 = torch.empty((1, 10_000), dtype=torch.float32, device="cuda")

    def scan():
        ms.maxsim_fwd_i8_tok(Q8, qs, D8, ds, scores=s8)

    total, _ = time_steps(torch, scan, steps, warmup)
    t_scan = total / steps
    ops = 2 * 128 * 1024 * 1024 * 10_000

    def pipeline():
        ms.two_stage_topk(Q8, qs, D8, ds, Qf, Df, 10, 100)

    total, _ = time_steps(torch, pipeline, steps, warmup)
    t_all = total / steps
    return {"workload": "int8tok_1x10000_lq1024_ld1024_top100_rescore_fp16_top10",
            "ms": t_all, "docs_per_s": 10_000 / (t_all * 1e-3),
            "int8_scan_ms": t_scan,
            "roofline": roofline("mfma", ops / (t_scan * 1e-3) / 1e12, INT8_PEAK_TOPS, "TOP/s"),
            "note": "roofline is the per-token INT8 scan kernel; ms is the whole four-call scan",
            "kernel": "fwd_dense_kernel (per-token int8), topk_kernel, fwd_dense_kernel (pairs)"}


def bench_topk(torch, ms, synth, wl, steps, warmup):
    """Top-100 of one row of 100,000 scores (the reranking workload's output)."""
    v = synth.random_scores(7, 1, 100_000).cuda()
    idx = torch.empty((1, 100), dtype=torch.int32, device="cuda")
    val = torch.empty((1, 100), dtype=torch.float32, device="cuda")

    def step():
        ms.maxsim_topk(v, 100, idx=idx, val=val)

    total, times = time_steps(torch, step, steps, warmup, flush_bytes=FLUSH_BYTES)
    t = statistics.median(times)
    nbytes = 100_000 * 4
    return {"workload": "topk_1x100000_k100", "ms": t, **spread(times),
            "roofline": roofline("hbm", nbytes / (t * 1e-3) / 1e9, HBM_PEAK_GBS, "GB/s"),
            "note": "one workgroup per row: threshold from a leading sample, one filtering pass, select and sort in LDS", "kernel": "topk_kernel"}


def bench_copy(torch, ms, synth, wl, steps, warmup):
    """A plain 1 GiB device-to-device copy: the reference kernel that the HBM
    byte counters are calibrated against (it must read and write 1 GiB)."""
    n = 1 << 30
    x = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)

    def step():
        y.copy_(x)

    total, _ = time_steps(torch, step, steps, warmup)
    t = total / steps
    return {"workload": "copy_1GiB", "ms": t, "bytes_read": n, "bytes_written": n,
            "roofline": roofline("hbm", 2 * n / (t * 1e-3) / 1e9, HBM_PEAK_GBS, "GB/s")}


def bench_yardstick(torch, ms, synth, wl, steps, warmup):
    """Not a path of this library: what plain, vendor-tuned kernels reach on
    this part, timed the same way, as a yardstick for the fractions of peak
    reported for the fused kernels. The vendor's GEMMs (torch.mm and
    torch._int_mm, served by the ROCm BLAS libraries) on square 8192^3 bf16
    and int8 operands, against the nominal dense MFMA peaks; and torch's
    integer sum over buffers of the headline's size (4.48 GB) and of the
    width sweep's corpus sizes, streaming reads, against the HBM peak; and
    torch's row gather at the backward's gather volume."""
    n = 8192
    gen = torch.Generator(device="cuda").manual_seed(0)
    a = torch.randn(n, n, device="cuda", dtype=torch.bfloat16, generator=gen)
    b = torch.randn(n, n, device="cuda", dtype=torch.bfloat16, generator=gen)
    ai = torch.randint(-127, 128, (n, n), device="cuda", dtype=torch.int8, generator=gen)
    bi = torch.randint(-127, 128, (n, n), device="cuda", dtype=torch.int8, generator=gen)
    ops = 2 * n ** 3
    k = min(steps, 20)
    out = {}
    for name, fn, peak, unit in (("gemm_bf16_8192", lambda: torch.mm(a, b), BF16_PEAK_TFLOPS, "TFLOP/s"),
                                 ("gemm_int8_8192", lambda: torch._int_mm(ai, bi), INT8_PEAK_TOPS, "TOP/s")):
        total, _ = time_steps(torch, fn, k, min(warmup, 5))
        t = total / k
        out[name] = {"ms": t, "roofline": roofline("mfma", ops / (t * 1e-3) / 1e12, peak, unit)}
    del a, b, ai, bi
    nbytes = 4_483_489_623 // 64 * 64
    x = torch.ones(nbytes // 8, dtype=torch.int64, device="cuda")
    total, _ = time_steps(torch, lambda: x.sum(), k, min(warmup, 5))
    t = total / k
    out["read_sum_4.48GB"] = {"ms": t, "bytes": nbytes,
                             "roofline": roofline("hbm", nbytes / (t * 1e-3) / 1e9, HBM_PEAK_GBS, "GB/s")}
    del x
    # the same read at the width sweep's corpus sizes (10,000 docs x 128
    # tokens x d x 2 bytes), each launch after a cache flush like the sweep's
    for d in DIM_SWEEP:
        nb = 10_000 * 128 * d * 2
        x = torch.ones(nb // 8, dtype=torch.int64, device="cuda")
        _, times = time_steps(torch, lambda: x.sum(), min(steps, 10), min(warmup, 5), flush_bytes=FLUSH_BYTES)
        t = statistics.median(times)
        out[f"read_sum_d{d}"] = {"ms": t, "bytes": nb,
                                 "roofline": roofline("hbm", nb / (t * 1e-3) / 1e9, HBM_PEAK_GBS, "GB/s")}
        del x
    # random row gathers of the backward's volume: 2,097,152 rows of 256 bytes
    # (bf16, d = 128) picked from a 32 MiB matrix, torch's index_select (it
    # also writes the 537 MB it gathers)
    src = torch.ones((128 * 1024, 128), dtype=torch.bfloat16, device="cuda")
    idx = torch.randint(0, 128 * 1024, (128 * 128 * 128,), device="cuda", generator=gen)
    _, times = time_steps(torch, lambda: torch.index_select(src, 0, idx), min(steps, 10), min(warmup, 5),
                          flush_bytes=FLUSH_BYTES)
    t = statistics.median(times)
    nb = idx.numel() * 256
    out["gather_rows_537MB"] = {"ms": t, "bytes_gathered": nb, "gathered_GBps": round(nb / (t * 1e-3) / 1e9, 1)}
    return {"workload": "vendor_yardstick", **out}


def host_info() -> dict:
    """The host the oracle runs on: CPU model, logical CPUs, oracle threads."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    from oracle import oracle
    return {"cpu_model": model, "nproc": os.cpu_count(), "oracle_threads": oracle.default_threads()}


def _timed(fn, reps=1):
    t0 = time.perf_counter()
    for _ in range(reps):
        fn()
    return time.perf_counter() - t0


def cpu_baseline(w, target_s: float = 12.0) -> dict:
    """The oracle, as it stands, on the headline workload: a 300-doc run sizes
    the sample for about `target_s` seconds of work, taken as the first n docs
    or, when all 100,000 docs take less, as repeated passes over all of them."""
    import numpy as np
    from oracle import oracle
    cu = w.cu_d.numpy().astype(np.int64)
    threads = oracle.default_threads()
    n_all = len(cu) - 1

    def run(n, reps=1):
        D = w.D[:cu[n]]
        t0 = time.perf_counter()
        for _ in range(reps):
            oracle.fwd_varlen(w.Q, w.cu_q, w.max_lq, D, w.cu_d[:n + 1], want_argmax=False,
                              threads=threads)
        return time.perf_counter() - t0

    t_small = run(300)
    n = int(min(n_all, max(300, 300 * target_s / max(t_small, 1e-3))))
    reps = 1
    if n == n_all:
        t_one = run(n)
        reps = max(1, int(round(target_s / max(t_one, 1e-3))))
    t = run(n, reps)
    what = f"first {n} of the {n_all:,} docs" if n < n_all else f"all {n_all:,} docs x {reps} passes"
    return {"value": round(n * reps / t, 3), "unit": "docs/s", "cores": threads, "kind": "oracle",
            "sample": f"{what} ({int(cu[n])} tokens per pass), 32-token query, "
                      f"fp64 on {threads} threads, {t:.2f} s"}


def cpu_baseline_tiny(w, target_s: float = 2.0) -> dict:
    from oracle import oracle
    th = oracle.default_threads()
    run = lambda: oracle.fwd(w.Q, w.D, threads=th)  # noqa: E731
    reps = max(1, int(target_s / max(_timed(run), 1e-4)))
    t = _timed(run, reps)
    return {"value": round(128 * reps / t, 3), "unit": "pairs/s", "cores": th, "kind": "oracle",
            "sample": f"the whole 4 x 32 workload with argmax x {reps} passes, fp64 on {th} threads, {t:.2f} s"}


def cpu_baseline_colpali(w, target_s: float = 6.0) -> dict:
    from oracle import oracle
    th = oracle.default_threads()

    def run(nq):
        return _timed(lambda: oracle.fwd(w.Q[:nq], w.D, w.q_mask[:nq], w.d_mask, threads=th))

    t2 = run(2)
    nq = int(min(128, max(2, 2 * target_s / max(t2, 1e-3))))
    t = run(nq)
    return {"value": round(nq * 128 / t, 3), "unit": "pairs/s", "cores": th, "kind": "oracle",
            "sample": f"the first {nq} of the 128 queries against all 128 docs, masks and argmax, "
                      f"fp64 on {th} threads, {t:.2f} s"}


def cpu_baseline_int8(w, target_s: float = 6.0) -> dict:
    from oracle import oracle
    th = oracle.default_threads()

    def run(nd):
        return _timed(lambda: oracle.fwd_i8(w.Q, w.q_scale, w.D[:nd], w.d_scale, want_argmax=False,
                                            threads=th))

    t20 = run(20)
    nd = int(min(10_000, max(20, 20 * target_s / max(t20, 1e-3))))
    t = run(nd)
    return {"value": round(nd / t, 3), "unit": "docs/s", "cores": th, "kind": "oracle",
            "sample": f"the first {nd} of the 10,000 docs, 1024-token query, int64 on {th} threads, {t:.2f} s"}


def cpu_baseline_backward(keep, target_s: float = 6.0) -> dict:
    from oracle import oracle
    th = oracle.default_threads()
    fw, argmax, g = keep
    run = lambda: oracle.bwd(fw.Q, fw.D, argmax, g, fw.q_mask, fw.d_mask, threads=th)  # noqa: E731
    reps = max(1, int(round(target_s / max(_timed(run), 1e-3))))
    t = _timed(run, reps)
    return {"value": round(128 * 128 * reps / t, 3), "unit": "pairs/s", "cores": th, "kind": "oracle",
            "sample": f"the whole backward (CSR, dQ, dD) through the GPU forward's argmax x {reps} passes, "
                      f"fp64 on {th} threads, {t:.2f} s"}


CPU_SAMPLES = {"tiny": cpu_baseline_tiny, "colpali": cpu_baseline_colpali,
               "int8": cpu_baseline_int8, "backward": cpu_baseline_backward}

FNS = {"rerank": bench_rerank, "tiny": bench_tiny, "colpali": bench_colpali,
       "int8": bench_int8, "backward": bench_backward, "backward_varlen": bench_backward_varlen,
       "pairs_varlen": bench_pairs_varlen, "two_stage": bench_two_stage,
       "topk": bench_topk, "chamfer": bench_chamfer, "dim_sweep": bench_dim_sweep,
       "copy": bench_copy, "yardstick": bench_yardstick, "batch_sweep": bench_batch_sweep}
DEFAULT = [HEADLINE, "tiny", "colpali", "int8", "backward", "backward_varlen", "pairs_varlen",
           "two_stage", "topk", "chamfer", "dim_sweep"]
MARK = "@@bench-result "


# ------------------------------------------------------------------ main

def run_child(args) -> int:
    """One workload in this process: its timing, then (with --cpu) its oracle
    sample; prints one marked JSON line."""
    import torch
    import maxsim_scoring_amd as ms
    from maxsim_scoring_amd import synth, workload as wl
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    ms.binding.lib()  # fails loudly without the built library
    flush_buffer(torch)  # written before the workload's warm-up and timing
    name = args.child
    _log(f"workload {name}: generating inputs and timing {args.steps} steps")
    r = FNS[name](torch, ms, synth, wl, args.steps, args.warmup)
    w = None
    if name == HEADLINE:
        r, w = r
    r["warmup_runs"] = [{"launches": n, "s": s} for n, s in WARMUP_LOG]
    cpu = None
    if args.cpu:
        torch.cuda.synchronize()
        if name == HEADLINE:
            _log("oracle CPU baseline on a bounded sample")
            cpu = cpu_baseline(w)
        elif name in CPU_SAMPLES:
            _log(f"workload {name}: oracle sample")
            cpu = CPU_SAMPLES[name](KEEP[name])
    print(MARK + json.dumps({"name": name, "result": r, "cpu": cpu}), flush=True)
    return 0


def under_profiler() -> bool:
    """True when a GPU profiler's library is preloaded: it may initialise the
    GPU in this process before main(), and a process whose GPU is initialised
    must not start other programs, so the workloads then run in this process."""
    return "rocprof" in os.environ.get("LD_PRELOAD", "") or any(k.startswith("ROCPROF") for k in os.environ)


def run_in_process(name: str, args, cpu: bool) -> dict:
    """The child's work in this process (used under a profiler)."""
    import io
    import contextlib
    args.child, args.cpu = name, cpu
    buf = io.StringIO()
    with contextlib.redirect_stdout(buf):
        rc = run_child(args)
    WARMUP_LOG.clear()
    KEEP.clear()
    import torch
    torch.cuda.empty_cache()
    lines = [l for l in buf.getvalue().splitlines() if l.startswith(MARK)]
    if rc != 0 or not lines:
        return {"error": f"workload returned status {rc}"}
    return json.loads(lines[-1][len(MARK):])


def run_in_child(name: str, args, cpu: bool) -> dict:
    cmd = [sys.executable, "-u", os.path.abspath(__file__), "--child", name, "--steps", str(args.steps),
           "--warmup", str(args.warmup), "--min-warmup-s", str(args.min_warmup_s)]
    if cpu:
        cmd.append("--cpu")
    p = subprocess.run(cmd, stdout=subprocess.PIPE, text=True, timeout=900)
    lines = [l for l in p.stdout.splitlines() if l.startswith(MARK)]
    if p.returncode != 0 or not lines:
        return {"error": f"child process exited with status {p.returncode}"}
    return json.loads(lines[-1][len(MARK):])


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--min-warmup-s", type=float, default=1.0,
                    help="minimum seconds of untimed launches before each timed region")
    ap.add_argument("--only", default="",
                    help="run one workload: " + "|".join(FNS))
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baselines")
    ap.add_argument("--child", default="", help=argparse.SUPPRESS)
    ap.add_argument("--cpu", action="store_true", help=argparse.SUPPRESS)
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this path has no multi-GPU mode "
              "(docs shard across GPUs with no exchange but a final gather of scores).",
              file=sys.stderr)
        return 2
    global MIN_WARMUP_S
    MIN_WARMUP_S = max(0.0, args.min_warmup_s)
    if args.child:
        return run_child(args)

    # the parent: runs every workload in a child process and never touches the
    # GPU (under a profiler, in this process instead)
    names = [args.only] if args.only else DEFAULT
    per, head = {}, None
    inproc = under_profiler()
    for n in names:
        _log(f"workload {n}: {'in this process (profiler)' if inproc else 'child process'}")
        r = (run_in_process if inproc else run_in_child)(n, args, cpu=not args.no_cpu)
        if n == HEADLINE:
            if "error" in r:
                print(f"bench.py: the headline workload failed ({r['error']})", file=sys.stderr)
                return 1
            head = r
        elif "error" in r:
            per[n] = r
        else:
            per[n] = dict(r["result"], **({"cpu_baseline": r["cpu"]} if r["cpu"] else {}))
        _log(f"workload {n}: done")

    if head is None:  # a single non-headline workload was asked for
        n, r = next(iter(per.items()))
        print(json.dumps({"metric": METRIC, "workload": r.get("workload", n), "result": r}), flush=True)
        return 0

    h = head["result"]
    cpu = head["cpu"]
    if cpu is not None:
        cpu = dict(cpu, host=host_info())
    line = {
        "metric": METRIC,
        "value": round(h["docs_per_s"], 1),
        "unit": "docs/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_min_s": MIN_WARMUP_S,
        "warmup_launches": h["warmup_runs"][0]["launches"] if h.get("warmup_runs") else None,
        "ms_per_step": round(h["ms"], 4),
        "per_launch_ms": h["per_launch_ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": h["workload"], "queries": 1, "query_tokens": 32,
                   "docs": 100_000, "doc_tokens": "U{50..300}", "packed_tokens": h["tokens"],
                   "d": 128, "seed": 2},
        "roofline": h["roofline"],
        "kernel": h["kernel"],
        "cpu_baseline": cpu,
        "per_config": per,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
