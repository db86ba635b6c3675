"""Writes int8_long_query_expected.json: the oracle's results for the long-query
INT8 workload (one query of 1024 tokens against 10,000 docs of 1024 tokens,
d = 128, per-tensor scales, seed 4; "Flash-MaxSim" Sec. 4.3.1), for the GPU
parity test that compares every doc.

Stored: every doc's exact int32 max-sum, every fp32 score (the hex of its
little-endian bits), and for each block of 100 docs a digest of their argmax
rows (the first 16 hex digits of the SHA-256 of the block's [100, 1024] int32
indices, little-endian), so the test checks every index bit for bit without
keeping 40 MB of indices and recomputes only a differing block. Digests of
the generated inputs are stored too, so the test can tell a change of inputs
from a parity failure.

Only the seeded generators and oracle/ are called. Run from the repository
root:  python tests/golden/make_int8_long_query.py   (a few minutes of CPU)
"""

import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

from maxsim_scoring_amd import synth  # noqa: E402
from oracle import oracle  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "int8_long_query_expected.json")


def sha(a) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


BLOCK = 100


def block_digests(argmax) -> list:
    a = np.ascontiguousarray(np.asarray(argmax, dtype="<i4"))
    return [hashlib.sha256(a[0, j:j + BLOCK].tobytes()).hexdigest()[:16]
            for j in range(0, a.shape[1], BLOCK)]


def main() -> None:
    t0 = time.time()
    w = synth.int8_long_query()
    Q, D = w.Q.numpy(), w.D.numpy()
    inputs = {"Q": sha(Q), "D": sha(D), "q_scale": float(w.q_scale), "d_scale": float(w.d_scale)}
    print(f"inputs generated in {time.time() - t0:.1f} s", flush=True)
    t0 = time.time()
    si, sf, a = oracle.fwd_i8(Q, w.q_scale, D, w.d_scale, want_argmax=True)
    print(f"oracle in {time.time() - t0:.1f} s on {oracle.default_threads()} threads", flush=True)
    out = {
        "what": "oracle results of the long-query INT8 workload, every doc",
        "citation": "Flash-MaxSim Sec. 4.3.1 (INT8 x INT8 scoring with a fused scale epilogue)",
        "workload": w.name, "seed": w.seed,
        "inputs_sha256": inputs,
        "argmax_digest": ("sha256 of argmax[0, b:b+100, :] as little-endian int32, first 16 hex "
                          "digits, for b = 0, 100, ..."),
        "argmax_block": BLOCK,
        "scores_i32": [int(x) for x in si[0]],
        "scores_f32_hex": sf[0].astype("<f4").tobytes().hex(),
        "argmax_block_digests": block_digests(a),
    }
    with open(OUT, "w") as f:
        json.dump(out, f, separators=(",", ":"))
        f.write("\n")
    print(f"wrote {OUT}")


if __name__ == "__main__":
    main()
