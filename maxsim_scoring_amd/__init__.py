"""MaxSim scoring on MI355X (gfx950): fused late-interaction scoring kernels.

The product is the HIP library ``libmaxsim_amd.so`` behind the C ABI in
``include/maxsim.h``; ``binding`` exposes the same entry points to Python
(torch tensors in GPU memory, argument marshalling only). ``synth`` draws the
seeded synthetic workloads and ``workload`` holds the byte/flop model.
"""

from .binding import (MaxSimError, maxsim_abi_version, maxsim_bwd, maxsim_bwd_varlen,
                      maxsim_chamfer_bwd, maxsim_chamfer_fwd, maxsim_fwd,
                      maxsim_fwd_i8, maxsim_fwd_i8_tok, maxsim_fwd_pairs, maxsim_fwd_pairs_varlen,
                      maxsim_fwd_varlen, maxsim_status_string, maxsim_topk, two_stage_topk)

__all__ = ["MaxSimError", "maxsim_fwd", "maxsim_fwd_varlen", "maxsim_fwd_i8", "maxsim_fwd_i8_tok",
           "maxsim_fwd_pairs", "maxsim_fwd_pairs_varlen", "maxsim_topk", "two_stage_topk",
           "maxsim_bwd", "maxsim_bwd_varlen", "maxsim_chamfer_fwd", "maxsim_chamfer_bwd",
           "maxsim_status_string", "maxsim_abi_version"]
