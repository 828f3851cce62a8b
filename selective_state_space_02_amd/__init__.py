"""MI355X-native (gfx950) selective-scan hot path.

The product is ``libssmscan.so`` (HIP kernels behind a C ABI, declared in
``include/ssm_scan.h``); ``binding`` is its thin Python binding.  ``workloads`` and
``synth`` hold the synthetic workload shapes and seeded input generators.  Importing
the package does not load the library; the first binding call does, and raises if it
is missing.
"""
from .binding import (SsmError, conv1d_causal_bwd, conv1d_causal_fwd,  # noqa: F401
                      conv1d_causal_step, load, new_ckpt, rmsnorm_bwd, rmsnorm_fwd, ssm_scan_bwd,
                      ssm_decode_step, ssm_scan_fused_bwd, ssm_scan_fused_fwd, ssm_scan_fused_step,
                      ssm_scan_fwd,
                      ssm_scan_step,
                      version)
