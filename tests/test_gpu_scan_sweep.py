"""GPU parity of the scan over a seeded random sweep of shapes and options.

Twenty cases drawn once from a fixed seed: B in [1, 5], L in [1, 700], D in [1, 300]
(every residue mod 4 and mod 64 occurs), N in {4, 8, 16}, f32 or bf16, with or without
h0 and stored checkpoints, plain or with the fused neighbours (time-step softplus and
bias, output gate).  Every output is compared with the oracle; the hand-picked cases in
the other scan tests stay the primary coverage, this catches combinations they miss.
"""
import numpy as np
import pytest

from selective_state_space_02_amd import synth
from selective_state_space_02_amd.workloads import custom
from tests.gpu_common import compare, say, scan_gpu, scan_oracle
from tests.test_gpu_scan_fused import FULL, fused_gpu, fused_inputs, fused_oracle, keys_for

pytestmark = pytest.mark.gpu


def _cases(n=20, seed=20261202):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        B = int(rng.integers(1, 6))
        L = int(rng.integers(1, 701))
        D = int(rng.integers(1, 301))
        N = int(rng.choice([4, 8, 16]))
        dtype = str(rng.choice(["f32", "bf16"]))
        out.append((i, custom(B=B, L=L, D=D, N=N, dtype=dtype), bool(rng.integers(0, 2)),
                    bool(rng.integers(0, 2)), bool(rng.integers(0, 2))))
    return out


CASES = _cases()


@pytest.mark.parametrize("i,w,with_h0,use_ckpt,fused", CASES,
                         ids=[f"{c[0]}-B{c[1].B}L{c[1].L}D{c[1].D}N{c[1].N}{c[1].dtype}"
                              f"{'-h0' if c[2] else ''}{'-ckpt' if c[3] else ''}"
                              f"{'-fused' if c[4] else ''}" for c in CASES])
def test_scan_random_shapes_match_oracle(i, w, with_h0, use_ckpt, fused):
    say(f"[scan sweep {i}] B={w.B} L={w.L} D={w.D} N={w.N} {w.dtype} h0={with_h0} "
        f"ckpt={use_ckpt} fused={fused}")
    if fused:
        p = fused_inputs(w, FULL, seed=100 + i, with_h0=with_h0)
        compare(fused_gpu(p, FULL, use_ckpt=use_ckpt), fused_oracle(p, FULL), keys_for(FULL),
                label=f"sweep {i} fused")
    else:
        p = synth.scan_inputs(w, seed=100 + i, with_h0=with_h0)
        compare(scan_gpu(p, use_ckpt=use_ckpt), scan_oracle(p),
                ("y", "h_last", "dx", "ddelta", "dA", "dB", "dC", "dD", "dh0"),
                label=f"sweep {i}")
