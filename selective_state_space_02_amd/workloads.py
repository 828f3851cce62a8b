"""The five synthetic workloads the scan path is tested and measured on.

Shapes and value distributions only (no arithmetic of the method).  B batch, L
sequence length, D inner channels (d_inner), N state size (d_state), K conv width
(d_conv); the RMSNorm backward runs over ``[rms_rows, rms_dim]``.  ``dtype`` is the
storage type of the activations; state and accumulation are always f32.

The ``delta_mu``/``delta_sigma`` pair parameterises the time step as
softplus(z), z ~ N(mu, sigma) (sigma is a standard deviation).  ``A[d, n] = -(n+1)``
for every workload.
"""
from dataclasses import dataclass


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    L: int
    D: int
    N: int
    K: int
    dtype: str          # "f32" or "bf16": storage type of activations
    delta_mu: float
    delta_sigma: float
    rms_rows: int
    rms_dim: int

    @property
    def elems(self) -> int:
        return self.B * self.L * self.D


WORKLOADS = [
    # tiny f32 case the oracle finishes instantly; RMSNorm rows = B*L
    Workload("tiny", 2, 8, 8, 4, 4, "f32", -2.0, 0.5, 16, 8),
    # the short-sequence, wide-batch shape of the ml-alpha stack (seq_len <= 32, state 16)
    Workload("alpha-stack", 256, 32, 64, 16, 4, "f32", -2.0, 0.5, 256 * 32, 64),
    # a Mamba-130M-shaped layer
    Workload("mamba-130m", 8, 2048, 1536, 16, 4, "f32", -3.0, 1.0, 8 * 2048, 768),
    # long sequence, bf16 activations
    Workload("long-bf16", 4, 8192, 2560, 16, 4, "bf16", -3.0, 1.0, 4 * 8192, 1280),
    # a Mamba-2.8B-shaped layer, bf16 activations
    Workload("mamba-2.8b", 2, 16384, 5120, 16, 4, "bf16", -4.0, 1.0, 2 * 16384, 2560),
]

BY_NAME = {w.name: w for w in WORKLOADS}


def custom(name="custom", B=2, L=64, D=32, N=16, K=4, dtype="f32", delta_mu=-2.0,
           delta_sigma=0.5, rms_rows=None, rms_dim=None) -> Workload:
    """A workload with the tiny case's distributions and arbitrary sizes (tests)."""
    return Workload(name, B, L, D, N, K, dtype, delta_mu, delta_sigma,
                    rms_rows if rms_rows is not None else B * L,
                    rms_dim if rms_dim is not None else D)
