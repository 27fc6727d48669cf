"""Seeded synthetic inputs and the named workloads.

This module holds no attention arithmetic: it only draws random numbers and
names shapes. Both the GPU path's tests/bench and the CPU oracle's tests take
their inputs from here, so the two sides see the same values.

Recipe: a CPU ``torch.Generator`` seeded with ``seed`` draws Q, then K, then
V, each ``torch.randn(B, H, N, d)`` in fp32; each is multiplied by ``sigma``
and cast to the workload dtype (round to nearest even). The oracle receives
these cast values upcast to fp64; the GPU receives them as they are.

The backward's upstream gradient dO is drawn the same way from a generator
seeded with ``seed + 7919`` (so it is independent of Q, K and V), with
sigma 1.
"""
from dataclasses import dataclass

import torch

DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str          # "f32" | "f16" | "bf16"
    causal: bool
    sigma: float = 1.0

    @property
    def torch_dtype(self):
        return DTYPES[self.dtype]

    @property
    def scale(self):
        """fp32(1/sqrt(d)), the value handed to the kernel and the oracle."""
        return float(torch.tensor(1.0 / self.d ** 0.5, dtype=torch.float32))

    def flops(self):
        """Two N x N x d contractions per head, halved when causal."""
        f = 4.0 * self.B * self.H * self.N * self.N * self.d
        return f / 2 if self.causal else f

    def flops_exact_causal(self):
        """Exact lower-triangle count 2*B*H*d*N*(N+1) (causal only)."""
        return 2.0 * self.B * self.H * self.d * self.N * (self.N + 1)

    def bwd_flops(self):
        """The five N x N x d contractions of the backward (S recomputed, dP,
        dV, dK, dQ), halved when causal: 2.5x the forward's."""
        return 2.5 * self.flops()

    def bwd_algorithmic_bytes(self, o_dtype="f32", grad_dtype="f32"):
        """Read Q, K, V, dO, O and LSE once; write dQ, dK, dV once."""
        e_in = torch.tensor([], dtype=self.torch_dtype).element_size()
        e_o = torch.tensor([], dtype=DTYPES[o_dtype]).element_size()
        e_g = torch.tensor([], dtype=DTYPES[grad_dtype]).element_size()
        n = self.B * self.H * self.N
        return (4 * e_in + e_o + 3 * e_g) * n * self.d + 4 * n

    def algorithmic_bytes(self, out_dtype=None):
        """Read Q, K, V once; write O (out dtype) and an fp32 LSE per row."""
        e_in = torch.tensor([], dtype=self.torch_dtype).element_size()
        e_out = torch.tensor([], dtype=DTYPES[out_dtype or self.dtype]).element_size()
        n = self.B * self.H * self.N
        return (3 * e_in + e_out) * n * self.d + 4 * n


# The five workloads: a single-head fp32 case, a short bf16 case, the causal
# headline case, a long causal case with large logits, and an fp16 case whose
# N is not a multiple of any tile size.
WORKLOADS = {
    "single_head_f32": Workload("single_head_f32", 1, 1, 128, 64, "f32", False),
    "b4h16_n1024_d64_bf16": Workload("b4h16_n1024_d64_bf16", 4, 16, 1024, 64, "bf16", False),
    "b2h32_n4096_d128_bf16_causal": Workload("b2h32_n4096_d128_bf16_causal", 2, 32, 4096, 128,
                                             "bf16", True),
    "b1h16_n16384_d128_bf16_sigma3_causal": Workload("b1h16_n16384_d128_bf16_sigma3_causal", 1, 16,
                                                     16384, 128, "bf16", True, 3.0),
    "b8h12_n3000_d64_f16": Workload("b8h12_n3000_d64_f16", 8, 12, 3000, 64, "f16", False),
}
HEADLINE = "b2h32_n4096_d128_bf16_causal"


def make_qkv(B, H, N, d, dtype="bf16", sigma=1.0, seed=0):
    """Q, K, V on the CPU, drawn in that order from one seeded generator."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    tdt = DTYPES[dtype] if isinstance(dtype, str) else dtype
    out = []
    for _ in range(3):
        x = torch.randn(B, H, N, d, generator=g, dtype=torch.float32)
        if sigma != 1.0:
            x = x * float(sigma)
        out.append(x.to(tdt).contiguous())
    return tuple(out)


def make_dout(B, H, N, d, dtype="bf16", seed=0):
    """Upstream gradient dO for the backward, on the CPU."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed) + 7919)
    tdt = DTYPES[dtype] if isinstance(dtype, str) else dtype
    return torch.randn(B, H, N, d, generator=g, dtype=torch.float32).to(tdt).contiguous()


def workload_qkv(w: Workload, seed=0):
    return make_qkv(w.B, w.H, w.N, w.d, w.dtype, w.sigma, seed)
