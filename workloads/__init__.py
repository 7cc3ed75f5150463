"""Seeded synthetic inputs for the retention workloads.

This module holds no retention arithmetic: it only draws seeded random tensors
of the workloads' shapes and writes down their fixed parameters (per-head decay
constants and rotation frequencies).  Both the GPU tests and the oracle-side
checks take their inputs from here; nothing here depends on either side.

Recipe: ``torch.Generator('cpu').manual_seed(1000 * c + j)`` where ``c`` is the
workload's seed group (tiny 1, parallel 2, chunkwise 3, decode 4, MSR layer 5;
ad-hoc test shapes pass an explicit seed)
and ``j`` the tensor's index in a fixed draw order (Q=0, K=1, V=2, W_Q=3, W_K=4,
W_V=5, W_G=6, W_O=7); ``torch.randn`` in fp32, scaled in fp32, then cast to the
workload dtype (round to nearest even for bf16).  Values are i.i.d. Gaussian:
the pages describe no structure in the data.
"""
from dataclasses import dataclass, field
from typing import Optional

import torch


def multiscale_gamma(H: int) -> torch.Tensor:
    """Per-head decay constants gamma_h = 1 - 2^(-5-h), h = 0..H-1 (gated
    multi-scale retention, "Retentive Network" paper summary, Sec. 2.2).
    Exact in fp32 for h <= 18."""
    return torch.tensor([1.0 - 2.0 ** (-5 - h) for h in range(H)], dtype=torch.float32)


def rotation_theta(dk: int) -> torch.Tensor:
    """Rotation frequencies theta_i = 10000^(-2i/dk), i < dk/2, as fp32 (the
    fp32 values are the definition both sides use)."""
    return torch.tensor([10000.0 ** (-2.0 * i / dk) for i in range(dk // 2)], dtype=torch.float32)


def randn(shape, seed: int, scale: float = 1.0, dtype=torch.float32) -> torch.Tensor:
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    x = torch.randn(*shape, generator=g, dtype=torch.float32)
    if scale != 1.0:
        x = x * torch.tensor(scale, dtype=torch.float32)
    return x.to(dtype)


@dataclass
class RetentionWorkload:
    name: str
    B: int
    H: int
    L: int
    dk: int
    dv: int
    chunk: int
    dtype: torch.dtype
    scale: float
    gn_eps: Optional[float]
    seed_group: int
    pos0: int = 0

    def gamma(self):
        return multiscale_gamma(self.H)

    def theta(self):
        return rotation_theta(self.dk)

    def qkv(self, seed_base: Optional[int] = None):
        base = 1000 * self.seed_group if seed_base is None else seed_base
        q = randn((self.B, self.H, self.L, self.dk), base + 0, self.scale, self.dtype)
        k = randn((self.B, self.H, self.L, self.dk), base + 1, self.scale, self.dtype)
        v = randn((self.B, self.H, self.L, self.dv), base + 2, self.scale, self.dtype)
        return q, k, v

    @property
    def tokens(self):
        return self.B * self.L


# tiny check, all three forms (fp32)
TINY = RetentionWorkload("tiny-fp32 B1 H2 L64 dk16 dv16 chunk16", 1, 2, 64, 16, 16, 16,
                         torch.float32, 1.0, None, 1)
# parallel form, bf16, GroupNorm on the output
PARALLEL_2K = RetentionWorkload("parallel B8 H8 L2048 dk256 dv512 bf16 +GN", 8, 8, 2048, 256, 512,
                                2048, torch.bfloat16, 256 ** -0.5, 1e-5, 2)
# chunkwise form, long context
CHUNKWISE_32K = RetentionWorkload("chunkwise B1 H8 L32768 dk128 dv256 chunk256 bf16", 1, 8, 32768,
                                  128, 256, 256, torch.bfloat16, 128 ** -0.5, None, 3)


@dataclass
class DecodeWorkload:
    name: str = "decode B128 H16 dk128 dv256 prefill512 steps1024 bf16"
    B: int = 128
    H: int = 16
    dk: int = 128
    dv: int = 256
    prefill: int = 512
    steps: int = 1024
    chunk: int = 256
    scale: float = 128 ** -0.5
    seed_group: int = 4

    def gamma(self):
        return multiscale_gamma(self.H)

    def theta(self):
        return rotation_theta(self.dk)

    def prefill_qkv(self):
        b = 1000 * self.seed_group
        q = randn((self.B, self.H, self.prefill, self.dk), b + 0, self.scale, torch.bfloat16)
        k = randn((self.B, self.H, self.prefill, self.dk), b + 1, self.scale, torch.bfloat16)
        v = randn((self.B, self.H, self.prefill, self.dv), b + 2, self.scale, torch.bfloat16)
        return q, k, v

    def step_qkv(self, steps: Optional[int] = None):
        """All decode-step inputs at once: [steps, B, H, d]."""
        n = self.steps if steps is None else steps
        b = 1000 * self.seed_group
        q = randn((n, self.B, self.H, self.dk), b + 3, self.scale, torch.bfloat16)
        k = randn((n, self.B, self.H, self.dk), b + 4, self.scale, torch.bfloat16)
        v = randn((n, self.B, self.H, self.dv), b + 5, self.scale, torch.bfloat16)
        return q, k, v


DECODE = DecodeWorkload()


@dataclass
class MSRWorkload:
    name: str = "msr-layer B4 L4096 dmodel2048 H8 dk256 dv512 chunk512 bf16"
    B: int = 4
    L: int = 4096
    d_model: int = 2048
    H: int = 8
    dk: int = 256
    dv: int = 512
    chunk: int = 512
    gn_eps: float = 1e-5
    w_std: float = 0.02
    seed_group: int = 5

    def gamma(self):
        return multiscale_gamma(self.H)

    def theta(self):
        return rotation_theta(self.dk)

    def inputs(self, seed_base: Optional[int] = None):
        """x [B,L,d_model]; weights stored [out, in]: w_q, w_k [H*dk, d_model],
        w_v, w_g [H*dv, d_model], w_o [d_model, H*dv]."""
        b = 1000 * self.seed_group if seed_base is None else seed_base
        bf = torch.bfloat16
        x = randn((self.B, self.L, self.d_model), b + 0, 1.0, bf)
        w_q = randn((self.H * self.dk, self.d_model), b + 3, self.w_std, bf)
        w_k = randn((self.H * self.dk, self.d_model), b + 4, self.w_std, bf)
        w_v = randn((self.H * self.dv, self.d_model), b + 5, self.w_std, bf)
        w_g = randn((self.H * self.dv, self.d_model), b + 6, self.w_std, bf)
        w_o = randn((self.d_model, self.H * self.dv), b + 7, self.w_std, bf)
        return x, w_q, w_k, w_v, w_g, w_o

    @property
    def tokens(self):
        return self.B * self.L


MSR_LAYER = MSRWorkload()
