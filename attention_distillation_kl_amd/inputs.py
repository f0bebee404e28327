"""Seeded synthetic inputs shared by the tests, the benchmark and the smoke check.

This module holds no arithmetic of the method: it only draws Gaussian
teacher/student query and key tensors.  Both the HIP path and the fp64 oracle
are fed the very same tensors built here (the oracle receives an exact float64
copy).

Recipe (the StreamKL summary page measures on synthetic long-context shapes
and names no dataset): all tensors are [B, H, N, d], d innermost.  The teacher
(Q1, K1) is i.i.d. N(0, 1); the student is either independent i.i.d. N(0, 1)
("iid") or teacher + sigma * N(0, 1) ("student").  Draws happen in float32 in
the order Q1, K1, noise_Q, noise_K (or Q1, K1, Q2, K2 for "iid") from one
``torch.Generator`` seeded with ``seed``; noise is added in float32 and the
result is cast to the working dtype last.  scale = 1/sqrt(d).
"""
import math
from dataclasses import dataclass, asdict

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    NQ: int
    NK: int
    d: int
    dtype: str          # "f32" | "bf16"
    causal: bool
    mode: str           # "iid" | "student"
    sigma: float
    seed: int
    passes: str         # "fwd" | "fwd+bwd"

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def fwd_flops(self) -> float:
        """4 * N_Q * N_K * d per head, halved when causal."""
        f = 4.0 * self.B * self.H * self.NQ * self.NK * self.d
        return f / 2 if self.causal else f

    def fwdbwd_flops(self) -> float:
        """16 * N_Q * N_K * d per head (fwd 4 + bwd 12), halved when causal."""
        return 4.0 * self.fwd_flops()

    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    def fwd_bytes(self) -> float:
        """Algorithmic HBM bytes of one forward: Q1, Q2, K1, K2 read once,
        KL, LSE1, LSE2 written (12 B per query row)."""
        bh = self.B * self.H
        return float(bh * (2 * (self.NQ + self.NK) * self.d * self.elem_bytes() + 12 * self.NQ))

    def bwd_bytes(self, kernel: str) -> float:
        """Algorithmic HBM bytes of one backward kernel: the four inputs and
        16 B per query row (KL, LSE1, LSE2, upstream gradient) read, its
        gradients written ('bwd_dk': dK1, dK2; 'bwd_dq': dQ1, dQ2;
        'bwd_fused': all four)."""
        bh = self.B * self.H
        rows = {"bwd_dk": self.NK, "bwd_dq": self.NQ, "bwd_fused": self.NQ + self.NK}[kernel]
        return float(bh * (2 * (self.NQ + self.NK) * self.d * self.elem_bytes() + 16 * self.NQ
                           + 2 * rows * self.d * self.elem_bytes()))

    def as_dict(self):
        return asdict(self)


WORKLOADS = {
    "c1": Workload("c1", 1, 1, 256, 256, 64, "f32", False, "iid", 0.0, 1001, "fwd"),
    "c2": Workload("c2", 1, 8, 2048, 2048, 64, "bf16", True, "student", 0.3, 1002, "fwd+bwd"),
    "c3": Workload("c3", 2, 32, 8192, 8192, 128, "bf16", True, "student", 0.1, 1003, "fwd+bwd"),
    "c4": Workload("c4", 1, 32, 2048, 65536, 128, "bf16", False, "iid", 0.0, 1004, "fwd"),
    "c5": Workload("c5", 1, 32, 65536, 65536, 128, "bf16", True, "student", 0.2, 1005, "fwd+bwd"),
    "h32k": Workload("h32k", 1, 32, 32768, 32768, 128, "bf16", True, "student", 0.2, 1032, "fwd+bwd"),
    # one decoding row per head over 64K keys (the split-K forward's case)
    "decode": Workload("decode", 1, 32, 1, 65536, 128, "bf16", False, "iid", 0.0, 1006, "fwd"),
    # a short query block over 64K keys, forward and backward (the split-K
    # forward and the fused backward)
    "shortq": Workload("shortq", 1, 32, 64, 65536, 128, "bf16", False, "student", 0.2, 1064, "fwd+bwd"),
}


def make_inputs(B, H, NQ, NK, d, dtype=torch.bfloat16, mode="student", sigma=0.2,
                seed=0, device="cpu"):
    """Return (q1, k1, q2, k2), each contiguous [B, H, N, d] of ``dtype``."""
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    kw = dict(generator=gen, device=device, dtype=torch.float32)
    q1 = torch.randn(B, H, NQ, d, **kw)
    k1 = torch.randn(B, H, NK, d, **kw)
    if mode == "iid":
        q2 = torch.randn(B, H, NQ, d, **kw)
        k2 = torch.randn(B, H, NK, d, **kw)
    elif mode == "student":
        q2 = torch.randn(B, H, NQ, d, **kw).mul_(sigma).add_(q1)
        k2 = torch.randn(B, H, NK, d, **kw).mul_(sigma).add_(k1)
    else:
        raise ValueError(f"unknown mode {mode!r}")
    return tuple(t.to(dtype).contiguous() for t in (q1, k1, q2, k2))


def workload_inputs(w: Workload, device="cpu"):
    return make_inputs(w.B, w.H, w.NQ, w.NK, w.d, w.torch_dtype, w.mode, w.sigma,
                       w.seed, device)


def upstream_grad(B, H, NQ, seed=0, device="cpu"):
    """A random per-row upstream gradient (both signs, some exact zeros)."""
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed) + 7)
    g = torch.randn(B, H, NQ, generator=gen, device=device, dtype=torch.float32)
    g[..., ::5] = 0.0
    return g.contiguous()
