"""Seeded synthetic inputs for attention, shared by the tests, the bench and
the smoke check.  Holds no attention arithmetic: it only draws random numbers
and rounds them to bf16 bit patterns.

Recipe (one per workload, all bf16 Q/K/V laid out [B, H, N, d]):
  * numpy default_rng(seed) (PCG64); standard_normal(dtype=float32) draws in
    the order Q, K, V, then the per-row factor r (rescale workload) or dO
    (backward workload);
  * float32 -> bf16 by round-to-nearest-even on the bit pattern;
  * the rescale workload multiplies each query row (b, h, i) by its own
    r ~ U[0.5, 4) in float32 before the single bf16 rounding, so the running
    row maximum jumps part-way through a row.

The FlashAttention-4 pages benchmark forward attention at head dimension 128
in BF16 over sequence lengths 1k-32k ("Production Benchmarks on NVIDIA
Blackwell B200"); the workloads below cover that range with iid N(0, 1)
inputs.  No dataset is involved.
"""
from dataclasses import dataclass, field
import math

import numpy as np


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 array -> uint16 bf16 bit patterns, round-to-nearest-even.
    Inputs here are finite; NaN/Inf are not produced by the generators."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """uint16 bf16 bit patterns -> float32 (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    N: int
    d: int
    causal: bool
    seed: int
    row_scale: bool = False      # per-row Q factor r ~ U[0.5, 4)
    backward: bool = False       # also draw dO
    note: str = field(default="", compare=False)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    def fwd_flops(self) -> float:
        """Nominal forward FLOPs: 4*B*Hq*N^2*d, exactly halved when causal."""
        f = 4.0 * self.B * self.Hq * self.N * self.N * self.d
        return f / 2 if self.causal else f

    def bwd_flops(self) -> float:
        """Nominal backward FLOPs: 2.5x the forward count."""
        return 2.5 * self.fwd_flops()


# The five workloads (sizes, seeds 42..46).
WORKLOADS = {
    "fwd_small_d64": Workload("fwd_small_d64", 1, 2, 2, 128, 64, False, 42,
                              note="B1 H2 N128 d64 forward, non-causal"),
    "fwd_n4096": Workload("fwd_n4096", 4, 16, 16, 4096, 128, False, 43,
                          note="B4 H16 N4096 d128 forward, non-causal"),
    "fwd_causal_rowscale_n8192": Workload("fwd_causal_rowscale_n8192", 2, 16, 16, 8192, 128,
                                          True, 44, row_scale=True,
                                          note="B2 H16 N8192 d128 causal, Q rows x U[0.5,4)"),
    "fwd_causal_gqa_n32768": Workload("fwd_causal_gqa_n32768", 1, 32, 8, 32768, 128, True, 45,
                                      note="B1 Hq32 Hkv8 N32768 d128 causal GQA 4:1"),
    "fwdbwd_causal_n8192": Workload("fwdbwd_causal_n8192", 2, 16, 16, 8192, 128, True, 46,
                                    backward=True,
                                    note="B2 H16 N8192 d128 causal, forward + backward"),
}


def make_inputs(w: Workload, seed: int = None):
    """Draw the workload's inputs.  Returns dict of uint16 bf16 bit arrays:
    q [B,Hq,N,d], k, v [B,Hkv,N,d], and dout [B,Hq,N,d] when w.backward."""
    rng = np.random.default_rng(w.seed if seed is None else seed)
    qf = rng.standard_normal((w.B, w.Hq, w.N, w.d), dtype=np.float32)
    kf = rng.standard_normal((w.B, w.Hkv, w.N, w.d), dtype=np.float32)
    vf = rng.standard_normal((w.B, w.Hkv, w.N, w.d), dtype=np.float32)
    if w.row_scale:
        r = rng.uniform(0.5, 4.0, size=(w.B, w.Hq, w.N, 1)).astype(np.float32)
        qf = qf * r
    out = {"q": f32_to_bf16_bits(qf), "k": f32_to_bf16_bits(kf), "v": f32_to_bf16_bits(vf)}
    del qf, kf, vf
    if w.backward:
        out["dout"] = f32_to_bf16_bits(rng.standard_normal((w.B, w.Hq, w.N, w.d),
                                                           dtype=np.float32))
    return out


def random_bf16(shape, seed, scale=1.0):
    """iid N(0, scale^2) bf16 bit patterns of the given shape (small cases)."""
    rng = np.random.default_rng(seed)
    return f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32) * np.float32(scale))
