"""Seeded synthetic inputs shared by the oracle tests, the GPU tests and the benchmark.

This module only draws random numbers and names shapes. It holds none of the
attention arithmetic: neither the oracle nor the HIP library is imported here,
and neither of them imports this module. Tests draw one set of inputs here and
hand identical copies to both sides.

Workloads (all Gaussian, the shapes used by the Performer and RFA pages for
bidirectional attention, causal attention and recurrent decoding):

  bidir_small  fp32  B1 H1  L256  d16 dv16 m32   Q,K,V ~ N(0, 0.5^2)        seed 0
  bidir_fp32   fp32  B1 H8  L4096 d16 dv16 m128  Q,K,V ~ N(0, 1)            seed 1
  bidir_bf16   bf16  B8 H12 L4096 d64 dv64 m256  Q,K ~ N(0,1)/sqrt2, V~N(0,1) seed 2
  cross_bf16   bf16  B8 H12 Lq1024 Lk4096 d64 dv64 m256, as bidir_bf16     seed 6
               (a synthetic cross-attention shape: the pages fix none)
  causal_bf16  bf16  B4 H8  L8192 d64 dv64 m256  Q,K,V ~ 0.5 N(0, 1)        seed 3
  decode_bf16  bf16  256 sequences, H16 d64 dv64 m256; 2048 prior tokens
               build the state, then 1000 steps of q,k,v ~ N(0,1)         seed 4
  decode_gated_bf16  the same, each step with a gate g ~ U[0.9, 1) per
               (sequence, head) and input weight 1 - g                   seed 5
  trig_bf16    bf16  B8 H12 L4096 d64 dv64 m256 with trigonometric features
               (128 vectors, sine and cosine), Q,K ~ 0.4 N(0,1), V ~ N(0,1)  seed 7
  backward_bf16  bidir_bf16's inputs plus an upstream gradient dOut ~ N(0,1)
               [B,H,L,dv] (its own generator, seed + 100): the gradients
               of the bidirectional estimator                            seed 2
  causal_backward_bf16  causal_bf16's inputs plus dOut ~ N(0,1) drawn the same
               way: the gradients of the causal estimator                seed 3

Draw order for one workload: Q, then K, then V, each one `torch.randn` call on
a CPU generator seeded with the workload's seed, scaled, then rounded to the
workload's dtype with round-to-nearest-even.  Decode step inputs are large
(1.57 GB), so they are drawn on the device with torch's counter-based CUDA
generator; tests copy the slices they check back to the host.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    kind: str            # "bidir" | "cross" | "causal" | "decode" | "decode_gated" | "backward" | "features"
    dtype: str           # "f32" | "bf16"
    B: int
    H: int
    L: int
    d: int
    dv: int
    m: int
    seed: int
    q_scale: float
    k_scale: float
    v_scale: float
    steps: int = 0       # decode only
    prior: int = 0       # decode only: tokens folded into the initial state
    Lq: int = 0          # cross attention: query length (L is then the key length); 0 = L
    feature: str = "prf"  # feature map: "prf" or "trig" (Omega of m/2 vectors, each twice)

    @property
    def Lq_eff(self) -> int:
        return self.Lq if self.Lq else self.L

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    "bidir_small": Workload("bidir_small", "bidir", "f32", 1, 1, 256, 16, 16, 32, 0, 0.5, 0.5, 0.5),
    "bidir_fp32": Workload("bidir_fp32", "bidir", "f32", 1, 8, 4096, 16, 16, 128, 1, 1.0, 1.0, 1.0),
    "bidir_bf16": Workload("bidir_bf16", "bidir", "bf16", 8, 12, 4096, 64, 64, 256, 2,
                           1.0 / math.sqrt(2.0), 1.0 / math.sqrt(2.0), 1.0),
    "cross_bf16": Workload("cross_bf16", "cross", "bf16", 8, 12, 4096, 64, 64, 256, 6,
                           1.0 / math.sqrt(2.0), 1.0 / math.sqrt(2.0), 1.0, Lq=1024),
    "trig_bf16": Workload("trig_bf16", "bidir", "bf16", 8, 12, 4096, 64, 64, 256, 7, 0.4, 0.4, 1.0,
                          feature="trig"),
    "backward_bf16": Workload("backward_bf16", "backward", "bf16", 8, 12, 4096, 64, 64, 256, 2,
                              1.0 / math.sqrt(2.0), 1.0 / math.sqrt(2.0), 1.0),
    "causal_bf16": Workload("causal_bf16", "causal", "bf16", 4, 8, 8192, 64, 64, 256, 3, 0.5, 0.5, 0.5),
    "causal_backward_bf16": Workload("causal_backward_bf16", "causal_backward", "bf16", 4, 8, 8192, 64, 64, 256, 3,
                                     0.5, 0.5, 0.5),
    "features_bf16": Workload("features_bf16", "features", "bf16", 8, 12, 4096, 64, 64, 256, 2,
                              1.0 / math.sqrt(2.0), 1.0 / math.sqrt(2.0), 1.0),
    "decode_bf16": Workload("decode_bf16", "decode", "bf16", 256, 16, 1, 64, 64, 256, 4, 1.0, 1.0, 1.0,
                            steps=1000, prior=2048),
    "decode_gated_bf16": Workload("decode_gated_bf16", "decode_gated", "bf16", 256, 16, 1, 64, 64, 256, 5,
                                  1.0, 1.0, 1.0, steps=1000, prior=2048),
}


def _randn(gen: torch.Generator, shape, scale: float, dtype: torch.dtype, device="cpu") -> torch.Tensor:
    x = torch.randn(*shape, generator=gen, dtype=torch.float32, device=device)
    if scale != 1.0:
        x = x * scale
    return x.to(dtype)


def make_qkv(w: Workload, device: str = "cpu"):
    """Q [B,H,Lq,d] (Lq = L unless set), K [B,H,L,d] and V [B,H,L,dv], contiguous, in the workload dtype.

    Drawn on a CPU generator (so the values do not depend on the GPU) and then
    moved to `device`.
    """
    gen = torch.Generator("cpu").manual_seed(w.seed)
    q = _randn(gen, (w.B, w.H, w.Lq_eff, w.d), w.q_scale, w.torch_dtype)
    k = _randn(gen, (w.B, w.H, w.L, w.d), w.k_scale, w.torch_dtype)
    v = _randn(gen, (w.B, w.H, w.L, w.dv), w.v_scale, w.torch_dtype)
    if device != "cpu":
        q, k, v = q.to(device), k.to(device), v.to(device)
    return q, k, v


def make_decode_prior(w: Workload, n_seq: Optional[int] = None, device: str = "cpu"):
    """The `prior` tokens that build the initial decode state.

    Returns k [S,H,prior,d] and v [S,H,prior,dv] for the first `n_seq`
    sequences (all of them by default), drawn on a CPU generator in the
    workload dtype. Only K and V enter the state.
    """
    n = w.B if n_seq is None else n_seq
    gen = torch.Generator("cpu").manual_seed(w.seed * 1000003 + 17)
    k = _randn(gen, (n, w.H, w.prior, w.d), w.k_scale, w.torch_dtype)
    v = _randn(gen, (n, w.H, w.prior, w.dv), w.v_scale, w.torch_dtype)
    if device != "cpu":
        k, v = k.to(device), v.to(device)
    return k, v


def make_dout(w: Workload, device: str = "cpu") -> torch.Tensor:
    """Upstream gradient of the attention output, [B,H,Lq,dv] ~ N(0,1) in the workload dtype, drawn on a CPU
    generator seeded with the workload's seed + 100."""
    gen = torch.Generator("cpu").manual_seed(w.seed + 100)
    g = _randn(gen, (w.B, w.H, w.Lq_eff, w.dv), 1.0, w.torch_dtype)
    return g.to(device) if device != "cpu" else g


def make_decode_steps(w: Workload, device: str, steps: Optional[int] = None):
    """All decode-step inputs, pre-drawn so that no RNG runs inside a timed loop.

    q, k: [steps, S, H, d]; v: [steps, S, H, dv], in the workload dtype, drawn
    with a generator on `device` (torch's Philox generator on a GPU).
    """
    n_steps = w.steps if steps is None else steps
    gen = torch.Generator(device).manual_seed(w.seed)
    q = _randn(gen, (n_steps, w.B, w.H, w.d), w.q_scale, w.torch_dtype, device)
    k = _randn(gen, (n_steps, w.B, w.H, w.d), w.k_scale, w.torch_dtype, device)
    v = _randn(gen, (n_steps, w.B, w.H, w.dv), w.v_scale, w.torch_dtype, device)
    return q, k, v


def make_gates(shape, seed: int, lo: float = 0.9, hi: float = 1.0, device: str = "cpu") -> torch.Tensor:
    """Gate values ~ U[lo, hi) in fp32 (recency gates of the gated decode), drawn on `device`."""
    gen = torch.Generator(device).manual_seed(seed)
    return lo + (hi - lo) * torch.rand(*shape, generator=gen, dtype=torch.float32, device=device)


def make_tensor(shape, seed: int, scale: float = 1.0, dtype=torch.float32, device="cpu") -> torch.Tensor:
    """One seeded Gaussian tensor, for ad-hoc test cases."""
    gen = torch.Generator("cpu").manual_seed(seed)
    t = _randn(gen, shape, scale, dtype)
    return t.to(device) if device != "cpu" else t
