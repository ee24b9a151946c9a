"""Seeded synthetic inputs for the HLA2 workloads (no method arithmetic here).

Both the GPU path and the fp64 oracle are fed from these generators: values
are drawn in fp32 from a seeded torch CPU generator in the order q, k, v,
scaled/normalised as the workload states, then rounded ONCE to the element
type (bf16 round-to-nearest-even, or kept fp32).  The oracle consumes the same
rounded values upcast exactly to fp64, so input quantisation is not an error
source of any comparison.

Workloads (named by what they are; sizes are per the workload list of the
method's measurement plan):
  tiny_f32      B=1  H=1  n=64     d=16  dv=16   fp32, N(0,1)/sqrt(d), no decay, unnormalised, chunk 16
  norm_2k       B=4  H=8  n=2048   d=64  dv=64   bf16, N(0,1)/sqrt(d), ratio-normalised, chunk 64
  decay_8k      B=8  H=16 n=8192   d=64  dv=128  bf16, q,k ~ N(0,1)/sqrt(d) then unit-L2 rows, v ~ N(0,1),
                                                 decay 0.99, unnormalised, chunk 64
  long_64k      B=1  H=16 n=65536  d=128 dv=128  bf16, N(0,1)/sqrt(d), ratio-normalised, chunk 128
  decode_256x32 N=256 H=32 d=64 dv=64, fp32 state after a 4096-token N(0,1)/sqrt(d) prefix, then 128
                single-token steps with bf16 q,k,v ~ N(0,1)/sqrt(d), ratio-normalised
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    n: int
    d: int
    dv: int
    dtype: str            # "f32" | "bf16"
    decay: float
    normalize: bool
    chunk: int
    qk_unit_rows: bool = False
    v_scale: float | None = None  # None: 1/sqrt(d)
    seed: int = 0

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    @property
    def head_tokens(self) -> int:
        return self.B * self.H * self.n


@dataclass(frozen=True)
class DecodeWorkload:
    name: str
    N: int
    H: int
    d: int
    dv: int
    prefix: int
    steps: int
    decay: float
    normalize: bool
    dtype: str = "bf16"
    seed: int = 0

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16


WORKLOADS = {
    "tiny_f32": Workload("tiny_f32", 1, 1, 64, 16, 16, "f32", 1.0, False, 16),
    "norm_2k": Workload("norm_2k", 4, 8, 2048, 64, 64, "bf16", 1.0, True, 64),
    "decay_8k": Workload("decay_8k", 8, 16, 8192, 64, 128, "bf16", 0.99, False, 64, qk_unit_rows=True,
                         v_scale=1.0),
    "long_64k": Workload("long_64k", 1, 16, 65536, 128, 128, "bf16", 1.0, True, 128),
}
DECODE = DecodeWorkload("decode_256x32", 256, 32, 64, 64, 4096, 128, 1.0, True)


def make_qkv(w: Workload, B=None, H=None, n=None, seed=None):
    """q, k, v as CPU tensors [B, H, n, d|dv] of the workload's element type.

    B, H, n may be overridden to draw a smaller case with the same recipe."""
    B = w.B if B is None else B
    H = w.H if H is None else H
    n = w.n if n is None else n
    g = torch.Generator().manual_seed(w.seed if seed is None else seed)
    s = 1.0 / math.sqrt(w.d)
    q = torch.randn(B, H, n, w.d, generator=g, dtype=torch.float32) * s
    k = torch.randn(B, H, n, w.d, generator=g, dtype=torch.float32) * s
    v = torch.randn(B, H, n, w.dv, generator=g, dtype=torch.float32)
    v = v * (s if w.v_scale is None else w.v_scale)
    if w.qk_unit_rows:
        q = q / q.norm(dim=-1, keepdim=True)
        k = k / k.norm(dim=-1, keepdim=True)
    t = w.torch_dtype
    return q.to(t).contiguous(), k.to(t).contiguous(), v.to(t).contiguous()


def make_tokens(shape_qk, shape_v, d: int, seed: int, dtype=torch.bfloat16):
    """q, k ~ N(0,1)/sqrt(d) of shape_qk and v ~ N(0,1)/sqrt(d) of shape_v, rounded to dtype."""
    g = torch.Generator().manual_seed(seed)
    s = 1.0 / math.sqrt(d)
    q = torch.randn(*shape_qk, generator=g, dtype=torch.float32) * s
    k = torch.randn(*shape_qk, generator=g, dtype=torch.float32) * s
    v = torch.randn(*shape_v, generator=g, dtype=torch.float32) * s
    return q.to(dtype), k.to(dtype), v.to(dtype)


def decode_prefix_tokens(w: DecodeWorkload, seq: int, head: int, length: int | None = None):
    """Prefix q, k, v of one (sequence, head) as [length, d|dv] bf16 CPU tensors.

    Each head has its own seed so any subset of heads can be regenerated alone."""
    length = w.prefix if length is None else length
    seed = (w.seed * 1_000_003 + 1 + seq * w.H + head) & 0x7FFFFFFF
    return make_tokens((length, w.d), (length, w.dv), w.d, seed, w.torch_dtype)


def decode_step_tokens(w: DecodeWorkload, step: int, N=None, H=None):
    """Step `step` q, k, v for all heads as [N, H, d|dv] bf16 CPU tensors."""
    N = w.N if N is None else N
    H = w.H if H is None else H
    seed = (w.seed * 7_919 + 0x5EED + step) & 0x7FFFFFFF
    return make_tokens((N, H, w.d), (N, H, w.dv), w.d, seed, w.torch_dtype)


def sample_heads(B: int, H: int, count: int, seed: int = 1234):
    """A fixed spread of (b, h) pairs (first, last and seeded random ones)."""
    total = B * H
    picks = {0, total - 1}
    g = torch.Generator().manual_seed(seed)
    perm = torch.randperm(total, generator=g).tolist()
    for p in perm:
        if len(picks) >= min(count, total):
            break
        picks.add(p)
    return [(p // H, p % H) for p in sorted(picks)]
