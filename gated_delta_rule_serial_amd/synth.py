"""Seeded synthetic workloads for the gated delta-rule recurrence.

This module only draws random numbers and lays them out; it holds none of the
recurrence's or the gate prologue's arithmetic.  The test suite feeds the same
tensors to the oracle and to the HIP library; the benchmark uses it for its
inputs.

Recipe (one ``torch.Generator`` on the CPU per workload, seed 1234 + index,
values drawn in float32 in this order):
  1. sequence lengths (packed workload only): ``randint(lo, hi + 1, (N,))``
  2. q, k ~ N(0, 1), each (token, head) row divided by its L2 norm
  3. v ~ N(0, 1)
  4. b ~ N(0, 1)                 (beta = sigmoid(b))
  5. a ~ N(0, 1)                 (log-decay g = -exp(A_log) softplus(a + dt_bias))
  6. A_log ~ U(0, 1)  [h_v]
  7. dt_bias ~ U(-1, 1)  [h_v]
  8. initial state ~ N(0, 0.05^2)  [N, h_v, d_k, d_v]  (when the workload has one)
Then q, k, v, a, b are cast to the I/O dtype (round to nearest even for
bfloat16); A_log, dt_bias and the state stay float32.  The key normalisation
is a data-preparation step: the recurrence itself never normalises.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional

import torch


@dataclasses.dataclass(frozen=True)
class Shape:
    """Geometry of one workload."""
    name: str
    kind: str               # "prefill" or "decode"
    io_dtype: torch.dtype   # torch.float32 or torch.bfloat16
    h_qk: int
    h_v: int
    d_k: int
    d_v: int
    gate_mode: str          # "precomputed" (g, beta given) or "raw" (a, b, A_log, dt_bias)
    num_seqs: int
    seqlen: Optional[int]   # fixed length per sequence, or None for drawn lengths
    len_range: Optional[tuple] = None  # (lo, hi) inclusive, drawn lengths
    init_state: bool = False
    seed_index: int = 0


# The five workloads, in order.
WORKLOADS: List[Shape] = [
    Shape("tiny_prefill", "prefill", torch.float32, 2, 2, 16, 16, "precomputed",
          num_seqs=1, seqlen=64, seed_index=0),
    Shape("decode_b64", "decode", torch.bfloat16, 16, 32, 128, 128, "precomputed",
          num_seqs=64, seqlen=1, init_state=True, seed_index=1),
    Shape("prefill_t4096_fused_gates", "prefill", torch.bfloat16, 16, 32, 128, 128, "raw",
          num_seqs=1, seqlen=4096, seed_index=2),
    Shape("varlen_prefill_8seq", "prefill", torch.bfloat16, 16, 32, 128, 128, "precomputed",
          num_seqs=8, seqlen=None, len_range=(512, 8192), init_state=True, seed_index=3),
    Shape("wide_prefill_t32768_d256", "prefill", torch.float32, 8, 8, 256, 256, "precomputed",
          num_seqs=1, seqlen=32768, seed_index=4),
]

BY_NAME = {w.name: w for w in WORKLOADS}


@dataclasses.dataclass
class Inputs:
    shape: Shape
    seqlens: List[int]
    cu_seqlens: torch.Tensor     # int32 [N+1]
    q: torch.Tensor              # [T, h_qk, d_k] io dtype
    k: torch.Tensor              # [T, h_qk, d_k] io dtype
    v: torch.Tensor              # [T, h_v, d_v] io dtype
    a: torch.Tensor              # [T, h_v] io dtype
    b: torch.Tensor              # [T, h_v] io dtype
    A_log: torch.Tensor          # [h_v] float32
    dt_bias: torch.Tensor        # [h_v] float32
    initial_state: Optional[torch.Tensor]  # [N, h_v, d_k, d_v] float32

    @property
    def total_tokens(self) -> int:
        return int(self.cu_seqlens[-1])


def _unit_rows(x: torch.Tensor) -> torch.Tensor:
    return x / torch.linalg.vector_norm(x, dim=-1, keepdim=True)


def generate(shape: Shape, *, seqlen: Optional[int] = None, num_seqs: Optional[int] = None,
             seqlens: Optional[List[int]] = None, seed: Optional[int] = None) -> Inputs:
    """Draw a workload's inputs on the CPU.

    ``seqlen`` / ``num_seqs`` / ``seqlens`` shrink or override the geometry
    (for parity cases the oracle finishes in seconds); ``seed`` overrides
    1234 + index.
    """
    gen = torch.Generator(device="cpu")
    gen.manual_seed(1234 + shape.seed_index if seed is None else seed)
    n = shape.num_seqs if num_seqs is None else num_seqs
    if seqlens is not None:
        lens = [int(x) for x in seqlens]
        n = len(lens)
    elif shape.seqlen is None and seqlen is None:
        lo, hi = shape.len_range
        lens = torch.randint(lo, hi + 1, (n,), generator=gen).tolist()
    else:
        lens = [shape.seqlen if seqlen is None else seqlen] * n
    T = sum(lens)
    cu = torch.zeros(n + 1, dtype=torch.int32)
    if n:
        cu[1:] = torch.cumsum(torch.tensor(lens, dtype=torch.int64), 0).to(torch.int32)

    f32 = torch.float32
    q = _unit_rows(torch.randn(T, shape.h_qk, shape.d_k, generator=gen, dtype=f32))
    k = _unit_rows(torch.randn(T, shape.h_qk, shape.d_k, generator=gen, dtype=f32))
    v = torch.randn(T, shape.h_v, shape.d_v, generator=gen, dtype=f32)
    b = torch.randn(T, shape.h_v, generator=gen, dtype=f32)
    a = torch.randn(T, shape.h_v, generator=gen, dtype=f32)
    A_log = torch.rand(shape.h_v, generator=gen, dtype=f32)
    dt_bias = torch.rand(shape.h_v, generator=gen, dtype=f32) * 2.0 - 1.0
    s0 = None
    if shape.init_state:
        s0 = torch.randn(n, shape.h_v, shape.d_k, shape.d_v, generator=gen, dtype=f32) * 0.05
    dt = shape.io_dtype
    return Inputs(shape, lens, cu, q.to(dt), k.to(dt), v.to(dt), a.to(dt), b.to(dt),
                  A_log, dt_bias, s0)


@dataclasses.dataclass
class VariantGates:
    a_key: torch.Tensor        # [T, h_v, d_k] raw per-key-dim decay input
    A_log_key: torch.Tensor    # [h_v, d_k] float32
    dt_bias_key: torch.Tensor  # [h_v, d_k] float32
    b_shared: torch.Tensor     # [T] raw write-strength input shared by the heads


def variant_gates(T: int, h_v: int, d_k: int, *, seed: int, io_dtype: torch.dtype) -> VariantGates:
    """Raw gate inputs for the per-key-dim decay and shared-beta layouts, drawn
    like the per-head ones: a, b ~ N(0, 1), A_log ~ U(0, 1), dt_bias ~ U(-1, 1)."""
    gen = torch.Generator(device="cpu")
    gen.manual_seed(seed)
    f32 = torch.float32
    a = torch.randn(T, h_v, d_k, generator=gen, dtype=f32)
    A_log = torch.rand(h_v, d_k, generator=gen, dtype=f32)
    dt_bias = torch.rand(h_v, d_k, generator=gen, dtype=f32) * 2.0 - 1.0
    b = torch.randn(T, generator=gen, dtype=f32)
    return VariantGates(a.to(io_dtype), A_log, dt_bias, b.to(io_dtype))


# ---------------------------------------------------------------- the block's neighbouring ops
@dataclasses.dataclass(frozen=True)
class ConvShape:
    """Causal depthwise conv in front of the recurrence: channels = the q, k
    and v projections side by side (2 h_qk d_k + h_v d_v)."""
    name: str
    io_dtype: torch.dtype
    channels: int
    kernel_size: int
    dilation: int
    num_seqs: int
    seqlen: Optional[int]                 # tokens per sequence, or None for drawn lengths
    len_range: Optional[tuple] = None
    init_state: bool = True
    bias: bool = True
    seed_index: int = 10


@dataclasses.dataclass(frozen=True)
class NormShape:
    """Gated RMSNorm after the recurrence: rows = tokens, width = h_v d_v,
    one group per value head."""
    name: str
    io_dtype: torch.dtype
    rows: int
    width: int
    group: int
    seed_index: int = 20


# The decode and packed-prefill geometry of the recurrence (h_qk 16, h_v 32,
# d 128), with the block's usual width-4 convolution.
CONV_WORKLOADS: List[ConvShape] = [
    ConvShape("conv_step_b64", torch.bfloat16, 8192, 4, 1, num_seqs=64, seqlen=1, seed_index=10),
    # seed index 3: the lengths are the packed recurrence workload's (drawn first)
    ConvShape("conv_varlen_8seq", torch.bfloat16, 8192, 4, 1, num_seqs=8, seqlen=None, len_range=(512, 8192),
              seed_index=3),
]
NORM_WORKLOADS: List[NormShape] = [
    NormShape("gated_rmsnorm_t33173", torch.bfloat16, 33173, 32 * 128, 128, seed_index=20),
]
CONV_BY_NAME = {w.name: w for w in CONV_WORKLOADS}
NORM_BY_NAME = {w.name: w for w in NORM_WORKLOADS}


@dataclasses.dataclass
class ConvInputs:
    shape: ConvShape
    seqlens: List[int]
    cu_seqlens: torch.Tensor               # int32 [N+1]
    x: torch.Tensor                        # [T, C] io dtype
    weight: torch.Tensor                   # [C, K] io dtype
    bias: Optional[torch.Tensor]           # [C] io dtype
    initial_state: Optional[torch.Tensor]  # [N, carry, C] io dtype


def generate_conv(shape: ConvShape, *, seqlens: Optional[List[int]] = None, seed: Optional[int] = None) -> ConvInputs:
    """Draw the conv inputs on the CPU (seed 1234 + index), in float32, in this
    order: lengths (drawn workloads), x ~ N(0, 1) [T, C], weight ~ U(-1, 1) / sqrt(K)
    [C, K], bias ~ N(0, 0.1^2) [C], initial state ~ N(0, 1) [N, carry, C]; then
    every tensor is cast to the I/O dtype."""
    gen = torch.Generator(device="cpu")
    gen.manual_seed(1234 + shape.seed_index if seed is None else seed)
    if seqlens is not None:
        lens = [int(v) for v in seqlens]
    elif shape.seqlen is None:
        lo, hi = shape.len_range
        lens = torch.randint(lo, hi + 1, (shape.num_seqs,), generator=gen).tolist()
    else:
        lens = [shape.seqlen] * shape.num_seqs
    n, T, C, K = len(lens), sum(lens), shape.channels, shape.kernel_size
    cu = torch.zeros(n + 1, dtype=torch.int32)
    if n:
        cu[1:] = torch.cumsum(torch.tensor(lens, dtype=torch.int64), 0).to(torch.int32)
    f32 = torch.float32
    x = torch.randn(T, C, generator=gen, dtype=f32)
    w = (torch.rand(C, K, generator=gen, dtype=f32) * 2.0 - 1.0) / K ** 0.5
    b = torch.randn(C, generator=gen, dtype=f32) * 0.1
    carry = (K - 1) * shape.dilation
    s0 = torch.randn(n, carry, C, generator=gen, dtype=f32) if shape.init_state else None
    dt = shape.io_dtype
    return ConvInputs(shape, lens, cu, x.to(dt), w.to(dt), b.to(dt) if shape.bias else None,
                      None if s0 is None else s0.to(dt))


@dataclasses.dataclass
class NormInputs:
    shape: NormShape
    x: torch.Tensor       # [rows, width] io dtype
    gate: torch.Tensor    # [rows, width] io dtype
    scale: torch.Tensor   # [group] io dtype


def generate_norm(shape: NormShape, *, rows: Optional[int] = None, seed: Optional[int] = None) -> NormInputs:
    """Draw the norm inputs on the CPU (seed 1234 + index), in float32: x ~ N(0, 1),
    gate ~ N(0, 2^2) [rows, width], scale ~ N(1, 0.1^2) [group]; cast to the I/O dtype."""
    gen = torch.Generator(device="cpu")
    gen.manual_seed(1234 + shape.seed_index if seed is None else seed)
    r = shape.rows if rows is None else rows
    f32 = torch.float32
    x = torch.randn(r, shape.width, generator=gen, dtype=f32)
    gate = torch.randn(r, shape.width, generator=gen, dtype=f32) * 2.0
    scale = 1.0 + 0.1 * torch.randn(shape.group, generator=gen, dtype=f32)
    dt = shape.io_dtype
    return NormInputs(shape, x.to(dt), gate.to(dt), scale.to(dt))


# ---------------------------------------------------------------- inputs outside the workloads' domain
def rescale_rows(x: torch.Tensor, lo: float, hi: float, *, seed: int) -> torch.Tensor:
    """Multiply each last-axis row of x by its own factor ~ U(lo, hi) (one
    seeded draw per row, in float32), then cast back to x's dtype: applied to
    L2-normalised keys it gives keys with norms spread over [lo, hi]."""
    gen = torch.Generator(device="cpu")
    gen.manual_seed(seed)
    f = lo + (hi - lo) * torch.rand(x.shape[:-1] + (1,), generator=gen, dtype=torch.float32)
    return (x.float() * f).to(x.dtype)


def positive_log_decays(g: torch.Tensor, every: int, hi: float, *, seed: int) -> torch.Tensor:
    """A copy of the log-decays g [T, h_v] in which every `every`-th (token,
    head) entry (flattened order) is replaced by a draw ~ U(0, hi]: gates that
    grow the state instead of decaying it, which the gate prologue never gives
    but precomputed gates may carry."""
    gen = torch.Generator(device="cpu")
    gen.manual_seed(seed)
    flat = g.float().flatten().clone()
    idx = torch.arange(0, flat.numel(), every)
    flat[idx] = hi * (1.0 - torch.rand(idx.numel(), generator=gen, dtype=torch.float32))
    return flat.reshape(g.shape).to(g.dtype)


def output_norm_inputs(T: int, h_v: int, d_v: int, *, seed: int, io_dtype: torch.dtype):
    """Gate [T, h_v, d_v] ~ N(0, 2^2) and scale [d_v] ~ N(1, 0.1^2) of the
    recurrence's output norm (the gated RMSNorm workload's recipe), in float32
    then cast to the I/O dtype."""
    gen = torch.Generator(device="cpu")
    gen.manual_seed(seed)
    gate = torch.randn(T, h_v, d_v, generator=gen, dtype=torch.float32) * 2.0
    scale = 1.0 + 0.1 * torch.randn(d_v, generator=gen, dtype=torch.float32)
    return gate.to(io_dtype), scale.to(io_dtype)
