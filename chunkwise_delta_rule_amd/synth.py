"""Seeded synthetic inputs for the DeltaNet forward pass.

This module draws random tensors and nothing else: it holds none of the
method's arithmetic. Both the HIP path's tests/benchmark and the oracle's
tests take their inputs from here.

Distributions (the workloads of the pages: "Context Parallelism for DeltaNet"
section 3 uses T = 8192 with chunk 64; the 1.3B DeltaNet of "Parallelizing
Linear Transformers with the Delta Rule over Sequence Length" has hidden
size 2048 = 16 heads x 128):

* q, k ~ N(0, 1) per element, then L2-normalised per (token, head) over the
  key dimension in fp32, then rounded to the input dtype (round to nearest
  even). The rounded values are what every consumer receives; nobody
  renormalises them.
* v ~ N(0, 1), rounded to the input dtype.
* beta = sigmoid(N(0, 1)) in fp32, rounded to the input dtype.
* S0: zero, or N(0, std) in fp32 when requested.
* g (Gated DeltaNet, log decay per token and head, always fp32):
  g = log sigmoid(x), x ~ N(mu, 1) with mu = 2 by default, so a = exp(g)
  has mean about 0.85 and a chunk of 64 tokens decays by about e^-10 end to
  end; drawn from its own generator seeded with ``seed + 104729``.
* varlen lengths: integers uniform on the inclusive range [lo, hi].

Draw order: varlen lengths come from a CPU ``torch.Generator`` seeded with
``seed``; then q, k, v, beta logits and S0 come, in that order, from one
generator on the target device seeded with ``seed`` (a varlen S0 uses its own
generator seeded with ``seed + 7919``). The same seed on another device gives
other numbers; parity tests therefore draw once and hand the same tensors to
both sides.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import torch

DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16}


@dataclass(frozen=True)
class Workload:
    """One synthetic workload. ``N``/``len_lo``/``len_hi`` are set for varlen."""

    name: str
    B: int
    H: int
    T: int
    dk: int
    dv: int
    chunk: int = 64
    dtype: str = "bf16"
    s0_std: float = 0.0
    N: int = 0
    len_lo: int = 0
    len_hi: int = 0
    extra: dict = field(default_factory=dict)

    @property
    def varlen(self) -> bool:
        return self.N > 0


# The five workloads: a tiny fp32 correctness case, the paper-scale layer
# (the throughput workload), the 128-chunk case of the context-parallel
# example, the long-context case and the packed varlen batch.
WORKLOADS = {
    "tiny_f32": Workload("tiny_f32", B=1, H=1, T=256, dk=64, dv=64, dtype="f32"),
    "layer_b8_h16_t4096": Workload("layer_b8_h16_t4096", B=8, H=16, T=4096, dk=128, dv=128),
    "chunks128_b4_h16_t8192": Workload("chunks128_b4_h16_t8192", B=4, H=16, T=8192, dk=128,
                                       dv=128, s0_std=0.02),
    "long_b1_h16_t131072": Workload("long_b1_h16_t131072", B=1, H=16, T=131072, dk=128, dv=128),
    "varlen_n64_h32": Workload("varlen_n64_h32", B=1, H=32, T=0, dk=128, dv=128, N=64,
                               len_lo=512, len_hi=32768),
}


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def draw_lengths(N: int, lo: int, hi: int, seed: int) -> list[int]:
    """Sequence lengths, uniform integers on [lo, hi] (drawn on the CPU)."""
    g = _gen("cpu", seed)
    return torch.randint(lo, hi + 1, (N,), generator=g).tolist()


def make_inputs(B: int, H: int, T: int, dk: int, dv: int, dtype: str = "bf16", seed: int = 0,
                device: str = "cpu", s0_std: float = 0.0, zero_s0_as_none: bool = True,
                gen: torch.Generator | None = None):
    """Dense inputs q, k [B,T,H,dk], v [B,T,H,dv], beta [B,T,H], S0 [B,H,dv,dk] or None."""
    dt = DTYPES[dtype]
    g = gen if gen is not None else _gen(device, seed)

    def unit_rows(d):
        x = torch.randn((B, T, H, d), generator=g, device=device, dtype=torch.float32)
        x = x / x.norm(dim=-1, keepdim=True).clamp_min(1e-30)
        return x.to(dt)

    q = unit_rows(dk)
    k = unit_rows(dk)
    v = torch.randn((B, T, H, dv), generator=g, device=device, dtype=torch.float32).to(dt)
    beta = torch.sigmoid(torch.randn((B, T, H), generator=g, device=device,
                                     dtype=torch.float32)).to(dt)
    if s0_std > 0:
        S0 = torch.randn((B, H, dv, dk), generator=g, device=device,
                         dtype=torch.float32) * s0_std
    elif zero_s0_as_none:
        S0 = None
    else:
        S0 = torch.zeros((B, H, dv, dk), device=device, dtype=torch.float32)
    return q, k, v, beta, S0


def make_gates(shape, seed: int = 0, device: str = "cpu", mu: float = 2.0):
    """Log decays g = log sigmoid(N(mu, 1)), fp32, of the given shape ([B,T,H] or [T,H])."""
    g = _gen(device, seed + 104729)
    x = torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32) + mu
    return torch.nn.functional.logsigmoid(x)


def make_channel_gates(shape, seed: int = 0, device: str = "cpu", mu: float = 2.0):
    """Per-channel log decays for KDA, g = log sigmoid(N(mu, 1)) per element,
    fp32, shape [B, T, H, dk]; own generator seeded with ``seed + 130363``."""
    g = _gen(device, seed + 130363)
    x = torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32) + mu
    return torch.nn.functional.logsigmoid(x)


def make_varlen_inputs(lengths, H: int, dk: int, dv: int, dtype: str = "bf16", seed: int = 0,
                       device: str = "cpu", s0_std: float = 0.0):
    """Packed inputs for sequences of the given lengths.

    Returns q, k [T,H,dk], v [T,H,dv], beta [T,H], cu_seqlens int32 [N+1],
    S0 [N,H,dv,dk] or None, with T = sum(lengths).
    """
    lengths = [int(x) for x in lengths]
    T = sum(lengths)
    q, k, v, beta, _ = make_inputs(1, H, T, dk, dv, dtype=dtype, seed=seed, device=device)
    cu = torch.zeros(len(lengths) + 1, dtype=torch.int32)
    cu[1:] = torch.cumsum(torch.tensor(lengths, dtype=torch.int64), 0).to(torch.int32)
    S0 = None
    if s0_std > 0:
        g = _gen(device, seed + 7919)
        S0 = torch.randn((len(lengths), H, dv, dk), generator=g, device=device,
                         dtype=torch.float32) * s0_std
    return q[0], k[0], v[0], beta[0], cu.to(device), S0


def workload_inputs(w: Workload, seed: int = 0, device: str = "cpu"):
    """Inputs of a named workload (dense: 5-tuple; varlen: 6-tuple + lengths)."""
    if w.varlen:
        lengths = draw_lengths(w.N, w.len_lo, w.len_hi, seed)
        return make_varlen_inputs(lengths, w.H, w.dk, w.dv, dtype=w.dtype, seed=seed,
                                  device=device, s0_std=w.s0_std) + (lengths,)
    return make_inputs(w.B, w.H, w.T, w.dk, w.dv, dtype=w.dtype, seed=seed, device=device,
                       s0_std=w.s0_std)
