"""Seeded synthetic inputs for the gated delta rule workloads.

This module only draws random inputs; it holds none of the recurrence's
arithmetic.  The tests feed the same tensors to the HIP library and to the
fp64 oracle, and the benchmark uses it to build its batches.

Shapes follow the Qwen3.5-9B Gated DeltaNet layer (Qwen3.5-9B architecture
page, section Gated DeltaNet): 16 query/key heads, 32 value heads, head
dimension 128.  Laws:
  * q, k: standard Gaussians, L2-normalised per token and head in fp32, then
    rounded once to the io dtype;
  * v: standard Gaussian (the workloads do not fix it; the tiny fp32 one uses
    N(0,1) and that law is kept for all);
  * beta = sigmoid(N(0,1)), fp32;
  * g (log of the forget gate, always <= 0):
      "softplus": -softplus(N(1,1))                  (tiny fp32 workload)
      "uniform":  -U(0.5, 7.0)                        (Qwen3.5-9B workloads)
      "weak":     -U(0, 0.02)                         (long-memory stress, tests only)
    With `strong_segment`, tokens 64..127 of sequence 0, value head 0 are set
    to exactly -6.72, the per-step decay of the fp32 overflow regression on
    the Candle pull-request page (section Chunked GatedDeltaNet Scan);
  * initial state: N(0, std^2) fp32 when `s0_std` is given, else none (zero).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import torch

STRONG_DECAY = -6.72


@dataclass
class Workload:
    name: str
    lengths: List[int]
    hqk: int
    hv: int
    dk: int
    dv: int
    chunk: int
    io_dtype: torch.dtype
    g_law: str
    s0_std: Optional[float]
    seed: int
    strong_segment: bool = False
    decode: bool = False
    verify_tokens: int = 0          # verify block length per sequence (varlen workload)
    notes: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def total_tokens(self) -> int:
        return int(sum(self.lengths))


def varlen_lengths(seed: int, n: int = 16, lo: int = 256, hi: int = 8192) -> List[int]:
    gen = torch.Generator().manual_seed(seed)
    return [int(x) for x in torch.randint(lo, hi + 1, (n,), generator=gen)]


def workload(name: str) -> Workload:
    """The five workloads: tiny fp32, 9B prefill, decode batch, long prefill, varlen."""
    if name == "tiny_fp32":
        return Workload(name, [64], 2, 4, 32, 32, 16, torch.float32, "softplus", None, 1000)
    if name == "prefill_1k":
        return Workload(name, [1024], 16, 32, 128, 128, 64, torch.bfloat16, "uniform", None, 1001,
                        strong_segment=True)
    if name == "decode_64":
        return Workload(name, [1] * 64, 16, 32, 128, 128, 64, torch.bfloat16, "uniform", 0.05, 1002,
                        decode=True)
    if name == "prefill_32k":
        return Workload(name, [32768], 16, 32, 128, 128, 64, torch.bfloat16, "uniform", 0.05, 1003,
                        strong_segment=True)
    if name == "varlen_16":
        return Workload(name, varlen_lengths(1004), 16, 32, 128, 128, 64, torch.bfloat16, "uniform",
                        0.05, 1004, strong_segment=True, verify_tokens=16)
    raise KeyError(name)


WORKLOADS = ("tiny_fp32", "prefill_1k", "decode_64", "prefill_32k", "varlen_16")


def _unit_gaussian(gen, shape):
    x = torch.randn(*shape, generator=gen, dtype=torch.float32)
    return x / x.norm(dim=-1, keepdim=True).clamp_min(1e-12)


def draw_g(gen, shape, law: str) -> torch.Tensor:
    if law == "softplus":
        return -torch.nn.functional.softplus(torch.randn(*shape, generator=gen) + 1.0)
    if law == "uniform":
        return -(0.5 + 6.5 * torch.rand(*shape, generator=gen))
    if law == "weak":
        return -(0.02 * torch.rand(*shape, generator=gen))
    if law == "zero":
        return torch.zeros(*shape)
    raise KeyError(law)


def correlated_unit_keys(gen, T, hqk, dk, noise=0.1):
    """Highly correlated keys: per query/key head one shared random direction plus
    N(0, noise^2 / dk) per component, L2-normalised per token (cosine between two keys of
    a head about 1 / (1 + noise^2))."""
    shared = _unit_gaussian(gen, (1, hqk, dk))
    k = shared + noise * torch.randn(T, hqk, dk, generator=gen) / float(dk) ** 0.5
    return k / k.norm(dim=-1, keepdim=True).clamp_min(1e-12)


def make_inputs(lengths, hqk, hv, dk, dv, io_dtype=torch.bfloat16, seed=0, g_law="uniform",
                s0_std=None, strong_segment=False, key_law="gaussian"):
    """Draw one packed batch on the CPU.

    key_law "gaussian" draws the keys like the queries; "correlated" draws highly
    correlated keys (correlated_unit_keys).

    Returns a dict with q, k [T, HQK, dk] and v [T, HV, dv] in io_dtype;
    g, beta [T, HV] fp32; cu_seqlens [N+1] int32; initial_state
    [N, HV, dk, dv] fp32 or None.
    """
    gen = torch.Generator().manual_seed(int(seed))
    lengths = [int(x) for x in lengths]
    T = sum(lengths)
    n = len(lengths)
    q = _unit_gaussian(gen, (T, hqk, dk)).to(io_dtype)
    if key_law == "correlated":
        k = correlated_unit_keys(gen, T, hqk, dk).to(io_dtype)
    elif key_law == "gaussian":
        k = _unit_gaussian(gen, (T, hqk, dk)).to(io_dtype)
    else:
        raise KeyError(key_law)
    v = torch.randn(T, hv, dv, generator=gen).to(io_dtype)
    beta = torch.sigmoid(torch.randn(T, hv, generator=gen)).float()
    g = draw_g(gen, (T, hv), g_law).float()
    if strong_segment and lengths and lengths[0] >= 128:
        g[64:128, 0] = STRONG_DECAY
    cu = torch.zeros(n + 1, dtype=torch.int32)
    if n:
        cu[1:] = torch.cumsum(torch.tensor(lengths, dtype=torch.int64), 0).to(torch.int32)
    s0 = None
    if s0_std is not None:
        s0 = (torch.randn(n, hv, dk, dv, generator=gen) * float(s0_std)).float()
    return dict(q=q.contiguous(), k=k.contiguous(), v=v.contiguous(), g=g.contiguous(),
                beta=beta.contiguous(), cu_seqlens=cu, initial_state=s0)


def make_workload_inputs(w: Workload, seed_offset: int = 0, lengths=None):
    return make_inputs(lengths if lengths is not None else w.lengths, w.hqk, w.hv, w.dk, w.dv,
                       w.io_dtype, w.seed + seed_offset, w.g_law, w.s0_std, w.strong_segment)


def accept_counts(seed: int, n: int, block: int = 16) -> List[int]:
    """Accepted prefix length per sequence after a verify block: U{1..block-1}."""
    gen = torch.Generator().manual_seed(int(seed))
    return [int(x) for x in torch.randint(1, block, (n,), generator=gen)]


def make_norm_inputs(tokens, hv, dv, io_dtype=torch.bfloat16, seed=0):
    """Inputs of the gated RMSNorm after the DeltaNet output, drawn on the CPU.

    o [tokens, HV, dv] in io_dtype: N(0, 1) rows scaled per value head by an RMS drawn
    log-uniformly in [1e-3, 2e-2] (the per-head output RMS range the NPU page reports,
    section "How it works"); z [tokens, HV, dv] in io_dtype: N(0, 2^2); weight [dv] fp32:
    U(0.5, 1.5).
    """
    gen = torch.Generator().manual_seed(int(seed))
    rms = torch.exp(torch.empty(hv).uniform_(float(torch.log(torch.tensor(1e-3))),
                                             float(torch.log(torch.tensor(2e-2))), generator=gen))
    o = (torch.randn(tokens, hv, dv, generator=gen) * rms[None, :, None]).to(io_dtype)
    z = (2.0 * torch.randn(tokens, hv, dv, generator=gen)).to(io_dtype)
    w = torch.empty(dv).uniform_(0.5, 1.5, generator=gen).float()
    return dict(o=o.contiguous(), z=z.contiguous(), weight=w.contiguous())


def make_conv_inputs(lengths, hqk, hv, dk, dv, width=4, io_dtype=torch.bfloat16, seed=0, with_state=True):
    """Inputs of the depthwise causal conv ahead of the recurrence, drawn on the CPU.

    x [T, 2 HQK dk + HV dv] in io_dtype: N(0, 1) (the packed q, k, v projections);
    weight [C, width] fp32: N(0, 1 / width); cu_seqlens [N+1] int32; state [N, C, width-1]
    fp32 holding earlier inputs (N(0, 1) rounded to io_dtype, as a conv state holds past x),
    or None.
    """
    gen = torch.Generator().manual_seed(int(seed))
    lengths = [int(x) for x in lengths]
    T = sum(lengths)
    C = 2 * hqk * dk + hv * dv
    x = torch.randn(T, C, generator=gen).to(io_dtype)
    w = (torch.randn(C, width, generator=gen) / float(width) ** 0.5).float()
    cu = torch.zeros(len(lengths) + 1, dtype=torch.int32)
    if lengths:
        cu[1:] = torch.cumsum(torch.tensor(lengths, dtype=torch.int64), 0).to(torch.int32)
    state = None
    if with_state:
        state = torch.randn(len(lengths), C, width - 1, generator=gen).to(io_dtype).float()
    return dict(x=x.contiguous(), weight=w.contiguous(), cu_seqlens=cu, state=state)
