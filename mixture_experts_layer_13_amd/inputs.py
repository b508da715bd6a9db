"""Seeded synthetic inputs for the fused MoE layer.

This module only draws inputs; it holds none of the layer's arithmetic (no
routing, no alignment, no expert GEMM, no activation quantisation).  Both the
GPU path and the CPU oracle read the bytes it produces.

Workloads (the pages name no dataset and ship no weights; the "representative
MoE model" of the AWS post's introduction is unnamed, so these seeded tensors
stand in for it):

  tiny_fp32      T=16, H=256, I=512, E=8, top-2; fp32 x and weights ~N(0, 0.02^2),
                 logits ~N(0, 1).
  decode_bf16    T in {1, 8, 32, 64}, H=4096, I=1024, E=64, top-8; bf16 weights
                 ~N(0, 0.02^2), x ~N(0, 1), logits ~N(0, 1).
  decode_fp8     decode_bf16's shapes; weights stored as E4M3FN codes with one
                 fp32 scale per expert and matrix (amax / 448).
  large_fp8      T in {1, 16, 64, 256}, H=7168, I=2048, E=256, top-8, E4M3 weights;
                 logits carry a Zipf(s=1.1) popularity bias.
  prefill_bf16   T in {4096, 8192}, H=4096, I=1024, E=64, top-8, Zipf(1.1) logits.
  prefill_fp8    prefill_bf16 with E4M3 weights.

The topk=8 example and the aggregate N = k * I = 8192 come from the pages
(uniquestudio digest, "背景与事实"; AWS post, "Swap-AB for WGMMA utilization").

Seeds: seed = 1000 * workload_index + T; independent streams x = seed+1,
logits = seed+2, w13 = seed+3, w2 = seed+4.

FP8 weights are prepared here, once, as *inputs*: per expert and matrix the
scale is amax/448 and the codes come from torch's own float8_e4m3fn cast of
the clamped ratio.  The layer under test receives codes and scales.
"""
from dataclasses import dataclass, field
import math

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    index: int
    H: int
    I: int
    E: int
    topk: int
    tokens: tuple
    x_dtype: torch.dtype
    w_dtype: str  # "f32", "bf16" or "e4m3"
    out_dtype: torch.dtype
    zipf: float = 0.0  # 0 = uniform expert popularity
    x_std: float = 1.0
    w_std: float = 0.02
    renormalize: bool = True
    fp8_act: bool = False
    notes: str = field(default="", compare=False)


WORKLOADS = {
    "tiny_fp32": Workload("tiny_fp32", 0, 256, 512, 8, 2, (16,), torch.float32, "f32",
                          torch.float32, x_std=0.02),
    "decode_bf16": Workload("decode_bf16", 1, 4096, 1024, 64, 8, (1, 8, 32, 64),
                            torch.bfloat16, "bf16", torch.bfloat16),
    "decode_fp8": Workload("decode_fp8", 2, 4096, 1024, 64, 8, (1, 8, 32, 64),
                           torch.bfloat16, "e4m3", torch.bfloat16, fp8_act=True),
    "large_fp8": Workload("large_fp8", 3, 7168, 2048, 256, 8, (1, 16, 64, 256),
                          torch.bfloat16, "e4m3", torch.bfloat16, zipf=1.1, fp8_act=True),
    "prefill_bf16": Workload("prefill_bf16", 4, 4096, 1024, 64, 8, (4096, 8192),
                             torch.bfloat16, "bf16", torch.bfloat16, zipf=1.1),
    "prefill_fp8": Workload("prefill_fp8", 4, 4096, 1024, 64, 8, (4096, 8192),
                            torch.bfloat16, "e4m3", torch.bfloat16, zipf=1.1, fp8_act=True),
}


def seed_of(w: Workload, T: int) -> int:
    return 1000 * w.index + T


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def zipf_log_bias(E: int, s: float) -> torch.Tensor:
    """ln p_e with p_e proportional to (e+1)^-s, normalised (rank = id + 1)."""
    r = torch.arange(1, E + 1, dtype=torch.float64)
    p = r.pow(-s)
    p = p / p.sum()
    return p.log()


def make_logits(T, E, seed, zipf=0.0, device="cpu"):
    g = _gen(device, seed)
    l = torch.randn(T, E, generator=g, device=device, dtype=torch.float32)
    if zipf:
        l = l + zipf_log_bias(E, zipf).to(device=device, dtype=torch.float32)
    return l.contiguous()


def make_x(T, H, seed, dtype, std=1.0, device="cpu"):
    g = _gen(device, seed)
    x = torch.randn(T, H, generator=g, device=device, dtype=torch.float32) * std
    return x.to(dtype).contiguous()


def make_router(E, K, seed, dtype, device="cpu"):
    """Router weight [E, K] (hidden dimension contiguous), N(0, 1/K): logits
    of N(0,1) activations come out near N(0,1)."""
    g = _gen(device, seed)
    w = torch.randn(E, K, generator=g, device=device, dtype=torch.float32) / float(K) ** 0.5
    return w.to(dtype).contiguous()


def _e4m3_weights(E, R, C, seed, std, device):
    """Per expert: draw N(0, std^2) in fp32, scale = amax/448, codes by torch cast."""
    g = _gen(device, seed)
    q = torch.empty(E, R, C, dtype=torch.float8_e4m3fn, device=device)
    s = torch.empty(E, dtype=torch.float32, device=device)
    for e in range(E):
        w = torch.randn(R, C, generator=g, device=device, dtype=torch.float32) * std
        amax = w.abs().max()
        sc = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
        q[e] = (w / sc).clamp(-448.0, 448.0).to(torch.float8_e4m3fn)
        s[e] = sc
    return q, s


def make_weights(E, H, I, seed13, seed2, w_dtype, std=0.02, device="cpu"):
    """w13 [E, 2I, H] and w2 [E, H, I] (+ per-expert scales for E4M3)."""
    if w_dtype == "e4m3":
        w13, s13 = _e4m3_weights(E, 2 * I, H, seed13, std, device)
        w2, s2 = _e4m3_weights(E, H, I, seed2, std, device)
        return w13, w2, s13, s2
    dt = {"f32": torch.float32, "bf16": torch.bfloat16}[w_dtype]
    g13 = _gen(device, seed13)
    g2 = _gen(device, seed2)
    w13 = torch.empty(E, 2 * I, H, dtype=dt, device=device)
    w2 = torch.empty(E, H, I, dtype=dt, device=device)
    for e in range(E):
        w13[e] = (torch.randn(2 * I, H, generator=g13, device=device) * std).to(dt)
    for e in range(E):
        w2[e] = (torch.randn(H, I, generator=g2, device=device) * std).to(dt)
    return w13, w2, None, None


def make_inputs(w: Workload, T: int, device="cpu", seed=None, H=None, I=None, E=None,
                topk=None):
    """All tensors of one call.  Shape overrides (H, I, E, topk) keep the
    workload's distributions and dtypes; they serve small parity cases."""
    H = H or w.H
    I = I or w.I
    E = E or w.E
    k = topk or w.topk
    s = seed_of(w, T) if seed is None else seed
    x = make_x(T, H, s + 1, w.x_dtype, w.x_std, device)
    logits = make_logits(T, E, s + 2, w.zipf, device)
    w13, w2, s13, s2 = make_weights(E, H, I, s + 3, s + 4, w.w_dtype, w.w_std, device)
    return {"x": x, "logits": logits, "w13": w13, "w2": w2, "w13_scale": s13,
            "w2_scale": s2, "T": T, "H": H, "I": I, "E": E, "topk": k,
            "workload": w}


def to_numpy_bits(t: torch.Tensor):
    """Raw bytes of a tensor as numpy: f32 -> float32, bf16 -> uint16 bits,
    E4M3 -> uint8 codes.  (The oracle decodes the bits itself.)"""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.float32:
        return t.numpy()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view("uint16")
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).numpy()
    if t.dtype == torch.int32:
        return t.numpy()
    raise TypeError(t.dtype)


def uniform_active_experts(T, E, k):
    """Expected number of distinct experts hit by T tokens under uniform
    routing (for reporting only)."""
    return E * (1.0 - math.prod((E - 1 - j) / (E - j) for j in range(k)) ** T)
