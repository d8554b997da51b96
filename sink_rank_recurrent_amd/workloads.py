"""Seeded synthetic decode workloads for the shallow-state engine.

This module only draws random inputs; it holds none of the method's
arithmetic.  Both the CPU oracle's tests and the HIP path's tests and
benchmark take their inputs from here, so the two sides always see the same
values (bf16 inputs are drawn in fp32 and rounded once; consumers upcast the
stored bf16 values exactly).

The shapes follow the heads the SEED pages describe: 128x128 Gated DeltaNet
and Kimi Delta Attention heads, Mamba-2 heads in the d_k = d_B = 128,
d_v = d_x = 64 orientation (SEED figures and tables, thelatestinai.com,
Table 17 note), rank R = 16 (Fig. 7 caption), fp32 recurrent states
(Table 2 caption).  No trace, checkpoint or dataset from the pages is used:
every value is drawn here.

Distributions per (request, head, step):
  * k, q ~ N(0, I), then divided by their L2 norm;
  * v = vbar + 0.3 * N(0, I), with vbar ~ N(0, I) fixed per (layer, head);
  * Gated DeltaNet: alpha ~ U(0.9, 0.999), beta ~ U(0, 1);
  * Kimi Delta Attention: alpha_i ~ U(0.95, 0.9999) per key channel,
    beta ~ U(0, 1);
  * Mamba-2: alpha = exp(-softplus(z) * 0.1), z ~ N(0, 1); no beta.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import torch

GDN, KDA, MAMBA2 = "gdn", "kda", "mamba2"
RULES = (GDN, KDA, MAMBA2)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    rule: str
    batch: int            # resident requests
    heads: int            # heads per layer
    layers: int           # recurrent layers (each is its own launch)
    d_k: int
    d_v: int
    R: int
    W: int
    steps: int            # decode steps
    prefill: int          # dense prefill steps before the conversion
    in_dtype: torch.dtype  # q, k, v storage type
    seed: int

    @property
    def cap(self) -> int:
        return self.R + self.W

    @property
    def heads_per_launch(self) -> int:
        return self.batch * self.heads


# The five workloads.  Prefill length 512 for every workload (the first one
# states it; the others inherit it).
WORKLOADS = {
    1: Workload("gdn_1x1_r16w16_f32", GDN, 1, 1, 1, 128, 128, 16, 16, 256, 512,
                torch.float32, 1001),
    2: Workload("gdn_64x16_r16w32_bf16", GDN, 64, 16, 1, 128, 128, 16, 32, 1024, 512,
                torch.bfloat16, 1002),
    3: Workload("mamba2_128x64_r16w32_bf16", MAMBA2, 128, 64, 1, 128, 64, 16, 32, 2048, 512,
                torch.bfloat16, 1003),
    4: Workload("kda_64x32_r16w64_bf16", KDA, 64, 32, 1, 128, 128, 16, 64, 4096, 512,
                torch.bfloat16, 1004),
    5: Workload("gdn_36Lx32x256_r16w32_bf16", GDN, 256, 32, 36, 128, 128, 16, 32, 16384, 512,
                torch.bfloat16, 1005),
}


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _mix(*parts: int) -> int:
    """Deterministic 63-bit seed from integer parts (splitmix-style)."""
    x = 0x9E3779B97F4A7C15
    for p in parts:
        x ^= (int(p) + 0x9E3779B97F4A7C15 + ((x << 6) & 0xFFFFFFFFFFFFFFFF) + (x >> 2))
        x &= 0xFFFFFFFFFFFFFFFF
        x = (x * 0xBF58476D1CE4E5B9) & 0xFFFFFFFFFFFFFFFF
        x ^= x >> 31
    return x & 0x7FFFFFFFFFFFFFFF


def make_vbar(heads: int, d_v: int, seed: int, layer: int = 0,
              device="cpu") -> torch.Tensor:
    """Per-head fixed direction vbar ~ N(0, I), fp32, shape [heads, d_v]."""
    g = _gen(device, _mix(seed, 0xBA5, layer))
    return torch.randn(heads, d_v, generator=g, device=device, dtype=torch.float32)


def make_step(rule: str, batch: int, heads: int, d_k: int, d_v: int,
              vbar: torch.Tensor, seed: int, t: int, layer: int = 0,
              in_dtype: torch.dtype = torch.float32, device="cpu") -> dict:
    """Inputs of decode step t (negative t: prefill) for one layer.

    Returns q, k [batch, heads, d_k] and v [batch, heads, d_v] in `in_dtype`;
    g [batch, heads] (Kimi Delta Attention: [batch, heads, d_k]) and beta
    [batch, heads] in fp32 (beta is None for Mamba-2).
    """
    if rule not in RULES:
        raise ValueError(f"unknown rule {rule!r}")
    gen = _gen(device, _mix(seed, 0x57E9, layer, t + (1 << 40)))
    f32 = torch.float32
    k = torch.randn(batch, heads, d_k, generator=gen, device=device, dtype=f32)
    q = torch.randn(batch, heads, d_k, generator=gen, device=device, dtype=f32)
    k = k / torch.linalg.vector_norm(k, dim=-1, keepdim=True)
    q = q / torch.linalg.vector_norm(q, dim=-1, keepdim=True)
    v = vbar.to(device=device, dtype=f32).unsqueeze(0) + 0.3 * torch.randn(
        batch, heads, d_v, generator=gen, device=device, dtype=f32)
    beta: Optional[torch.Tensor]
    if rule == GDN:
        g = 0.9 + 0.099 * torch.rand(batch, heads, generator=gen, device=device, dtype=f32)
        beta = torch.rand(batch, heads, generator=gen, device=device, dtype=f32)
    elif rule == KDA:
        g = 0.95 + 0.0499 * torch.rand(batch, heads, d_k, generator=gen, device=device, dtype=f32)
        beta = torch.rand(batch, heads, generator=gen, device=device, dtype=f32)
    else:
        z = torch.randn(batch, heads, generator=gen, device=device, dtype=f32)
        g = torch.exp(-torch.nn.functional.softplus(z) * 0.1)
        beta = None
    return {"q": q.to(in_dtype).contiguous(), "k": k.to(in_dtype).contiguous(),
            "v": v.to(in_dtype).contiguous(), "g": g.contiguous(),
            "beta": None if beta is None else beta.contiguous()}


def workload_step(w: Workload, vbar: torch.Tensor, t: int, layer: int = 0,
                  device="cpu", batch: Optional[int] = None) -> dict:
    """Inputs of step t of workload `w` (optionally only the first `batch` requests)."""
    return make_step(w.rule, w.batch if batch is None else batch, w.heads, w.d_k, w.d_v,
                     vbar, w.seed, t, layer, w.in_dtype, device)


def to_f64(x: Optional[torch.Tensor]):
    """Exact upcast of a stored input (fp32 or bf16) to a float64 numpy array."""
    if x is None:
        return None
    return x.detach().to("cpu", torch.float64).numpy()
