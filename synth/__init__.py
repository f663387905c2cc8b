"""Seeded synthetic KV-cache tensors for the HQMQ workloads.

This module only draws inputs.  It holds none of the codec's arithmetic and
is the one piece of code that both the HIP path (through the tests and the
benchmark) and the CPU oracle (through the tests) consume: a tensor drawn
here is handed to the library on the device and, read back byte for byte,
to the oracle on the host.

The workloads have the KV shapes of the models the pages evaluate (five
open models; the Llama-3-70B 128k-context cache is the pages' storage
example).  Real activations are not available, so every value is drawn from
a seeded distribution with the structure the pages describe: per-channel
scale spread, a few outlier channels per head whose chunk norms reach tens
of times the median, and rare token spikes (the outlier-heavy GQA models,
gist.science/nl/paper/2605.27646, "Technische Samenvatting",
"Probleemstelling" and Methodology 3).

Values are clamped to +-65504 and rounded to fp16 (fp32 for workload 1).
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace

import torch


@dataclass(frozen=True)
class Workload:
    wid: int
    name: str
    layers: int
    heads: int
    tokens: int            # tokens per (layer, head) slice
    head_dim: int
    dtype: str             # "f16" or "f32"
    S: int
    med_batch_tokens: int  # 0 = Med3x off
    roles: tuple           # 0 = K, 1 = V
    dist: str
    sequences: int = 1     # decode-step workload: sequences stacked along tokens
    append_tokens: int = 0  # decode-step workload: new tokens per step per (layer, head)
    med_C: float = 3.0
    data_seed: int = 0
    codebook_seed: int = 0
    notes: str = field(default="", compare=False)

    @property
    def chunks_per_role(self) -> int:
        return self.layers * self.heads * self.tokens * (self.head_dim // 4)

    @property
    def torch_dtype(self):
        return torch.float16 if self.dtype == "f16" else torch.float32

    def scaled(self, **kw) -> "Workload":
        """Same distribution at another shape (tests use small shapes)."""
        return replace(self, **kw)


WORKLOADS = {
    1: Workload(1, "single-head-k-fp32", 1, 1, 4096, 128, "f32", 8, 0, (0,),
                "normal", data_seed=1001,
                notes="K only, i.i.d. N(0,1), fp32"),
    2: Workload(2, "mistral7b-kv-32k", 32, 8, 32768, 128, "f16", 8, 0, (0, 1),
                "lognormal-channels", data_seed=1002,
                notes="N(0, sigma_c^2), sigma_c ~ lognormal(0, 0.5) per channel"),
    3: Workload(3, "qwen-outlier-kv-32k", 28, 4, 32768, 128, "f16", 32, 4096, (0, 1),
                "qwen-outliers", data_seed=1003,
                notes="N(0,1); 2% channels x U(20,100); 0.01% token spikes x50"),
    4: Workload(4, "llama3-70b-kv-128k", 80, 8, 131072, 128, "f16", 32, 4096, (0, 1),
                "llama70b", data_seed=1004,
                notes="K: lognormal channels + 1% channels x30; V: N(0,1)"),
    5: Workload(5, "llama3-8b-decode-32x32k", 32, 8, 32 * 32768, 128, "f16", 32, 4096,
                (0, 1), "outlier-channel", sequences=32, append_tokens=32,
                data_seed=1005,
                notes="N(0,1) + 1% channels x30; 32 sequences stacked on tokens"),
}


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _layer_seed(w: Workload, role: int, layer: int, salt: int = 0) -> int:
    return (w.data_seed * 1_000_003 + role * 10_007 + layer * 101 + salt) & 0x7FFFFFFFFFFFFFFF


def generate_layer(w: Workload, role: int, layer: int, device, tokens: int | None = None,
                   token_offset_seed: int = 0) -> torch.Tensor:
    """One layer [heads, tokens, head_dim] of workload ``w`` for ``role``."""
    T = w.tokens if tokens is None else tokens
    H, D = w.heads, w.head_dim
    g = _gen(_layer_seed(w, role, layer, token_offset_seed), device)
    x = torch.randn((H, T, D), generator=g, device=device, dtype=torch.float32)
    # per-(layer, head, role) structure is drawn from a second stream so that
    # it does not depend on the token count
    gs = _gen(_layer_seed(w, role, layer, 7_777_777), device)
    if w.dist == "normal":
        pass
    elif w.dist == "lognormal-channels" or (w.dist == "llama70b" and role == 0):
        sigma = torch.exp(0.5 * torch.randn((H, 1, D), generator=gs, device=device))
        x.mul_(sigma)
        if w.dist == "llama70b":
            n_out = max(1, round(0.01 * D))
            _scale_channels(x, n_out, 30.0, 30.0, gs)
    elif w.dist == "llama70b":  # V of the 70B cache
        pass
    elif w.dist == "qwen-outliers":
        n_out = max(1, round(0.02 * D))
        _scale_channels(x, n_out, 20.0, 100.0, gs)
        spikes = torch.rand((H, T, 1), generator=g, device=device) < 1e-4
        x.mul_(torch.where(spikes, 50.0, 1.0))
    elif w.dist == "outlier-channel":
        n_out = max(1, round(0.01 * D))
        _scale_channels(x, n_out, 30.0, 30.0, gs)
    else:
        raise ValueError(f"unknown distribution {w.dist}")
    x.clamp_(-65504.0, 65504.0)
    return x.to(w.torch_dtype)


def _scale_channels(x: torch.Tensor, n: int, lo: float, hi: float, g: torch.Generator):
    H, _, D = x.shape
    for h in range(H):
        ch = torch.randperm(D, generator=g, device=x.device)[:n]
        f = lo + (hi - lo) * torch.rand((n,), generator=g, device=x.device)
        x[h, :, ch] *= f


def generate(w: Workload, role: int, device, out: torch.Tensor | None = None,
             tokens: int | None = None) -> torch.Tensor:
    """Whole tensor [layers, heads, tokens, head_dim] (written into ``out``
    when given, one layer at a time so that fp32 staging stays small)."""
    T = w.tokens if tokens is None else tokens
    if out is None:
        out = torch.empty((w.layers, w.heads, T, w.head_dim), dtype=w.torch_dtype,
                          device=device)
    for l in range(w.layers):
        out[l].copy_(generate_layer(w, role, l, device, tokens=T))
    return out


def generate_append(w: Workload, role: int, step: int, device) -> torch.Tensor:
    """New tokens of one decode step: [layers, heads, append_tokens, head_dim]
    (one new token per sequence, the sequences stacked on the token axis)."""
    T = w.append_tokens
    out = torch.empty((w.layers, w.heads, T, w.head_dim), dtype=w.torch_dtype, device=device)
    for l in range(w.layers):
        out[l].copy_(generate_layer(w, role, l, device, tokens=T,
                                    token_offset_seed=1 + step))
    return out


def fp16_bytes(w: Workload) -> int:
    """Size of the uncompressed cache at 2 bytes per element, all roles."""
    return w.layers * w.heads * w.tokens * w.head_dim * 2 * len(w.roles)


def describe(w: Workload) -> str:
    return (f"{w.name}: [{w.layers}, {w.heads}, {w.tokens}, {w.head_dim}] {w.dtype}, "
            f"S={w.S}, Med3x B={w.med_batch_tokens}, roles={w.roles}; {w.notes}")


__all__ = ["Workload", "WORKLOADS", "generate", "generate_layer", "generate_append",
           "fp16_bytes", "describe"]
