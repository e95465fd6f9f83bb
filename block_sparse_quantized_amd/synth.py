"""Seeded synthetic attention inputs shaped like the pages' workloads.

This module holds none of the method's arithmetic: it only draws Q, K, V (and a
block mask for the custom-mask workload) from seeded torch generators.  It runs on
any torch device, so large inputs can be drawn directly in GPU memory; a given
(workload, seed, device) always yields the same tensors, and every head is drawn
from its own stream, so a workload cut to fewer heads reproduces the first heads
of the full one.

Workloads (the pages' model families, [chapterpal] method and results paragraphs;
[readme] "Supported models"):
  tiny      B=1 H=2  N=512    D=64  fp32; per 64-token block a shared N(0,1) mean plus
            N(0, 0.3^2) noise per token
  llm8k     B=1 H=32 N=8192   D=128 bf16; N(0,1) noise around a random-walk mean that
            steps by N(0, 0.05^2) per channel once per 64-token block (Llama-3.1-8B
            attention shape)
  llm128k   the llm8k recipe at N=131072 (Llama 3.1 at 128K context)
  video     B=2 H=30 N=17776  D=64  bf16; 226 N(0,1) text tokens, then a 13x30x45
            (t, y, x) grid of a Gaussian-smoothed (sigma 2 cells, reflect) white field,
            standardised per channel, plus 0.2*N(0,1) (CogVideoX-2b shape)
  image     B=1 H=24 N=4608   D=128 bf16; 512 N(0,1) text tokens, then a 64x64 smooth
            field (sigma 2, standardised, no noise); Bernoulli(0.3) block mask of
            shape (1, 24, 36, 72) with the two K blocks inside each Q block forced
            on (Flux shape)
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import Dict, Optional, Tuple

import torch
import torch.nn.functional as F

STREAM_Q, STREAM_K, STREAM_V, STREAM_MASK = 0, 1, 2, 3


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str
    B: int
    H: int
    N: int
    D: int
    dtype: torch.dtype
    seed: int
    causal: bool = False
    topk: float = 0.5
    filter_on: bool = True
    qk_int8: bool = False
    pv_fp16: bool = False
    pv_fp8: bool = False
    api: str = "topk"              # "topk" or "block_sparse"
    text: int = 0                  # text-token prefix length (visual workloads)
    grid: Tuple[int, ...] = ()     # visual grid shape after the prefix
    hilbert: bool = False
    mask_p: float = 0.3
    extra: Dict = field(default_factory=dict)


WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload("tiny", "blockmean", 1, 2, 512, 64, torch.float32, 0,
                     causal=False, topk=0.5, filter_on=False),
    "llm8k": Workload("llm8k", "drift", 1, 32, 8192, 128, torch.bfloat16, 1,
                      causal=True, topk=0.5, filter_on=True),
    "video": Workload("video", "video", 2, 30, 17776, 64, torch.bfloat16, 2,
                      causal=False, topk=0.3, filter_on=True, text=226, grid=(13, 30, 45),
                      hilbert=True),
    "image": Workload("image", "image", 1, 24, 4608, 128, torch.bfloat16, 3,
                      causal=False, filter_on=False, api="block_sparse", text=512,
                      grid=(64, 64), mask_p=0.3),
    "llm128k": Workload("llm128k", "drift", 1, 32, 131072, 128, torch.bfloat16, 4,
                        causal=True, topk=0.5, filter_on=True, qk_int8=True, pv_fp16=True),
}


def workload(name: str, **overrides) -> Workload:
    return replace(WORKLOADS[name], **overrides)


def _gen(seed: int, stream: int, b: int, h: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(((seed * 8 + stream) * 4096 + b) * 65536 + h + 1)
    return g


def _normal(shape, g, device) -> torch.Tensor:
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32)


def _gaussian_taps(sigma: float, device) -> torch.Tensor:
    r = int(math.ceil(4 * sigma))
    x = torch.arange(-r, r + 1, dtype=torch.float64, device=device)
    w = torch.exp(-0.5 * (x / sigma) ** 2)
    return (w / w.sum()).to(torch.float32)


def smooth_field(white: torch.Tensor, sigma: float) -> torch.Tensor:
    """Separable Gaussian smoothing over every axis but the first, reflect borders.

    ``white`` has shape (C, *grid); returns the same shape.  Each axis is one fixed
    sequence of elementwise products and sums over shifted copies (no convolution
    library call), so every device rounds it the same way.
    """
    taps = _gaussian_taps(sigma, white.device)
    r = (taps.numel() - 1) // 2
    out = white
    nd = out.dim() - 1
    for ax in range(1, nd + 1):
        moved = out.movedim(ax, -1)
        shp = moved.shape
        L = shp[-1]
        flat = moved.reshape(-1, 1, L)
        pad = min(r, L - 1)
        flat = F.pad(flat, (pad, pad), mode="reflect")
        if pad < r:
            flat = F.pad(flat, (r - pad, r - pad), mode="replicate")
        acc = taps[0] * flat[..., 0:L]
        for t in range(1, 2 * r + 1):
            acc = acc + taps[t] * flat[..., t:t + L]
        out = acc.reshape(shp).movedim(-1, ax)
    return out


def _standardise(x: torch.Tensor) -> torch.Tensor:
    # x: (C, cells); zero mean, unit variance per channel (statistics in fp64, so a
    # device's reduction order does not reach the fp32 result in practice)
    xd = x.double()
    mu = xd.mean(dim=1, keepdim=True)
    sd = xd.std(dim=1, unbiased=False, keepdim=True).clamp_min(1e-12)
    return ((xd - mu) / sd).float()


def _head(wl: Workload, stream: int, b: int, h: int, device) -> torch.Tensor:
    """One (N, D) float32 head of one tensor."""
    N, D = wl.N, wl.D
    g = _gen(wl.seed, stream, b, h, device)
    if wl.kind == "blockmean":
        nb = (N + 63) // 64
        mu = _normal((nb, D), g, device)
        eps = _normal((N, D), g, device)
        return mu.repeat_interleave(64, dim=0)[:N] + 0.3 * eps
    if wl.kind == "drift":
        nb = (N + 63) // 64
        steps = _normal((nb, D), g, device).double() * 0.05
        mu = torch.cumsum(steps, dim=0).float()
        eps = _normal((N, D), g, device)
        return mu.repeat_interleave(64, dim=0)[:N] + eps
    if wl.kind in ("video", "image"):
        cells = 1
        for s in wl.grid:
            cells *= s
        assert wl.text + cells == N, "text prefix + grid must equal N"
        text = _normal((wl.text, D), g, device)
        white = _normal((D,) + tuple(wl.grid), g, device)
        fld = _standardise(smooth_field(white, 2.0).reshape(D, cells)).t()
        if wl.kind == "video":
            fld = fld + 0.2 * _normal((cells, D), g, device)
        return torch.cat([text, fld], dim=0)
    raise ValueError(f"unknown workload kind {wl.kind}")


def make_qkv(wl: Workload, device="cpu") -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """(B, H, N, D) contiguous Q, K, V in the workload's dtype on ``device``."""
    out = []
    for stream in (STREAM_Q, STREAM_K, STREAM_V):
        t = torch.empty((wl.B, wl.H, wl.N, wl.D), dtype=wl.dtype, device=device)
        for b in range(wl.B):
            for h in range(wl.H):
                t[b, h] = _head(wl, stream, b, h, device).to(wl.dtype)
        out.append(t)
    return tuple(out)


def make_block_mask(wl: Workload, device="cpu") -> torch.Tensor:
    """(B, H, ceil(N/128), ceil(N/64)) uint8 0/1 mask: Bernoulli(mask_p), the K blocks
    lying inside each Q block's own token range forced to 1."""
    nQ, nK = (wl.N + 127) // 128, (wl.N + 63) // 64
    m = torch.empty((wl.B, wl.H, nQ, nK), dtype=torch.uint8, device=device)
    for b in range(wl.B):
        for h in range(wl.H):
            g = _gen(wl.seed, STREAM_MASK, b, h, device)
            u = torch.rand((nQ, nK), generator=g, device=device)
            mm = (u < wl.mask_p).to(torch.uint8)
            i = torch.arange(nQ, device=device)
            for jj in (2 * i, 2 * i + 1):
                ok = jj < nK
                mm[i[ok], jj[ok]] = 1
            m[b, h] = mm
    return m


def checksum(t: torch.Tensor) -> str:
    """Stable hex digest of a tensor's bytes (detects generator drift)."""
    import hashlib
    return hashlib.sha256(t.detach().cpu().contiguous().view(torch.uint8).numpy().tobytes()).hexdigest()[:16]


def fingerprint(t: torch.Tensor) -> list:
    """Three fp64 sums of a tensor, computed where it lives: of x, of x^2 and of
    x * cos(flat index).  A change of seed or recipe moves them far more than
    last-bit differences between devices do."""
    x = t.detach().double().reshape(-1)
    w = torch.cos(torch.arange(x.numel(), device=x.device, dtype=torch.float64))
    return [float(x.sum()), float((x * x).sum()), float((x * w).sum())]
