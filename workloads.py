"""Seeded synthetic inputs for the NVFP4 fake-quantized attention QAT path.

This module only draws random tensors.  It holds none of the method's
arithmetic, so both the CPU oracle's tests and the GPU path's tests and
benchmark can take their inputs from here without sharing any computation.

Every workload is drawn on the CPU with ``torch.Generator('cpu')`` in fp32,
in the order Q, K, V, dO (each ``randn(B, H, N, D)``), then the workload's
modifier is applied and the result is cast to bf16 (round-to-nearest-even).
The shapes follow the workloads on the pages: the BHSD tensor contract of
"NVFP4 Attention QAT Backward" (cuDNN frontend docs, §Tensor contract), the
Wan-2.1 480p latent (21x30x52 = 32760 tokens, H=40, D=128) and LLM training
shapes of the Attn-QAT summary (§Results), which stand in for datasets and
trained weights that are not used here.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    heads: int
    seqlen: int
    head_dim: int
    causal: bool
    seed: int
    softmax_scale: float
    modifier: str  # "none" | "outlier_channels" | "channel_offset" | "token_lognormal"
    description: str

    @property
    def shape(self):
        return (self.batch, self.heads, self.seqlen, self.head_dim)

    def bwd_flops(self) -> float:
        """Counted backward work: 10*B*H*N^2*D, halved when causal."""
        f = 10.0 * self.batch * self.heads * self.seqlen ** 2 * self.head_dim
        return f / 2 if self.causal else f

    def fwd_flops(self) -> float:
        """Counted forward work: 4*B*H*N^2*D, halved when causal."""
        f = 4.0 * self.batch * self.heads * self.seqlen ** 2 * self.head_dim
        return f / 2 if self.causal else f


WORKLOADS = {
    "tiny": Workload("tiny", 1, 1, 128, 64, False, 0, 1.0 / 8.0, "none",
                     "tiny non-causal B1 H1 N128 D64"),
    "small_causal": Workload("small_causal", 1, 4, 1024, 64, True, 1, 1.0 / 8.0, "none",
                             "small causal B1 H4 N1024 D64"),
    "ref_shape": Workload("ref_shape", 1, 16, 4096, 128, False, 2, 1.0 / math.sqrt(128.0),
                          "outlier_channels",
                          "reference shape non-causal B1 H16 N4096 D128, 4 outlier channels x8 per head"),
    "llm_causal": Workload("llm_causal", 2, 40, 8192, 128, True, 3, 1.0 / math.sqrt(128.0),
                           "channel_offset",
                           "LLM-training-like causal B2 H40 N8192 D128, per-channel mean offsets on Q/K"),
    "video_dit": Workload("video_dit", 1, 40, 32760, 128, False, 4, 1.0 / math.sqrt(128.0),
                          "token_lognormal",
                          "video-DiT-like non-causal B1 H40 N32760 D128, per-token lognormal Q/K scale"),
}

ORDER = ["tiny", "small_causal", "ref_shape", "llm_causal", "video_dit"]


def make_inputs(w: Workload | str, seqlen: int | None = None, heads: int | None = None,
                batch: int | None = None):
    """Draw (q, k, v, do) as bf16 CPU tensors of shape (B, H, N, D).

    ``seqlen``/``heads``/``batch`` override the workload's sizes (same seed and
    recipe) for reduced-size test cases.
    """
    if isinstance(w, str):
        w = WORKLOADS[w]
    B = batch if batch is not None else w.batch
    H = heads if heads is not None else w.heads
    N = seqlen if seqlen is not None else w.seqlen
    D = w.head_dim
    g = torch.Generator("cpu").manual_seed(w.seed)
    q = torch.randn(B, H, N, D, generator=g)
    k = torch.randn(B, H, N, D, generator=g)
    v = torch.randn(B, H, N, D, generator=g)
    do = torch.randn(B, H, N, D, generator=g)
    if w.modifier == "outlier_channels":
        # The same 4 random head-dim channels of Q, K and V are scaled x8 in each head.
        for b in range(B):
            for h in range(H):
                ch = torch.randperm(D, generator=g)[:4]
                q[b, h, :, ch] *= 8.0
                k[b, h, :, ch] *= 8.0
                v[b, h, :, ch] *= 8.0
    elif w.modifier == "channel_offset":
        q += 0.5 * torch.randn(B, H, 1, D, generator=g)
        k += 0.5 * torch.randn(B, H, 1, D, generator=g)
    elif w.modifier == "token_lognormal":
        q *= torch.exp(0.3 * torch.randn(B, H, N, 1, generator=g))
        k *= torch.exp(0.3 * torch.randn(B, H, N, 1, generator=g))
    elif w.modifier != "none":
        raise ValueError(f"unknown modifier {w.modifier}")
    return (q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16),
            do.to(torch.bfloat16))


def random_bf16(shape, seed: int, scale: float = 1.0, dist: str = "normal"):
    """A seeded bf16 CPU tensor for codec tests (normal or log-uniform magnitudes)."""
    g = torch.Generator("cpu").manual_seed(seed)
    if dist == "normal":
        x = torch.randn(*shape, generator=g) * scale
    elif dist == "loguniform":
        mag = torch.exp2(torch.rand(*shape, generator=g) * 40.0 - 30.0)
        sign = torch.where(torch.rand(*shape, generator=g) < 0.5, -1.0, 1.0)
        x = mag * sign * scale
    else:
        raise ValueError(dist)
    return x.to(torch.bfloat16)


def random_f32(shape, seed: int, scale: float = 1.0):
    g = torch.Generator("cpu").manual_seed(seed)
    return torch.randn(*shape, generator=g) * scale
