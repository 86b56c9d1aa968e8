"""Seeded synthetic Q/K/V workloads (shared by the tests, the smoke check and
the benchmark; holds none of the attention method's arithmetic).

The pages measure only on video-generation models (Wan2.1/2.2 text-to-video
and image-to-video at 480p and 720p, HunyuanVideo, CogVideoX) whose weights and
activations are not available, so seeded Gaussian inputs with the models'
attention shapes stand in for them:

* ``video_1p3b_480p``: one 480p clip of a 1.3B video DiT, latent grid
  21 x 30 x 52 = 32760 tokens, 12 heads of 128 channels.
* ``video_14b_720p``: one 720p clip of a 14B video DiT, latent grid
  21 x 45 x 80 = 75600 tokens, 40 heads of 128 channels.
* ``tiny``: 2 heads, 1024 tokens: the case the CPU oracle finishes in seconds.
* ``causal_prefill``: an LLM-prefill-shaped causal case, 4 x 32 heads x 8192.
* ``outlier``: 2 x 24 heads x 17550 tokens of 64 channels with outlier key
  channels and outlier query tokens (stresses smoothing and scales).

Recipe (all draws in fp32 from one ``torch.Generator`` seeded with ``seed``,
then rounded to bf16): Q, V ~ N(0, 1); K ~ N(0, 1) + o[b, h, c] with a
per-(batch, head, channel) offset o ~ N(0, sigma^2) shared by all tokens
(sigma = 3, or 2 for the causal case).  Outlier case: Q, K, V ~ N(0, 1); per
(b, h) round(1% of d) = 1 channel of K gets o ~ N(0, 20^2), and
round(0.5% of N) query tokens are multiplied by 30 (chosen without replacement).
Optional ``q_sigma`` (any workload): Q also gets a per-(batch, head, channel)
offset ~ N(0, q_sigma^2) shared by all tokens, drawn after everything above
(the inputs that Q smoothing is for; without it nothing changes).

``output_grad`` gives a workload the upstream gradient of its attention
output for the backward pass: dO ~ N(0, 1) of the output's shape, bf16, from
its own generator seeded with the workload's seed + 500000.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import torch

# name -> (B, H, N, d, causal, offset_sigma, kind)
WORKLOADS = {
    "tiny": (1, 2, 1024, 128, False, 3.0, "offset"),
    "video_1p3b_480p": (1, 12, 32760, 128, False, 3.0, "offset"),
    "video_14b_720p": (1, 40, 75600, 128, False, 3.0, "offset"),
    "causal_prefill": (4, 32, 8192, 128, True, 2.0, "offset"),
    "outlier": (2, 24, 17550, 64, False, 20.0, "outlier"),
}
ORDER = ["tiny", "video_1p3b_480p", "video_14b_720p", "causal_prefill", "outlier"]


@dataclass
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    causal: bool
    sm_scale: float
    seed: int
    q: torch.Tensor  # bf16 [B, H, N, d]
    k: torch.Tensor
    v: torch.Tensor
    outlier_tokens: torch.Tensor | None = None  # int64 [B, H, n_out] (outlier case)


def default_seed(name: str) -> int:
    return 1000 + ORDER.index(name)


def make(name: str, seed: int | None = None, device="cpu", B=None, H=None, N=None,
         q_sigma: float | None = None) -> Workload:
    """Generate workload ``name`` (sizes may be overridden for reduced tests)."""
    B0, H0, N0, d, causal, sigma, kind = WORKLOADS[name]
    B = B0 if B is None else B
    H = H0 if H is None else H
    N = N0 if N is None else N
    seed = default_seed(name) if seed is None else seed
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    shape = (B, H, N, d)
    q = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    k = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    v = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    outl = None
    if kind == "offset":
        o = torch.randn((B, H, 1, d), generator=g, device=device, dtype=torch.float32) * sigma
        k += o
    else:
        n_ch = max(1, int(round(0.01 * d)))
        n_tok = max(1, int(round(0.005 * N)))
        # channel choice and token choice per (b, h), without replacement
        ch = torch.argsort(torch.rand((B, H, d), generator=g, device=device), dim=-1)[..., :n_ch]
        o = torch.randn((B, H, n_ch), generator=g, device=device, dtype=torch.float32) * sigma
        offs = torch.zeros((B, H, 1, d), device=device, dtype=torch.float32)
        offs.scatter_(-1, ch.unsqueeze(2), o.unsqueeze(2))
        k += offs
        outl = torch.argsort(torch.rand((B, H, N), generator=g, device=device), dim=-1)[..., :n_tok]
        scale = torch.ones((B, H, N), device=device, dtype=torch.float32)
        scale.scatter_(-1, outl, 30.0)
        q *= scale.unsqueeze(-1)
    if q_sigma is not None:
        q += torch.randn((B, H, 1, d), generator=g, device=device, dtype=torch.float32) * q_sigma
    return Workload(name=name, B=B, H=H, N=N, d=d, causal=causal, sm_scale=1.0 / math.sqrt(d),
                    seed=seed, q=q.to(torch.bfloat16), k=k.to(torch.bfloat16),
                    v=v.to(torch.bfloat16), outlier_tokens=outl)


def output_grad(wl: Workload, layout: str = "HND") -> torch.Tensor:
    """The upstream gradient dO ~ N(0, 1) of ``wl``'s output, bf16, [B, H, N, d]
    (HND) or [B, N, H, d] (NHD), on the device of ``wl.q``."""
    dev = wl.q.device
    g = torch.Generator(device=dev)
    g.manual_seed(wl.seed + 500000)
    do = torch.randn((wl.B, wl.H, wl.N, wl.d), generator=g, device=dev, dtype=torch.float32)
    do = do.to(torch.bfloat16)
    return do if layout == "HND" else do.permute(0, 2, 1, 3).contiguous()


def bf16_codes(t: torch.Tensor):
    """A bf16 tensor's bit patterns as a numpy uint16 array (on the CPU)."""
    return t.detach().to("cpu").contiguous().view(torch.int16).numpy().view("uint16")
