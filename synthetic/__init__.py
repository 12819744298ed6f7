"""Seeded synthetic inputs for frame-windowed sparse attention.

This module is shared by the CPU oracle (``oracle/``) and the HIP path's tests
and benchmark. It holds workload shapes and random draws only: nothing here
computes any part of the attention method (no mask, no plan, no norms, no
softmax). Both sides receive the very same bf16 tensors from ``make_inputs``.

Workloads (the SR transformer's frame-windowed self-attention of the HeyGen /
Google Cloud Avatar IV article, section on removing the mask): every query
frame attends a window of neighbouring frames plus one global reference frame,
over tens of thousands of tokens. The article prints no tensor shape; the five
shapes below are synthetic stand-ins for its production SR activations, which
are not available:

* ``tiny``          1 x 2 heads x 400 tokens (5 frames x 80), D=64, window +-1
* ``sr720``         1 x 8 x 25,200 (21 x 1200, a 30x40 latent), D=128, +-1
* ``sr1080``        1 x 8 x 46,800 (13 x 3600, a 45x80 latent), D=128, +-2
* ``bound_stress``  the ``sr720`` shape with heavy-tailed q/k row norms
* ``dense``         1 x 8 x 16,800 (14 x 1200), D=128, window covers all frames
* ``key_offset``    the ``sr720`` shape with a large offset shared by all keys
                    of a head (the "common component" that key centring removes,
                    article section on freeing the softmax)

All use reference frame 0 and scale 1/sqrt(D) rounded to fp32.
"""
from __future__ import annotations

import dataclasses
import math

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    heads: int
    head_dim: int
    frames: int
    tokens_per_frame: int
    window: int
    ref_frame: int
    dist: str = "normal"          # "normal" or "bound_stress"
    seed: int = 0

    @property
    def seq_len(self) -> int:
        return self.frames * self.tokens_per_frame

    @property
    def scale(self) -> float:
        """1/sqrt(D) rounded to fp32 (the value both sides receive)."""
        return float(torch.tensor(1.0 / math.sqrt(self.head_dim), dtype=torch.float32))

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    "tiny": Workload("tiny", 1, 2, 64, 5, 80, 1, 0),
    "sr720": Workload("sr720", 1, 8, 128, 21, 1200, 1, 0),
    "sr1080": Workload("sr1080", 1, 8, 128, 13, 3600, 2, 0),
    "bound_stress": Workload("bound_stress", 1, 8, 128, 21, 1200, 1, 0, dist="bound_stress"),
    "dense": Workload("dense", 1, 8, 128, 14, 1200, 13, 0),
    "key_offset": Workload("key_offset", 1, 8, 128, 21, 1200, 1, 0, dist="key_offset"),
}

# Heavy-tailed inputs for ``bound_stress``: q and k rows are multiplied by
# exp(sigma * z), z ~ N(0, 1) per row (a log-normal norm with mu = 0), then a
# fixed fraction of key rows per head is multiplied by a constant.
STRESS_SIGMA = 1.0
STRESS_KEY_FRACTION = 0.05
STRESS_KEY_FACTOR = 8.0

# ``key_offset``: per (b, h) one direction u ~ N(0, I_D), scaled to this length,
# is added to every key row of the head.
KEY_OFFSET_NORM = 40.0


def make_inputs(wl: Workload, device: str = "cpu"):
    """Draw q, k, v as bf16 [B, H, N, D] tensors, seeded and deterministic.

    One ``torch.Generator('cpu')`` seeded with ``wl.seed`` draws q, k, v (in
    that order) as fp32 N(0, 1), which are then rounded to bf16 (RNE). For
    ``bound_stress`` the same generator continues after v with the q row
    factors, the k row factors, and per (b, h) one ``randperm`` whose first
    round(0.05 N) entries pick the key rows that are scaled x8; the rounding to
    bf16 happens after all scaling. For ``key_offset`` the generator continues
    after v with one offset direction per (b, h), added to that head's keys
    before the rounding.
    """
    g = torch.Generator("cpu").manual_seed(wl.seed)
    shape = (wl.batch, wl.heads, wl.seq_len, wl.head_dim)
    q = torch.randn(shape, generator=g, dtype=torch.float32)
    k = torch.randn(shape, generator=g, dtype=torch.float32)
    v = torch.randn(shape, generator=g, dtype=torch.float32)
    if wl.dist == "bound_stress":
        zq = torch.randn(shape[:3], generator=g, dtype=torch.float32)
        zk = torch.randn(shape[:3], generator=g, dtype=torch.float32)
        q *= torch.exp(STRESS_SIGMA * zq).unsqueeze(-1)
        k *= torch.exp(STRESS_SIGMA * zk).unsqueeze(-1)
        n_big = int(round(STRESS_KEY_FRACTION * wl.seq_len))
        for b in range(wl.batch):
            for h in range(wl.heads):
                idx = torch.randperm(wl.seq_len, generator=g)[:n_big]
                k[b, h, idx] *= STRESS_KEY_FACTOR
    elif wl.dist == "key_offset":
        u = torch.randn((wl.batch, wl.heads, 1, wl.head_dim), generator=g, dtype=torch.float32)
        k += u * (KEY_OFFSET_NORM / u.norm(dim=-1, keepdim=True))
    elif wl.dist != "normal":
        raise ValueError(f"unknown distribution {wl.dist!r}")
    out = [t.to(torch.bfloat16) for t in (q, k, v)]
    if device != "cpu":
        out = [t.to(device) for t in out]
    return tuple(out)


def make_device_normal(shape, seed: int, device: str):
    """q, k, v as bf16 N(0, 1) tensors of ``shape``, drawn on ``device`` by one
    ``torch.Generator(device)`` seeded with ``seed`` (q, k, v in that order),
    for shapes too large to draw on the host. Deterministic for a given device
    type and seed; the tests hand the oracle host copies of the slices it needs."""
    g = torch.Generator(device).manual_seed(seed)
    return tuple(torch.randn(shape, generator=g, dtype=torch.float32, device=device).to(torch.bfloat16)
                 for _ in range(3))


# Inputs of the fused pre-attention chain (article section "Bố cục là ABI"):
# token activations x [B, N, C], a per-channel norm gain and the q/k/v
# projection weight [3 H D, C]. The article gives no model width; C = H D.
@dataclasses.dataclass(frozen=True)
class PreWorkload:
    name: str
    batch: int
    seq_len: int
    channels: int
    heads: int
    head_dim: int
    seed: int = 0


PRE_WORKLOADS = {
    "pre_tiny": PreWorkload("pre_tiny", 1, 400, 128, 2, 64),
    "pre720": PreWorkload("pre720", 1, 25200, 1024, 8, 128),
}


def make_pre_inputs(wl: PreWorkload):
    """x ~ N(0, 1) as bf16 [B, N, C]; gain = 1 + 0.1 N(0, 1) as fp32 [C];
    w ~ N(0, 1/C) as bf16 [3 H D, C] (so the projections have unit variance).
    One ``torch.Generator('cpu')`` seeded with ``wl.seed`` draws x, gain, w in
    that order."""
    g = torch.Generator("cpu").manual_seed(wl.seed)
    x = torch.randn((wl.batch, wl.seq_len, wl.channels), generator=g, dtype=torch.float32)
    gain = 1.0 + 0.1 * torch.randn((wl.channels,), generator=g, dtype=torch.float32)
    w = torch.randn((3 * wl.heads * wl.head_dim, wl.channels), generator=g, dtype=torch.float32)
    w /= math.sqrt(wl.channels)
    return x.to(torch.bfloat16), gain, w.to(torch.bfloat16)


def to_f64(t: torch.Tensor):
    """Exact fp64 numpy copy of a bf16 tensor (every bf16 value is an fp64 value)."""
    return t.detach().to("cpu").to(torch.float64).numpy()


def sample_rows(wl: Workload, count: int, seed: int = 1):
    """Seeded sample of (b, h, i) query rows, always including the first and
    last row of frame 0, of the reference frame and of the last frame."""
    g = torch.Generator("cpu").manual_seed(seed)
    n = wl.seq_len
    b = torch.randint(0, wl.batch, (count,), generator=g)
    h = torch.randint(0, wl.heads, (count,), generator=g)
    i = torch.randint(0, n, (count,), generator=g)
    fixed = [0, wl.tokens_per_frame - 1, n - wl.tokens_per_frame, n - 1,
             wl.ref_frame * wl.tokens_per_frame]
    rows = {(int(b[j]), int(h[j]), int(i[j])) for j in range(count)}
    for t in fixed:
        rows.add((0, 0, t))
        rows.add((wl.batch - 1, wl.heads - 1, t))
    return sorted(rows)
