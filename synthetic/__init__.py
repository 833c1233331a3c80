"""Seeded synthetic KV-cache and query generators.

Shared by the tests, the benchmark and the CPU baseline.  This module holds
none of the quantizer's arithmetic: it only draws inputs.

The pages measure on LLaMA / Mistral layers with public text datasets that are
not available here.  These tensors stand in for them: they take those layers'
shapes (32 query heads, 8 KV heads, head_dim 128) and the per-channel structure
the workloads name -- N(0,1) noise times a per-channel lognormal(0, 0.5) scale
plus a per-channel offset (N(0, 2), i.e. variance 2, or Student-t(3)), with an
optional 1% of (head, channel) pairs scaled x10 as outliers.  Per-channel
parameters are per (KV head, channel), shared across batch and tokens; K and V
come from independent streams.
"""

from __future__ import annotations

import dataclasses

import numpy as np

__all__ = ["Workload", "WORKLOADS", "channel_params", "make_kv", "make_queries", "make_kv_numpy"]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    L: int
    d: int
    g: int            # sub-vector length: 8 -> 1 bit/elem, 4 -> 2 bit/elem
    kind: str         # channel model: "normal" | "outlier" | "student_t"
    dtype: str        # "f16" | "f32"
    ops: tuple        # which steps the workload exercises

    @property
    def bits(self) -> int:
        return 8 // self.g


WORKLOADS = {
    "single-head-fp32-1bit": Workload("single-head-fp32-1bit", 1, 1, 1, 256, 128, 8, "normal", "f32",
                                      ("encode", "dequantize", "attention")),
    "llama8b-layer-encode-2bit": Workload("llama8b-layer-encode-2bit", 1, 32, 8, 4096, 128, 4, "outlier", "f16",
                                          ("encode",)),
    "decode-2bit-b16-s32k": Workload("decode-2bit-b16-s32k", 16, 32, 8, 32768, 128, 4, "normal", "f16",
                                     ("encode", "attention")),
    "decode-step-1bit-b64-s8k": Workload("decode-step-1bit-b64-s8k", 64, 32, 8, 8192, 128, 8, "normal", "f16",
                                         ("encode", "step")),
    "mistral7b-long-2bit": Workload("mistral7b-long-2bit", 1, 32, 8, 131072, 128, 4, "student_t", "f16",
                                    ("encode", "attention")),
}


def channel_params(seed: int, H: int, d: int, kind: str):
    """Per-(head, channel) scale sigma and offset mu, plus the outlier factor."""
    rng = np.random.Generator(np.random.PCG64(seed))
    sigma = np.exp(0.5 * rng.standard_normal((H, d)))           # lognormal(0, 0.5)
    if kind == "student_t":
        z = rng.standard_normal((H, d))
        chi2 = rng.chisquare(3, size=(H, d))
        mu = z / np.sqrt(chi2 / 3.0)                               # Student-t(3)
    else:
        mu = np.sqrt(2.0) * rng.standard_normal((H, d))            # N(0, 2): variance 2
    factor = np.ones((H, d))
    if kind == "outlier":
        n_out = int(round(0.01 * H * d))
        pick = rng.choice(H * d, size=n_out, replace=False)
        factor.reshape(-1)[pick] = 10.0
    return sigma, mu, factor


def _stream_seed(seed: int, which: int) -> int:
    return (seed * 1_000_003 + which * 7919) & 0x7FFFFFFFFFFFFFFF


def make_kv(seed: int, B: int, H: int, L: int, d: int, kind: str, dtype: str = "f16", device="cpu"):
    """(K, V) torch tensors of shape (B, H, L, d), channel model ``kind``."""
    import torch

    tdt = torch.float16 if dtype == "f16" else torch.float32
    out = []
    for which in (0, 1):
        sigma, mu, factor = channel_params(_stream_seed(seed, 10 + which), H, d, kind)
        gen = torch.Generator(device=device)
        gen.manual_seed(_stream_seed(seed, which))
        x = torch.empty((B, H, L, d), dtype=tdt, device=device)
        sg = torch.tensor(sigma * factor, dtype=torch.float32, device=device)
        mg = torch.tensor(mu * factor, dtype=torch.float32, device=device)
        for b in range(B):
            for h in range(H):
                z = torch.randn((L, d), generator=gen, dtype=torch.float32, device=device)
                x[b, h] = (z * sg[h] + mg[h]).to(tdt)
        out.append(x)
    return out[0], out[1]


def make_kv_numpy(seed: int, B: int, H: int, L: int, d: int, kind: str, dtype: str = "f16"):
    """Same channel model as make_kv, drawn with NumPy (small CPU-only cases)."""
    npdt = np.float16 if dtype == "f16" else np.float32
    out = []
    for which in (0, 1):
        sigma, mu, factor = channel_params(_stream_seed(seed, 10 + which), H, d, kind)
        rng = np.random.Generator(np.random.PCG64(_stream_seed(seed, which)))
        z = rng.standard_normal((B, H, L, d))
        out.append((z * (sigma * factor)[None, :, None, :] + (mu * factor)[None, :, None, :]).astype(npdt))
    return out[0], out[1]


def make_queries(seed: int, B: int, Hq: int, d: int, device="cpu"):
    """Decode queries q ~ N(0, 1), fp16, shape (B, Hq, d)."""
    import torch

    gen = torch.Generator(device=device)
    gen.manual_seed(_stream_seed(seed, 99))
    return torch.randn((B, Hq, d), generator=gen, dtype=torch.float32, device=device).to(torch.float16)
