"""Seeded synthetic inputs for the routed-MoE layer (router -> align -> up -> down -> finalize).

This module is plumbing shared by the tests, the benchmark and the smoke check.  It
holds the layer workloads and the generators that fill their tensors; it holds
none of the layer's arithmetic.  Both the HIP path and the CPU oracle receive the
tensors produced here, so neither side ever sees inputs that the other made.

Workloads (the routed-MoE layer of an LLM decode/prefill step; hidden 7168, top_k 16
is the shape of the Kimi-K3 finalize on the FlashInfer MNNVL page, section 1-2, and
the AlphaMoE page names the GLM m8 / m128 / m512 / m2048 route workloads, sections 2-6):

  tiny           M=4,    H=256,  E=8,   k=2,  I=512,  block=16, no router bias
  decode_m8      M=8,    H=7168, E=256, k=16, I=2048, block=16, no router bias
  batch_m128     M=128,  H=7168, E=256, k=16, I=2048, block=64, no router bias
  batch_m512     M=512,  same layer, block=64, Zipf(1.0)-shaped router bias
  prefill_m2048  M=2048, same layer, block=64, Zipf(1.0)-shaped router bias
  prefill_m8192  M=8192, same layer, block=64, Zipf(1.0)-shaped router bias (a parity
                 case past the timed sizes: 131,072 flat ids)
  skew_m512      M=512,  same layer, block=64, the bias with s = 50 (a parity case: the
                 first dozen experts take every token, most experts none)

Value recipe (every tensor has its own seed so that any one of them, or any single
expert's weights, can be regenerated on its own):
  x, residual ~ N(0, 1) rounded to bf16
  router weight, W13[e], W2[e] ~ N(0, 0.02^2) rounded to bf16
  norm weight g = bf16(1 + 0.05 * N(0, 1))
  Zipf-shaped bias b[e] = -0.9 * s * ln(e + 1) with s = 1.0 (fp32): hot experts have
  low ids.  Exact Zipf popularity cannot be reached because an expert is picked at
  most once per token; this bias gives a log-log slope of about -1 in sorted counts.
  eps = 1e-5 (the RMS_EPS constant of the FlashInfer H7168/K16 benchmark driver).

bf16 tensors travel as torch.bfloat16; `bf16_bits` turns one into the uint16 bit
patterns that the oracle decodes by itself.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch

__all__ = [
    "LayerConfig", "CONFIGS", "make_layer", "LazyExperts", "bf16_bits",
    "SEED_X", "SEED_ROUTER", "SEED_RESIDUAL", "SEED_NORM", "SEED_W13", "SEED_W2",
]

SEED_X = 1
SEED_ROUTER = 2
SEED_RESIDUAL = 3
SEED_NORM = 4
SEED_W13 = 10_000   # + expert id
SEED_W2 = 20_000    # + expert id


@dataclasses.dataclass(frozen=True)
class LayerConfig:
    name: str
    M: int
    H: int
    E: int
    top_k: int
    I: int
    block: int
    zipf_s: Optional[float] = None   # None: no router bias ("uniform routing")
    eps: float = 1e-5
    w_std: float = 0.02

    def describe(self) -> dict:
        d = dataclasses.asdict(self)
        d["routing"] = "uniform" if self.zipf_s is None else f"zipf({self.zipf_s})"
        return d


CONFIGS = {
    "tiny": LayerConfig("tiny", M=4, H=256, E=8, top_k=2, I=512, block=16),
    "decode_m8": LayerConfig("decode_m8", M=8, H=7168, E=256, top_k=16, I=2048, block=16),
    "batch_m128": LayerConfig("batch_m128", M=128, H=7168, E=256, top_k=16, I=2048, block=64),
    "batch_m512": LayerConfig("batch_m512", M=512, H=7168, E=256, top_k=16, I=2048, block=64,
                              zipf_s=1.0),
    "prefill_m2048": LayerConfig("prefill_m2048", M=2048, H=7168, E=256, top_k=16, I=2048,
                                 block=64, zipf_s=1.0),
    "prefill_m8192": LayerConfig("prefill_m8192", M=8192, H=7168, E=256, top_k=16, I=2048,
                                 block=64, zipf_s=1.0),
    "skew_m512": LayerConfig("skew_m512", M=512, H=7168, E=256, top_k=16, I=2048, block=64,
                             zipf_s=50.0),
}


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _normal_bf16(shape, std: float, mean: float, device, seed: int) -> torch.Tensor:
    g = _gen(device, seed)
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    if mean != 0.0:
        t.add_(mean)
    return t.to(torch.bfloat16)


def zipf_bias(E: int, s: float) -> torch.Tensor:
    """Router bias b[e] = -0.9 * s * ln(e + 1), fp32 (workload recipe, see module doc)."""
    return torch.tensor([-0.9 * s * math.log(e + 1.0) for e in range(E)], dtype=torch.float32)


def expert_w13(cfg: LayerConfig, e: int, device="cpu", seed: int = 0) -> torch.Tensor:
    """W13[e] as [2I, H] bf16 (rows [0, I) gate, rows [I, 2I) up)."""
    return _normal_bf16((2 * cfg.I, cfg.H), cfg.w_std, 0.0, device, seed + SEED_W13 + e)


def expert_w2(cfg: LayerConfig, e: int, device="cpu", seed: int = 0) -> torch.Tensor:
    """W2[e] as [H, I] bf16."""
    return _normal_bf16((cfg.H, cfg.I), cfg.w_std, 0.0, device, seed + SEED_W2 + e)


class LazyExperts:
    """Indexable stand-in for a stacked expert weight: item e is generated on demand.

    Used where the full [E, ...] stack would not fit in host memory (the CPU timing
    sample); item e equals what `make_layer` puts at index e on the same device.
    """

    def __init__(self, cfg: LayerConfig, kind: str, device="cpu", seed: int = 0, as_bits=True):
        assert kind in ("w13", "w2")
        self.cfg, self.kind, self.device, self.seed, self.as_bits = cfg, kind, device, seed, as_bits

    def __len__(self):
        return self.cfg.E

    def __getitem__(self, e):
        fn = expert_w13 if self.kind == "w13" else expert_w2
        t = fn(self.cfg, int(e), self.device, self.seed)
        return bf16_bits(t) if self.as_bits else t


def make_layer(cfg: LayerConfig, device="cpu", seed: int = 0, with_experts: bool = True,
               M: Optional[int] = None) -> dict:
    """All tensors of one layer invocation, on `device`.

    Keys: x [M,H], router_w [E,H], router_bias [E] fp32 or None, w13 [E,2I,H], w2 [E,H,I],
    residual [M,H], norm_w [H] (bf16 unless noted), eps (float), cfg.
    `M` overrides the token count (same layer, fewer or more tokens).
    """
    M = cfg.M if M is None else int(M)
    out = {
        "cfg": cfg,
        "M": M,
        "x": _normal_bf16((M, cfg.H), 1.0, 0.0, device, seed + SEED_X),
        "router_w": _normal_bf16((cfg.E, cfg.H), cfg.w_std, 0.0, device, seed + SEED_ROUTER),
        "router_bias": None if cfg.zipf_s is None else zipf_bias(cfg.E, cfg.zipf_s).to(device),
        "residual": _normal_bf16((M, cfg.H), 1.0, 0.0, device, seed + SEED_RESIDUAL),
        "norm_w": _normal_bf16((cfg.H,), 0.05, 1.0, device, seed + SEED_NORM),
        "eps": float(cfg.eps),
    }
    if with_experts:
        w13 = torch.empty((cfg.E, 2 * cfg.I, cfg.H), dtype=torch.bfloat16, device=device)
        w2 = torch.empty((cfg.E, cfg.H, cfg.I), dtype=torch.bfloat16, device=device)
        for e in range(cfg.E):
            w13[e].copy_(expert_w13(cfg, e, device, seed))
            w2[e].copy_(expert_w2(cfg, e, device, seed))
        out["w13"], out["w2"] = w13, w2
    return out


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """Host numpy uint16 array holding the bit patterns of a bf16 tensor."""
    assert t.dtype == torch.bfloat16
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


class DeviceExpertsAsBits:
    """Indexable host view of a device-resident [E, ...] bf16 stack: item e is copied on demand."""

    def __init__(self, stack: torch.Tensor):
        self.stack = stack

    def __len__(self):
        return self.stack.shape[0]

    def __getitem__(self, e):
        return bf16_bits(self.stack[int(e)])


__all__ += ["DeviceExpertsAsBits", "zipf_bias", "expert_w13", "expert_w2"]
