"""Seeded synthetic inputs shared by the GPU path, the tests and the benchmark.

This module only draws random inputs.  It holds none of the layer's
arithmetic: no quantisation, no routing, no expert math.  Everything is
drawn with torch generators seeded per (workload seed, layer, tensor), so any
tensor can be regenerated on its own, on the CPU or on the GPU.  A tensor
drawn on one device differs from the same tensor drawn on another; each side
of a comparison reads the one copy that was drawn.

Workloads (shapes follow the 48-layer, 512-expert, top-10 model of the pages;
hidden, intermediate and format are the workload's own definition):

  tiny      hidden 64, 8 experts, top-2, inter 32, shared inter 32, 2-bit,
            fp32 router and activations, no router bias, 4 tokens
  decode1   hidden 2048, 512 experts, top-10, inter 704, shared 704, 2-bit,
            bf16 router/activations, Zipf(1.1) router bias, 1 token, 1 layer
  decode16  as decode1, 16 tokens per step through 48 stacked layers
  prefill   as decode1, 32,768 tokens, 1 layer
  prefill3  as decode1 but 3-bit, uniform routing (no bias), 4,096 tokens
            through 48 stacked layers
"""

from __future__ import annotations

import dataclasses

import numpy as np
import torch


@dataclasses.dataclass(frozen=True)
class MoEShape:
    hidden: int
    inter: int
    n_experts: int
    top_k: int
    shared_inter: int
    qbits: int


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    shape: MoEShape
    tokens: int
    layers: int
    seed: int
    act_dtype: torch.dtype      # dtype of x and of the router weights
    zipf_bias: bool
    weight_std: float = 0.02


FULL = dict(hidden=2048, inter=704, n_experts=512, top_k=10, shared_inter=704)

WORKLOADS = {
    "tiny": Workload("tiny", MoEShape(64, 32, 8, 2, 32, 2), 4, 1, 0, torch.float32, False),
    "decode1": Workload("decode1", MoEShape(qbits=2, **FULL), 1, 1, 1, torch.bfloat16, True),
    "decode16": Workload("decode16", MoEShape(qbits=2, **FULL), 16, 48, 2, torch.bfloat16, True),
    "prefill": Workload("prefill", MoEShape(qbits=2, **FULL), 32768, 1, 3, torch.bfloat16, True),
    "prefill3": Workload("prefill3", MoEShape(qbits=3, **FULL), 4096, 48, 4, torch.bfloat16, False),
    # the 4-bit block variant (codes -8..7), one layer of 4,096 tokens, uniform routing
    "prefill4": Workload("prefill4", MoEShape(qbits=4, **FULL), 4096, 1, 6, torch.bfloat16, False),
    # a speculative-decoding verify window: the token plus three drafts, through the stack
    "verify4": Workload("verify4", MoEShape(qbits=2, **FULL), 4, 48, 5, torch.bfloat16, True),
}

ZIPF_S = 1.1

_TAGS = {"router": 1, "bias": 2, "gate": 3, "up": 4, "down": 5,
         "sgate": 6, "sup": 7, "sdown": 8, "x": 9}


def derive_seed(seed: int, layer: int, tag: str, extra: int = 0) -> int:
    """Independent 63-bit seed for one tensor of one layer."""
    ss = np.random.SeedSequence([int(seed), int(layer), _TAGS[tag], int(extra)])
    return int(ss.generate_state(1, np.uint64)[0] & np.uint64((1 << 63) - 1))


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def normal(shape, std: float, seed: int, device) -> torch.Tensor:
    g = _gen(device, seed)
    out = torch.randn(*shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        out.mul_(std)
    return out


def expert_weights(wl: Workload, layer: int, device, experts=None):
    """fp32 N(0, std) routed-expert weights of one layer:
    gate [E, I, H], up [E, I, H], down [E, H, I].  `experts` (a slice or
    None) restricts the draw to a contiguous range, drawn with its own
    per-expert seeds so that any range reproduces the full draw."""
    s = wl.shape
    e_lo, e_hi = (0, s.n_experts) if experts is None else (experts.start, experts.stop)
    n = e_hi - e_lo
    gate = torch.empty(n, s.inter, s.hidden, device=device, dtype=torch.float32)
    up = torch.empty_like(gate)
    down = torch.empty(n, s.hidden, s.inter, device=device, dtype=torch.float32)
    for i, e in enumerate(range(e_lo, e_hi)):
        gate[i] = normal((s.inter, s.hidden), wl.weight_std, derive_seed(wl.seed, layer, "gate", e), device)
        up[i] = normal((s.inter, s.hidden), wl.weight_std, derive_seed(wl.seed, layer, "up", e), device)
        down[i] = normal((s.hidden, s.inter), wl.weight_std, derive_seed(wl.seed, layer, "down", e), device)
    return gate, up, down


def shared_weights(wl: Workload, layer: int, device):
    """fp32 shared-expert weights: gate [Is, H], up [Is, H], down [H, Is], or None."""
    s = wl.shape
    if s.shared_inter == 0:
        return None
    return (normal((s.shared_inter, s.hidden), wl.weight_std, derive_seed(wl.seed, layer, "sgate"), device),
            normal((s.shared_inter, s.hidden), wl.weight_std, derive_seed(wl.seed, layer, "sup"), device),
            normal((s.hidden, s.shared_inter), wl.weight_std, derive_seed(wl.seed, layer, "sdown"), device))


def router(wl: Workload, layer: int, device):
    """Router weights [E, H] in the workload's activation dtype (bf16 by
    round-to-nearest-even from fp32, or fp32) and the fp32 router bias [E]
    (None when the workload has no bias).

    Bias reading: a Zipf(s) prior over a seeded random ranking pi of the
    experts, b_e = -s * ln(pi(e) + 1), so expert popularity is skewed."""
    s = wl.shape
    w = normal((s.n_experts, s.hidden), wl.weight_std, derive_seed(wl.seed, layer, "router"), device)
    w = w.to(wl.act_dtype)
    bias = None
    if wl.zipf_bias:
        g = _gen("cpu", derive_seed(wl.seed, layer, "bias"))
        rank = torch.randperm(s.n_experts, generator=g).to(torch.float64)
        bias = (-ZIPF_S * torch.log(rank + 1.0)).to(torch.float32).to(device)
    return w, bias


def tokens(wl: Workload, device, layer: int = 0, n_tokens: int | None = None) -> torch.Tensor:
    """Activations x [T, H], N(0, 1), in the workload's activation dtype."""
    t = wl.tokens if n_tokens is None else n_tokens
    x = normal((t, wl.shape.hidden), 1.0, derive_seed(wl.seed, layer, "x"), device)
    return x.to(wl.act_dtype)


def custom(name: str, hidden: int, inter: int, n_experts: int, top_k: int, shared_inter: int,
           qbits: int, tokens_: int, seed: int, act_dtype=torch.bfloat16, zipf_bias: bool = False,
           layers: int = 1) -> Workload:
    """A workload of arbitrary shape (tests use it for ragged and edge cases)."""
    return Workload(name, MoEShape(hidden, inter, n_experts, top_k, shared_inter, qbits),
                    tokens_, layers, seed, act_dtype, zipf_bias)
