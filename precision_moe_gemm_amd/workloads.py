"""Device-resident workload builders (harness code over the library).

Turns the seeded synthetic draws of :mod:`synth` into the NVFP4 operands the
hot path consumes, with the library's own kernels: weights quantized once
(static), MXFP4 experts encoded with ``mxfp4_quantize`` and remapped with
``mxfp4_to_nvfp4`` (the fused [w1; w3] matrix as one tensor, so one
power-of-two global covers both halves), routing drawn on the host.
Expert weights are drawn and quantized one expert at a time, so a
384-expert layer never holds more than one expert in bf16.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

from . import NVFP4Tensor, mxfp4_quantize, mxfp4_to_nvfp4, nvfp4_quantize
from . import synth


def expert_view(t: NVFP4Tensor, e: int) -> NVFP4Tensor:
    return NVFP4Tensor(t.packed[e:e + 1], t.scales[e:e + 1], t.global_[e:e + 1], t.rows, t.cols, 1, t.flags)


@dataclass
class MoEWeights:
    w13: NVFP4Tensor          # batch E, [2I, H]
    w2: NVFP4Tensor           # batch E, [H, I]
    mx13: tuple | None = None  # (packed [E, 2I, H/2], e8m0 [E, 2I, H/32]) for MXFP4 experts
    mx2: tuple | None = None


def build_moe_weights(cfg: synth.MoE, device="cuda", keep_mx: bool = False) -> MoEWeights:
    E, H, I = cfg.E, cfg.H, cfg.I
    dev = torch.device(device)
    if not cfg.mx:
        w13 = NVFP4Tensor.empty(2 * I, H, E, dev)
        w2 = NVFP4Tensor.empty(H, I, E, dev)
        for e in range(E):
            nvfp4_quantize(cfg.w13(e, dev), out=expert_view(w13, e))
            nvfp4_quantize(cfg.w2(e, dev), out=expert_view(w2, e))
        return MoEWeights(w13, w2)
    p13 = torch.empty((E, 2 * I, H // 2), dtype=torch.uint8, device=dev)
    s13 = torch.empty((E, 2 * I, H // 32), dtype=torch.uint8, device=dev)
    p2 = torch.empty((E, H, I // 2), dtype=torch.uint8, device=dev)
    s2 = torch.empty((E, H, I // 32), dtype=torch.uint8, device=dev)
    for e in range(E):
        a, b = mxfp4_quantize(cfg.w13(e, dev))
        p13[e].copy_(a)
        s13[e].copy_(b)
        a, b = mxfp4_quantize(cfg.w2(e, dev))
        p2[e].copy_(a)
        s2[e].copy_(b)
    w13 = mxfp4_to_nvfp4(p13, s13, 2 * I, H, E, in_place=not keep_mx)
    w2 = mxfp4_to_nvfp4(p2, s2, H, I, E, in_place=not keep_mx)
    if keep_mx:
        return MoEWeights(w13, w2, (p13, s13), (p2, s2))
    return MoEWeights(w13, w2)


def build_dense_mlp(cfg: synth.DenseMLP, device="cuda") -> MoEWeights:
    """The dense SwiGLU MLP as a one-expert MoE (E=1, top-1, weight 1)."""
    dev = torch.device(device)
    w13 = nvfp4_quantize(cfg.w13(dev))
    w2 = nvfp4_quantize(cfg.w2(dev))
    return MoEWeights(w13, w2)


def routing(cfg: synth.MoE, device="cuda"):
    ids, w = cfg.routing("cpu")
    return ids.to(device), w.to(device)
