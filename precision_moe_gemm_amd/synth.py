"""Seeded synthetic inputs for the NVFP4 workloads.

This module draws random tensors and nothing else: it holds none of the
quantization, GEMM or MoE arithmetic.  Both the HIP path's tests/benchmark and
the CPU oracle take their inputs from here, so the two sides always see the
same bits.

Every tensor is identified by a tuple of integers (workload seed, tensor id,
expert id, ...).  Host draws use numpy's PCG64 seeded with that tuple, so any
one expert can be regenerated on its own; device draws (for the multi-GB
expert sets) use torch's Philox generator seeded with a 63-bit hash of the
same tuple.  Floats are drawn in fp32 and rounded to bf16 with
round-to-nearest-even.

The shapes follow the pages' models: a 27B-class dense MLP (hidden 5120,
intermediate 17408, page "Qwen3.8-27B-NVFP4" section 2), a 512-expert top-10
MoE (page "Qwen3.8-Flash-Next-NVFP4"), a 384-expert MoE whose experts start as
MXFP4 (page "DeepSeek-V4.1-Flash-NVFP4"), and a 262144-token KV cache with
4 KV heads of 256 (page "Qwen3.8-2.4T-A95B-NVFP4").  The pages measure on
real checkpoints and evaluation suites; these synthetic draws stand in for
them.
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass, field

import numpy as np
import torch


def _seed63(parts) -> int:
    h = hashlib.sha256(repr(tuple(int(p) for p in parts)).encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def normal_bf16(shape, std: float, parts, device="cpu") -> torch.Tensor:
    """N(0, std^2) draws rounded to bf16 (a torch.bfloat16 tensor)."""
    device = torch.device(device)
    if device.type == "cpu":
        rng = np.random.Generator(np.random.PCG64(list(int(p) for p in parts)))
        a = rng.standard_normal(size=tuple(shape), dtype=np.float32)
        t = torch.from_numpy(a)
    else:
        g = torch.Generator(device=device)
        g.manual_seed(_seed63(parts))
        t = torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        t = t * std
    return t.to(torch.bfloat16)


def bits(t: torch.Tensor) -> np.ndarray:
    """Raw bf16 bits of a (CPU or device) bf16 tensor as a numpy uint16 array."""
    assert t.dtype == torch.bfloat16
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def from_bits(b: np.ndarray, device="cpu") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16).to(device)


def with_outliers(x: torch.Tensor, frac: float, factor: float, parts) -> torch.Tensor:
    """Multiply a fraction of entries (chosen uniformly without replacement)
    by ``factor`` (done in fp32, re-rounded to bf16)."""
    n = x.numel()
    cnt = int(round(frac * n))
    rng = np.random.Generator(np.random.PCG64(list(int(p) for p in parts)))
    idx = rng.choice(n, size=cnt, replace=False)
    y = x.float().flatten().cpu()
    y[torch.from_numpy(idx)] *= factor
    return y.reshape(x.shape).to(torch.bfloat16).to(x.device)


def route_topk(logits: torch.Tensor, k: int):
    """Top-k routing from fp32 logits: softmax over all experts, the k most
    probable experts (ties broken towards the lower id), weights = the
    selected probabilities (not renormalised).  Returns (ids int32 [T,k],
    weights fp32 [T,k])."""
    p = torch.softmax(logits.float(), dim=1)
    vals, idx = torch.sort(p, dim=1, descending=True, stable=True)
    return idx[:, :k].to(torch.int32).contiguous(), vals[:, :k].contiguous()


def zipf_bias(E: int, s: float, parts) -> torch.Tensor:
    """Expert bias b_e = -s * ln(rank_e), rank a seeded permutation of 1..E."""
    rng = np.random.Generator(np.random.PCG64(list(int(p) for p in parts)))
    rank = rng.permutation(E) + 1
    return torch.from_numpy(-s * np.log(rank.astype(np.float64))).float()


def lognormal_channel_kv(tokens: int, heads: int, dim: int, parts, device="cpu") -> torch.Tensor:
    """bf16 [tokens, heads, dim] = sigma[h, d] * z with sigma ~ LogNormal(0,1)
    per (head, dim) and z ~ N(0,1)."""
    rng = np.random.Generator(np.random.PCG64(list(int(p) for p in parts) + [0]))
    sigma = torch.from_numpy(np.exp(rng.standard_normal(size=(heads, dim))).astype(np.float32))
    z_parts = list(parts) + [1]
    device = torch.device(device)
    if device.type == "cpu":
        z_rng = np.random.Generator(np.random.PCG64(z_parts))
        z = torch.from_numpy(z_rng.standard_normal(size=(tokens, heads, dim), dtype=np.float32))
    else:
        g = torch.Generator(device=device)
        g.manual_seed(_seed63(z_parts))
        z = torch.randn((tokens, heads, dim), generator=g, device=device, dtype=torch.float32)
    return (z * sigma.to(z.device)).to(torch.bfloat16)


# --------------------------------------------------------------------------
# the five workloads
# --------------------------------------------------------------------------

# tensor ids inside a workload seed
X, W, W13, W2, W1, W3, LOGITS, BIAS, OUTL, KCACHE, VCACHE = range(11)


@dataclass(frozen=True)
class TinyLinear:
    """16x512 activations (1% of entries x20) times a 256x512 weight."""
    seed: int = 1
    M: int = 16
    N: int = 256
    K: int = 512

    def x(self, device="cpu"):
        x = normal_bf16((self.M, self.K), 1.0, (self.seed, X), device)
        return with_outliers(x, 0.01, 20.0, (self.seed, OUTL))

    def w(self, device="cpu"):
        return normal_bf16((self.N, self.K), 0.02, (self.seed, W), device)


@dataclass(frozen=True)
class DenseMLP:
    """27B-class SwiGLU MLP: gate_up 34816x5120, down 5120x17408."""
    seed: int = 2
    H: int = 5120
    I: int = 17408
    Ms: tuple = (1, 32, 8192)

    def w13(self, device="cpu"):
        return normal_bf16((2 * self.I, self.H), 0.02, (self.seed, W13), device)

    def w2(self, device="cpu"):
        return normal_bf16((self.H, self.I), 0.02, (self.seed, W2), device)

    def x(self, M, device="cpu"):
        return normal_bf16((M, self.H), 1.0, (self.seed, X, M), device)


@dataclass(frozen=True)
class MoE:
    """Routed-expert MoE layer.  ``mx`` marks experts that start as MXFP4."""
    seed: int
    E: int
    k: int
    H: int
    I: int
    T: int
    zipf: float = 0.0
    mx: bool = False

    def w13(self, e, device="cpu"):
        """gate rows [0, I) then up rows [I, 2I) of expert e (bf16 [2I, H])."""
        if self.mx:
            w1 = normal_bf16((self.I, self.H), 0.02, (self.seed, W1, e), device)
            w3 = normal_bf16((self.I, self.H), 0.02, (self.seed, W3, e), device)
            return torch.cat([w1, w3], dim=0)
        return normal_bf16((2 * self.I, self.H), 0.02, (self.seed, W13, e), device)

    def w2(self, e, device="cpu"):
        return normal_bf16((self.H, self.I), 0.02, (self.seed, W2, e), device)

    def x(self, device="cpu"):
        return normal_bf16((self.T, self.H), 1.0, (self.seed, X, self.T), device)

    def logits(self, device="cpu"):
        z = normal_bf16((self.T, self.E), 1.0, (self.seed, LOGITS, self.T), "cpu").float()
        if self.zipf:
            z = z + zipf_bias(self.E, self.zipf, (self.seed, BIAS))[None, :]
        return z.to(device)

    def routing(self, device="cpu"):
        ids, w = route_topk(self.logits("cpu"), self.k)
        return ids.to(device), w.to(device)

    def scaled(self, **kw):
        d = dict(seed=self.seed, E=self.E, k=self.k, H=self.H, I=self.I, T=self.T,
                 zipf=self.zipf, mx=self.mx)
        d.update(kw)
        return MoE(**d)


@dataclass(frozen=True)
class KVCache:
    """One sequence of 262144 tokens x 4 KV heads x 256, written in 2048-token chunks."""
    seed: int = 5
    tokens: int = 262144
    heads: int = 4
    dim: int = 256
    chunk: int = 2048

    def k(self, device="cpu"):
        return lognormal_channel_kv(self.tokens, self.heads, self.dim, (self.seed, KCACHE), device)

    def v(self, device="cpu"):
        return lognormal_channel_kv(self.tokens, self.heads, self.dim, (self.seed, VCACHE), device)


C1 = TinyLinear()
C2 = DenseMLP()
C3 = MoE(seed=3, E=512, k=10, H=4096, I=1024, T=4096)
C4_DECODE = MoE(seed=4, E=384, k=8, H=7168, I=2048, T=64, zipf=1.1, mx=True)
C4_PREFILL = MoE(seed=4, E=384, k=8, H=7168, I=2048, T=16384, zipf=1.1, mx=True)
C5 = KVCache()
