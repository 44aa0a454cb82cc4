"""Seeded synthetic workloads for the Stable LatentMoE layer.

This module only draws random numbers and packs them: shapes, seeds, the
per-expert logit offsets of the load-skew workload and the frozen bias of the
decode-like workload.  It holds none of the layer's arithmetic, so both the CPU
oracle (through the tests) and the GPU path take their inputs from here.

Shapes follow the five workloads of the layer (tiny fp32, mini-replica,
load-skew, K3 routing, decode-like).  The replica scale-down (experts 896/3.5 =
256, top-6) is the one described in "Pretraining a Mini Kimi K3" (review of the
e-book, scale-down capsules 4-8); K3's own 896-choose-16 routing is from the
same page and from the "K3 tops open source" blog (section on idle experts).

Recipe:
  * generator: numpy PCG64, ``np.random.default_rng([seed, stream])`` with
    ``seed = 1000 + workload id`` and one ``stream`` per purpose, so that the
    tensors of one purpose never depend on how many were drawn for another;
  * x ~ N(0, 1); weights ~ N(0, 1/fan_in) drawn in fp32 in the order
    W_r, W_sg, W_su, W_sd, W_dn, W_g, W_u, W_d, W_up; gamma = 1;
  * bf16 workloads round every drawn tensor to bf16 (round to nearest even).
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import numpy as np

__all__ = [
    "LayerShape", "WORKLOADS", "workload", "make_weights", "make_x",
    "zipf_logit_offset", "frozen_bias", "f32_to_bf16_bits", "bf16_bits_to_f32",
]

# stream ids of the seeded generator (second word of the seed sequence)
_S_WEIGHTS = 1
_S_X = 2
_S_OFFSET = 3
_S_BIAS = 4


@dataclasses.dataclass(frozen=True)
class LayerShape:
    """Sizes of one layer and one batch.

    T tokens; d model width; l latent width; E routed experts; k experts per
    token; f expert GLU hidden; f_s shared GLU hidden (0 = no shared expert);
    B histogram bins; dtype "bf16" or "f32".
    """
    name: str
    wid: int
    dtype: str
    T: int
    d: int
    l: int
    E: int
    k: int
    f: int
    f_s: int
    B: int = 256
    qb_frozen: bool = False
    rms_eps: float = 1e-6

    def with_tokens(self, T: int) -> "LayerShape":
        return dataclasses.replace(self, T=int(T))

    @property
    def seed(self) -> int:
        return 1000 + self.wid


WORKLOADS: Dict[str, LayerShape] = {
    "tiny": LayerShape("tiny", 1, "f32", T=256, d=256, l=64, E=16, k=2, f=128, f_s=256),
    "replica": LayerShape("replica", 2, "bf16", T=8192, d=1024, l=256, E=256, k=6, f=512, f_s=2048),
    "skew": LayerShape("skew", 3, "bf16", T=32768, d=1024, l=256, E=256, k=6, f=512, f_s=2048),
    "k3": LayerShape("k3", 4, "bf16", T=16384, d=4096, l=1024, E=896, k=16, f=512, f_s=4096),
    "decode": LayerShape("decode", 5, "bf16", T=131072, d=1024, l=256, E=256, k=6, f=512, f_s=2048,
                         qb_frozen=True),
}

# Zipf offset of the load-skew workload: c_e = ALPHA * rank_e ** -ZIPF_S
ZIPF_S = 1.2
ZIPF_ALPHA = 1.5


def workload(name: str, T: Optional[int] = None) -> LayerShape:
    s = WORKLOADS[name]
    return s if T is None else s.with_tokens(T)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest, ties to even.

    Finite inputs only (the generators never produce anything else)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _rng(shape: LayerShape, stream: int, sub: int = 0) -> np.random.Generator:
    return np.random.default_rng([shape.seed, stream, sub])


def _normal(rng: np.random.Generator, dims, std: float) -> np.ndarray:
    a = rng.standard_normal(dims, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


def _finish(a: np.ndarray, dtype: str) -> np.ndarray:
    """Round to the storage precision; returns fp32 values (exact bf16 values
    for bf16 workloads)."""
    if dtype == "bf16":
        return bf16_bits_to_f32(f32_to_bf16_bits(a))
    return a


def make_weights(shape: LayerShape) -> Dict[str, np.ndarray]:
    """All weights of one layer as fp32 arrays holding storage-precision values.

    PyTorch ``[out, in]`` convention, row-major: W_r[E,d], W_sg[f_s,d],
    W_su[f_s,d], W_sd[d,f_s], W_dn[l,d], W_g[E,f,l], W_u[E,f,l], W_d[E,l,f],
    W_up[d,l]; gamma[d] is fp32 ones.
    """
    s = shape
    rng = _rng(s, _S_WEIGHTS)
    w: Dict[str, np.ndarray] = {}
    w["gamma"] = np.ones(s.d, dtype=np.float32)
    w["W_r"] = _finish(_normal(rng, (s.E, s.d), 1.0 / np.sqrt(s.d)), s.dtype)
    w["W_sg"] = _finish(_normal(rng, (s.f_s, s.d), 1.0 / np.sqrt(s.d)), s.dtype)
    w["W_su"] = _finish(_normal(rng, (s.f_s, s.d), 1.0 / np.sqrt(s.d)), s.dtype)
    w["W_sd"] = _finish(_normal(rng, (s.d, s.f_s), 1.0 / np.sqrt(max(s.f_s, 1))), s.dtype)
    w["W_dn"] = _finish(_normal(rng, (s.l, s.d), 1.0 / np.sqrt(s.d)), s.dtype)
    w["W_g"] = _finish(_normal(rng, (s.E, s.f, s.l), 1.0 / np.sqrt(s.l)), s.dtype)
    w["W_u"] = _finish(_normal(rng, (s.E, s.f, s.l), 1.0 / np.sqrt(s.l)), s.dtype)
    w["W_d"] = _finish(_normal(rng, (s.E, s.l, s.f), 1.0 / np.sqrt(s.f)), s.dtype)
    w["W_up"] = _finish(_normal(rng, (s.d, s.l), 1.0 / np.sqrt(s.l)), s.dtype)
    return w


def make_x(shape: LayerShape, step: int = 0) -> np.ndarray:
    """Input activations x[T,d] ~ N(0,1) for a given step (fresh x per step)."""
    rng = _rng(shape, _S_X, step)
    return _finish(_normal(rng, (shape.T, shape.d), 1.0), shape.dtype)


def zipf_logit_offset(shape: LayerShape, alpha: float = ZIPF_ALPHA, s: float = ZIPF_S) -> np.ndarray:
    """Per-expert router-logit offset c_e = alpha * rank_e^-s, rank a seeded
    permutation of 1..E (fp32).  Gives a few experts > 10x the mean load."""
    rng = _rng(shape, _S_OFFSET)
    rank = rng.permutation(shape.E).astype(np.float64) + 1.0
    return (alpha * rank ** (-s)).astype(np.float32)


def frozen_bias(shape: LayerShape, std: float = 0.1, n_forced_empty: int = 0) -> np.ndarray:
    """Inference-time bias: N(0, std) per expert, optionally with the first
    ``n_forced_empty`` experts (in a seeded order) pushed to -1, then
    mean-centred in fp64 and stored as fp32."""
    rng = _rng(shape, _S_BIAS)
    b = rng.standard_normal(shape.E) * std
    if n_forced_empty:
        b[rng.permutation(shape.E)[:n_forced_empty]] = -1.0
    b = b - b.mean()
    return b.astype(np.float32)
