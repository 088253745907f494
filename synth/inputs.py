"""Seeded synthetic inputs for the int4 grouped-GEMM MoE layer.

This module only draws random inputs and stores them in the layer's input
formats. It holds none of the layer's arithmetic: no dequantisation, no
routing, no GEMM. Both the CPU oracle and the GPU path take their inputs from
here, so that both see the same bytes.

Every array comes from its own keyed PCG64 stream,
``numpy.random.default_rng([seed, cfg_id, layer, a, b])``. One expert's
weights can therefore be regenerated without drawing any other expert's.

Key layout:

* weights: ``a`` = expert index (``E`` for the shared expert),
  ``b = 10 * tensor + field``. ``tensor`` is 0 gate, 1 up, 2 down; ``field``
  is 0 packed nibbles, 1 scale, 2 bias.
* activations: ``a = X_KEY``, ``b`` = chunk or decode step.
* router logits: ``a = LOGIT_KEY``, ``b`` = chunk or decode step.
* Zipf expert permutation: ``a = ZIPF_KEY``, ``layer`` = 0, ``b`` = 0.

Weight format (groupwise-affine 4-bit, groups of 64 along K; the news.ainew.jp
Lily article, section "Prefill"): a matrix of shape ``[N, K]`` (out x in) is
stored as

* ``q``: uint8 ``[N, K/2]``. Byte ``i`` of a row holds element ``2i`` in its
  low nibble and element ``2i+1`` in its high nibble.
* ``scale``, ``bias``: bf16 bit patterns (uint16) ``[N, K/64]``.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Iterator, Optional, Tuple

import numpy as np

GROUP = 64
X_KEY = 1_000_000
LOGIT_KEY = 2_000_000
ZIPF_KEY = 3_000_000
ROUTER_KEY = 4_000_000
ZIPF_S = 1.1

GATE, UP, DOWN = 0, 1, 2
F_Q, F_SCALE, F_BIAS = 0, 1, 2


@dataclasses.dataclass(frozen=True)
class LayerConfig:
    """Shape and distribution of one synthetic workload."""

    name: str
    cfg_id: int
    T: int  # tokens per call (chunk size for chunked prefill)
    H: int  # hidden size
    F: int  # expert FFN size
    E: int  # routed experts
    k: int  # experts chosen per token
    layers: int = 1
    total_tokens: Optional[int] = None  # chunked prefill: tokens over all chunks
    steps: int = 1  # decode steps
    zipf: bool = False
    scale_lo: float = 0.005
    scale_hi: float = 0.02
    bias_std: float = 0.01

    @property
    def chunks(self) -> int:
        if self.total_tokens is None:
            return 1
        return self.total_tokens // self.T


CONFIGS: Dict[str, LayerConfig] = {
    c.name: c
    for c in (
        LayerConfig("tiny", 0, T=32, H=256, F=128, E=16, k=2),
        LayerConfig("prefill512", 1, T=512, H=2048, F=512, E=256, k=8),
        LayerConfig("prefill2048_zipf", 2, T=2048, H=2048, F=512, E=256, k=8, zipf=True),
        LayerConfig("stack40_T8192", 3, T=2048, H=2048, F=512, E=256, k=8, layers=40,
                    total_tokens=8192),
        LayerConfig("decode40", 4, T=1, H=2048, F=512, E=256, k=8, layers=40, steps=256),
        # one layer call at the long-prompt size, uniform routing (tile-height sweep)
        LayerConfig("prefill8192", 5, T=8192, H=2048, F=512, E=256, k=8),
    )
}


def rng(seed: int, cfg_id: int, layer: int, a: int, b: int) -> np.random.Generator:
    return np.random.default_rng([seed, cfg_id, layer, a, b])


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Store float32 samples as bf16 bit patterns (round to nearest even).

    The samples are finite, so no NaN handling is needed.
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def matrix_dims(cfg: LayerConfig, tensor: int) -> Tuple[int, int]:
    """(N, K) of a weight matrix: gate/up map H -> F, down maps F -> H."""
    return (cfg.F, cfg.H) if tensor in (GATE, UP) else (cfg.H, cfg.F)


def expert_matrix(cfg: LayerConfig, layer: int, expert: int, tensor: int, seed: int = 0):
    """One int4 matrix of one expert: (q [N,K/2] u8, scale [N,K/64] u16, bias [N,K/64] u16)."""
    N, K = matrix_dims(cfg, tensor)
    q = rng(seed, cfg.cfg_id, layer, expert, 10 * tensor + F_Q).integers(
        0, 256, size=(N, K // 2), dtype=np.uint8)
    s = rng(seed, cfg.cfg_id, layer, expert, 10 * tensor + F_SCALE).uniform(
        cfg.scale_lo, cfg.scale_hi, size=(N, K // GROUP)).astype(np.float32)
    b = rng(seed, cfg.cfg_id, layer, expert, 10 * tensor + F_BIAS).normal(
        0.0, cfg.bias_std, size=(N, K // GROUP)).astype(np.float32)
    return q, f32_to_bf16_bits(s), f32_to_bf16_bits(b)


@dataclasses.dataclass
class W4:
    """Stacked int4 matrices of several experts, canonical layout."""

    q: np.ndarray  # uint8 [n, N, K/2]
    scale: np.ndarray  # uint16 [n, N, K/64]
    bias: np.ndarray  # uint16 [n, N, K/64]


@dataclasses.dataclass
class LayerWeights:
    gate: W4  # [E, F, H/2]
    up: W4
    down: W4  # [E, H, F/2]
    sh_gate: W4  # [1, F, H/2]
    sh_up: W4
    sh_down: W4


def _stack(cfg, layer, experts, tensor, seed) -> W4:
    N, K = matrix_dims(cfg, tensor)
    n = len(experts)
    q = np.empty((n, N, K // 2), np.uint8)
    s = np.empty((n, N, K // GROUP), np.uint16)
    b = np.empty((n, N, K // GROUP), np.uint16)
    for i, e in enumerate(experts):
        q[i], s[i], b[i] = expert_matrix(cfg, layer, e, tensor, seed)
    return W4(q, s, b)


def layer_weights(cfg: LayerConfig, layer: int = 0, seed: int = 0) -> LayerWeights:
    """All weights of one layer (routed experts 0..E-1 and the shared expert E)."""
    routed = list(range(cfg.E))
    sh = [cfg.E]
    return LayerWeights(
        gate=_stack(cfg, layer, routed, GATE, seed),
        up=_stack(cfg, layer, routed, UP, seed),
        down=_stack(cfg, layer, routed, DOWN, seed),
        sh_gate=_stack(cfg, layer, sh, GATE, seed),
        sh_up=_stack(cfg, layer, sh, UP, seed),
        sh_down=_stack(cfg, layer, sh, DOWN, seed),
    )


def activations(cfg: LayerConfig, index: int = 0, seed: int = 0, T: Optional[int] = None) -> np.ndarray:
    """Token activations x, bf16 bits [T, H], drawn N(0,1)."""
    T = cfg.T if T is None else T
    g = rng(seed, cfg.cfg_id, 0, X_KEY, index)
    return f32_to_bf16_bits(g.standard_normal((T, cfg.H), dtype=np.float32))


def zipf_log_bias(cfg: LayerConfig, seed: int = 0) -> np.ndarray:
    """Per-expert log-probability of a Zipf(s=1.1) popularity over a random
    permutation of the experts, float32 [E]."""
    perm = rng(seed, cfg.cfg_id, 0, ZIPF_KEY, 0).permutation(cfg.E)
    p = (perm.astype(np.float64) + 1.0) ** (-ZIPF_S)
    p /= p.sum()
    return np.log(p).astype(np.float32)


def router_logits(cfg: LayerConfig, layer: int = 0, index: int = 0, seed: int = 0,
                  T: Optional[int] = None) -> np.ndarray:
    """Router logits, float32 [T, E]: N(0,1), plus the Zipf log-bias if the
    workload asks for uneven expert groups."""
    T = cfg.T if T is None else T
    g = rng(seed, cfg.cfg_id, layer, LOGIT_KEY, index)
    lg = g.standard_normal((T, cfg.E), dtype=np.float32)
    if cfg.zipf:
        lg = lg + zipf_log_bias(cfg, seed)[None, :]
    return np.ascontiguousarray(lg, dtype=np.float32)


def router_weights(cfg: LayerConfig, layer: int = 0, seed: int = 0) -> np.ndarray:
    """Router projection W_r, bf16 bits [E, H], drawn N(0, 1/H) so that
    x W_r^T of N(0,1) activations has unit variance, like the logits above."""
    g = rng(seed, cfg.cfg_id, layer, ROUTER_KEY, 0)
    w = g.standard_normal((cfg.E, cfg.H), dtype=np.float32) * np.float32(1.0 / np.sqrt(cfg.H))
    return f32_to_bf16_bits(w)


def iter_layer_weights(cfg: LayerConfig, seed: int = 0) -> Iterator[LayerWeights]:
    for layer in range(cfg.layers):
        yield layer_weights(cfg, layer, seed)
