"""Seeded synthetic workloads for the WNA16 / W4A8 quantized linear layer.

This module only draws random numbers and rounds them to the storage types
(uint8 codes, bf16 bit patterns).  It holds none of the method's arithmetic:
no packing, no dequantization, no products.  It is the one module that both
the CPU oracle side (tests, CPU baseline) and the GPU side (tests, bench,
smoke) take their inputs from.

Value structure follows the pages:
  * codes are uniform unsigned b-bit integers (the compressed-tensors WNA16
    scheme for b in 2..8; "vLLM Can Run INT5-7", section 1);
  * one symmetric scale per group of 128 input features, about half of them
    negative (model card "Qwen3.8-27B-INT6-Mixed-AutoRound", Findings; club-3090
    discussion #733, "Under the hood": AutoRound emits about half negative
    group scales);
  * activations are bf16, with optional outlier channels for the W4A8 case.

Draw order inside one workload: codes, then scales, then activations, all
from ``numpy.random.default_rng(seed)`` (PCG64).  bf16 values are produced by
round-to-nearest-even from float32.
"""
from __future__ import annotations

import dataclasses

import numpy as np

GROUP = 128


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even).

    Returns the bf16 bit patterns as uint16.  Inputs are finite here.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to float32 exactly."""
    return (np.ascontiguousarray(h, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclasses.dataclass
class Workload:
    """One synthetic linear layer: activations, weight codes and group scales.

    A: bf16 bits uint16 [M, K]; codes: uint8 [N, K] in [0, 2**b);
    scales: bf16 bits uint16 [N, K // 128].
    """
    A: np.ndarray
    codes: np.ndarray
    scales: np.ndarray
    b: int
    group: int = GROUP

    @property
    def M(self) -> int:
        return self.A.shape[0]

    @property
    def N(self) -> int:
        return self.codes.shape[0]

    @property
    def K(self) -> int:
        return self.codes.shape[1]


def draw_codes(rng: np.random.Generator, N: int, K: int, b: int) -> np.ndarray:
    return rng.integers(0, 1 << b, size=(N, K), dtype=np.uint8)


def draw_scales_uniform(rng: np.random.Generator, N: int, G: int, lim: float = 0.02) -> np.ndarray:
    """Scales ~U(-lim, lim): about half negative."""
    return f32_to_bf16_bits(rng.uniform(-lim, lim, size=(N, G)).astype(np.float32))


def draw_scales_halfnormal_signed(rng: np.random.Generator, N: int, G: int,
                                  sigma: float = 0.01) -> np.ndarray:
    """Scales |N(0, sigma)| with an independent random sign (about half negative)."""
    mag = np.abs(rng.normal(0.0, sigma, size=(N, G)))
    sign = np.where(rng.integers(0, 2, size=(N, G)) == 1, -1.0, 1.0)
    return f32_to_bf16_bits((mag * sign).astype(np.float32))


def draw_act(rng: np.random.Generator, M: int, K: int, outlier_frac: float = 0.0,
             outlier_gain: float = 20.0) -> np.ndarray:
    """Activations ~N(0, 1), optionally with a fixed set of outlier columns.

    The outlier columns (round(outlier_frac * K) of them, drawn once) are
    multiplied by ``outlier_gain`` before the bf16 rounding.
    """
    a = rng.normal(0.0, 1.0, size=(M, K)).astype(np.float32)
    n_out = int(round(outlier_frac * K))
    if n_out:
        cols = rng.choice(K, size=n_out, replace=False)
        a[:, cols] *= np.float32(outlier_gain)
    return f32_to_bf16_bits(a)


# --- the five workloads the method is measured on ---------------------------

def tiny(seed: int = 0) -> Workload:
    """A bf16[4,512] ~N(0,1); b=6 codes, N=256; scales ~U(-0.02, 0.02)."""
    rng = np.random.default_rng(seed)
    M, N, K, b = 4, 256, 512, 6
    codes = draw_codes(rng, N, K, b)
    scales = draw_scales_uniform(rng, N, K // GROUP)
    A = draw_act(rng, M, K)
    return Workload(A, codes, scales, b)


def decode(M: int, b: int, seed: int = 1, N: int = 17408, K: int = 5120) -> Workload:
    """Decode-shape layer: M in {1,4,16}, K=5120, N=17408, scales |N(0,0.01)| signed."""
    rng = np.random.default_rng(seed)
    codes = draw_codes(rng, N, K, b)
    scales = draw_scales_halfnormal_signed(rng, N, K // GROUP)
    A = draw_act(rng, M, K)
    return Workload(A, codes, scales, b)


def prefill(M: int = 4096, N: int = 17408, K: int = 5120, b: int = 6, seed: int = 2) -> Workload:
    """Prefill-shape layer (up: K=5120,N=17408; down: K=17408,N=5120), b=6."""
    rng = np.random.default_rng(seed)
    codes = draw_codes(rng, N, K, b)
    scales = draw_scales_halfnormal_signed(rng, N, K // GROUP)
    A = draw_act(rng, M, K)
    return Workload(A, codes, scales, b)


def w4a8(M: int = 2048, N: int = 17408, K: int = 5120, seed: int = 3) -> Workload:
    """W4A8 layer: int4 codes, signed group scales, A with 1% outlier columns x20."""
    rng = np.random.default_rng(seed)
    codes = draw_codes(rng, N, K, 4)
    scales = draw_scales_halfnormal_signed(rng, N, K // GROUP)
    A = draw_act(rng, M, K, outlier_frac=0.01, outlier_gain=20.0)
    return Workload(A, codes, scales, 4)


def layer_bits(layer: int, n_layers: int = 64) -> int:
    """Depth-tiered allocation of the 64-layer stack: 7 bits on the 20 edge
    layers (0-9 and 54-63), 5 on even and 6 on odd middle layers."""
    if layer < 10 or layer >= n_layers - 10:
        return 7
    return 5 if layer % 2 == 0 else 6


# --- the mixed-bit 64-layer stack with an 8-bit vocabulary head --------------

STACK_LAYERS = 64
STACK_HIDDEN = 5120
STACK_INTER = 17408
STACK_VOCAB = 248320


def stack_scale_sigma(K: int, b: int) -> float:
    """Gain-normalising scale magnitude for chained layers: sigma =
    1 / (sqrt(K) * rms(q)) with rms(q) = 2^(b-1) / sqrt(3) for uniform codes,
    so each layer keeps activations at unit scale and 128 chained layers stay
    finite."""
    return float(np.sqrt(3.0) / (np.sqrt(K) * (1 << (b - 1))))


def stack_weights(b: int, kind: str, seed: int = 4, N: int | None = None,
                  K: int | None = None):
    """One weight set of the stack: kind 'up' (K 5120 -> N 17408), 'down'
    (K 17408 -> N 5120) or 'head' (K 5120 -> N 248320, b = 8).  Codes uniform,
    scales |N(0, sigma)| with a random sign.  Returns (codes, scales)."""
    dims = {"up": (STACK_INTER, STACK_HIDDEN), "down": (STACK_HIDDEN, STACK_INTER),
            "head": (STACK_VOCAB, STACK_HIDDEN)}[kind]
    N = dims[0] if N is None else N
    K = dims[1] if K is None else K
    sub = {"up": 0, "down": 1, "head": 2}[kind]
    rng = np.random.default_rng([seed, b, sub])
    codes = draw_codes(rng, N, K, b)
    scales = draw_scales_halfnormal_signed(rng, N, K // GROUP, sigma=stack_scale_sigma(K, b))
    return codes, scales


def stack_input(M: int, seed: int = 4, K: int = STACK_HIDDEN) -> np.ndarray:
    """Stack input activations ~N(0, 1), bf16 bits [M, K]."""
    return draw_act(np.random.default_rng([seed, 99, M]), M, K)


EMBED_VOCAB = 248320
EMBED_HIDDEN = 5120


def embed_table(V: int = EMBED_VOCAB, K: int = EMBED_HIDDEN, b: int = 8, seed: int = 5):
    """Quantized embedding table in the dense layout ("vLLM Can Run INT5-7",
    section 3: vocabulary 248,320 x hidden 5,120).  With K*b a multiple of 32
    a dense row has no padding bits, so every 32-bit pattern is a row of
    uniform b-bit codes: the words themselves are drawn (no packing step).
    Scales |N(0, 0.01)| with a random sign.  Returns (words uint32 [V, K*b/32],
    scales bf16 bits [V, K/128])."""
    assert (K * b) % 32 == 0 and K % GROUP == 0
    rng = np.random.default_rng([seed, b, V, K])
    words = rng.integers(0, 1 << 32, size=(V, K * b // 32), dtype=np.uint32)
    scales = draw_scales_halfnormal_signed(rng, V, K // GROUP)
    return words, scales


def embed_ids(T: int, V: int = EMBED_VOCAB, seed: int = 5) -> np.ndarray:
    """Token ids uniform in [0, V), int64 [T]."""
    return np.random.default_rng([seed, 7, T]).integers(0, V, size=T, dtype=np.int64)
