"""Shared helpers for the GPU parity tests: device upload of the synthetic
workloads and the parity criteria.

Criteria:
  * unpacked codes, activation codes and scales: bit-exact;
  * WNA16 (bf16 output, fp32 accumulation):
        |Y - y_ref| <= 4e-3 * sum_k |a*w| + 1e-3   per element;
  * W4A8 fp32 output: |Y - y_ref| <= 1e-5 * sum_g |s * acc_g| * |s_a|;
    W4A8 bf16 output: that plus one bf16 rounding, 2^-8 |y_ref|.
"""
import numpy as np
import torch

import weight_only_bit_wq_amd as wq
from weight_only_bit_wq_amd import synth

WNA16_REL = 4e-3
WNA16_ABS = 1e-3
A8_REL = 1e-5


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def dev_words(packed: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(packed).view(np.int32)).cuda()


def host_bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def bf16_values(bits: np.ndarray) -> np.ndarray:
    return synth.bf16_bits_to_f32(bits).astype(np.float64)


class Layer:
    """A workload's weights on the device in one layout."""

    def __init__(self, w: synth.Workload, layout: int, packed: np.ndarray | None = None):
        self.w = w
        self.layout = layout
        self.packed = wq.wq_pack(w.codes, w.b) if packed is None else packed
        self.packed_d = dev_words(self.packed)
        self.scales_d = dev_bf16(w.scales)
        if layout == wq.WQ_LAYOUT_TILED:
            self.W_d = wq.wq_repack(self.packed_d, self.scales_d, w.K, w.b)
            self.S_d = None
        else:
            self.W_d = self.packed_d
            self.S_d = self.scales_d

    def gemm(self, A_bits: np.ndarray | None = None) -> np.ndarray:
        A = self.w.A if A_bits is None else A_bits
        Y = wq.wq_gemm(dev_bf16(A), self.W_d, self.layout, self.S_d, self.w.N, self.w.b)
        torch.cuda.synchronize()
        return host_bf16_bits(Y)

    def gemm_a8(self, out_dtype=wq.WQ_OUT_F32, A_bits: np.ndarray | None = None) -> np.ndarray:
        A = self.w.A if A_bits is None else A_bits
        Y = wq.wq_gemm_a8(dev_bf16(A), self.W_d, self.layout, self.S_d, self.w.N, self.w.b,
                          out_dtype=out_dtype)
        torch.cuda.synchronize()
        if out_dtype == wq.WQ_OUT_F32:
            return Y.cpu().numpy().astype(np.float64)
        return bf16_values(host_bf16_bits(Y))


def assert_wna16(Y_bits: np.ndarray, y_ref: np.ndarray, mag: np.ndarray, what: str = ""):
    y = bf16_values(Y_bits)
    err = np.abs(y - y_ref)
    bound = WNA16_REL * mag + WNA16_ABS
    bad = err > bound
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError("%s: %d of %d outside tolerance; first %s: got %s ref %s mag %s"
                             % (what, bad.sum(), bad.size, idx.tolist(),
                                y[tuple(idx.T)], y_ref[tuple(idx.T)], mag[tuple(idx.T)]))
    assert np.all(np.isfinite(y))


def assert_a8(Y: np.ndarray, y_ref: np.ndarray, mag: np.ndarray, bf16_out: bool, what: str = ""):
    bound = A8_REL * mag
    if bf16_out:
        bound = bound + 2.0 ** -8 * np.abs(y_ref)
    err = np.abs(Y - y_ref)
    bad = err > bound
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError("%s: %d of %d outside tolerance; first %s: got %s ref %s mag %s"
                             % (what, bad.sum(), bad.size, idx.tolist(),
                                Y[tuple(idx.T)], y_ref[tuple(idx.T)], mag[tuple(idx.T)]))


def sample_points(M: int, N: int, count: int, seed: int):
    rng = np.random.default_rng(seed)
    mi = rng.integers(0, M, count)
    ni = rng.integers(0, N, count)
    # always include the corners and the ragged edges
    mi = np.concatenate([mi, [0, 0, M - 1, M - 1]])
    ni = np.concatenate([ni, [0, N - 1, 0, N - 1]])
    return mi, ni
