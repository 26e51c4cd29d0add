"""Python access to the CPU oracle (``oracle/oracle.c``).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg use this module; the GPU library and its Python binding never
import it.  Arrays are numpy; bf16 values travel as their uint16 bit patterns.

Functions mirror the C entry points:
  words_per_row(K, b)           ceil(K*b/32) (dense pack-quantized row length)
  pack(codes, b)                codes uint8 [N,K] -> packed uint32 [N, W]
  unpack(packed, K, b)          inverse of pack
  wna16(A, packed, scales, b)   fp64 y = A . dequant(W)^T and sum |a*w|
  wna16_points(...)             the same at chosen (m, n) positions
  quant_act_i8(A)               fp32 per-token int8 quantization -> (Aq, s_a)
  w4a8(A, packed, scales, b=4)  fp64 int8-activation result and magnitude (b = 4: W4A8)
  w4a8_points(Aq, sa, ...)      the same at chosen positions
  wna16_grouped(A, packed, scales, b, offsets)  grouped (mixture-of-experts) layer
  bf16_rne(x)                   fp64 values -> nearest bf16 bit patterns (ties to even)
  embed(packed, scales, K, b, ids)  quantized embedding gather -> bf16 bits [T, K]
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc (-O2, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                               "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build(force=True)
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    i64 = ctypes.c_int64
    ci = ctypes.c_int
    lib.oracle_words_per_row.argtypes = [i64, ci]
    lib.oracle_words_per_row.restype = i64
    lib.oracle_pack.argtypes = [P, i64, i64, ci, P]
    lib.oracle_unpack.argtypes = [P, i64, i64, ci, P]
    lib.oracle_wna16.argtypes = [P, i64, i64, i64, P, P, P, ci, ci, P, P]
    lib.oracle_wna16_points.argtypes = [P, i64, i64, i64, P, P, P, ci, ci, P, P, i64, P, P]
    lib.oracle_quant_act_i8.argtypes = [P, i64, i64, P, P]
    lib.oracle_w4a8.argtypes = [P, i64, i64, i64, P, P, P, ci, ci, P, P, P, P]
    lib.oracle_w4a8_points.argtypes = [P, P, i64, i64, i64, P, P, P, ci, ci, P, P, i64, P, P]
    lib.oracle_wna16_grouped.argtypes = [P, i64, i64, i64, P, P, P, ci, ci, P, i64, P, P]
    lib.oracle_bf16_rne.argtypes = [ctypes.c_double]
    lib.oracle_bf16_rne.restype = ctypes.c_uint16
    lib.oracle_embed.argtypes = [P, P, P, i64, i64, ci, ci, P, i64, P]
    for f in ("oracle_pack", "oracle_unpack", "oracle_wna16", "oracle_wna16_points",
              "oracle_quant_act_i8", "oracle_w4a8", "oracle_w4a8_points", "oracle_embed",
              "oracle_wna16_grouped",
              "oracle_num_threads", "oracle_abi", "oracle_little_endian"):
        getattr(lib, f).restype = ci
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _zeros(zeros, N: int, K: int):
    """Zero points uint8 [N, K/128] as (array, pointer), or (None, NULL) for symmetric groups."""
    if zeros is None:
        return None, None
    z = _c(zeros, np.uint8)
    assert z.shape == (N, K // 128)
    return z, _ptr(z)


def num_threads() -> int:
    return _load().oracle_num_threads()


def words_per_row(K: int, b: int) -> int:
    return int(_load().oracle_words_per_row(K, b))


def pack(codes: np.ndarray, b: int) -> np.ndarray:
    codes = _c(codes, np.uint8)
    N, K = codes.shape
    out = np.empty((N, words_per_row(K, b)), dtype=np.uint32)
    if _load().oracle_pack(_ptr(codes), N, K, b, _ptr(out)) != 0:
        raise ValueError("oracle_pack: code out of range for b=%d" % b)
    return out


def unpack(packed: np.ndarray, K: int, b: int) -> np.ndarray:
    packed = _c(packed, np.uint32)
    N = packed.shape[0]
    assert packed.shape[1] == words_per_row(K, b)
    out = np.empty((N, K), dtype=np.uint8)
    if _load().oracle_unpack(_ptr(packed), N, K, b, _ptr(out)) != 0:
        raise RuntimeError("oracle_unpack failed")
    return out


def wna16(A: np.ndarray, packed: np.ndarray, scales: np.ndarray, b: int, group: int = 128,
          zeros=None):
    """Return (y, mag), fp64 [M, N].  zeros: uint8 [N, K/128] zero points, or None
    for symmetric groups (z = 2^(b-1)); group = K is per-channel scales."""
    A = _c(A, np.uint16)
    packed = _c(packed, np.uint32)
    scales = _c(scales, np.uint16)
    M, K = A.shape
    N = packed.shape[0]
    assert packed.shape[1] == words_per_row(K, b) and scales.shape == (N, K // group)
    z, zp = _zeros(zeros, N, K)
    y = np.empty((M, N), dtype=np.float64)
    mag = np.empty((M, N), dtype=np.float64)
    r = _load().oracle_wna16(_ptr(A), M, N, K, _ptr(packed), _ptr(scales), zp, b, group,
                             _ptr(y), _ptr(mag))
    if r != 0:
        raise RuntimeError("oracle_wna16 failed (%d)" % r)
    return y, mag


def wna16_points(A, packed, scales, b, m_idx, n_idx, group: int = 128, zeros=None):
    A = _c(A, np.uint16)
    packed = _c(packed, np.uint32)
    scales = _c(scales, np.uint16)
    m_idx = _c(m_idx, np.int64)
    n_idx = _c(n_idx, np.int64)
    M, K = A.shape
    N = packed.shape[0]
    assert packed.shape[1] == words_per_row(K, b) and scales.shape == (N, K // group)
    P = m_idx.size
    z, zp = _zeros(zeros, N, K)
    y = np.empty(P, dtype=np.float64)
    mag = np.empty(P, dtype=np.float64)
    r = _load().oracle_wna16_points(_ptr(A), M, N, K, _ptr(packed), _ptr(scales), zp, b, group,
                                    _ptr(m_idx), _ptr(n_idx), P, _ptr(y), _ptr(mag))
    if r != 0:
        raise RuntimeError("oracle_wna16_points failed (%d)" % r)
    return y, mag


def wna16_grouped(A, packed, scales, b, offsets, group: int = 128, zeros=None):
    """Grouped layer: packed [E*N, W], scales [E*N, K/group], zero points
    [E*N, K/128] or None; rows [offsets[e], offsets[e+1]) of A through expert e.
    Return (y, mag) fp64 [M, N]."""
    A = _c(A, np.uint16)
    packed = _c(packed, np.uint32)
    scales = _c(scales, np.uint16)
    off = _c(offsets, np.int64)
    M, K = A.shape
    E = off.size - 1
    N = packed.shape[0] // E
    assert packed.shape == (E * N, words_per_row(K, b)) and scales.shape == (E * N, K // group)
    z, zp = _zeros(zeros, E * N, K)
    y = np.zeros((M, N), dtype=np.float64)
    mag = np.zeros((M, N), dtype=np.float64)
    r = _load().oracle_wna16_grouped(_ptr(A), M, N, K, _ptr(packed), _ptr(scales), zp, b, group,
                                     _ptr(off), E, _ptr(y), _ptr(mag))
    if r != 0:
        raise RuntimeError("oracle_wna16_grouped failed (%d)" % r)
    return y, mag


def bf16_rne(x) -> np.ndarray:
    """Nearest bf16 bit patterns (ties to even) of fp64 values."""
    x = np.asarray(x, dtype=np.float64)
    f = _load().oracle_bf16_rne
    return np.array([f(float(v)) for v in x.ravel()], dtype=np.uint16).reshape(x.shape)


def embed(packed: np.ndarray, scales: np.ndarray, K: int, b: int, ids, group: int = 128,
          zeros=None):
    """Quantized embedding gather: bf16 bits [T, K] of rows ids of the dequantized table."""
    packed = _c(packed, np.uint32)
    scales = _c(scales, np.uint16)
    ids = _c(ids, np.int64).ravel()
    V = packed.shape[0]
    assert packed.shape[1] == words_per_row(K, b) and scales.shape == (V, K // group)
    z, zp = _zeros(zeros, V, K)
    out = np.empty((ids.size, K), dtype=np.uint16)
    r = _load().oracle_embed(_ptr(packed), _ptr(scales), zp, V, K, b, group, _ptr(ids), ids.size,
                             _ptr(out))
    if r != 0:
        raise RuntimeError("oracle_embed failed (%d)" % r)
    return out


def quant_act_i8(A: np.ndarray):
    """Return (Aq int8 [M,K], s_a float32 [M])."""
    A = _c(A, np.uint16)
    M, K = A.shape
    Aq = np.empty((M, K), dtype=np.int8)
    sa = np.empty(M, dtype=np.float32)
    _load().oracle_quant_act_i8(_ptr(A), M, K, _ptr(Aq), _ptr(sa))
    return Aq, sa


def w4a8(A: np.ndarray, packed: np.ndarray, scales: np.ndarray, group: int = 128, b: int = 4,
         zeros=None):
    """Return (y, mag, Aq, s_a) for the int8-activation layer on b-bit codes
    (b = 4: W4A8)."""
    A = _c(A, np.uint16)
    packed = _c(packed, np.uint32)
    scales = _c(scales, np.uint16)
    M, K = A.shape
    N = packed.shape[0]
    assert packed.shape[1] == words_per_row(K, b) and scales.shape == (N, K // group)
    z, zp = _zeros(zeros, N, K)
    Aq = np.empty((M, K), dtype=np.int8)
    sa = np.empty(M, dtype=np.float32)
    y = np.empty((M, N), dtype=np.float64)
    mag = np.empty((M, N), dtype=np.float64)
    r = _load().oracle_w4a8(_ptr(A), M, N, K, _ptr(packed), _ptr(scales), zp, b, group,
                            _ptr(Aq), _ptr(sa), _ptr(y), _ptr(mag))
    if r != 0:
        raise RuntimeError("oracle_w4a8 failed (%d)" % r)
    return y, mag, Aq, sa


def w4a8_points(Aq, sa, packed, scales, m_idx, n_idx, group: int = 128, b: int = 4, zeros=None):
    Aq = _c(Aq, np.int8)
    sa = _c(sa, np.float32)
    packed = _c(packed, np.uint32)
    scales = _c(scales, np.uint16)
    m_idx = _c(m_idx, np.int64)
    n_idx = _c(n_idx, np.int64)
    M, K = Aq.shape
    N = packed.shape[0]
    P = m_idx.size
    z, zp = _zeros(zeros, N, K)
    y = np.empty(P, dtype=np.float64)
    mag = np.empty(P, dtype=np.float64)
    r = _load().oracle_w4a8_points(_ptr(Aq), _ptr(sa), M, N, K, _ptr(packed), _ptr(scales),
                                   zp, b, group, _ptr(m_idx), _ptr(n_idx), P, _ptr(y), _ptr(mag))
    if r != 0:
        raise RuntimeError("oracle_w4a8_points failed (%d)" % r)
    return y, mag
