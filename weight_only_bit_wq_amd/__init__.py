"""weight_only_bit_wq_amd -- b-bit weight-only quantized linear layers (WNA16)
and the int8-activation variant (W4A8) on AMD Instinct MI355X (gfx950).

This module is the Python binding of ``libwq.so`` (built from ``csrc/`` by
``build.py``).  Every function has the name of the C entry point it calls
(declared in ``include/wq.h``) and only marshals arguments: host arrays are
numpy, device buffers are torch CUDA tensors (torch supplies device memory and
the current stream).  All computation happens in the library's HIP kernels;
there is no CPU fallback, and a missing library raises ``WQError`` at the
first call.
"""
from __future__ import annotations

import ctypes
import os
import re
import threading

import numpy as np

__all__ = [
    "WQError", "lib_path", "declared_functions",
    "WQ_OK", "WQ_LAYOUT_DENSE", "WQ_LAYOUT_TILED", "WQ_OP_GEMM", "WQ_OP_GEMM_A8",
    "WQ_OUT_BF16", "WQ_OUT_F32",
    "wq_abi_version", "wq_status_str", "wq_last_hip_error", "wq_device_supported",
    "wq_packed_words_per_row", "wq_pack", "wq_unpack", "wq_repacked_bytes", "wq_repack",
    "wq_unpack_dev", "wq_workspace_bytes", "wq_gemm", "wq_gemm_noalloc", "wq_quant_act_i8",
    "wq_gemm_a8",
    "wq_embed", "wq_gemm_grouped", "wq_grouped_workspace_bytes",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_ROOT = os.path.dirname(_HERE)
lib_path = os.path.join(_HERE, "libwq.so")
header_path = os.path.join(_ROOT, "include", "wq.h")

WQ_OK = 0
WQ_ERR_INVALID_ARG = 1
WQ_ERR_UNSUPPORTED_BITS = 2
WQ_ERR_BAD_GROUP = 3
WQ_ERR_MISALIGNED = 4
WQ_ERR_CODE_RANGE = 5
WQ_ERR_WORKSPACE = 6
WQ_ERR_BAD_LAYOUT = 7
WQ_ERR_UNSUPPORTED_DEVICE = 8
WQ_ERR_HIP = 9
WQ_ERR_ZERO_POINTS = 10
WQ_ERR_SCRATCH_LIMIT = 11
WQ_NOALLOC_SCRATCH_BYTES = 64 << 20

WQ_LAYOUT_DENSE = 0
WQ_LAYOUT_TILED = 1
WQ_OP_GEMM = 0
WQ_OP_GEMM_A8 = 1
WQ_OUT_BF16 = 0
WQ_OUT_F32 = 1
GROUP = 128
# Leading workspace bytes that must be zero before a call and are zero after it.
WORKSPACE_ZERO_BYTES = 1 << 16


class WQError(RuntimeError):
    def __init__(self, func: str, status: int, detail: str = ""):
        self.status = status
        msg = "%s failed: status %d (%s)" % (func, status, _status_text(status))
        if detail:
            msg += ": " + detail
        super().__init__(msg)


_lib = None
_lock = threading.Lock()


def _status_text(status: int) -> str:
    try:
        return _load().wq_status_str(status).decode()
    except Exception:  # pragma: no cover - only when the library is absent
        return "libwq not loaded"


def _load():
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(lib_path):
            raise WQError("load", -1, "libwq.so not built (run weight_only_bit_wq_amd/build.py)")
        lib = ctypes.CDLL(lib_path)
        P, I, L = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
        sig = {
            "wq_abi_version": ([], I),
            "wq_status_str": ([I], ctypes.c_char_p),
            "wq_last_hip_error": ([], I),
            "wq_device_supported": ([I], I),
            "wq_packed_words_per_row": ([L, I], L),
            "wq_pack": ([P, L, L, I, I, P], I),
            "wq_unpack": ([P, L, L, I, P], I),
            "wq_repacked_bytes": ([I, L, L, I, I], L),
            "wq_repack": ([P, P, L, L, I, I, I, P, P], I),
            "wq_unpack_dev": ([P, I, L, L, I, I, P, P], I),
            "wq_workspace_bytes": ([I, L, L, L, I, I], L),
            "wq_gemm": ([P, L, L, L, P, I, P, P, I, I, P, P, L, P], I),
            "wq_gemm_noalloc": ([P, L, L, L, P, I, P, P, I, I, P, P], I),
            "wq_quant_act_i8": ([P, L, L, P, P, P], I),
            "wq_gemm_a8": ([P, L, L, L, P, I, P, P, I, I, P, I, P, L, P], I),
            "wq_embed": ([P, P, P, L, L, I, I, P, L, P, P], I),
            "wq_gemm_grouped": ([P, L, L, L, P, L, P, P, L, I, I, P, P, L, P], I),
            "wq_grouped_workspace_bytes": ([P, L, L, L, I, I], L),
        }
        for name, (args, res) in sig.items():
            f = getattr(lib, name)
            f.argtypes = args
            f.restype = res
        _lib = lib
        return lib


def declared_functions() -> list[str]:
    """Names of the functions include/wq.h declares."""
    with open(header_path) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(wq_\w+)\s*\(", text, re.M)))


def _check(func: str, status: int):
    if status != WQ_OK:
        raise WQError(func, status)


def _ptr(x):
    """Address of a numpy array, torch tensor or None."""
    if x is None:
        return None
    if isinstance(x, np.ndarray):
        return ctypes.c_void_p(x.ctypes.data)
    return ctypes.c_void_p(x.data_ptr())


def _torch_stream(stream=None):
    """The torch stream a call runs on: `stream`, else torch's current one."""
    import torch
    return stream if stream is not None else torch.cuda.current_stream()


def _stream(stream=None):
    return ctypes.c_void_p(_torch_stream(stream).cuda_stream)


def _require_cuda(name: str, t, dtype=None, shape=None):
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError("%s must be a CUDA (HIP) torch tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise TypeError("%s has dtype %s" % (name, t.dtype))
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))


# --- plain calls ---------------------------------------------------------------

def wq_abi_version() -> int:
    return _load().wq_abi_version()


def wq_status_str(status: int) -> str:
    return _load().wq_status_str(status).decode()


def wq_last_hip_error() -> int:
    return _load().wq_last_hip_error()


def wq_device_supported(device: int = 0) -> bool:
    return bool(_load().wq_device_supported(device))


def wq_packed_words_per_row(K: int, b: int) -> int:
    return int(_load().wq_packed_words_per_row(K, b))


def wq_pack(codes: np.ndarray, b: int, group: int = GROUP) -> np.ndarray:
    """Host: uint8 codes [N, K] -> dense packed uint32 [N, ceil(K*b/32)]."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    N, K = codes.shape
    out = np.empty((N, max(0, wq_packed_words_per_row(K, b))), dtype=np.uint32)
    _check("wq_pack", _load().wq_pack(_ptr(codes), N, K, b, group, _ptr(out)))
    return out


def wq_unpack(packed: np.ndarray, K: int, b: int) -> np.ndarray:
    """Host: dense packed uint32 [N, ceil(K*b/32)] -> uint8 codes [N, K]."""
    packed = np.ascontiguousarray(packed, dtype=np.uint32)
    N = packed.shape[0]
    if packed.shape[1] != wq_packed_words_per_row(K, b):
        raise ValueError("packed has %d words per row, expected %d"
                         % (packed.shape[1], wq_packed_words_per_row(K, b)))
    out = np.empty((N, K), dtype=np.uint8)
    _check("wq_unpack", _load().wq_unpack(_ptr(packed), N, K, b, _ptr(out)))
    return out


def wq_repacked_bytes(layout: int, N: int, K: int, b: int, group: int = GROUP) -> int:
    return int(_load().wq_repacked_bytes(layout, N, K, b, group))


def wq_repack(packed_d, scales_d, K: int, b: int, group: int = GROUP,
              layout: int = WQ_LAYOUT_TILED, out=None, stream=None):
    """Device: dense words (int32/uint32 [N, W]) + bf16 scales [N, K/group] -> blob (uint8).
    group = K (per-channel scales [N, 1]) writes the row's scale into every group."""
    import torch
    N = packed_d.shape[0]
    _require_cuda("packed_d", packed_d, (torch.int32, torch.uint32),
                  (N, wq_packed_words_per_row(K, b)))
    _require_cuda("scales_d", scales_d, (torch.bfloat16, torch.int16), (N, K // group))
    nbytes = wq_repacked_bytes(layout, N, K, b, group)
    if nbytes < 0:
        raise WQError("wq_repacked_bytes", WQ_ERR_INVALID_ARG)
    ts = _torch_stream(stream)
    if out is None:
        out = _empty_on(ts, nbytes, torch.uint8, packed_d.device)
    else:
        _require_cuda("out", out, torch.uint8, (nbytes,))
    _check("wq_repack", _load().wq_repack(_ptr(packed_d), _ptr(scales_d), N, K, b, group, layout,
                                          _ptr(out), _stream(ts)))
    return out


def wq_unpack_dev(W_d, layout: int, N: int, K: int, b: int, group: int = GROUP, out=None,
                  stream=None):
    """Device: codes of a weight buffer in `layout` -> uint8 [N, K]."""
    import torch
    _require_cuda("W_d", W_d)
    ts = _torch_stream(stream)
    if out is None:
        out = _empty_on(ts, (N, K), torch.uint8, W_d.device)
    else:
        _require_cuda("out", out, torch.uint8, (N, K))
    _check("wq_unpack_dev", _load().wq_unpack_dev(_ptr(W_d), layout, N, K, b, group, _ptr(out),
                                                  _stream(ts)))
    return out


def wq_workspace_bytes(op: int, M: int, N: int, K: int, b: int, group: int = GROUP) -> int:
    return int(_load().wq_workspace_bytes(op, M, N, K, b, group))


# One zero-filled workspace per (device, stream); the library leaves it zeroed.
# It is allocated and zeroed on the stream whose calls use it (inside
# torch.cuda.stream(s)), so its zero fill is ordered before those calls and
# torch's caching allocator ties the memory to that stream: a buffer
# replaced by a larger one is only reused by later work on the same stream.
_ws_cache: dict = {}


def _workspace(nbytes: int, device, ts):
    import torch
    if nbytes <= 0:
        return None, 0
    key = (str(device), int(ts.cuda_stream))
    buf = _ws_cache.get(key)
    if buf is None or buf.numel() < nbytes:
        with torch.cuda.stream(ts):
            buf = torch.zeros(max(nbytes, 1 << 20), dtype=torch.uint8, device=device)
        _ws_cache[key] = buf
    return buf, buf.numel()


def _empty_on(ts, shape, dtype, device):
    """An output allocated on the stream that writes it (see _workspace)."""
    import torch
    with torch.cuda.stream(ts):
        return torch.empty(shape, dtype=dtype, device=device)


def _require_zeros(zeros_d, N: int, K: int):
    if zeros_d is not None:
        import torch
        _require_cuda("zeros_d", zeros_d, torch.uint8, (N, K // GROUP))


def wq_gemm(A_d, W_d, layout: int, scales_d, N: int, b: int, group: int = GROUP, Y=None,
            ws=None, stream=None, zeros=None):
    """Device: Y bf16 [M, N] = A_d bf16 [M, K] . dequant(W)^T.  zeros: optional
    uint8 zero points [N, K/128] (b = 4 or 8)."""
    import torch
    _require_cuda("A_d", A_d, torch.bfloat16)
    _require_cuda("W_d", W_d)
    M, K = A_d.shape
    if scales_d is not None:
        _require_cuda("scales_d", scales_d, (torch.bfloat16, torch.int16), (N, K // group))
    _require_zeros(zeros, N, K)
    ts = _torch_stream(stream)
    if Y is None:
        Y = _empty_on(ts, (M, N), torch.bfloat16, A_d.device)
    else:
        _require_cuda("Y", Y, torch.bfloat16, (M, N))
    st = _stream(ts)
    need = wq_workspace_bytes(WQ_OP_GEMM, M, N, K, b, group)
    if ws is None:
        ws_buf, ws_bytes = _workspace(need, A_d.device, ts)
    else:
        ws_buf, ws_bytes = ws, ws.numel() * ws.element_size()
    _check("wq_gemm", _load().wq_gemm(_ptr(A_d), M, N, K, _ptr(W_d), layout, _ptr(scales_d),
                                      _ptr(zeros), b, group, _ptr(Y), _ptr(ws_buf), ws_bytes, st))
    return Y


def wq_gemm_noalloc(A_d, W_d, layout: int, scales_d, N: int, b: int, group: int = GROUP,
                    Y=None, stream=None, zeros=None):
    """Device: wq_gemm with the library's static per-GPU scratch instead of a
    workspace.  Y must be given by a caller that cannot allocate (else a new
    tensor is returned); calls that overlap on one GPU race."""
    import torch
    _require_cuda("A_d", A_d, torch.bfloat16)
    _require_cuda("W_d", W_d)
    M, K = A_d.shape
    if scales_d is not None:
        _require_cuda("scales_d", scales_d, (torch.bfloat16, torch.int16), (N, K // group))
    _require_zeros(zeros, N, K)
    ts = _torch_stream(stream)
    if Y is None:
        Y = _empty_on(ts, (M, N), torch.bfloat16, A_d.device)
    else:
        _require_cuda("Y", Y, torch.bfloat16, (M, N))
    _check("wq_gemm_noalloc", _load().wq_gemm_noalloc(_ptr(A_d), M, N, K, _ptr(W_d), layout,
                                                      _ptr(scales_d), _ptr(zeros), b, group,
                                                      _ptr(Y), _stream(ts)))
    return Y


def wq_grouped_workspace_bytes(offsets, N: int, K: int, b: int, group: int = GROUP) -> int:
    """Workspace bytes of a grouped call with these host offsets (-1: invalid)."""
    off = np.ascontiguousarray(offsets, dtype=np.int64)
    return int(_load().wq_grouped_workspace_bytes(_ptr(off), off.size - 1, N, K, b, group))


def wq_gemm_grouped(A_d, W_d, expert_bytes: int, offsets, N: int, b: int, group: int = GROUP,
                    Y=None, ws=None, stream=None, zeros=None):
    """Device: grouped (mixture-of-experts) layer.  W_d: E tiled blobs at
    expert_bytes apart (uint8); offsets: host int64 [E + 1], rows of A_d sorted
    by expert.  Returns Y bf16 [M, N]."""
    import torch
    _require_cuda("A_d", A_d, torch.bfloat16)
    _require_cuda("W_d", W_d)
    M, K = A_d.shape
    off = np.ascontiguousarray(offsets, dtype=np.int64)
    E = off.size - 1
    if zeros is not None:
        _require_cuda("zeros_d", zeros, torch.uint8, (E * N, K // GROUP))
    ts = _torch_stream(stream)
    if Y is None:
        Y = _empty_on(ts, (M, N), torch.bfloat16, A_d.device)
    else:
        _require_cuda("Y", Y, torch.bfloat16, (M, N))
    st = _stream(ts)
    need = int(_load().wq_grouped_workspace_bytes(_ptr(off), E, N, K, b, group))
    if need < 0:
        raise WQError("wq_grouped_workspace_bytes", WQ_ERR_INVALID_ARG)
    if ws is None:
        ws_buf, ws_bytes = _workspace(need, A_d.device, ts)
    else:
        ws_buf, ws_bytes = ws, ws.numel() * ws.element_size()
    _check("wq_gemm_grouped", _load().wq_gemm_grouped(
        _ptr(A_d), M, N, K, _ptr(W_d), expert_bytes, _ptr(zeros), _ptr(off), E, b, group,
        _ptr(Y), _ptr(ws_buf), ws_bytes, st))
    return Y


def wq_quant_act_i8(A_d, Aq=None, sa=None, stream=None):
    """Device: per-token int8 quantization -> (Aq int8 [M, K], s_a float32 [M])."""
    import torch
    _require_cuda("A_d", A_d, torch.bfloat16)
    M, K = A_d.shape
    ts = _torch_stream(stream)
    if Aq is None:
        Aq = _empty_on(ts, (M, K), torch.int8, A_d.device)
    if sa is None:
        sa = _empty_on(ts, (M,), torch.float32, A_d.device)
    _check("wq_quant_act_i8", _load().wq_quant_act_i8(_ptr(A_d), M, K, _ptr(Aq), _ptr(sa),
                                                      _stream(ts)))
    return Aq, sa


def wq_embed(ids_d, W_d, scales_d, K: int, b: int, group: int = GROUP, Y=None, stream=None,
             zeros=None):
    """Device: quantized embedding gather from the dense layout -> bf16 [T, K]
    (rows of ids outside [0, V) are zero).  group 128 or K (per-channel
    scales); zeros: optional uint8 zero points [V, K/128] (b = 4 or 8)."""
    import torch
    _require_cuda("ids_d", ids_d, torch.int64)
    V = W_d.shape[0]
    _require_cuda("W_d", W_d, (torch.int32, torch.uint32), (V, wq_packed_words_per_row(K, b)))
    _require_cuda("scales_d", scales_d, (torch.bfloat16, torch.int16), (V, K // group))
    _require_zeros(zeros, V, K)
    T = ids_d.numel()
    ts = _torch_stream(stream)
    if Y is None:
        Y = _empty_on(ts, (T, K), torch.bfloat16, W_d.device)
    else:
        _require_cuda("Y", Y, torch.bfloat16, (T, K))
    _check("wq_embed", _load().wq_embed(_ptr(W_d), _ptr(scales_d), _ptr(zeros), V, K, b, group,
                                        _ptr(ids_d), T, _ptr(Y), _stream(ts)))
    return Y


def wq_gemm_a8(A_d, W_d, layout: int, scales_d, N: int, b: int = 4, group: int = GROUP,
               out_dtype: int = WQ_OUT_BF16, Y=None, ws=None, stream=None, zeros=None):
    """Device: int8-activation layer on b-bit weights (b = 4: W4A8) -> Y [M, N]
    (bf16 or float32).  zeros: optional uint8 zero points [N, K/128] (b = 4)."""
    import torch
    _require_cuda("A_d", A_d, torch.bfloat16)
    _require_cuda("W_d", W_d)
    M, K = A_d.shape
    if scales_d is not None:
        _require_cuda("scales_d", scales_d, (torch.bfloat16, torch.int16), (N, K // group))
    _require_zeros(zeros, N, K)
    ydt = torch.float32 if out_dtype == WQ_OUT_F32 else torch.bfloat16
    ts = _torch_stream(stream)
    if Y is None:
        Y = _empty_on(ts, (M, N), ydt, A_d.device)
    else:
        _require_cuda("Y", Y, ydt, (M, N))
    st = _stream(ts)
    need = wq_workspace_bytes(WQ_OP_GEMM_A8, M, N, K, b, group)
    if ws is None:
        ws_buf, ws_bytes = _workspace(need, A_d.device, ts)
    else:
        ws_buf, ws_bytes = ws, ws.numel() * ws.element_size()
    _check("wq_gemm_a8", _load().wq_gemm_a8(_ptr(A_d), M, N, K, _ptr(W_d), layout,
                                            _ptr(scales_d), _ptr(zeros), b, group, _ptr(Y),
                                            out_dtype, _ptr(ws_buf), ws_bytes, st))
    return Y
