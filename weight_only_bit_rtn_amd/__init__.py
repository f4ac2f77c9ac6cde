"""Python binding of liblowbit (weight-only 2/3/4/8-bit RTN linear layers, gfx950).

Argument marshalling only: every step of quantization, packing and the
dequantize-and-multiply products runs in the HIP kernels of ``liblowbit.so``,
reached through its C ABI (``include/lowbit.h``).  torch is used for device
memory and streams.  There is no CPU fallback: if the library is missing or
no GPU is present the calls raise.

Functions mirror the C entry points:

  quantize_rtn(w, bits, group_size, codes=True, packed=True, symmetric=False) -> dict
  pack(codes, bits) -> packed
  qgemv(x, packed, scales, zeros, K, bits, group_size) -> y      (1 <= B <= 15)
  qgemm(x, packed, scales, zeros, K, bits, group_size) -> y      (any B)
  pack_meta(scales, zeros) -> (meta, saturated)                   compact group words
  qgemv_meta / qgemm_meta(x, packed, meta, K, bits, group_size) -> y
  quantize_gptq(w, x_calib, bits, group_size, damp=0.01, symmetric=False) -> dict
                                                                  error-feedback codes
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblowbit.so")

LOWBIT_OK = 0
LOWBIT_ERR_ARG = -1
LOWBIT_ERR_SHAPE = -2
LOWBIT_ERR_UNSUPPORTED = -3
LOWBIT_ERR_HIP = -4
LOWBIT_ERR_SCRATCH = -5
QGEMV_MAX_B = 15
QUANTIZE_MAX_K = 131072
GPTQ_NOALLOC_MAX_BYTES = 72 << 20

EXPORTED = ("lowbit_quantize_rtn", "lowbit_quantize_rtn_sym", "lowbit_pack", "lowbit_qgemv", "lowbit_qgemm",
            "lowbit_pack_meta", "lowbit_qgemv_meta", "lowbit_qgemm_meta", "lowbit_gptq_workspace_bytes",
            "lowbit_quantize_gptq", "lowbit_quantize_gptq_sym", "lowbit_quantize_gptq_noalloc",
            "lowbit_status_string")

_lib = None


class LowbitError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} (status {status})")


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load liblowbit.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m "
                          f"weight_only_bit_rtn_amd.build` (or __graft_entry__.build())")
    lib = ctypes.CDLL(path)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.lowbit_quantize_rtn.argtypes = [vp, i64, i64, i32, i64, vp, vp, vp, vp, vp]
    lib.lowbit_quantize_rtn_sym.argtypes = [vp, i64, i64, i32, i64, vp, vp, vp, vp, vp]
    lib.lowbit_pack.argtypes = [vp, i64, i64, i32, vp, vp]
    lib.lowbit_qgemv.argtypes = [vp, i64, vp, vp, vp, i64, i64, i32, i64, vp, vp]
    lib.lowbit_qgemm.argtypes = [vp, i64, vp, vp, vp, i64, i64, i32, i64, vp, vp]
    lib.lowbit_pack_meta.argtypes = [vp, vp, i64, i64, vp, vp, vp]
    lib.lowbit_gptq_workspace_bytes.argtypes = [i64, i64]
    lib.lowbit_gptq_workspace_bytes.restype = i64
    lib.lowbit_quantize_gptq.argtypes = [vp, i64, i64, vp, i64, ctypes.c_double, i32, i64, vp,
                                         vp, vp, vp, vp, i64, vp]
    lib.lowbit_quantize_gptq_sym.argtypes = lib.lowbit_quantize_gptq.argtypes
    lib.lowbit_quantize_gptq_noalloc.argtypes = [vp, i64, i64, vp, i64, ctypes.c_double, i32,
                                                 i64, vp, vp, vp, vp, vp, vp]
    lib.lowbit_qgemv_meta.argtypes = [vp, i64, vp, vp, i64, i64, i32, i64, vp, vp]
    lib.lowbit_qgemm_meta.argtypes = [vp, i64, vp, vp, i64, i64, i32, i64, vp, vp]
    for name in ("lowbit_quantize_rtn", "lowbit_quantize_rtn_sym", "lowbit_pack", "lowbit_qgemv",
                 "lowbit_qgemm", "lowbit_pack_meta", "lowbit_qgemv_meta", "lowbit_qgemm_meta",
                 "lowbit_quantize_gptq", "lowbit_quantize_gptq_sym",
                 "lowbit_quantize_gptq_noalloc"):
        getattr(lib, name).restype = ctypes.c_int
    lib.lowbit_status_string.argtypes = [ctypes.c_int]
    lib.lowbit_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().lowbit_status_string(int(status)).decode()


def _check(status: int, what: str) -> None:
    if status != LOWBIT_OK:
        raise LowbitError(status, what)


def _torch():
    import torch
    return torch


def _stream_handle(device) -> int:
    torch = _torch()
    return torch.cuda.current_stream(device).cuda_stream


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _require_gpu_tensor(t, name: str, dtype) -> None:
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must live on the GPU")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def groups(K: int, group_size: int) -> int:
    return 1 if group_size == 0 else K // group_size


def packed_words(K: int, bits: int) -> int:
    return K * bits // 32


# ---------------------------------------------------------------------------
# raw entry points (device pointers as ints; the caller owns every buffer)
# ---------------------------------------------------------------------------
def quantize_rtn_raw(w, N, K, bits, group_size, codes, packed, scales, zeros, stream) -> int:
    return load_library().lowbit_quantize_rtn(w, N, K, bits, group_size, codes, packed, scales,
                                              zeros, stream)


def quantize_rtn_sym_raw(w, N, K, bits, group_size, codes, packed, scales, zeros, stream) -> int:
    return load_library().lowbit_quantize_rtn_sym(w, N, K, bits, group_size, codes, packed,
                                                  scales, zeros, stream)


def pack_raw(codes, N, K, bits, packed, stream) -> int:
    return load_library().lowbit_pack(codes, N, K, bits, packed, stream)


def qgemv_raw(x, B, packed, scales, zeros, N, K, bits, group_size, y, stream) -> int:
    return load_library().lowbit_qgemv(x, B, packed, scales, zeros, N, K, bits, group_size, y,
                                       stream)


def qgemm_raw(x, B, packed, scales, zeros, N, K, bits, group_size, y, stream) -> int:
    return load_library().lowbit_qgemm(x, B, packed, scales, zeros, N, K, bits, group_size, y,
                                       stream)


def pack_meta_raw(scales, zeros, N, G, meta, saturated, stream) -> int:
    return load_library().lowbit_pack_meta(scales, zeros, N, G, meta, saturated, stream)


def qgemv_meta_raw(x, B, packed, meta, N, K, bits, group_size, y, stream) -> int:
    return load_library().lowbit_qgemv_meta(x, B, packed, meta, N, K, bits, group_size, y,
                                            stream)


def qgemm_meta_raw(x, B, packed, meta, N, K, bits, group_size, y, stream) -> int:
    return load_library().lowbit_qgemm_meta(x, B, packed, meta, N, K, bits, group_size, y,
                                            stream)


# ---------------------------------------------------------------------------
# tensor front end
# ---------------------------------------------------------------------------
def quantize_rtn(w, bits: int, group_size: int, codes: bool = True, packed: bool = True,
                 out: dict | None = None, symmetric: bool = False) -> dict:
    """RTN quantization of fp16 ``w[N][K]`` on the GPU: the min-max grid, or
    with ``symmetric=True`` the signed symmetric grid (``lowbit_quantize_rtn_sym``).

    Returns a dict with ``scales`` (fp16 [N][G]), ``zeros`` (int32 [N][G]) and,
    as requested, ``codes`` (uint8 [N][K]) and ``packed`` (int32 view of the
    uint32 words, [N][K*bits/32]).  ``out`` may supply preallocated buffers.
    """
    torch = _torch()
    _require_gpu_tensor(w, "w", torch.float16)
    N, K = w.shape
    G = groups(K, group_size)
    out = dict(out or {})
    dev = w.device
    if "scales" not in out:
        out["scales"] = torch.empty((N, G), dtype=torch.float16, device=dev)
    if "zeros" not in out:
        out["zeros"] = torch.empty((N, G), dtype=torch.int32, device=dev)
    if codes and "codes" not in out:
        out["codes"] = torch.empty((N, K), dtype=torch.uint8, device=dev)
    if packed and "packed" not in out:
        out["packed"] = torch.empty((N, packed_words(K, bits)), dtype=torch.int32, device=dev)
    raw, name = ((quantize_rtn_sym_raw, "lowbit_quantize_rtn_sym") if symmetric
                 else (quantize_rtn_raw, "lowbit_quantize_rtn"))
    st = raw(w.data_ptr(), N, K, bits, group_size,
             _ptr(out.get("codes") if codes else None),
             _ptr(out.get("packed") if packed else None),
             out["scales"].data_ptr(), out["zeros"].data_ptr(), _stream_handle(dev))
    _check(st, name)
    return out


def pack(codes, bits: int, out=None):
    torch = _torch()
    _require_gpu_tensor(codes, "codes", torch.uint8)
    N, K = codes.shape
    if out is None:
        out = torch.empty((N, packed_words(K, bits)), dtype=torch.int32, device=codes.device)
    _check(pack_raw(codes.data_ptr(), N, K, bits, out.data_ptr(), _stream_handle(codes.device)),
           "lowbit_pack")
    return out


def _product(raw, name, x, packed, scales, zeros, K, bits, group_size, out):
    torch = _torch()
    _require_gpu_tensor(x, "x", torch.float16)
    _require_gpu_tensor(packed, "packed", torch.int32)
    _require_gpu_tensor(scales, "scales", torch.float16)
    _require_gpu_tensor(zeros, "zeros", torch.int32)
    B = x.shape[0]
    N = packed.shape[0]
    if x.shape[1] != K:
        raise ValueError("x.shape[1] != K")
    if out is None:
        out = torch.empty((B, N), dtype=torch.float16, device=x.device)
    _check(raw(x.data_ptr(), B, packed.data_ptr(), scales.data_ptr(), zeros.data_ptr(), N, K,
               bits, group_size, out.data_ptr(), _stream_handle(x.device)), name)
    return out


def qgemv(x, packed, scales, zeros, K: int, bits: int, group_size: int, out=None):
    """y = x * deq(packed)^T, fp16 [B][N], 1 <= B <= 15 (VALU kernel)."""
    return _product(qgemv_raw, "lowbit_qgemv", x, packed, scales, zeros, K, bits, group_size,
                    out)


def qgemm(x, packed, scales, zeros, K: int, bits: int, group_size: int, out=None):
    """y = x * deq(packed)^T, fp16 [B][N], any B (matrix-core kernel)."""
    return _product(qgemm_raw, "lowbit_qgemm", x, packed, scales, zeros, K, bits, group_size,
                    out)


def pack_meta(scales, zeros, out=None, saturated=None):
    """Compact group words (int32 view of fp16 scale | int16 zero << 16),
    shape of ``scales``.  ``saturated``: optional device int32 tensor of one
    element to which the number of saturated zero points is added."""
    torch = _torch()
    _require_gpu_tensor(scales, "scales", torch.float16)
    _require_gpu_tensor(zeros, "zeros", torch.int32)
    if scales.shape != zeros.shape or scales.dim() != 2:
        raise ValueError("scales and zeros must both be [N][G]")
    N, G = scales.shape
    if out is None:
        out = torch.empty((N, G), dtype=torch.int32, device=scales.device)
    if saturated is not None:
        _require_gpu_tensor(saturated, "saturated", torch.int32)
    _check(pack_meta_raw(scales.data_ptr(), zeros.data_ptr(), N, G, out.data_ptr(),
                         _ptr(saturated), _stream_handle(scales.device)), "lowbit_pack_meta")
    return out


def _product_meta(raw, name, x, packed, meta, K, bits, group_size, out):
    torch = _torch()
    _require_gpu_tensor(x, "x", torch.float16)
    _require_gpu_tensor(packed, "packed", torch.int32)
    _require_gpu_tensor(meta, "meta", torch.int32)
    B = x.shape[0]
    N = packed.shape[0]
    if x.shape[1] != K:
        raise ValueError("x.shape[1] != K")
    if out is None:
        out = torch.empty((B, N), dtype=torch.float16, device=x.device)
    _check(raw(x.data_ptr(), B, packed.data_ptr(), meta.data_ptr(), N, K, bits, group_size,
               out.data_ptr(), _stream_handle(x.device)), name)
    return out


def qgemv_meta(x, packed, meta, K: int, bits: int, group_size: int, out=None):
    """qgemv with compact group words."""
    return _product_meta(qgemv_meta_raw, "lowbit_qgemv_meta", x, packed, meta, K, bits,
                         group_size, out)


def qgemm_meta(x, packed, meta, K: int, bits: int, group_size: int, out=None):
    """qgemm with compact group words."""
    return _product_meta(qgemm_meta_raw, "lowbit_qgemm_meta", x, packed, meta, K, bits,
                         group_size, out)


def gptq_workspace_bytes(N: int, K: int) -> int:
    return int(load_library().lowbit_gptq_workspace_bytes(N, K))


def quantize_gptq_raw(w, N, K, x, n, damp, bits, group_size, codes, packed, scales, zeros,
                      workspace, workspace_bytes, stream) -> int:
    return load_library().lowbit_quantize_gptq(w, N, K, x, n, float(damp), bits, group_size,
                                               codes, packed, scales, zeros, workspace,
                                               workspace_bytes, stream)


def quantize_gptq_sym_raw(w, N, K, x, n, damp, bits, group_size, codes, packed, scales, zeros,
                          workspace, workspace_bytes, stream) -> int:
    return load_library().lowbit_quantize_gptq_sym(w, N, K, x, n, float(damp), bits, group_size,
                                                   codes, packed, scales, zeros, workspace,
                                                   workspace_bytes, stream)


def quantize_gptq_noalloc_raw(w, N, K, x, n, damp, bits, group_size, codes, packed, scales,
                              zeros, status, stream) -> int:
    """lowbit_quantize_gptq_noalloc: the min-max error-feedback quantizer in the
    library's static device scratch (no workspace argument, nothing allocated);
    `status` is a device int32 address or None."""
    return load_library().lowbit_quantize_gptq_noalloc(w, N, K, x, n, float(damp), bits,
                                                       group_size, codes, packed, scales, zeros,
                                                       status, stream)


def quantize_gptq(w, x_calib, bits: int, group_size: int, damp: float = 0.01,
                  codes: bool = True, packed: bool = True, workspace=None,
                  symmetric: bool = False) -> dict:
    """Error-feedback (GPTQ) quantization of fp16 w[N][K] with the Hessian of
    the fp16 calibration rows x_calib[n][K], on the GPU in fp64.  Returns the
    outputs of quantize_rtn plus ``status`` (device int32: 0, or 1 when the
    Hessian was not positive definite).  ``workspace``: optional uint8 device
    tensor of at least gptq_workspace_bytes(N, K) bytes.  ``symmetric`` selects
    the signed symmetric grid of quantize_rtn(symmetric=True)."""
    torch = _torch()
    _require_gpu_tensor(w, "w", torch.float16)
    _require_gpu_tensor(x_calib, "x_calib", torch.float16)
    N, K = w.shape
    if x_calib.dim() != 2 or x_calib.shape[1] != K:
        raise ValueError("x_calib must be [n][K]")
    G = groups(K, group_size)
    dev = w.device
    need = gptq_workspace_bytes(N, K)
    if need < 0:
        _check(need, "lowbit_gptq_workspace_bytes")
    if workspace is None:
        workspace = torch.empty(need + 256, dtype=torch.uint8, device=dev)
    off = (-workspace.data_ptr()) % 256
    ws_ptr = workspace.data_ptr() + off
    out = {"scales": torch.empty((N, G), dtype=torch.float16, device=dev),
           "zeros": torch.empty((N, G), dtype=torch.int32, device=dev)}
    if codes:
        out["codes"] = torch.empty((N, K), dtype=torch.uint8, device=dev)
    if packed:
        out["packed"] = torch.empty((N, packed_words(K, bits)), dtype=torch.int32, device=dev)
    raw, name = ((quantize_gptq_sym_raw, "lowbit_quantize_gptq_sym") if symmetric
                 else (quantize_gptq_raw, "lowbit_quantize_gptq"))
    st = raw(w.data_ptr(), N, K, x_calib.data_ptr(), x_calib.shape[0], damp, bits, group_size,
             _ptr(out.get("codes")), _ptr(out.get("packed")), out["scales"].data_ptr(),
             out["zeros"].data_ptr(), ws_ptr, workspace.numel() - off, _stream_handle(dev))
    _check(st, name)
    out["status"] = workspace[off:off + 4].view(torch.int32)
    return out
