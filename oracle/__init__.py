"""CPU oracle for weight-only low-bit RTN quantization (test infrastructure).

TEST INFRASTRUCTURE ONLY: the test suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` are the only callers.  The product path (the
HIP library ``weight_only_bit_rtn_amd``) never imports this package, and this
package never imports the product path; the two share no code.

The arithmetic lives in ``lowbit_oracle.c`` (plain C, single-threaded); this
module only marshals numpy arrays into it.  The C source's header states the
passage each step follows and the readings taken where the pages are silent.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build as _build


def _c(a: np.ndarray, dtype) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != dtype:
        raise TypeError(f"expected {np.dtype(dtype)}, got {a.dtype}")
    return a


def _bits16(a: np.ndarray) -> np.ndarray:
    """fp16 arrays are passed to the C code as their uint16 bit patterns."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.float16:
        return a.view(np.uint16)
    return _c(a, np.uint16)


def _ok(rc: int, what: str) -> None:
    if rc != 0:
        raise ValueError(f"oracle {what}: bad argument (rc={rc})")


def groups(K: int, group_size: int) -> int:
    return 1 if group_size == 0 else K // group_size


class Oracle:
    """numpy front end of one build of the C oracle (a path to its .so)."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        i64, i32, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
        lib.orc_f16_to_f64.argtypes = [ctypes.c_uint16]
        lib.orc_f16_to_f64.restype = ctypes.c_double
        lib.orc_f64_to_f16.argtypes = [ctypes.c_double]
        lib.orc_f64_to_f16.restype = ctypes.c_uint16
        lib.orc_quantize_rtn.argtypes = [vp, i64, i64, i32, i64, vp, vp, vp]
        lib.orc_quantize_rtn_sym.argtypes = [vp, i64, i64, i32, i64, vp, vp, vp]
        lib.orc_pack.argtypes = [vp, i64, i64, i32, vp]
        lib.orc_unpack.argtypes = [vp, i64, i64, i32, vp]
        lib.orc_dequant.argtypes = [vp, vp, vp, i64, i64, i32, i64, vp]
        lib.orc_matmul_f64.argtypes = [vp, vp, i64, i64, i64, vp]
        lib.orc_pack_meta.argtypes = [vp, vp, i64, vp]
        lib.orc_pack_meta.restype = ctypes.c_int64
        lib.orc_unpack_meta.argtypes = [vp, i64, vp, vp]
        lib.orc_unpack_meta.restype = ctypes.c_int
        lib.orc_hessian.argtypes = [vp, i64, i64, ctypes.c_double, vp]
        lib.orc_hessian.restype = ctypes.c_int
        lib.orc_quantize_gptq.argtypes = [vp, i64, i64, vp, i32, i64, vp, vp, vp, vp]
        lib.orc_quantize_gptq.restype = ctypes.c_int
        lib.orc_quantize_gptq_sym.argtypes = [vp, i64, i64, vp, i32, i64, vp, vp, vp, vp]
        lib.orc_quantize_gptq_sym.restype = ctypes.c_int
        for name in ("orc_quantize_rtn", "orc_quantize_rtn_sym", "orc_pack", "orc_unpack",
                     "orc_dequant", "orc_matmul_f64"):
            getattr(lib, name).restype = ctypes.c_int
        self.lib = lib
        self.path = path

    def f16_to_f64(self, h: int) -> float:
        return self.lib.orc_f16_to_f64(int(h) & 0xFFFF)

    def f64_to_f16(self, v: float) -> int:
        return int(self.lib.orc_f64_to_f16(float(v)))

    def quantize_rtn(self, w: np.ndarray, bits: int, group_size: int):
        """RTN min-max quantization of fp16 ``w[N][K]``.

        Returns ``(codes uint8[N][K], scales fp16[N][G], zeros int32[N][G])``.
        """
        wb = _bits16(w)
        N, K = wb.shape
        G = groups(K, group_size)
        codes = np.empty((N, K), np.uint8)
        scales = np.empty((N, G), np.uint16)
        zeros = np.empty((N, G), np.int32)
        _ok(self.lib.orc_quantize_rtn(wb.ctypes.data, N, K, bits, group_size,
                                      codes.ctypes.data, scales.ctypes.data,
                                      zeros.ctypes.data), "quantize_rtn")
        return codes, scales.view(np.float16), zeros

    def quantize_rtn_sym(self, w: np.ndarray, bits: int, group_size: int):
        """Signed symmetric RTN quantization of fp16 ``w[N][K]`` (codes stored
        with the zero point 2^(bits-1)); same outputs as ``quantize_rtn``."""
        wb = _bits16(w)
        N, K = wb.shape
        G = groups(K, group_size)
        codes = np.empty((N, K), np.uint8)
        scales = np.empty((N, G), np.uint16)
        zeros = np.empty((N, G), np.int32)
        _ok(self.lib.orc_quantize_rtn_sym(wb.ctypes.data, N, K, bits, group_size,
                                          codes.ctypes.data, scales.ctypes.data,
                                          zeros.ctypes.data), "quantize_rtn_sym")
        return codes, scales.view(np.float16), zeros

    def pack(self, codes: np.ndarray, bits: int) -> np.ndarray:
        codes = _c(codes, np.uint8)
        N, K = codes.shape
        out = np.empty((N, K * bits // 32), np.uint32)
        _ok(self.lib.orc_pack(codes.ctypes.data, N, K, bits, out.ctypes.data), "pack")
        return out

    def unpack(self, packed: np.ndarray, K: int, bits: int) -> np.ndarray:
        packed = _c(packed, np.uint32)
        N = packed.shape[0]
        out = np.empty((N, K), np.uint8)
        _ok(self.lib.orc_unpack(packed.ctypes.data, N, K, bits, out.ctypes.data), "unpack")
        return out

    def hessian(self, x: np.ndarray, damp: float) -> np.ndarray:
        """H = (2/n) X^T X + damp * mean(diag) * I for fp16 x[n][K], fp64."""
        xb = _bits16(x)
        n, K = xb.shape
        H = np.empty((K, K), np.float64)
        _ok(self.lib.orc_hessian(xb.ctypes.data, n, K, float(damp), H.ctypes.data), "hessian")
        return H

    def quantize_gptq(self, w: np.ndarray, H: np.ndarray, bits: int, group_size: int,
                      symmetric: bool = False):
        """Error-feedback codes of fp16 w[N][K] on the RTN grid of w (min-max,
        or signed symmetric), with the Hessian H[K][K]; returns (codes,
        scales, zeros) as quantize_rtn."""
        wb = _bits16(w)
        N, K = wb.shape
        Hc = np.ascontiguousarray(H, dtype=np.float64)
        assert Hc.shape == (K, K)
        G = groups(K, group_size)
        codes = np.empty((N, K), np.uint8)
        scales = np.empty((N, G), np.uint16)
        zeros = np.empty((N, G), np.int32)
        work = np.empty(3 * K * K + N * K, np.float64)
        fn = self.lib.orc_quantize_gptq_sym if symmetric else self.lib.orc_quantize_gptq
        _ok(fn(wb.ctypes.data, N, K, Hc.ctypes.data, bits, group_size, codes.ctypes.data,
               scales.ctypes.data, zeros.ctypes.data, work.ctypes.data), "quantize_gptq")
        return codes, scales.view(np.float16), zeros

    def pack_meta(self, scales: np.ndarray, zeros: np.ndarray):
        """Compact words (fp16 scale | int16 zero << 16), same shape as
        ``scales``, and the number of zero points saturated to int16."""
        sb = _bits16(scales)
        zz = np.ascontiguousarray(zeros, dtype=np.int32)
        assert sb.shape == zz.shape
        out = np.empty(sb.shape, np.uint32)
        n = self.lib.orc_pack_meta(sb.ctypes.data, zz.ctypes.data, sb.size, out.ctypes.data)
        if n < 0:
            raise ValueError("oracle pack_meta: bad argument")
        return out, int(n)

    def unpack_meta(self, meta: np.ndarray):
        m = np.ascontiguousarray(meta, dtype=np.uint32)
        sb = np.empty(m.shape, np.uint16)
        zz = np.empty(m.shape, np.int32)
        _ok(self.lib.orc_unpack_meta(m.ctypes.data, m.size, sb.ctypes.data, zz.ctypes.data),
            "unpack_meta")
        return sb.view(np.float16), zz

    def dequant(self, codes: np.ndarray, scales: np.ndarray, zeros: np.ndarray, bits: int,
                group_size: int) -> np.ndarray:
        codes = _c(codes, np.uint8)
        sb = _bits16(scales)
        zeros = _c(zeros, np.int32)
        N, K = codes.shape
        out = np.empty((N, K), np.float64)
        _ok(self.lib.orc_dequant(codes.ctypes.data, sb.ctypes.data, zeros.ctypes.data, N, K,
                                 bits, group_size, out.ctypes.data), "dequant")
        return out

    def matmul_f64(self, x: np.ndarray, deq: np.ndarray) -> np.ndarray:
        xb = _bits16(x)
        db = _c(deq, np.float64)
        B, K = xb.shape
        N = db.shape[0]
        if db.shape[1] != K:
            raise ValueError("x and deq disagree on K")
        y = np.empty((B, N), np.float64)
        _ok(self.lib.orc_matmul_f64(xb.ctypes.data, db.ctypes.data, B, N, K, y.ctypes.data),
            "matmul_f64")
        return y

    def reference_y(self, x: np.ndarray, packed: np.ndarray, scales: np.ndarray,
                    zeros: np.ndarray, K: int, bits: int, group_size: int) -> np.ndarray:
        """fp64 y = x * deq(packed)^T for the rows present in ``packed``."""
        codes = self.unpack(packed, K, bits)
        deq = self.dequant(codes, scales, zeros, bits, group_size)
        return self.matmul_f64(x, deq)


_DEFAULT: Oracle | None = None


def default() -> Oracle:
    """The oracle built from ``lowbit_oracle.c`` (compiled on first use)."""
    global _DEFAULT
    if _DEFAULT is None:
        path = _build.library_path()
        src = os.path.join(os.path.dirname(os.path.abspath(__file__)), "lowbit_oracle.c")
        if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(src):
            _build.build()
        _DEFAULT = Oracle(path)
    return _DEFAULT


def pack_meta(scales, zeros):
    return default().pack_meta(scales, zeros)


def unpack_meta(meta):
    return default().unpack_meta(meta)


def hessian(x, damp):
    return default().hessian(x, damp)


def quantize_gptq(w, H, bits, group_size, symmetric=False):
    return default().quantize_gptq(w, H, bits, group_size, symmetric)


def f16_to_f64(h):
    return default().f16_to_f64(h)


def f64_to_f16(v):
    return default().f64_to_f16(v)


def quantize_rtn(w, bits, group_size):
    return default().quantize_rtn(w, bits, group_size)


def quantize_rtn_sym(w, bits, group_size):
    return default().quantize_rtn_sym(w, bits, group_size)


def pack(codes, bits):
    return default().pack(codes, bits)


def unpack(packed, K, bits):
    return default().unpack(packed, K, bits)


def dequant(codes, scales, zeros, bits, group_size):
    return default().dequant(codes, scales, zeros, bits, group_size)


def matmul_f64(x, deq):
    return default().matmul_f64(x, deq)


def reference_y(x, packed, scales, zeros, K, bits, group_size):
    return default().reference_y(x, packed, scales, zeros, K, bits, group_size)
