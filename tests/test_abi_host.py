"""Host-side checks of the C ABI (no GPU needed, nothing is launched).

The library must load, export exactly the entry points ``include/lowbit.h``
declares, and reject bad arguments on the host before touching a device.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lowbit.h")


@pytest.fixture(scope="module")
def lw():
    import weight_only_bit_rtn_amd as lw
    if not os.path.exists(lw.LIB_PATH):
        from weight_only_bit_rtn_amd import build
        build.build()
    lw.load_library()
    return lw


def declared_entry_points():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"LOWBIT_API\s+[\w\s\*]+?\b(lowbit_\w+)\s*\(", text)))


def test_header_declares_the_abi():
    assert declared_entry_points() == sorted(
        ["lowbit_pack", "lowbit_pack_meta", "lowbit_qgemm", "lowbit_qgemm_meta", "lowbit_qgemv",
         "lowbit_qgemv_meta", "lowbit_quantize_gptq", "lowbit_quantize_gptq_sym",
         "lowbit_quantize_gptq_noalloc", "lowbit_quantize_rtn",
         "lowbit_quantize_rtn_sym", "lowbit_gptq_workspace_bytes", "lowbit_status_string"])


def test_library_exports_every_declared_symbol(lw):
    lib = ctypes.CDLL(lw.LIB_PATH)
    for name in declared_entry_points():
        assert hasattr(lib, name), name
    assert set(lw.EXPORTED) == set(declared_entry_points())


def test_header_constants_match_binding(lw):
    text = open(HEADER).read()
    consts = dict(re.findall(r"#define\s+(LOWBIT_\w+)\s+\(?(-?\d+)\)?", text))
    assert int(consts["LOWBIT_OK"]) == lw.LOWBIT_OK
    assert int(consts["LOWBIT_ERR_ARG"]) == lw.LOWBIT_ERR_ARG
    assert int(consts["LOWBIT_ERR_SHAPE"]) == lw.LOWBIT_ERR_SHAPE
    assert int(consts["LOWBIT_ERR_UNSUPPORTED"]) == lw.LOWBIT_ERR_UNSUPPORTED
    assert int(consts["LOWBIT_ERR_HIP"]) == lw.LOWBIT_ERR_HIP
    assert int(consts["LOWBIT_QGEMV_MAX_B"]) == lw.QGEMV_MAX_B
    assert int(consts["LOWBIT_QUANTIZE_MAX_K"]) == lw.QUANTIZE_MAX_K
    assert int(consts["LOWBIT_ERR_SCRATCH"]) == lw.LOWBIT_ERR_SCRATCH
    assert int(consts["LOWBIT_GPTQ_NOALLOC_MAX_BYTES"]) == lw.GPTQ_NOALLOC_MAX_BYTES


def test_status_strings(lw):
    for st in (0, -1, -2, -3, -4, -5, 17):
        s = lw.status_string(st)
        assert isinstance(s, str) and s
    assert lw.status_string(0) == "ok"


# Fake, never-dereferenced addresses: every call below must fail validation
# (or be an empty problem) and return before any HIP call.
P = 0x7F0000000000
MIS = P + 4


HOST_VALIDATION_CASES = [
    # bit width
    (lambda lw: lw.quantize_rtn_raw(P, 4, 128, 5, 0, P, P, P, P, None), "UNSUPPORTED"),
    (lambda lw: lw.pack_raw(P, 4, 128, 1, P, None), "UNSUPPORTED"),
    (lambda lw: lw.qgemv_raw(P, 1, P, P, P, 4, 128, 6, 0, P, None), "UNSUPPORTED"),
    (lambda lw: lw.qgemm_raw(P, 1, P, P, P, 4, 128, 7, 0, P, None), "UNSUPPORTED"),
    (lambda lw: lw.quantize_rtn_sym_raw(P, 4, 128, 5, 0, P, P, P, P, None), "UNSUPPORTED"),
    (lambda lw: lw.qgemm_raw(P, 1, P, P, P, 4, 128, 0, 0, P, None), "UNSUPPORTED"),
    # shapes
    (lambda lw: lw.quantize_rtn_raw(P, 4, 0, 4, 0, P, P, P, P, None), "SHAPE"),
    (lambda lw: lw.quantize_rtn_raw(P, 4, 48, 4, 0, P, P, P, P, None), "SHAPE"),
    (lambda lw: lw.quantize_rtn_raw(P, 4, 96, 3, 0, P, P, P, P, None), "SHAPE"),
    (lambda lw: lw.quantize_rtn_raw(P, 4, 96, 2, 0, P, P, P, P, None), "SHAPE"),
    (lambda lw: lw.quantize_rtn_raw(P, 4, 256, 4, 48, P, P, P, P, None), "SHAPE"),
    (lambda lw: lw.quantize_rtn_raw(P, 4, 256, 4, 96, P, P, P, P, None), "SHAPE"),
    (lambda lw: lw.quantize_rtn_raw(P, 4, 262144, 4, 0, P, P, P, P, None), "SHAPE"),
    (lambda lw: lw.qgemv_raw(P, 1, P, P, P, 4, 160, 4, 64, P, None), "SHAPE"),
    (lambda lw: lw.pack_raw(P, 4, 64, 3, P, None), "SHAPE"),
    # arguments
    (lambda lw: lw.quantize_rtn_raw(P, -1, 128, 4, 0, P, P, P, P, None), "ARG"),
    (lambda lw: lw.quantize_rtn_raw(P, 4, 128, 4, -32, P, P, P, P, None), "ARG"),
    (lambda lw: lw.quantize_rtn_raw(None, 4, 128, 4, 0, P, P, P, P, None), "ARG"),
    (lambda lw: lw.quantize_rtn_raw(P, 4, 128, 4, 0, None, None, P, P, None), "ARG"),
    (lambda lw: lw.quantize_rtn_raw(P, 4, 128, 4, 0, MIS, None, P, P, None), "ARG"),
    (lambda lw: lw.pack_raw(None, 4, 128, 4, P, None), "ARG"),
    # the symmetric entry point shares the validation
    (lambda lw: lw.quantize_rtn_sym_raw(P, 4, 128, 1, 0, P, P, P, P, None), "UNSUPPORTED"),
    (lambda lw: lw.quantize_rtn_sym_raw(P, 4, 256, 4, 96, P, P, P, P, None), "SHAPE"),
    (lambda lw: lw.quantize_rtn_sym_raw(P, 4, 262144, 2, 0, P, P, P, P, None), "SHAPE"),
    (lambda lw: lw.quantize_rtn_sym_raw(P, 4, 128, 4, 0, None, None, P, P, None), "ARG"),
    (lambda lw: lw.quantize_rtn_sym_raw(P, 4, 128, 4, 0, P, MIS, P, P, None), "ARG"),
    (lambda lw: lw.quantize_rtn_sym_raw(None, 0, 128, 4, 0, None, None, None, None, None),
     "OK"),
    (lambda lw: lw.qgemv_raw(P, 16, P, P, P, 4, 128, 4, 0, P, None), "ARG"),
    (lambda lw: lw.qgemv_raw(P, -1, P, P, P, 4, 128, 4, 0, P, None), "ARG"),
    (lambda lw: lw.qgemv_raw(P, 1, None, P, P, 4, 128, 4, 0, P, None), "ARG"),
    (lambda lw: lw.qgemm_raw(P, 1, P, P, P, 4, 128, 4, 0, MIS, None), "ARG"),
    (lambda lw: lw.qgemm_raw(MIS, 1, P, P, P, 4, 128, 4, 0, P, None), "ARG"),
    # activations off a 16-byte boundary, at a batch the matrix-core GEMV takes
    (lambda lw: lw.qgemv_raw(MIS, 12, P, P, P, 4100, 2048, 2, 64, P, None), "ARG"),
    (lambda lw: lw.qgemv_meta_raw(MIS, 12, P, P, 4100, 2048, 2, 64, P, None), "ARG"),
    # compact metadata entry points
    (lambda lw: lw.pack_meta_raw(P, P, -1, 4, P, None, None), "ARG"),
    (lambda lw: lw.pack_meta_raw(None, P, 4, 4, P, None, None), "ARG"),
    (lambda lw: lw.pack_meta_raw(P, P, 4, 4, MIS, None, None), "ARG"),
    (lambda lw: lw.pack_meta_raw(P, P, 4, 4, P, P + 2, None), "ARG"),
    (lambda lw: lw.qgemv_meta_raw(P, 16, P, P, 4, 128, 4, 0, P, None), "ARG"),
    (lambda lw: lw.qgemv_meta_raw(P, 1, P, None, 4, 128, 4, 0, P, None), "ARG"),
    (lambda lw: lw.qgemm_meta_raw(P, 1, P, MIS, 4, 128, 4, 0, P, None), "ARG"),
    (lambda lw: lw.qgemm_meta_raw(P, 1, P, P, 4, 128, 5, 0, P, None), "UNSUPPORTED"),
    (lambda lw: lw.qgemv_meta_raw(P, 1, P, P, 4, 160, 4, 64, P, None), "SHAPE"),
    (lambda lw: lw.pack_meta_raw(None, None, 0, 4, None, None, None), "OK"),
    (lambda lw: lw.qgemm_meta_raw(None, 0, None, None, 4, 128, 4, 0, None, None), "OK"),
    # error-feedback quantization (workspace of 1 MiB at a fake 256-aligned address)
    (lambda lw: lw.quantize_gptq_raw(P, 4, 128, P, 64, 0.01, 6, 0, P, P, P, P, P, 1 << 20, None),
     "UNSUPPORTED"),
    (lambda lw: lw.quantize_gptq_raw(P, 4, 96, P, 64, 0.01, 4, 64, P, P, P, P, P, 1 << 20, None),
     "SHAPE"),
    (lambda lw: lw.quantize_gptq_raw(P, 4, 128, P, 64, 0.0, 4, 0, P, P, P, P, P, 1 << 20, None),
     "ARG"),
    (lambda lw: lw.quantize_gptq_raw(P, 4, 128, P, 0, 0.01, 4, 0, P, P, P, P, P, 1 << 20, None),
     "ARG"),
    (lambda lw: lw.quantize_gptq_raw(P, 4, 128, P, 64, 0.01, 4, 0, P, P, P, P, P + 16, 1 << 20,
                                     None), "ARG"),
    (lambda lw: lw.quantize_gptq_raw(P, 4, 128, P, 64, 0.01, 4, 0, P, P, P, P, P, 1024, None),
     "ARG"),
    (lambda lw: lw.quantize_gptq_raw(P, 4, 128, None, 64, 0.01, 4, 0, P, P, P, P, P, 1 << 20,
                                     None), "ARG"),
    (lambda lw: lw.quantize_gptq_raw(None, 0, 128, None, 64, 0.01, 4, 0, None, None, None, None,
                                     None, 0, None), "OK"),
    (lambda lw: lw.quantize_gptq_sym_raw(P, 4, 128, P, 64, 0.01, 5, 0, P, P, P, P, P, 1 << 20,
                                         None), "UNSUPPORTED"),
    (lambda lw: lw.quantize_gptq_sym_raw(P, 4, 128, P, 64, -1.0, 4, 0, P, P, P, P, P, 1 << 20,
                                         None), "ARG"),
    (lambda lw: lw.quantize_gptq_sym_raw(P, 4, 128, P, 64, 0.01, 4, 0, P, P, P, P, P, 1024,
                                         None), "ARG"),
    (lambda lw: lw.quantize_gptq_sym_raw(None, 0, 128, None, 64, 0.01, 4, 0, None, None, None,
                                         None, None, 0, None), "OK"),
    # the no-allocation error-feedback entry point: same checks, plus the
    # static scratch bound (11008 x 4096 needs ~513 MB) and the status word
    (lambda lw: lw.quantize_gptq_noalloc_raw(P, 4, 128, P, 64, 0.01, 6, 0, P, P, P, P, None,
                                             None), "UNSUPPORTED"),
    (lambda lw: lw.quantize_gptq_noalloc_raw(P, 4, 96, P, 64, 0.01, 4, 64, P, P, P, P, None,
                                             None), "SHAPE"),
    (lambda lw: lw.quantize_gptq_noalloc_raw(P, 4, 128, P, 64, 0.0, 4, 0, P, P, P, P, None,
                                             None), "ARG"),
    (lambda lw: lw.quantize_gptq_noalloc_raw(P, 4, 128, P, 64, 0.01, 4, 0, P, P, P, P, P + 2,
                                             None), "ARG"),
    (lambda lw: lw.quantize_gptq_noalloc_raw(P, 4, 128, None, 64, 0.01, 4, 0, P, P, P, P, None,
                                             None), "ARG"),
    (lambda lw: lw.quantize_gptq_noalloc_raw(P, 11008, 4096, P, 64, 0.01, 2, 64, P, P, P, P, P,
                                             None), "SCRATCH"),
    (lambda lw: lw.quantize_gptq_noalloc_raw(None, 0, 128, None, 64, 0.01, 4, 0, None, None,
                                             None, None, None, None), "OK"),
    # empty problems are valid and launch nothing
    (lambda lw: lw.quantize_rtn_raw(None, 0, 128, 4, 0, None, None, None, None, None), "OK"),
    (lambda lw: lw.qgemv_raw(None, 0, None, None, None, 8, 128, 4, 0, None, None), "OK"),
    (lambda lw: lw.qgemm_raw(None, 5, None, None, None, 0, 128, 4, 0, None, None), "OK"),
    (lambda lw: lw.pack_raw(None, 0, 128, 4, None, None), "OK"),
]


def expected_status(lw, status: str) -> int:
    return {"OK": lw.LOWBIT_OK, "ARG": lw.LOWBIT_ERR_ARG, "SHAPE": lw.LOWBIT_ERR_SHAPE,
            "UNSUPPORTED": lw.LOWBIT_ERR_UNSUPPORTED, "SCRATCH": lw.LOWBIT_ERR_SCRATCH}[status]


@pytest.mark.parametrize("call,status", HOST_VALIDATION_CASES)
def test_host_validation(lw, call, status):
    assert call(lw) == expected_status(lw, status)


def test_binding_refuses_cpu_tensors(lw):
    import torch
    w = torch.zeros(4, 128, dtype=torch.float16)
    with pytest.raises(ValueError):
        lw.quantize_rtn(w, 4, 0)


def test_gptq_noalloc_scratch_bound(lw):
    """The largest workspace the static scratch holds: the 2048 x 2048 layer
    fits, the Llama-7B 11008 x 4096 layer does not."""
    assert lw.gptq_workspace_bytes(2048, 2048) <= lw.GPTQ_NOALLOC_MAX_BYTES
    assert lw.gptq_workspace_bytes(11008, 4096) > lw.GPTQ_NOALLOC_MAX_BYTES


def test_gptq_workspace_size(lw):
    K, N = 4096, 11008
    up = lambda b: (b + 255) // 256 * 256
    nt = (K + 63) // 64  # 64 x 64 Cholesky tiles per side, one int32 counter each
    assert lw.gptq_workspace_bytes(N, K) == (256 + up(K * K * 8) + up(K * N * 8) + up(N * K)
                                             + up(nt * nt * 4))
    assert lw.gptq_workspace_bytes(-1, K) < 0
    assert lw.gptq_workspace_bytes(N, 0) < 0
