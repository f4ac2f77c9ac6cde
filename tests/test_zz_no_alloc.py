"""lowbit_quantize_gptq_noalloc (the entry point that allocates nothing: its
workspace is the library's static device scratch) against
lowbit_quantize_gptq with a caller workspace, through the C ABI: codes,
packed words, scales, zeros and the status word identical, on two calls in a
row (the second smaller, so it runs over what the first left in the
scratch), then a calibration set of zeros (Hessian not positive definite,
status 1 from both)."""
from __future__ import annotations

import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu


def _say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def lw():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import weight_only_bit_rtn_amd as lw
    lw.load_library()
    return lw


def _run_both(lw, w: np.ndarray, x: np.ndarray, bits: int, g: int):
    import torch
    dev = torch.device("cuda:0")
    N, K = w.shape
    n = x.shape[0]
    G = 1 if g == 0 else K // g
    stream = torch.cuda.current_stream().cuda_stream
    wd = torch.from_numpy(w).to(dev)
    xd = torch.from_numpy(x).to(dev)

    def outputs():
        return {"codes": torch.full((N, K), 0xAB, dtype=torch.uint8, device=dev),
                "packed": torch.full((N, K * bits // 32), -1, dtype=torch.int32, device=dev),
                "scales": torch.zeros((N, G), dtype=torch.float16, device=dev),
                "zeros": torch.full((N, G), 77, dtype=torch.int32, device=dev),
                "status": torch.full((4,), -9, dtype=torch.int32, device=dev)}

    ref = outputs()
    need = lw.gptq_workspace_bytes(N, K)
    ws = torch.empty(need + 256, dtype=torch.uint8, device=dev)
    off = (-ws.data_ptr()) % 256
    st = lw.quantize_gptq_raw(wd.data_ptr(), N, K, xd.data_ptr(), n, 0.01, bits, g,
                              ref["codes"].data_ptr(), ref["packed"].data_ptr(),
                              ref["scales"].data_ptr(), ref["zeros"].data_ptr(),
                              ws.data_ptr() + off, need, stream)
    assert st == 0, lw.status_string(st)
    torch.cuda.synchronize()
    ref["status"][0] = int(ws[off:off + 4].view(torch.int32).item())

    got = outputs()
    st = lw.quantize_gptq_noalloc_raw(wd.data_ptr(), N, K, xd.data_ptr(), n, 0.01, bits, g,
                                      got["codes"].data_ptr(), got["packed"].data_ptr(),
                                      got["scales"].data_ptr(), got["zeros"].data_ptr(),
                                      got["status"].data_ptr(), stream)
    assert st == 0, lw.status_string(st)
    torch.cuda.synchronize()
    return ({k: v.cpu().numpy() for k, v in ref.items()},
            {k: v.cpu().numpy() for k, v in got.items()})


def _inputs(N, K, n, seed, zero_x=False):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    x = np.zeros((n, K), np.float16) if zero_x else rng.standard_normal((n, K)).astype(np.float16)
    return w, x


def _assert_same(ref, got, what):
    for key in ("codes", "packed", "zeros"):
        bad = np.argwhere(ref[key] != got[key])
        assert bad.size == 0, f"{what}: {key} differ at {bad[:5].tolist()}"
    assert np.array_equal(ref["scales"].view(np.uint16), got["scales"].view(np.uint16)), what
    assert ref["status"][0] == got["status"][0], (what, ref["status"][0], got["status"][0])


def test_noalloc_matches_workspace_entry_two_calls(lw):
    # first call: 300 x 512, 4-bit groups of 128; second, smaller: 130 x 256,
    # 2-bit groups of 64 (it runs over the first call's leftovers)
    cases = [(300, 512, 1024, 4, 128, 1), (130, 256, 512, 2, 64, 2)]
    for N, K, n, bits, g, seed in cases:
        what = f"N={N} K={K} bits={bits} g={g}"
        _say(f"[noalloc] {what}")
        w, x = _inputs(N, K, n, seed)
        ref, got = _run_both(lw, w, x, bits, g)
        assert got["status"][0] == 0
        _assert_same(ref, got, what)


def test_noalloc_reports_not_positive_definite(lw):
    _say("[noalloc] zero calibration inputs")
    w, x = _inputs(64, 128, 32, 3, zero_x=True)
    ref, got = _run_both(lw, w, x, 4, 0)
    assert ref["status"][0] == 1 and got["status"][0] == 1


def test_noalloc_largest_layer(lw):
    """The 2048 x 2048 layer, the largest workload shape the scratch holds."""
    _say("[noalloc] 2048 x 2048, 4-bit, groups of 128")
    w, x = _inputs(2048, 2048, 2048, 4)
    ref, got = _run_both(lw, w, x, 4, 128)
    assert got["status"][0] == 0
    _assert_same(ref, got, "2048x2048")


def test_noalloc_rejects_too_large(lw):
    st = lw.quantize_gptq_noalloc_raw(16, 11008, 4096, 16, 64, 0.01, 2, 64, 16, 16, 16, 16,
                                      None, None)
    assert st == lw.LOWBIT_ERR_SCRATCH
