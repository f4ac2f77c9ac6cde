"""Compact group metadata on the GPU: lowbit_pack_meta against the oracle's
words (bit-exact, with the saturation count), and the products reading the
words (lowbit_qgemv_meta / lowbit_qgemm_meta) against the products reading
separate scales and zeros (bit-identical y) and against the oracle (within
|y - y_ref| <= 1e-3 |y_ref| + 1e-4), for every width and scale layout,
ragged shapes and the two grouped workload layers at full size."""
from __future__ import annotations

import sys

import numpy as np
import pytest

import harness
import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lw():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import weight_only_bit_rtn_amd as lw
    lw.load_library()
    return lw


def _say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def _to_gpu(a):
    import torch
    if a.dtype == np.uint32:
        a = a.view(np.int32)
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")


@pytest.mark.parametrize("N,G", [(1, 1), (7, 3), (129, 64), (1000, 172), (4096, 1)])
def test_pack_meta_matches_oracle(lw, N, G):
    import torch
    rng = np.random.default_rng(N + G)
    sb = rng.integers(0, 0x7C00, (N, G)).astype(np.uint16)
    z = rng.integers(-60000, 60000, (N, G)).astype(np.int32)
    z[::2] = rng.integers(-300, 300, z[::2].shape)     # mostly in range
    want, want_sat = harness.oracle.pack_meta(sb.view(np.float16), z)
    sat = torch.full((1,), 5, dtype=torch.int32, device="cuda:0")   # the count is added
    meta = lw.pack_meta(_to_gpu(sb.view(np.float16)), _to_gpu(z), saturated=sat)
    torch.cuda.synchronize()
    assert np.array_equal(meta.cpu().numpy().view(np.uint32), want)
    assert int(sat.item()) == 5 + want_sat


def _products_agree(lw, w, bits, g, batches, what):
    import torch
    N, K = w.shape
    codes, scales, zeros, packed = harness.oracle_quantize(w, bits, g)
    meta_ref, sat = harness.oracle.pack_meta(scales, zeros)
    assert sat == 0
    p, s, z = _to_gpu(packed), _to_gpu(scales), _to_gpu(zeros)
    meta = lw.pack_meta(s, z)
    torch.cuda.synchronize()
    assert np.array_equal(meta.cpu().numpy().view(np.uint32), meta_ref), what
    for B in batches:
        x = _to_gpu(synth.normal_f16(B, K, 1.0, seed=B + 3, stream=2))
        kerns = [("qgemv", "qgemv_meta")] if B <= lw.QGEMV_MAX_B else []
        kerns.append(("qgemm", "qgemm_meta"))
        y_ref = harness.oracle_y(x.cpu().numpy(), packed, scales, zeros, K, bits, g)
        for plain, compact in kerns:
            y1 = getattr(lw, plain)(x, p, s, z, K, bits, g)
            y2 = getattr(lw, compact)(x, p, meta, K, bits, g)
            torch.cuda.synchronize()
            assert torch.equal(y1.view(torch.int16), y2.view(torch.int16)), \
                f"{what} {compact} B={B}: differs from {plain}"
            harness.assert_y_close(y2.cpu().numpy(), y_ref, f"{what} {compact} B={B}")


CASES = [(2, 67, 4160, 64), (2, 33, 8256, 0), (2, 21, 1408, 128), (2, 17, 4160, 32),
         (3, 67, 4224, 0), (3, 33, 8320, 64), (3, 19, 4224, 96),
         (4, 67, 4128, 96), (4, 70, 4224, 128), (4, 17, 1280, 256), (4, 40, 8192, 1024),
         (8, 67, 4128, 0), (8, 33, 640, 128), (8, 21, 4224, 32)]


@pytest.mark.parametrize("bits,N,K,g", CASES)
def test_meta_products(lw, bits, N, K, g):
    _say(f"[meta products] bits={bits} N={N} K={K} g={g}")
    rng = np.random.default_rng(bits * 100 + N)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    w[1::5] = np.float16(-0.37)          # constant rows: zero points at the grid's end
    _products_agree(lw, w, bits, g, [1, 4, 9, 16, 33, 64], f"bits={bits} N={N} K={K} g={g}")


def test_meta_saturation_is_counted(lw):
    import torch
    w = np.zeros((3, 256), np.float16)
    w[0, :128] = np.float16(40000.0)     # a constant group: zero = -40000
    w[1, 128:] = np.float16(-33000.0)    # zero = 33000
    out = lw.quantize_rtn(_to_gpu(w), 4, 128)
    sat = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    meta = lw.pack_meta(out["scales"], out["zeros"], saturated=sat)
    torch.cuda.synchronize()
    assert int(sat.item()) == 2
    hi = (meta.cpu().numpy().view(np.uint32) >> 16).astype(np.uint16).view(np.int16)
    assert hi[0, 0] == -32768 and hi[1, 1] == 32767


FULL = [L for L in harness.all_layers() if L.group_size > 0 and L.name in (
    "llama7b_up_11008x4096", "llama70b_up_28672x8192")]


@pytest.mark.parametrize("layer", FULL, ids=lambda L: L.name)
def test_meta_full_size(lw, layer):
    """The grouped workload layers at full size, in the launch configuration
    the benchmark times: compact-word products bit-identical to the plain ones."""
    import torch
    _say(f"[meta full size] {layer.name}")
    d = harness.layer_data(layer)
    p, s, z = _to_gpu(d.packed), _to_gpu(d.scales), _to_gpu(d.zeros)
    meta = lw.pack_meta(s, z)
    K, bits, g = layer.K, layer.bits, layer.group_size
    for B in layer.batches:
        x = _to_gpu(d.x(B))
        plain, compact = ("qgemv", "qgemv_meta") if B <= lw.QGEMV_MAX_B else ("qgemm", "qgemm_meta")
        y1 = getattr(lw, plain)(x, p, s, z, K, bits, g)
        y2 = getattr(lw, compact)(x, p, meta, K, bits, g)
        torch.cuda.synchronize()
        assert torch.equal(y1.view(torch.int16), y2.view(torch.int16)), f"{layer.name} B={B}"
