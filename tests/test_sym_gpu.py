"""The signed symmetric RTN grid on the GPU (lowbit_quantize_rtn_sym) against
the oracle's symmetric quantizer, and the two products on its output.

Bars as for the min-max grid: scales, zeros, codes and packed words
bit-exact; y within |y - y_ref| <= 1e-3 |y_ref| + 1e-4 per element.  The
shapes reach all three reduction layouts of the quantizer (one group per row,
groups inside a wave, groups spread over waves through LDS) with ragged last
rounds; the degenerate groups are all-zero, one-signed, a single nonzero,
values on the half-way points of the grid and groups whose largest magnitude
is negative.
"""
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


def _weights(kind: str, N: int, K: int, seed: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    if kind == "normal":
        return (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    if kind == "mixed":          # tiny, normal, constant and zero rows
        w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
        w[::3] *= 1e-3
        w[1::5] = -0.37
        w[2::7] = 0.0
        return w.astype(np.float16)
    if kind == "skewed":         # one-signed rows and negative extremes
        w = rng.uniform(0.1, 0.9, (N, K)).astype(np.float32)
        w[1::2] = -w[1::2] * 3
        return w.astype(np.float16)
    if kind == "wide":
        return (rng.standard_normal((N, K)) * 30).astype(np.float16)
    if kind == "tiny":           # subnormal scales
        return (rng.standard_normal((N, K)) * 3e-5).astype(np.float16)
    raise ValueError(kind)


def _check_quantize(lw, w, bits, g, what, codes_too=(True, False)):
    codes, scales, zeros, packed = harness.oracle_quantize(w, bits, g, symmetric=True)
    assert (zeros == 1 << (bits - 1)).all()
    for want_codes in codes_too:
        out = lw.quantize_rtn(_to_gpu(w), bits, g, codes=want_codes, packed=True,
                              symmetric=True)
        res = {k: v.cpu().numpy() for k, v in out.items()}
        sc = res["scales"].view(np.uint16)
        bad = np.argwhere(sc != scales.view(np.uint16))
        assert bad.size == 0, f"{what}: scales differ at {bad[:5].tolist()}"
        assert np.array_equal(res["zeros"], zeros), f"{what}: zeros"
        if want_codes:
            bad = np.argwhere(res["codes"] != codes)
            assert bad.size == 0, f"{what}: codes differ at {bad[:5].tolist()}"
        bad = np.argwhere(res["packed"].view(np.uint32) != packed)
        assert bad.size == 0, f"{what}: packed words differ at {bad[:5].tolist()}"
    return codes, scales, zeros, packed


SHAPES = {
    4: [(1, 32), (5, 96), (17, 2080), (67, 4128)],
    2: [(1, 64), (5, 192), (17, 4160), (67, 8256)],
    3: [(1, 128), (5, 384), (17, 4224), (67, 8320)],
}


def _shape_cases():
    for bits, shapes in SHAPES.items():
        for (N, K) in shapes:
            for g in (0, 32, 96, 128, 192):
                if g == 0 or K % g == 0:
                    yield bits, N, K, g


@pytest.mark.parametrize("bits,N,K,g", list(_shape_cases()))
@pytest.mark.parametrize("kind", ["normal", "mixed", "skewed"])
def test_sym_quantize_shapes(lw, bits, N, K, g, kind):
    w = _weights(kind, N, K, seed=N * 131 + K + bits)
    _check_quantize(lw, w, bits, g, f"sym bits={bits} N={N} K={K} g={g} {kind}", (True,))


# Every reduction layout: groups of 32 and 64 lanes, power-of-two groups
# larger than a wave, groups that are not a power of two (LDS), the longest
# row (1024 threads, 16 chunks each) and ragged last rounds.
PATH_CASES = [
    (4, 6, 4096, 256),
    (2, 6, 4096, 512),
    (3, 5, 8192, 1024),
    (4, 7, 12320, 160),
    (3, 2, 98304, 96),
    (2, 3, 65600, 0),
    (4, 2, 131072, 0),
    (3, 2, 131072, 64),
    (4, 2, 131072, 16384),
]


@pytest.mark.parametrize("bits,N,K,g", PATH_CASES)
def test_sym_quantize_group_paths(lw, bits, N, K, g):
    _say(f"[sym paths] bits={bits} N={N} K={K} g={g}")
    w = _weights("mixed", N, K, seed=K + g + bits)
    _check_quantize(lw, w, bits, g, f"sym paths bits={bits} N={N} K={K} g={g}")


def _tie_rows(bits: int, K: int) -> np.ndarray:
    """Rows whose weights sit exactly on the half-way points k + 1/2 of the
    grid (rint must take the even neighbour), with the extremes that set a
    power-of-two scale."""
    qmax = (1 << (bits - 1)) - 1
    s = 0.25                               # amax = qmax * s is exact in fp16
    half = (np.arange(-qmax, qmax) + 0.5) * s
    row = np.resize(np.concatenate([half, [qmax * s, -qmax * s]]), K)
    rows = [row, -row, row * 2.0, np.roll(row, 3)]
    return np.stack(rows).astype(np.float16)


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("g", [0, 32, 96])
def test_sym_quantize_degenerate(lw, bits, g):
    K = 384
    cases = {
        "zero": np.zeros((3, K), np.float16),
        "single": np.zeros((3, K), np.float16),
        "negative_extreme": None,
        "ties": _tie_rows(bits, K),
        "tiny": _weights("tiny", 5, K, seed=bits),
        "wide": _weights("wide", 5, K, seed=bits),
    }
    cases["single"][0, 5] = 0.75
    cases["single"][1, K - 1] = -3.0
    cases["single"][2, 0] = np.float16(6.1e-5)
    neg = _weights("normal", 4, K, seed=bits + 1).astype(np.float32)
    neg[:, 7] = -1.0                        # the largest magnitude is negative
    cases["negative_extreme"] = neg.astype(np.float16)
    for name, w in cases.items():
        _say(f"[sym degenerate] {name} bits={bits} g={g}")
        codes, scales, zeros, _ = _check_quantize(lw, w, bits, g, f"sym {name} bits={bits} g={g}")
        assert codes.min() >= 1 and codes.max() <= (1 << bits) - 1


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_sym_scale_of_zero_group_is_one(lw, bits):
    w = np.zeros((2, 256), np.float16)
    w[1, 128:] = 0.5
    out = lw.quantize_rtn(_to_gpu(w), bits, 128, symmetric=True)
    sc = out["scales"].cpu().numpy().view(np.uint16)
    assert sc[0, 0] == 0x3C00 and sc[0, 1] == 0x3C00 and sc[1, 0] == 0x3C00
    assert (out["codes"].cpu().numpy()[0] == 1 << (bits - 1)).all()


def _check_products(lw, w, bits, g, batches, kernel, what):
    import torch
    N, K = w.shape
    codes, scales, zeros, packed = _check_quantize(lw, w, bits, g, what, (False,))
    args = [_to_gpu(packed), _to_gpu(scales), _to_gpu(zeros), K, bits, g]
    for B in batches:
        x = synth.normal_f16(B, K, 1.0, seed=B + 5, stream=2)
        y = getattr(lw, kernel)(_to_gpu(x), *args)
        torch.cuda.synchronize()
        y_ref = harness.oracle_y(x, packed, scales, zeros, K, bits, g)
        harness.assert_y_close(y.cpu().numpy(), y_ref, f"{what} {kernel} B={B}")


PRODUCT_CASES = [(4, 67, 4128, 0), (4, 70, 4224, 128), (3, 67, 4224, 0), (3, 33, 8320, 64),
                 (2, 67, 4160, 64), (2, 17, 8256, 0)]


@pytest.mark.parametrize("bits,N,K,g", PRODUCT_CASES)
def test_sym_products(lw, bits, N, K, g):
    what = f"sym bits={bits} N={N} K={K} g={g}"
    _say(f"[sym products] {what}")
    w = _weights("normal", N, K, seed=N + 7 * K + bits)
    _check_products(lw, w, bits, g, [1, 4, 15], "qgemv", what)
    _check_products(lw, w, bits, g, [16, 33, 64], "qgemm", what)


# The workload layer shapes, quantized on the symmetric grid at full size;
# every row checked bit-exact, every output of the products in tolerance.
SYM_LAYERS = [L for L in harness.all_layers() if L.name in (
    "outlier_2048", "llama7b_up_11008x4096", "llama70b_up_28672x8192",
    "opt175b_attn_12288")]


@pytest.mark.parametrize("layer", SYM_LAYERS, ids=lambda L: L.name)
def test_sym_workload_layers(lw, layer):
    import torch
    _say(f"[sym workload] {layer.name} N={layer.N} K={layer.K} bits={layer.bits} "
         f"g={layer.group_size}")
    w = layer.weights()
    codes, scales, zeros, packed = _check_quantize(
        lw, w, layer.bits, layer.group_size, f"sym {layer.name}", (False,))
    K, bits, g = layer.K, layer.bits, layer.group_size
    args = [_to_gpu(packed), _to_gpu(scales), _to_gpu(zeros), K, bits, g]
    for B in layer.batches:
        x = layer.activations(B)
        kernel = "qgemv" if B < 16 else "qgemm"
        y = getattr(lw, kernel)(_to_gpu(x), *args)
        torch.cuda.synchronize()
        y_ref = harness.oracle_y(x, packed, scales, zeros, K, bits, g)
        harness.assert_y_close(y.cpu().numpy(), y_ref, f"sym {layer.name} B={B}")
