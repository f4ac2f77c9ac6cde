"""Edge cases of the HIP path against the oracle: ragged shapes that span
several tiles with partial tails, every batch size of the matrix-vector
kernel, batches around the matrix-core tile edges, degenerate groups (constant,
all-zero, one-signed, tiny and far-from-zero weights that force the exact
slow decode), round-half-to-even ties, empty problems and error returns."""
from __future__ import annotations

import ctypes
import sys

import numpy as np
import pytest

import harness

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lw():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import weight_only_bit_rtn_amd as lw
    lw.load_library()
    return lw


def _to_gpu(a):
    import torch
    if a.dtype == np.uint32:
        a = a.view(np.int32)
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")


def _say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def _sync():
    import torch
    torch.cuda.synchronize()


def _weights(kind: str, N: int, K: int, seed: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    if kind == "normal":
        return (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    if kind == "wide":
        return (rng.standard_normal((N, K)) * 30).astype(np.float16)
    if kind == "tiny":           # scales far below 2^-7: exact slow decode
        return (rng.standard_normal((N, K)) * 3e-5).astype(np.float16)
    if kind == "offset":         # one-signed groups far from zero: large |zero|
        return (100 + 0.1 * rng.standard_normal((N, K))).astype(np.float16)
    if kind == "mixed":          # some rows tiny, some normal, some constant
        w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
        w[::3] *= 1e-3
        w[1::5] = 0.37
        w[2::7] = 0.0
        w[:, :: max(1, K // 7)] = -0.5
        return w.astype(np.float16)
    if kind == "positive":
        return rng.uniform(0.1, 0.9, (N, K)).astype(np.float16)
    if kind == "negative":
        return rng.uniform(-2.0, -1.0, (N, K)).astype(np.float16)
    if kind == "ties":           # the worked examples' values, tiled
        base = np.array([-1.5, -0.5, 0.0, 0.5, 1.5, -0.5, 2.5, 0.25], np.float32)
        return np.resize(base, (N, K)).astype(np.float16)
    raise ValueError(kind)


SHAPES = {
    4: [(1, 32), (5, 96), (17, 2080), (67, 4128)],
    2: [(1, 64), (5, 192), (17, 4160), (67, 8256)],
    3: [(1, 128), (5, 384), (17, 4224), (67, 8320)],
}


def _groups(K):
    gs = [0, 32]
    for g in (96, 128, 192):
        if K % g == 0:
            gs.append(g)
    return gs


def _quant_cases():
    for bits, shapes in SHAPES.items():
        for (N, K) in shapes:
            for g in _groups(K):
                yield bits, N, K, g


@pytest.mark.parametrize("bits,N,K,g", list(_quant_cases()))
@pytest.mark.parametrize("kind", ["normal", "mixed"])
def test_quantize_shapes(lw, bits, N, K, g, kind):
    w = _weights(kind, N, K, seed=N * 131 + K + bits)
    codes, scales, zeros, packed = harness.oracle_quantize(w, bits, g)
    out = lw.quantize_rtn(_to_gpu(w), bits, g)
    _sync()
    assert np.array_equal(out["scales"].cpu().numpy().view(np.uint16), scales.view(np.uint16))
    assert np.array_equal(out["zeros"].cpu().numpy(), zeros)
    assert np.array_equal(out["codes"].cpu().numpy(), codes)
    assert np.array_equal(out["packed"].cpu().numpy().view(np.uint32), packed)


# Group sizes and row lengths that reach every reduction layout of the
# quantizer: groups of 32 and 64 lanes, power-of-two groups larger than a
# wave, groups that are not a power of two, rows of 1024 threads with up to
# 16 chunks per thread (the largest row), and ragged last rounds.
GROUP_PATH_CASES = [
    (4, 6, 4096, 256),
    (2, 6, 4096, 512),
    (3, 5, 8192, 1024),
    (4, 4, 8192, 2048),
    (4, 7, 12320, 160),
    (3, 2, 98304, 96),
    (2, 3, 65600, 0),
    (2, 3, 131072, 0),
    (3, 2, 131072, 64),
    (4, 2, 131072, 16384),
]


@pytest.mark.parametrize("bits,N,K,g", GROUP_PATH_CASES)
@pytest.mark.parametrize("kind", ["normal", "mixed"])
def test_quantize_group_paths(lw, bits, N, K, g, kind):
    _say(f"[quantize paths] bits={bits} N={N} K={K} g={g} {kind}")
    w = _weights(kind, N, K, seed=K + g + bits)
    codes, scales, zeros, packed = harness.oracle_quantize(w, bits, g)
    for want_codes in (True, False):
        out = lw.quantize_rtn(_to_gpu(w), bits, g, codes=want_codes, packed=True)
        _sync()
        assert np.array_equal(out["scales"].cpu().numpy().view(np.uint16), scales.view(np.uint16))
        assert np.array_equal(out["zeros"].cpu().numpy(), zeros)
        if want_codes:
            assert np.array_equal(out["codes"].cpu().numpy(), codes)
        assert np.array_equal(out["packed"].cpu().numpy().view(np.uint32), packed)


def _scale_tie_groups(bits: int, count: int) -> list:
    """(lo, hi) fp16 pairs whose fp32 quotient (hi - lo) / M lies exactly
    half-way between two fp16 values, so the stored scale depends on the
    quotient being rounded to fp32 before fp16 (ties to even)."""
    M = np.float32((1 << bits) - 1)
    found = []
    for lo in (np.float16(-0.5), np.float16(-1.0), np.float16(0.25)):
        his = np.arange(0x2000, 0x3C00, dtype=np.uint16).view(np.float16)
        his = his[his.astype(np.float32) > np.float32(lo)]
        d = his.astype(np.float32) - np.float32(lo)
        s32 = (d / M).astype(np.float32)
        s16 = s32.astype(np.float16)
        down = np.nextafter(s16, np.float16(-np.inf))
        up = np.nextafter(s16, np.float16(np.inf))
        half_dn = (s16.astype(np.float64) + down.astype(np.float64)) / 2
        half_up = (s16.astype(np.float64) + up.astype(np.float64)) / 2
        tie = (s32.astype(np.float64) == half_dn) | (s32.astype(np.float64) == half_up)
        found += [(lo, h) for h in his[tie][:count]]
    assert found, "no halfway scale found"
    return found[: count]


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("g", [0, 32, 96])
def test_quantize_scale_ties(lw, bits, g):
    """Regression: the scale is rounded to fp32, then to fp16, never once."""
    _say(f"[quantize scale ties] bits={bits} g={g}")
    pairs = _scale_tie_groups(bits, 12)
    gs = g if g else 384
    rng = np.random.default_rng(bits * 7 + g)
    rows = []
    for lo, hi in pairs:
        grp = rng.uniform(float(lo), float(hi), gs).astype(np.float16)
        grp[rng.integers(0, gs)] = lo
        grp[rng.integers(0, gs)] = hi
        grp = np.clip(grp, lo, hi)
        reps = 384 // gs
        rows.append(np.tile(grp, reps))
    w = np.stack(rows).astype(np.float16)
    codes, scales, zeros, packed = harness.oracle_quantize(w, bits, g)
    out = lw.quantize_rtn(_to_gpu(w), bits, g)
    _sync()
    assert np.array_equal(out["scales"].cpu().numpy().view(np.uint16), scales.view(np.uint16))
    assert np.array_equal(out["zeros"].cpu().numpy(), zeros)
    assert np.array_equal(out["codes"].cpu().numpy(), codes)
    assert np.array_equal(out["packed"].cpu().numpy().view(np.uint32), packed)


@pytest.mark.parametrize("kind", ["wide", "tiny", "offset", "positive", "negative", "ties"])
@pytest.mark.parametrize("bits", [2, 3, 4])
def test_quantize_degenerate(lw, kind, bits):
    N, K = 9, 384 if bits != 2 else 448
    if bits == 3:
        K = 384
    for g in (0, 32, 64 if K % 64 == 0 else 32):
        w = _weights(kind, N, K, seed=bits)
        codes, scales, zeros, packed = harness.oracle_quantize(w, bits, g)
        for want_codes, want_packed in ((True, False), (False, True)):
            out = lw.quantize_rtn(_to_gpu(w), bits, g, codes=want_codes, packed=want_packed)
            _sync()
            assert np.array_equal(out["scales"].cpu().numpy().view(np.uint16),
                                  scales.view(np.uint16)), (kind, g)
            assert np.array_equal(out["zeros"].cpu().numpy(), zeros), (kind, g)
            if want_codes:
                assert np.array_equal(out["codes"].cpu().numpy(), codes), (kind, g)
            if want_packed:
                assert np.array_equal(out["packed"].cpu().numpy().view(np.uint32), packed), (kind, g)


def _product_cases():
    for bits, shapes in SHAPES.items():
        for (N, K) in shapes:
            for g in _groups(K)[:3]:
                yield bits, N, K, g


def _check_product(lw, w, bits, g, batches, kernel, stress=False):
    import torch
    N, K = w.shape
    codes, scales, zeros, packed = harness.oracle_quantize(w, bits, g)
    args = [_to_gpu(packed), _to_gpu(scales), _to_gpu(zeros), K, bits, g]
    for B in batches:
        x = harness.synth.normal_f16(B, K, 1.0, seed=B + 7, stream=2)
        y = getattr(lw, kernel)(_to_gpu(x), *args)
        torch.cuda.synchronize()
        y_ref = harness.oracle_y(x, packed, scales, zeros, K, bits, g)
        terms = harness.oracle_abs_y(x, packed, scales, zeros, K, bits, g) if stress else None
        harness.assert_y_close(y.cpu().numpy(), y_ref,
                               f"{kernel} bits={bits} N={N} K={K} g={g} B={B}", terms, K)


@pytest.mark.parametrize("bits,N,K,g", list(_product_cases()))
def test_qgemv_shapes(lw, bits, N, K, g):
    w = _weights("normal", N, K, seed=N + 3 * K + bits)
    _check_product(lw, w, bits, g, [1, 2, 3, 5, 8, 15] if K <= 4224 else [1, 4], "qgemv")


@pytest.mark.parametrize("bits,N,K,g", list(_product_cases()))
def test_qgemm_shapes(lw, bits, N, K, g):
    w = _weights("normal", N, K, seed=N + 5 * K + bits)
    _check_product(lw, w, bits, g, [1, 16, 17, 33, 64, 70], "qgemm")


# Groups that hold a matrix-core step's unit spans whole (4-bit g >= 128,
# 2-bit g >= 256; the 2-bit g = 128 cases take the two-operand form), with K
# not a multiple of the 512-long step: the last step of every row runs past
# the row end.
WIDE_GROUP_CASES = [(4, 33, 640, 128), (4, 17, 1280, 256), (2, 9, 640, 128), (2, 21, 1408, 128),
                    (4, 40, 2176, 128), (2, 19, 1280, 256)]


@pytest.mark.parametrize("bits,N,K,g", WIDE_GROUP_CASES)
@pytest.mark.parametrize("kind", ["normal", "mixed"])
def test_products_wide_groups_ragged(lw, bits, N, K, g, kind):
    _say(f"[wide groups] bits={bits} N={N} K={K} g={g} {kind}")
    w = _weights(kind, N, K, seed=N + 11 * K + bits)
    _check_product(lw, w, bits, g, [1, 16, 17, 33, 64], "qgemm")
    _check_product(lw, w, bits, g, [1, 4], "qgemv")


# The small-batch matrix-core GEMV (grouped 2- and 4-bit codes; 5 to 8
# activation rows on two 8-wave workgroups per CU, 9 to 15 on one of 16
# waves): one to three 16-row tiles per CU (257 tiles: two on one CU),
# activations staged in several rounds (K up to 8256 at 15 rows) whose length
# is cut to fill every wave's share (5, 6 and 7 rows), a last step running
# past the row end (units per row not a multiple of four), one, two, three
# and four units per group, ragged tiles; compared on every output with the
# oracle, and bit for bit with the compact group words.
MMA_CASES = [(2, 4100, 8256, 64), (2, 4100, 4224, 128), (2, 33, 1344, 192), (4, 4100, 4128, 32),
             (4, 4100, 2016, 96), (4, 700, 8192, 128), (4, 50, 4224, 64)]


@pytest.mark.parametrize("bits,N,K,g", MMA_CASES)
def test_qgemv_matrix_core_batches(lw, bits, N, K, g):
    import torch
    _say(f"[small-batch matrix-core] bits={bits} N={N} K={K} g={g}")
    w = _weights("mixed", N, K, seed=N + 11 * K + bits)
    codes, scales, zeros, packed = harness.oracle_quantize(w, bits, g)
    p, s, z = _to_gpu(packed), _to_gpu(scales), _to_gpu(zeros)
    meta = lw.pack_meta(s, z)
    for B in (5, 6, 7, 8, 9, 12, 15):
        x = harness.synth.normal_f16(B, K, 1.0, seed=B + 29, stream=2)
        xg = _to_gpu(x)
        y = lw.qgemv(xg, p, s, z, K, bits, g)
        ym = lw.qgemv_meta(xg, p, meta, K, bits, g)
        torch.cuda.synchronize()
        assert torch.equal(ym.view(torch.int16), y.view(torch.int16)), f"B={B} compact words"
        y_ref = harness.oracle_y(x, packed, scales, zeros, K, bits, g)
        harness.assert_y_close(y.cpu().numpy(), y_ref, f"qgemv bits={bits} N={N} K={K} g={g} B={B}")


# Layers of more than three 16-row tiles per CU (on 256 CUs) hand grouped
# 2- and 4-bit products of 5 to 8 activation rows to the matrix-core GEMM.
@pytest.mark.parametrize("bits,N,K,g", [(4, 12320, 1024, 128), (2, 12320, 1024, 64)])
def test_qgemv_tall_layers(lw, bits, N, K, g):
    _say(f"[tall layers] bits={bits} N={N} K={K} g={g}")
    w = _weights("normal", N, K, seed=N + 7 * K + bits)
    _check_product(lw, w, bits, g, [4, 5, 8], "qgemv")


# At least five 16-row groups per workgroup (on 256 CUs), so a whole 512-k
# step sits in one K part, and G a multiple of 8, with the group exactly a
# step run's span: at batch tiles of 16 and 32 rows the matrix-core product
# copies each wave's scales and zeros into LDS and reads them there, while the
# 64-row tile loads them per step.  Every output row must come out with the
# same bits either way, and the same as from the compact group words.
STAGED_CASES = [(4, 20487, 1024, 128), (8, 20487, 1024, 128), (2, 20487, 2048, 256)]


@pytest.mark.parametrize("bits,N,K,g", STAGED_CASES)
def test_qgemm_staged_group_parameters(lw, bits, N, K, g):
    import torch
    _say(f"[staged parameters] bits={bits} N={N} K={K} g={g}")
    w = _weights("mixed", N, K, seed=N + 13 * K + bits)
    codes, scales, zeros, packed = harness.oracle_quantize(w, bits, g)
    p, s, z = _to_gpu(packed), _to_gpu(scales), _to_gpu(zeros)
    meta = lw.pack_meta(s, z)
    x = harness.synth.normal_f16(48, K, 1.0, seed=17, stream=2)
    xg = _to_gpu(x)
    y48 = lw.qgemm(xg, p, s, z, K, bits, g)
    for B in (16, 32):
        xb = xg[:B].contiguous()
        yb = lw.qgemm(xb, p, s, z, K, bits, g)
        ym = lw.qgemm_meta(xb, p, meta, K, bits, g)
        torch.cuda.synchronize()
        assert torch.equal(yb.view(torch.int16), y48[:B].view(torch.int16)), f"B={B} vs B=48"
        assert torch.equal(ym.view(torch.int16), yb.view(torch.int16)), f"B={B} compact words"
    y_ref = harness.oracle_y(x, packed, scales, zeros, K, bits, g)
    harness.assert_y_close(y48.cpu().numpy(), y_ref, f"qgemm bits={bits} N={N} K={K} g={g} B=48")


# 64-row batch tiles stage each step's group parameters in LDS when every
# round of every workgroup (one per CU, 256 CUs) holds at least five 16-row
# groups: 13 groups per workgroup (rounds of 8 and 5: staged), 12 (8 and 4:
# loaded per lane), and shares of 5 and 6 groups with a ragged last tile
# (staged).  Each must match the oracle, give the same bits from compact group
# words, and give the 16-row tile's bits in its first 16 rows (the same K
# split, parameters copied per round or loaded per step).
STEP_STAGED_CASES = [(4, 13 * 256 * 16, 1024, 128), (4, 12 * 256 * 16, 1024, 128),
                     (4, (5 * 256 + 100) * 16 - 3, 1024, 128), (2, 13 * 256 * 16, 1024, 256),
                     (8, (5 * 256 + 100) * 16 - 3, 1024, 128)]


@pytest.mark.parametrize("bits,N,K,g", STEP_STAGED_CASES)
def test_qgemm_step_staged_parameters(lw, bits, N, K, g):
    import torch
    _say(f"[step-staged parameters] bits={bits} N={N} K={K} g={g}")
    w = _weights("mixed", N, K, seed=N + 31 * K + bits)
    codes, scales, zeros, packed = harness.oracle_quantize(w, bits, g)
    p, s, z = _to_gpu(packed), _to_gpu(scales), _to_gpu(zeros)
    meta = lw.pack_meta(s, z)
    x = harness.synth.normal_f16(64, K, 1.0, seed=23, stream=2)
    xg = _to_gpu(x)
    y64 = lw.qgemm(xg, p, s, z, K, bits, g)
    m64 = lw.qgemm_meta(xg, p, meta, K, bits, g)
    y16 = lw.qgemm(xg[:16].contiguous(), p, s, z, K, bits, g)
    torch.cuda.synchronize()
    assert torch.equal(m64.view(torch.int16), y64.view(torch.int16)), "compact words"
    assert torch.equal(y16.view(torch.int16), y64[:16].view(torch.int16)), "B=16 vs B=64"
    y_ref = harness.oracle_y(x, packed, scales, zeros, K, bits, g)
    harness.assert_y_close(y64.cpu().numpy(), y_ref, f"qgemm bits={bits} N={N} K={K} g={g} B=64")


@pytest.mark.parametrize("kind", ["wide", "tiny", "offset", "mixed", "positive", "negative", "ties"])
@pytest.mark.parametrize("bits", [2, 3, 4])
def test_products_degenerate(lw, kind, bits):
    N, K = 70, 4224 if bits == 3 else 4160
    w = _weights(kind, N, K, seed=11 * bits)
    stress = kind in ("wide", "offset")
    for g in (0, 64):
        _check_product(lw, w, bits, g, [1, 4], "qgemv", stress)
        _check_product(lw, w, bits, g, [16, 40], "qgemm", stress)


@pytest.mark.parametrize("kind", ["wide", "offset", "tiny", "negative"])
@pytest.mark.parametrize("bits,g", [(4, 128), (4, 256), (2, 256)])
def test_products_wide_groups_degenerate(lw, kind, bits, g):
    """The matrix-core layout that scales each unit's sum (groups holding
    the unit spans whole), on weights whose zero points fall outside
    +-1024 (offset) or whose scales are large or tiny: the exact per-code
    path inside that layout."""
    N, K = 37, 4096
    _say(f"[wide degenerate] kind={kind} bits={bits} g={g}")
    w = _weights(kind, N, K, seed=5 * bits + g)
    stress = kind in ("wide", "offset")
    _check_product(lw, w, bits, g, [16, 40, 64], "qgemm", stress)
    _check_product(lw, w, bits, g, [1, 4], "qgemv", stress)


def test_products_are_deterministic(lw):
    import torch
    N, K, bits, g = 1000, 4096, 4, 128
    w = _weights("normal", N, K, 1)
    codes, scales, zeros, packed = harness.oracle_quantize(w, bits, g)
    x = _to_gpu(harness.synth.normal_f16(8, K, 1.0, 0, 2))
    a = [_to_gpu(packed), _to_gpu(scales), _to_gpu(zeros), K, bits, g]
    for kern in ("qgemv", "qgemm"):
        y1 = getattr(lw, kern)(x, *a)
        y2 = getattr(lw, kern)(x, *a)
        torch.cuda.synchronize()
        assert torch.equal(y1.view(torch.int16), y2.view(torch.int16)), kern


def test_empty_problems_launch_nothing(lw):
    import torch
    stream = torch.cuda.current_stream().cuda_stream
    dummy = torch.zeros(64, dtype=torch.int32, device="cuda:0")
    p = dummy.data_ptr()
    assert lw.quantize_rtn_raw(p, 0, 128, 4, 0, p, p, p, p, stream) == lw.LOWBIT_OK
    assert lw.pack_raw(p, 0, 128, 4, p, stream) == lw.LOWBIT_OK
    assert lw.qgemv_raw(p, 0, p, p, p, 16, 128, 4, 0, p, stream) == lw.LOWBIT_OK
    assert lw.qgemm_raw(p, 3, p, p, p, 0, 128, 4, 0, p, stream) == lw.LOWBIT_OK
    torch.cuda.synchronize()
    assert int(dummy.abs().sum()) == 0


def test_error_returns_on_gpu(lw):
    import torch
    stream = torch.cuda.current_stream().cuda_stream
    buf = torch.zeros(1 << 16, dtype=torch.int32, device="cuda:0")
    p = buf.data_ptr()
    assert lw.qgemv_raw(p, 16, p, p, p, 8, 128, 4, 0, p, stream) == lw.LOWBIT_ERR_ARG
    assert lw.qgemv_raw(p, 1, p, p, p, 8, 128, 5, 0, p, stream) == lw.LOWBIT_ERR_UNSUPPORTED
    assert lw.qgemm_raw(p, 1, p, p, p, 8, 96, 3, 0, p, stream) == lw.LOWBIT_ERR_SHAPE
    assert lw.qgemm_raw(p + 2, 1, p, p, p, 8, 128, 4, 0, p, stream) == lw.LOWBIT_ERR_ARG
    assert lw.quantize_rtn_raw(p, 8, 128, 4, 48, p, p, p, p, stream) == lw.LOWBIT_ERR_SHAPE
    assert lw.quantize_rtn_raw(p, 8, 128, 4, 0, None, None, p, p, stream) == lw.LOWBIT_ERR_ARG
    torch.cuda.synchronize()
    assert int(buf.abs().sum()) == 0


def test_calls_follow_the_callers_stream(lw):
    """Every entry point enqueues on the stream it is given (here a
    side stream of default priority): results match the default-stream ones,
    and work queued behind an event on that stream sees the outputs."""
    import torch
    N, K, bits, g = 257, 2048, 4, 128
    w = _weights("normal", N, K, 3)
    x = _to_gpu(harness.synth.normal_f16(4, K, 1.0, 0, 2))
    ref = lw.quantize_rtn(_to_gpu(w), bits, g)
    y_ref = lw.qgemv(x, ref["packed"], ref["scales"], ref["zeros"], K, bits, g)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    wg = _to_gpu(w)
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        q = lw.quantize_rtn(wg, bits, g)
        y = lw.qgemv(x, q["packed"], q["scales"], q["zeros"], K, bits, g)
        y2 = lw.qgemm(x, q["packed"], q["scales"], q["zeros"], K, bits, g)
        done = torch.cuda.Event()
        done.record(side)
    torch.cuda.current_stream().wait_event(done)
    assert torch.equal(q["packed"], ref["packed"])
    assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16))
    y_host = harness.oracle_y(x.cpu().numpy(), ref["packed"].cpu().numpy().view(np.uint32),
                              ref["scales"].cpu().numpy(), ref["zeros"].cpu().numpy(), K, bits, g)
    harness.assert_y_close(y2.cpu().numpy(), y_host, "qgemm on a side stream")

