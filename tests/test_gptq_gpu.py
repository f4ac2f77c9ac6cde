"""Error-feedback (GPTQ) quantization on the GPU (lowbit_quantize_gptq, fp64)
against the oracle's inverse-Hessian formulation.

Bar: codes, packed words, scales and zeros bit-exact.  Both sides decide every
code in fp64; they compute the running weights in different (algebraically
equal) ways, so a code could differ only where a quotient falls within about
1e-12 of a rounding midpoint, which seeded continuous inputs do not produce.
Shapes cover K that is not a multiple of the 64-column block, ragged row
tiles (16-, 32-, 48- and 64-row workgroups), every width, per-row and grouped grids (power-of-two and other group
sizes), and one workload layer at full size (every row through the oracle).
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


def _calibration(n: int, K: int, seed: int, correlated: bool) -> np.ndarray:
    """Synthetic calibration inputs: N(0, 1), optionally mixed across channels
    so that the Hessian has off-diagonal structure."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, K))
    if correlated:
        x = x @ (np.eye(K) + rng.standard_normal((K, K)) / np.sqrt(K))
    return x.astype(np.float16)


def _check(lw, w, x, bits, g, damp, what, codes=True, packed=True, symmetric=False):
    import torch
    H = harness.oracle.hessian(x, damp)
    rc, rs, rz = harness.oracle.quantize_gptq(w, H, bits, g, symmetric=symmetric)
    out = lw.quantize_gptq(_to_gpu(w), _to_gpu(x), bits, g, damp, codes=codes, packed=packed,
                           symmetric=symmetric)
    torch.cuda.synchronize()
    assert int(out["status"].item()) == 0, f"{what}: Hessian reported not positive definite"
    assert np.array_equal(out["scales"].cpu().numpy().view(np.uint16), rs.view(np.uint16)), what
    assert np.array_equal(out["zeros"].cpu().numpy(), rz), what
    if codes:
        got = out["codes"].cpu().numpy()
        bad = np.argwhere(got != rc)
        assert bad.size == 0, f"{what}: {len(bad)} codes differ, first {bad[:5].tolist()}"
    if packed:
        want = harness.oracle.pack(rc, bits)
        assert np.array_equal(out["packed"].cpu().numpy().view(np.uint32), want), what
    return rc


# The row kernel takes the fewest of 16, 32, 48 and 64 rows per workgroup
# whose workgroups all fit on the CUs at once (256 on MI355X): the 4100-row
# shape takes the 32-row form (4100 = 128 * 32 + 4), the 8200-row shapes the
# 48-row form (8200 = 170 * 48 + 40), the 16448-row shapes the 64-row form,
# all others the 16-row form.
CASES = [(5, 32, 4, 0), (17, 128, 3, 0), (64, 192, 2, 32), (67, 128, 4, 64), (130, 96, 8, 0),
         (70, 160, 4, 32), (33, 352, 4, 0), (129, 512, 3, 128), (40, 480, 4, 96),
         (21, 320, 2, 64), (66, 256, 8, 32), (4100, 128, 3, 32), (8200, 96, 4, 32), (8200, 320, 2, 0),
         (16448, 128, 3, 0), (16448, 224, 4, 32)]


@pytest.mark.parametrize("N,K,bits,g", CASES)
@pytest.mark.parametrize("correlated", [False, True], ids=["iid", "mixed"])
def test_gptq_matches_oracle(lw, N, K, bits, g, correlated):
    _say(f"[gptq] N={N} K={K} bits={bits} g={g} correlated={correlated}")
    rng = np.random.default_rng(N * 7 + K)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    x = _calibration(2 * K, K, seed=K + bits, correlated=correlated)
    codes = _check(lw, w, x, bits, g, 0.01, f"N={N} K={K} bits={bits} g={g}")
    if correlated:
        rtn, _, _ = harness.oracle.quantize_rtn(w, bits, g)
        assert (codes != rtn).any(), "error feedback changed no code"


@pytest.mark.parametrize("want", [(True, False), (False, True)], ids=["codes", "packed"])
def test_gptq_single_output(lw, want):
    rng = np.random.default_rng(5)
    w = (rng.standard_normal((50, 128)) * 0.02).astype(np.float16)
    x = _calibration(200, 128, seed=5, correlated=True)
    _check(lw, w, x, 4, 32, 0.05, "single output", codes=want[0], packed=want[1])


def test_gptq_degenerate_rows(lw):
    """Constant, zero and one-signed rows, and few calibration samples (a
    low-rank X^T X that only the damping makes positive definite)."""
    rng = np.random.default_rng(9)
    w = (rng.standard_normal((20, 128)) * 0.02).astype(np.float32)
    w[3] = 0.0
    w[4] = 0.25
    w[5] = np.abs(w[5]) + 1.0
    w[6] *= 1e-3
    x = _calibration(8, 128, seed=9, correlated=False)
    for bits, g in ((2, 0), (4, 32), (8, 0)):
        _check(lw, w.astype(np.float16), x, bits, g, 0.01, f"degenerate bits={bits} g={g}")


SYM_CASES = [(5, 32, 4, 0), (17, 128, 3, 0), (64, 192, 2, 32), (67, 128, 4, 64),
             (130, 96, 8, 0), (40, 480, 4, 96), (66, 256, 8, 32)]


@pytest.mark.parametrize("N,K,bits,g", SYM_CASES)
def test_gptq_symmetric_matches_oracle(lw, N, K, bits, g):
    """lowbit_quantize_gptq_sym: the signed symmetric grid, codes in [1, M]."""
    _say(f"[gptq sym] N={N} K={K} bits={bits} g={g}")
    rng = np.random.default_rng(N * 5 + K)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    x = _calibration(2 * K, K, seed=K + bits + 1, correlated=True)
    codes = _check(lw, w, x, bits, g, 0.01, f"sym N={N} K={K} bits={bits} g={g}",
                   symmetric=True)
    assert codes.min() >= 1
    rtn, _, _ = harness.oracle.quantize_rtn_sym(w, bits, g)
    assert (codes != rtn).any(), "error feedback changed no code"


def test_gptq_symmetric_degenerate_rows(lw):
    rng = np.random.default_rng(19)
    w = (rng.standard_normal((12, 128)) * 0.02).astype(np.float32)
    w[2] = 0.0
    w[3] = -0.5
    w[4] = np.abs(w[4]) + 1.0
    x = _calibration(8, 128, seed=19, correlated=False)
    for bits, g in ((2, 0), (4, 32), (8, 0)):
        _check(lw, w.astype(np.float16), x, bits, g, 0.01, f"sym degenerate bits={bits} g={g}",
               symmetric=True)


def test_gptq_full_size(lw):
    """The 2048 x 2048, 4-bit, groups-of-128 layer with its 1% outlier input
    channels, 2048 calibration rows: every row's codes, scales, zeros and
    packed words against the oracle (rows are independent given the Hessian,
    so the oracle runs on row ranges in parallel threads)."""
    import torch
    layer = [L for L in harness.all_layers() if L.name == "outlier_2048"][0]
    _say(f"[gptq full size] {layer.name}")
    w = layer.weights()
    K = layer.K
    cols = synth.outlier_columns(K, layer.outlier_frac, layer.seed)
    xs = np.random.default_rng(11).standard_normal((2048, K))
    xs[:, cols] *= layer.outlier_scale
    x = xs.astype(np.float16)
    out = lw.quantize_gptq(_to_gpu(w), _to_gpu(x), layer.bits, layer.group_size, 0.01)
    torch.cuda.synchronize()
    assert int(out["status"].item()) == 0
    H = harness.oracle.hessian(x, 0.01)
    _say("[gptq full size] oracle on all rows")
    rc, rs, rz = harness.oracle_gptq(w, H, layer.bits, layer.group_size)
    got = out["codes"].cpu().numpy()
    bad = np.argwhere(got != rc)
    assert bad.size == 0, f"{len(bad)} codes differ, first {bad[:5].tolist()}"
    assert np.array_equal(out["scales"].cpu().numpy().view(np.uint16), rs.view(np.uint16))
    assert np.array_equal(out["zeros"].cpu().numpy(), rz)
    want = harness.oracle.pack(rc, layer.bits)
    assert np.array_equal(out["packed"].cpu().numpy().view(np.uint32), want)


def test_gptq_full_size_factor_11008x4096(lw):
    """The 11008 x 4096, 2-bit, groups-of-64 layer with 4096 calibration rows
    (the bench's size; the oracle's inverse-Hessian form is too slow here):
    the GPU's own intermediate in the caller's workspace, the Cholesky factor
    L of the index-reversed Hessian (64 x 64 tiles, 64 per side, in the
    lower triangle at byte 256), against numpy in fp64: rows of L L^T equal
    the same rows of reverse(H), H = (2/n) X^T X + damp mean(diag) I, on
    sampled rows (tile edges, both ends, random ones) and on the whole
    diagonal.  Also every code lies on the grid."""
    import torch
    N, K, bits, g, n, damp = 11008, 4096, 2, 64, 4096, 0.01
    _say(f"[gptq factor] N={N} K={K} n={n}")
    rng = np.random.default_rng(4096)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    x = rng.standard_normal((n, K)).astype(np.float16)
    need = lw.gptq_workspace_bytes(N, K)
    ws = torch.empty(need + 256, dtype=torch.uint8, device="cuda:0")
    off = (-ws.data_ptr()) % 256
    out = lw.quantize_gptq(_to_gpu(w), _to_gpu(x), bits, g, damp, workspace=ws)
    torch.cuda.synchronize()
    assert int(out["status"].item()) == 0
    A = ws[off + 256: off + 256 + K * K * 8].view(torch.float64).reshape(K, K).cpu().numpy()
    L = np.tril(A)
    x64 = x.astype(np.float64)
    H = (2.0 / n) * (x64.T @ x64)
    H += damp * np.mean(np.diag(H)) * np.eye(K)
    R = H[::-1, ::-1]
    rows = sorted(set([0, 1, 63, 64, 65, 127, 128, 2047, 2048, 4031, 4032, K - 2, K - 1]
                      + rng.choice(K, 48, replace=False).tolist()))
    scale = np.abs(np.diag(R)).max()
    err = np.abs(L[rows] @ L.T - R[rows]).max() / scale
    assert err < 1e-11, f"rows of L L^T differ from reverse(H) by {err:.3g} (relative)"
    dg = np.einsum("ij,ij->i", L, L)
    assert np.abs(dg - np.diag(R)).max() / scale < 1e-11
    assert np.all(np.diag(L) > 0)
    codes = out["codes"].cpu().numpy()
    assert codes.max() <= (1 << bits) - 1
