"""Test harness shared by the GPU parity tests: runs the HIP path through its
C ABI and the CPU oracle on the same seeded inputs, and compares them.

The oracle is plain single-threaded C; the harness only calls it on disjoint
row ranges from several Python threads (ctypes releases the GIL) so that the
full-size workloads finish in seconds.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

import oracle
import synth

Y_RTOL = 1e-3   # |y - y_ref| <= Y_RTOL * |y_ref| + Y_ATOL, per element
Y_ATOL = 1e-4


def threads() -> int:
    return max(1, min(16, len(os.sched_getaffinity(0))))


def row_chunks(N: int, parts: int):
    step = max(1, -(-N // parts))
    return [(r0, min(N, r0 + step)) for r0 in range(0, N, step)]


def oracle_quantize(w: np.ndarray, bits: int, group_size: int, symmetric: bool = False):
    """Oracle quantization of all rows (row ranges in parallel threads): the
    min-max grid, or the signed symmetric grid when ``symmetric``."""
    N, K = w.shape
    quantize = oracle.quantize_rtn_sym if symmetric else oracle.quantize_rtn
    G = oracle.groups(K, group_size)
    codes = np.empty((N, K), np.uint8)
    scales = np.empty((N, G), np.float16)
    zeros = np.empty((N, G), np.int32)

    def run(rng):
        r0, r1 = rng
        c, s, z = quantize(w[r0:r1], bits, group_size)
        codes[r0:r1], scales[r0:r1], zeros[r0:r1] = c, s, z

    with ThreadPoolExecutor(threads()) as ex:
        list(ex.map(run, row_chunks(N, 4 * threads())))
    packed = np.empty((N, K * bits // 32), np.uint32)

    def run_pack(rng):
        r0, r1 = rng
        packed[r0:r1] = oracle.pack(codes[r0:r1], bits)

    with ThreadPoolExecutor(threads()) as ex:
        list(ex.map(run_pack, row_chunks(N, 4 * threads())))
    return codes, scales, zeros, packed


def oracle_y(x: np.ndarray, packed: np.ndarray, scales: np.ndarray, zeros: np.ndarray,
             K: int, bits: int, group_size: int, rows: np.ndarray | None = None) -> np.ndarray:
    """fp64 reference y[B][len(rows)] for the selected weight rows."""
    if rows is not None:
        packed, scales, zeros = packed[rows], scales[rows], zeros[rows]
    N = packed.shape[0]
    out = np.empty((x.shape[0], N), np.float64)

    def run(rng):
        r0, r1 = rng
        out[:, r0:r1] = oracle.reference_y(x, packed[r0:r1], scales[r0:r1], zeros[r0:r1], K,
                                           bits, group_size)

    with ThreadPoolExecutor(threads()) as ex:
        list(ex.map(run, row_chunks(N, 4 * threads())))
    return out


def oracle_gptq(w: np.ndarray, H: np.ndarray, bits: int, group_size: int,
                symmetric: bool = False, parts: int | None = None):
    """Oracle error-feedback codes of every row of w, with the rows split into
    ``parts`` ranges run in parallel threads (rows are independent given H;
    each call repeats the oracle's inverse-Hessian work for its range)."""
    N, K = w.shape
    G = oracle.groups(K, group_size)
    codes = np.empty((N, K), np.uint8)
    scales = np.empty((N, G), np.float16)
    zeros = np.empty((N, G), np.int32)

    def run(rng):
        r0, r1 = rng
        c, s, z = oracle.quantize_gptq(w[r0:r1], H, bits, group_size, symmetric)
        codes[r0:r1], scales[r0:r1], zeros[r0:r1] = c, s, z

    with ThreadPoolExecutor(threads()) as ex:
        list(ex.map(run, row_chunks(N, parts or threads())))
    return codes, scales, zeros


def oracle_abs_y(x: np.ndarray, packed: np.ndarray, scales: np.ndarray, zeros: np.ndarray,
                 K: int, bits: int, group_size: int) -> np.ndarray:
    """sum_k |x[b][k] * deq[n][k]| (the size of the terms an output sums)."""
    codes = oracle.unpack(packed, K, bits)
    deq = oracle.dequant(codes, scales, zeros, bits, group_size)
    return oracle.matmul_f64(np.abs(x), np.abs(deq))


def assert_y_close(y_gpu: np.ndarray, y_ref: np.ndarray, what: str,
                   abs_terms: np.ndarray | None = None, K: int = 0) -> None:
    """Per-element tolerance check.

    The workloads use |y - y_ref| <= 1e-3 |y_ref| + 1e-4 exactly.  Stress
    inputs whose terms are orders of magnitude larger than the result (weights
    near 100, or spread 30, against N(0,1) activations) pass ``abs_terms`` =
    sum_k |x*deq|; the bound then also admits the rounding of an fp32 sum of
    K such terms, sqrt(K) * 2^-22 * sum_k |x*deq| (a 4x margin over the
    random-walk size of K fp32 roundings).
    """
    yg = y_gpu.astype(np.float64)
    err = np.abs(yg - y_ref)
    bound = Y_RTOL * np.abs(y_ref) + Y_ATOL
    if abs_terms is not None:
        bound = bound + np.sqrt(K) * 2.0 ** -22 * abs_terms
    bad = err > bound
    if bad.any():
        idx = np.argwhere(bad)[:5]
        detail = ", ".join(f"{tuple(i)}: gpu={yg[tuple(i)]!r} ref={y_ref[tuple(i)]!r}"
                           for i in idx)
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} outputs outside "
                             f"|dy| <= {Y_RTOL}|y| + {Y_ATOL}; first: {detail}")


class LayerData:
    """Seeded inputs of one workload layer and the oracle's artefacts for it."""

    def __init__(self, layer: synth.Layer):
        self.layer = layer
        self.w = layer.weights()
        (self.codes, self.scales, self.zeros,
         self.packed) = oracle_quantize(self.w, layer.bits, layer.group_size)

    def x(self, B: int) -> np.ndarray:
        return self.layer.activations(B)


_CACHE: dict[str, LayerData] = {}


def layer_data(layer: synth.Layer) -> LayerData:
    if layer.name not in _CACHE:
        _CACHE.clear()            # keep one (possibly multi-GB) layer resident
        _CACHE[layer.name] = LayerData(layer)
    return _CACHE[layer.name]


def all_layers():
    for name, layers in synth.WORKLOADS.items():
        for layer in layers:
            yield layer
