"""Seeded synthetic inputs and the workload catalogue.

This module holds input generation only: no step of the quantizer, the
packer or the matrix product lives here.  Both the CPU oracle's callers and
the HIP path's callers draw their inputs from it, so the two sides see
identical bytes.

Generator: numpy's PCG64 bit generator and its ``standard_normal(dtype=
float32)`` sampler.  A matrix is cut into blocks of ``ROWS_PER_BLOCK`` rows;
block i of input kind ``stream`` draws from ``SeedSequence([seed, stream,
i])``, so blocks can be drawn in parallel and a row's values do not depend on
how many rows follow it.  Samples are drawn in fp32, multiplied by the
standard deviation in fp32, and rounded to fp16 (round-to-nearest-even,
numpy's cast).
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

STREAM_W = 1        # weight matrix
STREAM_X = 2        # activations
STREAM_OUTLIER = 3  # choice of outlier input channels

ROWS_PER_BLOCK = 512


def _rng(seed: int, stream: int, block: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, stream, block])))


def _threads() -> int:
    return max(1, min(16, len(os.sched_getaffinity(0))))


def normal_f16(rows: int, cols: int, std: float, seed: int, stream: int,
               col_scale: np.ndarray | None = None) -> np.ndarray:
    """fp16 matrix with entries fp16(fp32(N(0,1)) * std [* col_scale])."""
    out = np.empty((rows, cols), np.float16)

    def block(i: int) -> None:
        r0 = i * ROWS_PER_BLOCK
        r1 = min(rows, r0 + ROWS_PER_BLOCK)
        a = _rng(seed, stream, i).standard_normal(size=(r1 - r0, cols), dtype=np.float32)
        a *= np.float32(std)
        if col_scale is not None:
            a *= col_scale[None, :]
        out[r0:r1] = a.astype(np.float16)

    nblocks = (rows + ROWS_PER_BLOCK - 1) // ROWS_PER_BLOCK
    if nblocks <= 1:
        for i in range(nblocks):
            block(i)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(block, range(nblocks)))
    return out


def outlier_columns(K: int, frac: float, seed: int) -> np.ndarray:
    """round(frac*K) distinct input-channel indices, sorted."""
    count = int(round(frac * K))
    rng = _rng(seed, STREAM_OUTLIER)
    return np.sort(rng.choice(K, size=count, replace=False))


@dataclass(frozen=True)
class Layer:
    """One quantized linear layer: W[N][K] (out x in), bits, group size."""
    name: str
    N: int
    K: int
    bits: int
    group_size: int            # 0 = one group per row
    batches: tuple             # activation batch sizes exercised
    outlier_frac: float = 0.0  # fraction of input channels scaled by outlier_scale
    outlier_scale: float = 10.0
    w_std: float = 0.02
    x_std: float = 1.0
    seed: int = 0

    def weights(self) -> np.ndarray:
        col_scale = None
        if self.outlier_frac > 0:
            cols = outlier_columns(self.K, self.outlier_frac, self.seed)
            col_scale = np.ones(self.K, np.float32)
            col_scale[cols] = np.float32(self.outlier_scale)
        return normal_f16(self.N, self.K, self.w_std, self.seed, STREAM_W, col_scale)

    def activations(self, B: int) -> np.ndarray:
        return normal_f16(B, self.K, self.x_std, self.seed, STREAM_X)


# The five workloads.  Shapes follow the linear layers the source pages talk
# about: a small single layer, a 2048-wide layer with outlier input channels,
# OPT-175B's attention-sized and fc1 layers at 3 bits per-row (the OPTQ card's
# 3-bit OPT-175B run), Llama-7B MLP up/down at 2 bits, and a Llama-70B MLP
# layer at 4 bits for the batched (MFMA) product.
WORKLOADS = {
    "single_256": [Layer("single_256", 256, 256, 4, 0, (1,))],
    "outlier_2048": [Layer("outlier_2048", 2048, 2048, 4, 128, (1,), outlier_frac=0.01)],
    "opt175b_3bit": [Layer("opt175b_attn_12288", 12288, 12288, 3, 0, (1,)),
                     Layer("opt175b_fc1_49152x12288", 49152, 12288, 3, 0, (1,))],
    "llama7b_mlp_2bit": [Layer("llama7b_up_11008x4096", 11008, 4096, 2, 64, (1, 4, 8)),
                         Layer("llama7b_down_4096x11008", 4096, 11008, 2, 64, (1, 4, 8))],
    "llama70b_mlp_4bit": [Layer("llama70b_up_28672x8192", 28672, 8192, 4, 128, (16, 32, 64))],
}
