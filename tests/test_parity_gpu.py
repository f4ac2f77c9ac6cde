"""HIP path vs the CPU oracle, element by element, through the C ABI.

Bars: codes, fp16 scale bits, int32 zeros and packed words bit-exact;
y within |y - y_ref| <= 1e-3 |y_ref| + 1e-4 per element.  The workload tests
run the five workloads at their full sizes in the launch configuration the
benchmark times, and compare every output element; the product tests feed the
ORACLE's quantized weights to the GPU kernels, so the quantizer and the
products are checked independently.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

import harness
import synth

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


def _dev():
    import torch
    return torch.device("cuda:0")


def _to_gpu(a: np.ndarray):
    import torch
    if a.dtype == np.uint32:
        a = a.view(np.int32)
    return torch.from_numpy(np.ascontiguousarray(a)).to(_dev())


def _gpu_quantize(lw, w: np.ndarray, bits: int, g: int, codes=True, packed=True):
    import torch
    out = lw.quantize_rtn(_to_gpu(w), bits, g, codes=codes, packed=packed)
    torch.cuda.synchronize()
    res = {k: v.cpu().numpy() for k, v in out.items()}
    if "packed" in res:
        res["packed"] = res["packed"].view(np.uint32)
    return res


def _assert_quant_equal(res, codes, scales, zeros, packed, what):
    assert np.array_equal(res["scales"].view(np.uint16), scales.view(np.uint16)), f"{what}: scales"
    assert np.array_equal(res["zeros"], zeros), f"{what}: zeros"
    if "codes" in res:
        bad = np.argwhere(res["codes"] != codes)
        assert bad.size == 0, f"{what}: codes differ at {bad[:5].tolist()}"
    if "packed" in res:
        bad = np.argwhere(res["packed"] != packed)
        assert bad.size == 0, f"{what}: packed words differ at {bad[:5].tolist()}"


LAYERS = list(harness.all_layers())


@pytest.mark.parametrize("layer", LAYERS, ids=lambda L: L.name)
def test_quantize_workload(lw, layer):
    _say(f"[quantize] {layer.name} N={layer.N} K={layer.K} bits={layer.bits} g={layer.group_size}")
    d = harness.layer_data(layer)
    res = _gpu_quantize(lw, d.w, layer.bits, layer.group_size)
    _assert_quant_equal(res, d.codes, d.scales, d.zeros, d.packed, layer.name)
    # the packer on the GPU's own codes gives the same words
    import torch
    p = lw.pack(_to_gpu(res["codes"]), layer.bits)
    torch.cuda.synchronize()
    assert np.array_equal(p.cpu().numpy().view(np.uint32), d.packed), f"{layer.name}: lowbit_pack"


def _product_cases():
    for layer in LAYERS:
        for B in layer.batches:
            yield layer, B


@pytest.mark.parametrize("layer,B", list(_product_cases()),
                         ids=lambda v: v.name if isinstance(v, synth.Layer) else f"B{v}")
def test_product_workload(lw, layer, B):
    import torch
    _say(f"[product] {layer.name} B={B}")
    d = harness.layer_data(layer)
    x = d.x(B)
    args = (_to_gpu(x), _to_gpu(d.packed), _to_gpu(d.scales), _to_gpu(d.zeros), layer.K,
            layer.bits, layer.group_size)
    fn = lw.qgemv if B <= lw.QGEMV_MAX_B else lw.qgemm
    y = fn(*args)
    torch.cuda.synchronize()
    y = y.cpu().numpy()
    # every output row against the oracle (threaded over row ranges)
    y_ref = harness.oracle_y(x, d.packed, d.scales, d.zeros, layer.K, layer.bits,
                             layer.group_size)
    harness.assert_y_close(y, y_ref, f"{layer.name} B={B}")
    # the matrix-core kernel agrees too, whatever the batch
    if fn is lw.qgemv:
        y2 = lw.qgemm(*args)
        torch.cuda.synchronize()
        harness.assert_y_close(y2.cpu().numpy(), y_ref, f"{layer.name} B={B} qgemm")
