"""Benchmark: fused dequantize-GEMV of 3-bit per-row RTN weights at batch 1.

Workload (the metric's): the two OPT-175B-shaped linear layers at 3 bits,
per-row asymmetric min-max, word-straddling pack --- W 12288x12288 and fc1
49152x12288 --- against one fp16 activation row.  A step is one batch-1
forward through both layers: two lowbit_qgemv calls, each reading its layer's
packed weights, fp16 scales and int32 zeros once from HBM.  The weights were
quantized and packed on the GPU (lowbit_quantize_rtn) before the timed region
and are resident in HBM; to keep the 256 MB last-level cache (MALL) from
serving repeated reads, every step uses the next of several copies of the
packed weights (>= 1 GB in total).

value = algorithmic bytes of the step (packed words + scales + zeros + x + y)
over the wall time of the timed steps; roofline.achieved = the same bytes per
GEMV launch over the average launch duration, from HIP events recorded on the
launch stream around the timed region (elapsed / launches).  The quantizer
(lowbit_quantize_rtn, and lowbit_quantize_rtn_sym for the signed symmetric
grid), every workload's products and the matrix-core product (lowbit_qgemm,
Llama-70B MLP shape at batch 16/32/64) are measured in the same run as
separate stages.  The CPU baseline times the C oracle (unpack + exact
dequantization + fp64 product, and quantize + pack) on bounded samples of the
same layers, single-threaded and with rows split over the host's cores.

Usage: python bench.py [--gpus 1] [--steps 50] [--warmup 10] [--no-cpu-baseline]
                       [--no-stages] [--stage-reps 20] [--gptq-only] [--counter-pass]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, published
MFMA_F16_PEAK_TFLOPS = 2500.0   # MI355X dense fp16 matrix, published
FP64_PEAK_TFLOPS = 78.6         # MI355X fp64 (vector and matrix), published
MALL_DEFEAT_BYTES = 1 << 30
PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "qgemv_opt175b_3bit_traffic.json")
GEMV_SOURCES = ["gemv.hip", "gemv3.hip", "gemv_kernel.h", "unit_decode.h", "common.h"]
GEMV_KERNEL = "qgemv_kernel<3,1,R,perrow>"


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def gemv_source_hash() -> str:
    h = hashlib.sha256()
    for name in GEMV_SOURCES:
        with open(os.path.join(ROOT, "weight_only_bit_rtn_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def product_bytes(N: int, K: int, bits: int, group_size: int, B: int) -> int:
    G = 1 if group_size == 0 else K // group_size
    return N * K * bits // 8 + N * G * 2 + N * G * 4 + B * K * 2 + B * N * 2


def product_bytes_meta(N: int, K: int, bits: int, group_size: int, B: int) -> int:
    """Algorithmic bytes with compact group words (4 bytes per group)."""
    G = 1 if group_size == 0 else K // group_size
    return N * K * bits // 8 + N * G * 4 + B * K * 2 + B * N * 2


def quantize_bytes(N: int, K: int, bits: int, group_size: int) -> int:
    G = 1 if group_size == 0 else K // group_size
    return N * K * 2 + N * K * bits // 8 + N * G * 6


class Prepared:
    """A layer quantized on the GPU, with `copies` copies of its packed form."""

    def __init__(self, lw, torch, layer, copies: int):
        import numpy as np
        self.layer = layer
        dev = torch.device("cuda:0")
        w = torch.from_numpy(layer.weights()).to(dev)
        q = lw.quantize_rtn(w, layer.bits, layer.group_size, codes=False, packed=True)
        self.w = w
        self.copies = [(q["packed"], q["scales"], q["zeros"])]
        for _ in range(copies - 1):
            self.copies.append(tuple(t.clone() for t in self.copies[0]))
        self.x = {B: torch.from_numpy(layer.activations(B)).to(dev) for B in layer.batches}
        self.y = {B: torch.empty((B, layer.N), dtype=torch.float16, device=dev)
                  for B in layer.batches}
        self.np = np

    def add_meta(self, lw) -> None:
        """Compact group words for every copy (4th element of each copy)."""
        self.copies = [(p, s, z, lw.pack_meta(s, z)) for (p, s, z) in self.copies]

    def footprint(self) -> int:
        L = self.layer
        return product_bytes(L.N, L.K, L.bits, L.group_size, 0)


def copies_for(footprint: int) -> int:
    return max(2, math.ceil(MALL_DEFEAT_BYTES / max(footprint, 1)))


def run_product(lw, prep: Prepared, B: int, c: int, stream: int, kernel: str) -> None:
    L = prep.layer
    cp = prep.copies[c % len(prep.copies)]
    packed, scales, zeros = cp[:3]
    if kernel.endswith("_meta"):
        raw = lw.qgemv_meta_raw if kernel == "qgemv_meta" else lw.qgemm_meta_raw
        st = raw(prep.x[B].data_ptr(), B, packed.data_ptr(), cp[3].data_ptr(), L.N, L.K, L.bits,
                 L.group_size, prep.y[B].data_ptr(), stream)
        if st != 0:
            raise RuntimeError(f"{kernel} failed: {lw.status_string(st)}")
        return
    raw = lw.qgemv_raw if kernel == "qgemv" else lw.qgemm_raw
    st = raw(prep.x[B].data_ptr(), B, packed.data_ptr(), scales.data_ptr(), zeros.data_ptr(),
             L.N, L.K, L.bits, L.group_size, prep.y[B].data_ptr(), stream)
    if st != 0:
        raise RuntimeError(f"{kernel} failed: {lw.status_string(st)}")


def time_launches(torch, fn, count: int, spread: bool = False):
    """Device time of `count` launches of fn(i), each bracketed by events:
    (average, median) in ms, and with spread=True also (p10, p90)."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(count)]
    for i, (a, b) in enumerate(evs):
        a.record()
        fn(i)
        b.record()
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in evs)
    avg, med = sum(ms) / len(ms), ms[len(ms) // 2]
    if not spread:
        return avg, med
    return avg, med, ms[(len(ms) - 1) // 10], ms[(9 * (len(ms) - 1)) // 10]


# The same shapes at 8 bits (the wider weight-only width): OPT-175B fc1 per
# row at batch 1 and 4, the Llama-70B MLP layer in groups of 128 at 16..64.
WIDE_LAYERS = (("opt175b_fc1_49152x12288_8bit", 49152, 12288, 8, 0, (1, 4)),
               ("llama70b_up_28672x8192_8bit", 28672, 8192, 8, 128, (16, 32, 64)))


# One GPU's share of the OPT-175B fc1 layer when it is split by output rows
# over two GPUs (the OPTQ card's 3-bit OPT-175B run on two GPUs): the same
# kernel on half the rows.
SHARD_LAYERS = (("opt175b_fc1_shard_24576x12288", 24576, 12288, 3, 0, (1,)),)


# Error-feedback (GPTQ) quantization, fp64: (layer name, calibration rows).
GPTQ_LAYERS = (("outlier_2048", 2048), ("llama7b_up_11008x4096", 4096))


def gptq_flops(N: int, K: int, n: int) -> float:
    """fp64 operations of one call: the Hessian (n K^2: one triangle of the
    symmetric matrix, 2 n per entry), its Cholesky factor (K^3 / 3) and the
    feedback product (N K^2)."""
    return float(n) * K * K + K ** 3 / 3.0 + float(N) * K * K


def measure_gptq(lw, torch, stream: int) -> dict:
    import numpy as np
    import synth
    stages = {}
    layers = {L.name: L for Ls in synth.WORKLOADS.values() for L in Ls}
    dev = torch.device("cuda:0")
    for name, n in GPTQ_LAYERS:
        L = layers[name]
        w = torch.from_numpy(L.weights()).to(dev)
        x = torch.from_numpy(synth.normal_f16(n, L.K, 1.0, L.seed, synth.STREAM_X)).to(dev)
        G = 1 if L.group_size == 0 else L.K // L.group_size
        need = lw.gptq_workspace_bytes(L.N, L.K)
        ws = torch.empty(need + 256, dtype=torch.uint8, device=dev)
        off = (-ws.data_ptr()) % 256
        packed = torch.empty((L.N, L.K * L.bits // 32), dtype=torch.int32, device=dev)
        scales = torch.empty((L.N, G), dtype=torch.float16, device=dev)
        zeros = torch.empty((L.N, G), dtype=torch.int32, device=dev)

        def run(_):
            st = lw.quantize_gptq_raw(w.data_ptr(), L.N, L.K, x.data_ptr(), n, 0.01, L.bits,
                                      L.group_size, None, packed.data_ptr(), scales.data_ptr(),
                                      zeros.data_ptr(), ws.data_ptr() + off, need, stream)
            if st != 0:
                raise RuntimeError(lw.status_string(st))

        run(0)
        avg, med, p10, p90 = time_launches(torch, run, 5, spread=True)
        status = int(ws[off:off + 4].view(torch.int32).item())
        fl = gptq_flops(L.N, L.K, n)
        stages[f"gptq/{name}"] = {
            "us": round(avg * 1e3, 1), "us_median": round(med * 1e3, 1),
            "us_p10": round(p10 * 1e3, 1), "us_p90": round(p90 * 1e3, 1),
            "calibration_rows": n, "fp64_flop": fl, "TFLOPs": round(fl / (avg * 1e-3) / 1e12, 2),
            "fp64_frac": round(fl / (avg * 1e-3) / 1e12 / FP64_PEAK_TFLOPS, 4), "status": status}
        del w, x, ws, packed, scales, zeros
        torch.cuda.empty_cache()
    return stages


def measure_stages(lw, torch, stream: int, reps: int) -> dict:
    import synth
    stages = {}
    wide = [synth.Layer(*spec) for spec in WIDE_LAYERS]
    shard = [synth.Layer(*spec) for spec in SHARD_LAYERS]
    # quantize + pack (reads 2 B per weight): the OPT-175B 3-bit per-row
    # layers and the Llama-70B 4-bit layer (groups of 128), on the min-max
    # grid and, for the larger two, on the signed symmetric grid
    runs = [(synth.WORKLOADS["opt175b_3bit"][0], False), (synth.WORKLOADS["opt175b_3bit"][1], False),
            (synth.WORKLOADS["opt175b_3bit"][1], True), (synth.WORKLOADS["llama70b_mlp_4bit"][0], False),
            (synth.WORKLOADS["llama70b_mlp_4bit"][0], True), (wide[0], False), (wide[1], True)]
    for layer, sym in runs:
        dev = torch.device("cuda:0")
        w = torch.from_numpy(layer.weights()).to(dev)
        G = 1 if layer.group_size == 0 else layer.K // layer.group_size
        packed = torch.empty((layer.N, layer.K * layer.bits // 32), dtype=torch.int32, device=dev)
        scales = torch.empty((layer.N, G), dtype=torch.float16, device=dev)
        zeros = torch.empty((layer.N, G), dtype=torch.int32, device=dev)
        raw = lw.quantize_rtn_sym_raw if sym else lw.quantize_rtn_raw

        def q(_):
            st = raw(w.data_ptr(), layer.N, layer.K, layer.bits, layer.group_size, None,
                     packed.data_ptr(), scales.data_ptr(), zeros.data_ptr(), stream)
            if st != 0:
                raise RuntimeError(lw.status_string(st))

        q(0)
        avg, med, p10, p90 = time_launches(torch, q, reps, spread=True)
        nbytes = quantize_bytes(layer.N, layer.K, layer.bits, layer.group_size)
        stages[f"{'quantize_pack_sym' if sym else 'quantize_pack'}/{layer.name}"] = {
            "us": round(avg * 1e3, 2), "us_median": round(med * 1e3, 2),
            "us_p10": round(p10 * 1e3, 2), "us_p90": round(p90 * 1e3, 2), "bytes": nbytes,
            "GBps": round(nbytes / (avg * 1e-3) / 1e9, 1),
            "roofline": {"bound": "hbm", "frac": round(nbytes / (avg * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}}
        del w, packed, scales, zeros
        torch.cuda.empty_cache()
    # every workload's products
    for name, layers in list(synth.WORKLOADS.items()) + [("shard", shard), ("8bit", wide)]:
        for layer in layers:
            prep = None
            # grouped layers are also timed with compact group words
            variants = ("", "_meta") if layer.group_size > 0 and layer.bits != 8 else ("",)
            for B, var in [(B, v) for v in variants for B in layer.batches]:
                kern = ("qgemv" if B <= lw.QGEMV_MAX_B else "qgemm") + var
                if prep is None:
                    fp = product_bytes(layer.N, layer.K, layer.bits, layer.group_size, 0)
                    prep = Prepared(lw, torch, layer, copies_for(fp))
                    if len(variants) > 1:
                        prep.add_meta(lw)
                for i in range(3):
                    run_product(lw, prep, B, i, stream, kern)
                avg, med, p10, p90 = time_launches(
                    torch, lambda i: run_product(lw, prep, B, i, stream, kern), reps, spread=True)
                nbytes = (product_bytes_meta if var else product_bytes)(
                    layer.N, layer.K, layer.bits, layer.group_size, B)
                gbps = nbytes / (avg * 1e-3) / 1e9
                rec = {"kernel": kern, "us": round(avg * 1e3, 2), "us_median": round(med * 1e3, 2),
                       "us_p10": round(p10 * 1e3, 2), "us_p90": round(p90 * 1e3, 2),
                       "bytes": nbytes, "GBps": round(gbps, 1),
                       "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4)}
                if kern.startswith("qgemm"):
                    tflops = 2.0 * B * layer.N * layer.K / (avg * 1e-3) / 1e12
                    rec["TFLOPs"] = round(tflops, 1)
                    rec["mfma_frac"] = round(tflops / MFMA_F16_PEAK_TFLOPS, 4)
                stages[f"{kern}/{layer.name}/B{B}"] = rec
            del prep
            torch.cuda.empty_cache()
    stages.update(measure_gptq(lw, torch, stream))
    # a measured streaming reference next to the published peak: a plain
    # device-to-device copy (read + write) of 1 GiB
    src = torch.empty(COPY_REF_BYTES // 2, dtype=torch.float16, device="cuda:0").normal_()
    dst = torch.empty_like(src)
    dst.copy_(src)
    avg, med, p10, p90 = time_launches(torch, lambda i: dst.copy_(src), 10, spread=True)
    moved = 2 * COPY_REF_BYTES
    stages["reference/device_copy_1GiB"] = {
        "us": round(avg * 1e3, 2), "us_median": round(med * 1e3, 2), "bytes_read_plus_written": moved,
        "GBps": round(moved / (avg * 1e-3) / 1e9, 1),
        "hbm_frac": round(moved / (avg * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}
    del src, dst
    torch.cuda.empty_cache()
    return stages


def _oracle_rate(work, nbytes: int, threads: int, budget_s: float):
    """Run work() repeatedly on `threads` Python threads (the oracle's C calls
    release the GIL) for about budget_s seconds of wall time; returns
    (bytes per second, calls, seconds)."""
    import threading
    calls = [0] * threads
    t0 = time.perf_counter()
    t_end = t0 + budget_s

    def loop(i: int) -> None:
        while True:
            work(i)
            calls[i] += 1
            if time.perf_counter() >= t_end:
                return

    ts = [threading.Thread(target=loop, args=(i,)) for i in range(threads)]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    wall = time.perf_counter() - t0
    return sum(calls) * nbytes / wall, sum(calls), wall


def cpu_baseline(budget_s: float = 5.0) -> dict:
    """The C oracle as it stands, on bounded samples of the metric's layers
    (K = 12288, 3-bit, one group per row): the product (unpack + exact
    dequantization + fp64 matrix-vector product, batch 1) and quantize + pack,
    each single-threaded and with rows split over the host's cores."""
    import numpy as np  # noqa: F401

    import oracle
    import synth
    layer = synth.WORKLOADS["opt175b_3bit"][1]
    rows = 256
    affinity = len(os.sched_getaffinity(0))
    cores = max(1, min(16, affinity))   # the host's CPU share for one GPU
    chunks = []
    for i in range(cores):
        w = synth.normal_f16(rows, layer.K, layer.w_std, layer.seed + 1000 + i, synth.STREAM_W)
        codes, scales, zeros = oracle.quantize_rtn(w, layer.bits, layer.group_size)
        chunks.append((w, oracle.pack(codes, layer.bits), scales, zeros))
    x = layer.activations(1)
    pbytes = product_bytes(rows, layer.K, layer.bits, layer.group_size, 1)
    qbytes = quantize_bytes(rows, layer.K, layer.bits, layer.group_size)

    def product(i):
        _, packed, scales, zeros = chunks[i % len(chunks)]
        oracle.reference_y(x, packed, scales, zeros, layer.K, layer.bits, layer.group_size)

    def quantize(i):
        w = chunks[i % len(chunks)][0]
        codes, _, _ = oracle.quantize_rtn(w, layer.bits, layer.group_size)
        oracle.pack(codes, layer.bits)

    p1, n1, s1 = _oracle_rate(product, pbytes, 1, budget_s)
    pn, nn, sn = _oracle_rate(product, pbytes, cores, budget_s)
    q1, m1, t1 = _oracle_rate(quantize, qbytes, 1, budget_s)
    qn, mn, tn = _oracle_rate(quantize, qbytes, cores, budget_s)
    return {"value": round(pn / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"{rows}-row chunks of the {layer.N}x{layer.K} 3-bit per-row layer "
                      f"(K={layer.K}), batch 1, through the oracle's unpack + exact "
                      f"dequantization + fp64 product: {nn} chunks in {sn:.1f} s on {cores} "
                      f"threads (rows split over the cores; {affinity} in the affinity mask)",
            "single_thread": {"value": round(p1 / 1e9, 4), "unit": "GB/s", "cores": 1,
                              "chunks": n1, "seconds": round(s1, 2)},
            "quantize_pack": {"value": round(qn / 1e9, 4), "unit": "GB/s", "cores": cores,
                              "chunks": mn, "seconds": round(tn, 2),
                              "single_thread": round(q1 / 1e9, 4),
                              "bytes_per_chunk": qbytes,
                              "what": "oracle quantize_rtn + pack of the same chunks "
                                      "(2 B read per weight + packed words + scales + zeros)"}}


def load_traffic(avg_bytes_per_launch: int):
    if not os.path.exists(PROFILE_TRAFFIC):
        return None
    try:
        with open(PROFILE_TRAFFIC) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("gemv_source_hash") != gemv_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


COPY_BYTES = 256 << 20
COPY_REF_BYTES = 1 << 30


def counter_pass(lw, torch, layers, stream: int) -> int:
    """Launch sequence profiled by the counter passes (FETCH_SIZE, WRITE_SIZE,
    MfmaUtil / VALUBusy): the quantizer once per GEMV layer, three GEMV launches
    per layer (distinct weight copies), two GEMV launches per batch (1, 4, 8)
    of each Llama-7B MLP layer, two matrix-core launches per batch of the
    Llama-70B MLP shape, then three plain device-to-device copies of
    COPY_BYTES whose counter readings calibrate the bytes per count."""
    import synth
    preps = [Prepared(lw, torch, L, 3) for L in layers]  # quantizes each layer once
    for p in preps:
        del p.w
    torch.cuda.synchronize()
    for p in preps:
        for i in range(3):
            run_product(lw, p, 1, i, stream, "qgemv")
    torch.cuda.synchronize()
    # the Llama-7B MLP layers, 2-bit groups of 64, at batch 1, 4 and 8
    small = []
    for L in synth.WORKLOADS["llama7b_mlp_2bit"]:
        ps = Prepared(lw, torch, L, 2)
        del ps.w
        for B in L.batches:
            for i in range(2):
                run_product(lw, ps, B, i, stream, "qgemv")
        torch.cuda.synchronize()
        small.append(L)
        del ps
    big = synth.WORKLOADS["llama70b_mlp_4bit"][0]
    pg = Prepared(lw, torch, big, 2)
    del pg.w
    for B in big.batches:
        for i in range(2):
            run_product(lw, pg, B, i, stream, "qgemm")
    torch.cuda.synchronize()
    del pg
    src = torch.empty(COPY_BYTES // 2, dtype=torch.float16, device="cuda:0").normal_()
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    per_launch = {p.layer.name: product_bytes(p.layer.N, p.layer.K, p.layer.bits,
                                              p.layer.group_size, 1) for p in preps}
    for L in small:
        for B in L.batches:
            per_launch[f"{L.name}/B{B}"] = product_bytes(L.N, L.K, L.bits, L.group_size, B)
    for B in big.batches:
        per_launch[f"{big.name}/B{B}"] = product_bytes(big.N, big.K, big.bits, big.group_size, B)
    for p in preps:
        L = p.layer
        per_launch[f"quantize/{L.name}"] = quantize_bytes(L.N, L.K, L.bits, L.group_size)
    print(json.dumps({"counter_pass": True, "copy_bytes": COPY_BYTES,
                      "algorithmic_bytes_per_launch": per_launch}), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-stages", action="store_true")
    ap.add_argument("--stage-reps", type=int, default=20)
    ap.add_argument("--gptq-only", action="store_true",
                    help="only the error-feedback (GPTQ) stages, printed as one JSON line")
    ap.add_argument("--counter-pass", action="store_true",
                    help="for rocprofv3 --pmc: the quantizer and a few GEMV launches on both "
                         "layers, a few matrix-core launches of the Llama-70B MLP shape, then a "
                         "plain device copy of COPY_BYTES (the counters' calibration)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on one GPU only: the quantized GEMV path has no multi-GPU "
              "component (it would shard by output rows, one row slice per GPU); rerun with "
              "--gpus 1", file=sys.stderr)
        return 2

    import torch

    import synth
    import weight_only_bit_rtn_amd as lw
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    lw.load_library()
    stream = torch.cuda.current_stream().cuda_stream

    layers = synth.WORKLOADS["opt175b_3bit"]
    if args.gptq_only:
        print(json.dumps({"gptq": measure_gptq(lw, torch, stream)}))
        return 0
    if args.counter_pass:
        return counter_pass(lw, torch, layers, stream)
    footprint = sum(product_bytes(L.N, L.K, L.bits, L.group_size, 0) for L in layers)
    copies = copies_for(footprint)
    log(f"[bench] preparing {len(layers)} layers, {copies} weight copies "
        f"({copies * footprint / 1e9:.2f} GB)")
    preps = [Prepared(lw, torch, L, copies) for L in layers]
    for p in preps:
        del p.w
    torch.cuda.synchronize()
    step_bytes = sum(product_bytes(L.N, L.K, L.bits, L.group_size, 1) for L in layers)

    def step(i: int) -> None:
        for p in preps:
            run_product(lw, p, 1, i, stream, "qgemv")

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # timed region: exactly `steps` steps, synchronized on both sides; HIP events
    # on the launch stream (torch's current stream) bracket the same region
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record()
    for i in range(args.steps):
        step(args.warmup + i)
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    value = step_bytes * args.steps / wall / 1e9
    launches = len(preps)
    avg_launch_ms = ev0.elapsed_time(ev1) / (args.steps * launches)
    avg_bytes = step_bytes / launches
    achieved = avg_bytes / (avg_launch_ms * 1e-3) / 1e9

    # per layer: the same back-to-back launches, one layer at a time, between
    # one pair of events on the launch stream (the kernel trace's view), and
    # each launch bracketed by its own events (median, p10, p90: launch
    # overhead included)
    per_layer, spread = {}, {}
    for p in preps:
        L = p.layer
        for i in range(3):
            run_product(lw, p, 1, i, stream, "qgemv")
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(args.steps):
            run_product(lw, p, 1, i, stream, "qgemv")
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / args.steps
        nb = product_bytes(L.N, L.K, L.bits, L.group_size, 1)
        per_layer[L.name] = {"bytes_per_launch": nb, "avg_launch_us": round(us, 3),
                             "achieved": round(nb / (us * 1e-6) / 1e9, 1),
                             "frac": round(nb / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)}
        _, med, p10, p90 = time_launches(
            torch, lambda i, p=p: run_product(lw, p, 1, i, stream, "qgemv"), args.steps,
            spread=True)
        spread[L.name] = {"median": round(med * 1e3, 2), "p10": round(p10 * 1e3, 2),
                          "p90": round(p90 * 1e3, 2)}
    traffic = load_traffic(avg_bytes)

    result = {
        "metric": "packed-weight GB/s & % HBM peak, 3/4-bit dequant-GEMV batch 1 (us/layer)",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "opt175b_3bit_gemv_b1",
                   "layers": [f"{L.N}x{L.K}" for L in layers], "bits": 3,
                   "group_size": "per-row", "batch": 1, "weight_copies": copies,
                   "w_dist": "N(0,0.02) fp16", "x_dist": "N(0,1) fp16", "seed": 0},
        "hbm_frac": round(value / HBM_PEAK_GBPS, 4),
        "us_per_layer": {name: rec["avg_launch_us"] for name, rec in per_layer.items()},
        "us_per_launch_single": spread,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": traffic,
                     "kernel": GEMV_KERNEL,
                     "bytes_per_launch": int(avg_bytes),
                     "avg_launch_us": round(avg_launch_ms * 1e3, 3),
                     "layers": per_layer},
    }
    if not args.no_stages:
        log("[bench] stages")
        result["stages"] = measure_stages(lw, torch, stream, args.stage_reps)
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle)")
        result["cpu_baseline"] = cpu_baseline()
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
