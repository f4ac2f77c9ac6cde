"""Pins for the CPU oracle: checks that tie it to something other than itself.

Every check takes an ``oracle.Oracle`` and raises ``AssertionError`` on a
mismatch.  None of them re-types the oracle's formulas: they use the worked
examples in ``tests/golden`` (derived by hand from the method's definition),
numpy's own IEEE binary16 conversions, exact rational / big-integer
arithmetic, invariants of min-max round-to-nearest quantization, and brute
force search over the quantization grid on tiny inputs.  The planted-mistake
tests run the same checks against deliberately broken builds of the oracle.
"""
from __future__ import annotations

import json
import os
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _f16_values_positive():
    """All positive finite fp16 values, ascending, as float64."""
    bits = np.arange(0x0001, 0x7C00, dtype=np.uint16)
    return bits.view(np.float16).astype(np.float64)


def _frac16(v) -> Fraction:
    return Fraction(float(np.float16(v)))


def _nearest_f16_bits(x: Fraction) -> int:
    """Round an exact rational to fp16 by searching the two neighbours.

    Ties go to the neighbour whose encoding is even.  Overflow follows IEEE:
    magnitudes at or above 65520 (half-way past the largest finite) are inf.
    """
    neg = x < 0
    a = -x if neg else x
    sign = 0x8000 if neg else 0
    if a >= Fraction(65520):
        return sign | 0x7C00
    pos = _POS_F16
    # float(a) is only used to find the bracket; the decision is exact.
    idx = int(np.searchsorted(pos, float(a)))
    cands = set()
    for i in (idx - 2, idx - 1, idx, idx + 1):
        if 0 <= i < len(pos):
            cands.add(i)
    best = None
    for i in sorted(cands):
        v = Fraction(float(pos[i]))
        d = abs(v - a)
        enc = i + 1  # encoding of pos[i]
        key = (d, enc & 1)
        if best is None or key < best[0]:
            best = (key, enc)
    zero_key = (a, 0)
    if zero_key < best[0]:
        return sign
    return sign | best[1]


_POS_F16 = _f16_values_positive()


# ---------------------------------------------------------------------------
# fp16 conversions against numpy's binary16 implementation
# ---------------------------------------------------------------------------
def check_f16_decode(o) -> None:
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([o.f16_to_f64(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan), "NaN decoding differs"
    assert np.array_equal(got[~nan], ref[~nan]), "fp16 -> double decoding differs from numpy"
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan])), "sign of zero differs"


def _encode_probe_values(rng) -> np.ndarray:
    pos = _POS_F16
    mids = (pos[:-1] + pos[1:]) / 2.0          # exact in double
    vals = [pos, mids, np.nextafter(mids, 0), np.nextafter(mids, np.inf),
            np.array([0.0, 2.0 ** -25, np.nextafter(2.0 ** -25, 1), 2.0 ** -26, 65504.0,
                      65519.99, 65520.0, 65536.0, 1e300, np.inf]),
            np.exp(rng.uniform(np.log(2.0 ** -30), np.log(2.0 ** 17), 20000))]
    v = np.concatenate(vals)
    return np.concatenate([v, -v])


def check_f16_encode(o) -> None:
    rng = np.random.default_rng(12345)
    vals = _encode_probe_values(rng)
    with np.errstate(over="ignore"):
        ref = vals.astype(np.float16).view(np.uint16)
    got = np.array([o.f64_to_f16(float(v)) for v in vals], dtype=np.uint16)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, (
        f"double -> fp16 rounding differs from numpy at {vals[bad[:5]]}: "
        f"got {[hex(g) for g in got[bad[:5]]]} want {[hex(r) for r in ref[bad[:5]]]}")


# ---------------------------------------------------------------------------
# Worked examples (tests/golden)
# ---------------------------------------------------------------------------
def check_worked_examples(o) -> None:
    for case in _load("rtn_worked_examples.json")["cases"]:
        w = np.array([case["w"]], np.float16)
        codes, scales, zeros = o.quantize_rtn(w, case["bits"], 0)
        name = case["name"]
        assert scales.view(np.uint16)[0, 0] == int(case["scale_f16_bits"], 16), name
        assert zeros[0, 0] == case["zero"], name
        assert codes[0].tolist() == case["codes"], name
        deq = o.dequant(codes, scales, zeros, case["bits"], 0)
        assert deq[0].astype(np.float64).tolist() == case["deq"], name


def check_pack_closed_forms(o) -> None:
    for case in _load("pack_closed_forms.json")["cases"]:
        codes = np.array([case["codes"]], np.uint8)
        words = o.pack(codes, case["bits"])
        assert [int(v) for v in words[0]] == [int(h, 16) for h in case["words"]], case["name"]
        assert np.array_equal(o.unpack(words, codes.shape[1], case["bits"]), codes), case["name"]


def check_pack_bigint(o) -> None:
    """Packing against a Python big-integer bitstream, plus the round trip."""
    rng = np.random.default_rng(7)
    for bits in (2, 3, 4, 8):
        for K in (32, 64, 96, 128, 160, 416):
            if (K * bits) % 32:
                continue
            codes = rng.integers(0, 1 << bits, size=(3, K), dtype=np.uint8)
            words = o.pack(codes, bits)
            assert words.shape == (3, K * bits // 32)
            for n in range(3):
                stream = 0
                for k in range(K):
                    stream |= int(codes[n, k]) << (bits * k)
                want = [(stream >> (32 * i)) & 0xFFFFFFFF for i in range(K * bits // 32)]
                assert [int(v) for v in words[n]] == want, (bits, K, n)
            assert np.array_equal(o.unpack(words, K, bits), codes), (bits, K)


# ---------------------------------------------------------------------------
# Invariants of min-max RTN on random inputs
# ---------------------------------------------------------------------------
def _random_weight_sets(rng):
    N, K = 12, 256
    yield "normal", (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    yield "uniform", rng.uniform(-3, 5, (N, K)).astype(np.float16)
    yield "positive", rng.uniform(0.5, 2.0, (N, K)).astype(np.float16)
    yield "negative", rng.uniform(-7.0, -0.01, (N, K)).astype(np.float16)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    w[:, rng.choice(K, 3, replace=False)] *= 10
    yield "outliers", w.astype(np.float16)
    yield "wide", (rng.standard_normal((N, K)) * 300).astype(np.float16)


def check_invariants(o) -> None:
    rng = np.random.default_rng(2024)
    for label, w in _random_weight_sets(rng):
        N, K = w.shape
        wf = w.astype(np.float64)
        for bits in (2, 3, 4, 8):
            M = (1 << bits) - 1
            for g in (0, 32, 64, 128):
                codes, scales, zeros = o.quantize_rtn(w, bits, g)
                gs = K if g == 0 else g
                G = K // gs
                assert codes.shape == (N, K) and scales.shape == (N, G) and zeros.shape == (N, G)
                assert codes.max() <= M, (label, bits, g, "code above M")
                deq = o.dequant(codes, scales, zeros, bits, g).astype(np.float64)
                s = scales.astype(np.float64)
                for n in range(N):
                    for j in range(G):
                        seg = slice(j * gs, (j + 1) * gs)
                        wseg = wf[n, seg]
                        cseg = codes[n, seg]
                        lo_i, hi_i = int(np.argmin(wseg)), int(np.argmax(wseg))
                        assert cseg[lo_i] == 0, (label, bits, g, "min must map to code 0")
                        if wseg[hi_i] > wseg[lo_i]:
                            assert cseg[hi_i] in (M - 1, M), (label, bits, g, "max code")
                        sj = s[n, j]
                        err = np.abs(deq[n, seg] - wseg)
                        bound = sj * (0.5 + M * 2.0 ** -10) + np.abs(wseg) * 2.0 ** -22
                        assert np.all(err <= bound), (label, bits, g, "reconstruction error")


def check_scale_is_nearest(o) -> None:
    """The stored scale is the fp16 nearest to the exact (max - min)/M.

    max - min is taken as one IEEE fp32 subtraction (numpy float32), and the
    nearest fp16 is found by exact rational search, so this does not go
    through any fp16 rounding routine.  A zero result must be stored as 1.0.
    """
    rng = np.random.default_rng(99)
    for label, w in _random_weight_sets(rng):
        for bits in (2, 3, 4, 8):
            M = (1 << bits) - 1
            for g in (0, 64):
                _, scales, _ = o.quantize_rtn(w, bits, g)
                N, K = w.shape
                gs = K if g == 0 else g
                sb = scales.view(np.uint16)
                for n in range(0, N, 3):
                    for j in range(0, K // gs, 2):
                        seg = w[n, j * gs:(j + 1) * gs].astype(np.float32)
                        d = np.float32(seg.max()) - np.float32(seg.min())
                        want = _nearest_f16_bits(Fraction(float(d)) / M)
                        if want & 0x7FFF == 0:
                            want = 0x3C00
                        assert sb[n, j] == want, (label, bits, g, hex(sb[n, j]), hex(want))


def check_dequant_is_exact(o) -> None:
    """deq is exactly the rational (q - zero) * scale, with no rounding (the
    fp16 scale taken as its exact rational value); also for zero points far
    outside the code range."""
    rng = np.random.default_rng(5)
    for label, w in _random_weight_sets(rng):
        for bits in (2, 4, 8):
            codes, scales, zeros = o.quantize_rtn(w, bits, 32)
            if label == "wide":
                zeros = zeros + rng.integers(-40000, 40000, zeros.shape).astype(np.int32)
            deq = o.dequant(codes, scales, zeros, bits, 32)
            for n in range(0, w.shape[0], 4):
                for k in range(0, w.shape[1], 7):
                    j = k // 32
                    exact = (int(codes[n, k]) - int(zeros[n, j])) * _frac16(scales[n, j])
                    assert Fraction(float(deq[n, k])) == exact, (label, bits, n, k)


# ---------------------------------------------------------------------------
# Brute force on tiny matrices: the codes are nearest grid points
# ---------------------------------------------------------------------------
def _rint_by_search(t: Fraction) -> int:
    """Nearest integer to t, ties to the even one, found by comparison."""
    lo = int(np.floor(float(t))) - 1
    best = None
    for c in range(lo, lo + 4):
        key = (abs(Fraction(c) - t), c & 1)
        if best is None or key < best[0]:
            best = (key, c)
    return best[1]


def check_rtn_bruteforce(o) -> None:
    rng = np.random.default_rng(31337)
    for trial in range(80):
        bits = (2, 3, 4, 8)[trial % 4]
        M = (1 << bits) - 1
        g = (0, 2, 4)[(trial // 4) % 3]
        w = (rng.standard_normal((4, 8)) * rng.choice([0.02, 1.0, 40.0])).astype(np.float16)
        if trial % 7 == 0:
            w[1, :4] = w[1, 0]                         # a constant group
        codes, scales, zeros = o.quantize_rtn(w, bits, g)
        gs = 8 if g == 0 else g
        for n in range(4):
            for j in range(8 // gs):
                s32 = np.float32(scales[n, j])
                seg = w[n, j * gs:(j + 1) * gs]
                lo = np.float32(seg.min())
                # zero point: the integer nearest the fp32 quotient -lo/s
                zq = Fraction(float(np.float32(-lo) / s32))
                assert zeros[n, j] == _rint_by_search(zq), ("zero", trial, n, j)
                z = int(zeros[n, j])
                for k in range(gs):
                    t = Fraction(float(np.float32(seg[k]) / s32))
                    # search the whole grid for the nearest level (q - z) to t
                    best = None
                    for q in range(M + 1):
                        key = (abs(Fraction(q - z) - t), (q - z) & 1)
                        if best is None or key < best[0]:
                            best = (key, q)
                    # a tie between two levels is broken toward an even (q - z)
                    # only when both are inside [0, M]; clamping otherwise picks
                    # the nearest end, which the search above also yields
                    assert codes[n, j * gs + k] == best[1], ("code", trial, n, j, k)


# ---------------------------------------------------------------------------
# Signed symmetric variant (zero point fixed at 2^(b-1))
# ---------------------------------------------------------------------------
def check_sym_worked_examples(o) -> None:
    for case in _load("rtn_sym_worked_examples.json")["cases"]:
        w = np.array([case["w"]], np.float16)
        codes, scales, zeros = o.quantize_rtn_sym(w, case["bits"], 0)
        name = case["name"]
        assert scales.view(np.uint16)[0, 0] == int(case["scale_f16_bits"], 16), name
        assert zeros[0, 0] == case["zero"], name
        assert codes[0].tolist() == case["codes"], name
        deq = o.dequant(codes, scales, zeros, case["bits"], 0)
        assert deq[0].astype(np.float64).tolist() == case["deq"], name


def check_sym_invariants(o) -> None:
    """Zero point 2^(b-1); codes in [1, 2^b - 1]; the largest magnitude maps to
    the end of the grid with its sign; quantizing -w mirrors the codes about
    the zero point (round-half-even is odd-symmetric); bounded reconstruction
    error."""
    rng = np.random.default_rng(4242)
    for label, w in _random_weight_sets(rng):
        N, K = w.shape
        wf = w.astype(np.float64)
        for bits in (2, 3, 4, 8):
            M, z, qmax = (1 << bits) - 1, 1 << (bits - 1), (1 << (bits - 1)) - 1
            for g in (0, 32, 128):
                codes, scales, zeros = o.quantize_rtn_sym(w, bits, g)
                neg_codes, neg_scales, _ = o.quantize_rtn_sym(-w, bits, g)
                assert np.all(zeros == z), (label, bits, g, "zero point")
                assert codes.min() >= 1 and codes.max() <= M, (label, bits, g, "code range")
                assert np.array_equal(neg_scales.view(np.uint16), scales.view(np.uint16))
                assert np.array_equal(neg_codes.astype(int), 2 * z - codes.astype(int)), \
                    (label, bits, g, "mirror")
                gs = K if g == 0 else g
                deq = o.dequant(codes, scales, zeros, bits, g).astype(np.float64)
                for n in range(N):
                    for j in range(K // gs):
                        seg = slice(j * gs, (j + 1) * gs)
                        wseg = wf[n, seg]
                        i = int(np.argmax(np.abs(wseg)))
                        if wseg[i] != 0:
                            want = z + qmax if wseg[i] > 0 else z - qmax
                            assert codes[n, seg][i] == want, (label, bits, g, "extreme code")
                        sj = float(scales[n, j])
                        err = np.abs(deq[n, seg] - wseg)
                        bound = sj * (0.5 + qmax * 2.0 ** -10) + np.abs(wseg) * 2.0 ** -22
                        assert np.all(err <= bound), (label, bits, g, "reconstruction error")


def check_sym_scale_is_nearest(o) -> None:
    """The stored scale is the fp16 nearest to the fp32 quotient max|w| / qmax
    (one IEEE fp32 division, numpy float32), found by exact rational search;
    a zero result is stored as 1.0."""
    rng = np.random.default_rng(606)
    for label, w in _random_weight_sets(rng):
        for bits in (2, 3, 4, 8):
            qmax = (1 << (bits - 1)) - 1
            for g in (0, 64):
                _, scales, _ = o.quantize_rtn_sym(w, bits, g)
                N, K = w.shape
                gs = K if g == 0 else g
                sb = scales.view(np.uint16)
                for n in range(0, N, 3):
                    for j in range(0, K // gs, 2):
                        amax = np.float32(np.abs(w[n, j * gs:(j + 1) * gs].astype(np.float32)).max())
                        q32 = amax / np.float32(qmax)
                        want = _nearest_f16_bits(Fraction(float(q32)))
                        if want & 0x7FFF == 0:
                            want = 0x3C00
                        assert sb[n, j] == want, (label, bits, g, hex(sb[n, j]), hex(want))


def check_sym_bruteforce(o) -> None:
    """Every code, less the zero point, is the grid level of [-qmax, qmax]
    nearest the fp32 quotient w / s (ties to the even level)."""
    rng = np.random.default_rng(8080)
    for trial in range(60):
        bits = (2, 3, 4, 8)[trial % 4]
        z, qmax = 1 << (bits - 1), (1 << (bits - 1)) - 1
        g = (0, 2, 4)[(trial // 4) % 3]
        w = (rng.standard_normal((4, 8)) * rng.choice([0.02, 1.0, 40.0])).astype(np.float16)
        if trial % 5 == 0:
            w[2, :4] = 0
        codes, scales, zeros = o.quantize_rtn_sym(w, bits, g)
        gs = 8 if g == 0 else g
        for n in range(4):
            for j in range(8 // gs):
                s32 = np.float32(scales[n, j])
                for k in range(gs):
                    t = Fraction(float(np.float32(w[n, j * gs + k]) / s32))
                    best = None
                    for q in range(-qmax, qmax + 1):
                        key = (abs(Fraction(q) - t), q & 1)
                        if best is None or key < best[0]:
                            best = (key, q)
                    assert codes[n, j * gs + k] == best[1] + z, ("sym code", trial, n, j, k)


# ---------------------------------------------------------------------------
# Compact metadata words (fp16 scale | int16 zero << 16)
# ---------------------------------------------------------------------------
def check_meta_words(o) -> None:
    cases = _load("meta_words.json")["cases"]
    for case in cases:
        s = np.array([int(case["scale_f16_bits"], 16)], np.uint16).view(np.float16)
        z = np.array([case["zero"]], np.int32)
        meta, sat = o.pack_meta(s, z)
        assert int(meta[0]) == int(case["word"], 16), case["name"]
        assert sat == case["saturated"], case["name"]
        s2, z2 = o.unpack_meta(meta)
        assert s2.view(np.uint16)[0] == s.view(np.uint16)[0], case["name"]
        assert z2[0] == max(-32768, min(32767, case["zero"])), case["name"]
    # all cases in one call: the count adds up
    s = np.array([int(c["scale_f16_bits"], 16) for c in cases], np.uint16).view(np.float16)
    z = np.array([c["zero"] for c in cases], np.int32)
    _, sat = o.pack_meta(s, z)
    assert sat == sum(c["saturated"] for c in cases)


def check_meta_round_trip(o) -> None:
    """In-range zero points survive the word; out-of-range ones saturate and
    are counted; the low half is the scale's bit pattern unchanged.  The RTN
    zero points of 2/3/4-bit groups with hi > lo fit (|z| <= M * 2^11 <= 30720)."""
    rng = np.random.default_rng(16)
    sb = rng.integers(0, 0x7C00, 4000).astype(np.uint16)
    z = rng.integers(-70000, 70000, 4000).astype(np.int32)
    meta, sat = o.pack_meta(sb.view(np.float16), z)
    assert np.array_equal((meta & 0xFFFF).astype(np.uint16), sb)
    hi = (meta >> 16).astype(np.uint16).view(np.int16).astype(np.int32)
    assert np.array_equal(hi, np.clip(z, -32768, 32767))
    assert sat == int(np.sum((z < -32768) | (z > 32767)))
    for label, w in _random_weight_sets(rng):
        for bits in (2, 3, 4):
            _, scales, zeros = o.quantize_rtn(w, bits, 32)
            meta, sat = o.pack_meta(scales, zeros)
            assert sat == 0, (label, bits)
            s2, z2 = o.unpack_meta(meta)
            assert np.array_equal(s2.view(np.uint16), scales.view(np.uint16))
            assert np.array_equal(z2, zeros)


# ---------------------------------------------------------------------------
# Error-feedback (GPTQ) quantization
# ---------------------------------------------------------------------------
def _hadamard(n: int) -> np.ndarray:
    h = np.array([[1.0]])
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


def check_gptq_worked_example(o) -> None:
    for case in _load("gptq_worked_example.json")["cases"]:
        x = np.array(case["x"], np.float16)
        w = np.array([case["w"]], np.float16)
        H = o.hessian(x, case["damp"])
        assert np.array_equal(H, np.array(case["hessian"])), case["name"]
        codes, _, _ = o.quantize_gptq(w, H, case["bits"], 0)
        assert codes[0].tolist() == case["gptq_codes"], case["name"]
        rtn, _, _ = o.quantize_rtn(w, case["bits"], 0)
        assert rtn[0].tolist() == case["rtn_codes"], case["name"]


def check_gptq_hessian_closed_form(o) -> None:
    """Hadamard calibration rows: X^T X = n I exactly, so H = 2 I + 2 damp I."""
    for K in (16, 64):
        x = _hadamard(K).astype(np.float16)
        for damp in (0.0, 0.01, 0.25):
            H = o.hessian(x, damp)
            assert np.array_equal(H, np.eye(K) * (2.0 + 2.0 * damp)), (K, damp)
        # scaled columns: X^T X = n diag(c^2)
        c = np.array([1.0, 2.0, 0.5, 4.0] * (K // 4))
        H = o.hessian((x * c).astype(np.float16), 0.0)
        assert np.array_equal(H, np.diag(2.0 * c * c)), K


def check_gptq_uncoupled_is_rtn(o) -> None:
    """With a diagonal Hessian no error reaches another column: the codes are
    the round-to-nearest codes (the fp64 and fp32 quotients give the same
    integers for these weights), on the same grid."""
    rng = np.random.default_rng(1717)
    K = 64
    had = _hadamard(K)
    for trial in range(8):
        c = rng.choice([0.5, 1.0, 2.0, 4.0], K)
        H = o.hessian((had * c).astype(np.float16), (0.0, 0.01)[trial % 2])
        w = (rng.standard_normal((6, K)) * 0.02).astype(np.float16)
        for bits in (2, 3, 4, 8):
            for g in (0, 16, 32):
                codes, scales, zeros = o.quantize_gptq(w, H, bits, g)
                rcodes, rscales, rzeros = o.quantize_rtn(w, bits, g)
                scodes, sscales, szeros = o.quantize_gptq(w, H, bits, g, symmetric=True)
                rs = o.quantize_rtn_sym(w, bits, g)
                assert np.array_equal(scodes, rs[0]), (trial, bits, g, "sym")
                assert np.array_equal(sscales.view(np.uint16), rs[1].view(np.uint16))
                assert np.array_equal(szeros, rs[2])
                assert np.array_equal(codes, rcodes), (trial, bits, g)
                assert np.array_equal(scales.view(np.uint16), rscales.view(np.uint16))
                assert np.array_equal(zeros, rzeros)


def _gptq_upper_cholesky_form(w, H, scales, zeros, bits, g, qlo=0):
    """The same method through the upper Cholesky factor U of H^-1 (H^-1 =
    U^T U): err = (w_i - deq_i) / U_ii, w_j -= err * U_ij."""
    N, K = w.shape
    M = (1 << bits) - 1
    U = np.linalg.cholesky(np.linalg.inv(H)).T
    cur = w.astype(np.float64)
    codes = np.zeros((N, K), np.uint8)
    gs = K if g == 0 else g
    for i in range(K):
        s = scales[:, i // gs].astype(np.float64)
        z = zeros[:, i // gs].astype(np.int64)
        q = np.clip(np.rint(cur[:, i] / s).astype(np.int64) + z, qlo, M)
        codes[:, i] = q
        deq = (q - z) * s
        err = (cur[:, i] - deq) / U[i, i]
        cur[:, i + 1:] -= np.outer(err, U[i, i + 1:])
    return codes


def _gptq_reverse_cholesky_form(w, H, scales, zeros, bits, g, qlo=0):
    """The same method through R with H = R R^T, R upper triangular (the
    Cholesky factor of H with the index order reversed), without an inverse:
    t_j = w_j + (sum_{i<j} d_i R_ij) / R_jj with d_i = w_i - deq_i on the
    ORIGINAL weights."""
    N, K = w.shape
    M = (1 << bits) - 1
    P = np.eye(K)[::-1]
    R = P @ np.linalg.cholesky(P @ H @ P) @ P
    wf = w.astype(np.float64)
    d = np.zeros((N, K))
    codes = np.zeros((N, K), np.uint8)
    gs = K if g == 0 else g
    for j in range(K):
        s = scales[:, j // gs].astype(np.float64)
        z = zeros[:, j // gs].astype(np.int64)
        t = wf[:, j] + d[:, :j] @ R[:j, j] / R[j, j]
        q = np.clip(np.rint(t / s).astype(np.int64) + z, qlo, M)
        codes[:, j] = q
        d[:, j] = wf[:, j] - (q - z) * s
    return codes


def check_gptq_other_formulations(o) -> None:
    """Two algebraically equal formulations, written independently in numpy,
    give the same codes on random correlated calibration data.  (They differ
    from the oracle only by fp64 rounding; a code could flip only when a
    quotient lands within ~1e-12 of a rounding midpoint.)"""
    rng = np.random.default_rng(2323)
    for trial in range(12):
        K = (32, 48, 64)[trial % 3]
        n = 3 * K
        mix = rng.standard_normal((K, K)) / np.sqrt(K) + np.eye(K)
        x = (rng.standard_normal((n, K)) @ mix).astype(np.float16)
        H = o.hessian(x, 0.01)
        w = (rng.standard_normal((5, K)) * rng.choice([0.02, 1.0])).astype(np.float16)
        bits = (2, 3, 4, 8)[trial % 4]
        g = (0, 16)[trial % 2]
        sym = trial % 3 == 2
        codes, scales, zeros = o.quantize_gptq(w, H, bits, g, symmetric=sym)
        qlo = 1 if sym else 0
        if sym:
            assert (zeros == 1 << (bits - 1)).all() and codes.min() >= 1, trial
        s = scales.astype(np.float64)
        assert np.array_equal(codes, _gptq_upper_cholesky_form(w, H, s, zeros, bits, g, qlo)), trial
        assert np.array_equal(codes, _gptq_reverse_cholesky_form(w, H, s, zeros, bits, g, qlo)), trial


def check_gptq_lowers_output_error(o) -> None:
    """The point of the feedback: on correlated inputs the layer-output error
    ||(W - deq(Q)) X^T|| is smaller than that of round-to-nearest."""
    rng = np.random.default_rng(99)
    K, n = 64, 256
    mix = rng.standard_normal((K, K)) / np.sqrt(K) + np.eye(K)
    x = (rng.standard_normal((n, K)) @ mix).astype(np.float16)
    H = o.hessian(x, 0.01)
    w = (rng.standard_normal((16, K)) * 0.02).astype(np.float16)
    xf = x.astype(np.float64)
    for bits in (2, 3, 4):
        qg, s, z = o.quantize_gptq(w, H, bits, 0)
        qr, _, _ = o.quantize_rtn(w, bits, 0)
        dg = o.dequant(qg, s, z, bits, 0).astype(np.float64)
        dr = o.dequant(qr, s, z, bits, 0).astype(np.float64)
        wf = w.astype(np.float64)
        eg = np.linalg.norm((wf - dg) @ xf.T)
        er = np.linalg.norm((wf - dr) @ xf.T)
        assert eg < er, (bits, eg, er)


# ---------------------------------------------------------------------------
# The reference product against exact integer arithmetic
# ---------------------------------------------------------------------------
def check_matmul_exact(o) -> None:
    rng = np.random.default_rng(77)
    for trial in range(20):
        B, N, K = 3, 4, 8
        x = (rng.standard_normal((B, K)) * 2).astype(np.float16)
        # dequantized weights are exact products (q - z) * s: up to 19 significant
        # bits, every one an integer multiple of 2^-24 like the fp16 values
        d = (rng.standard_normal((N, K)) * 0.05).astype(np.float16).astype(np.float64)
        d *= rng.integers(-255, 256, (N, K))
        if trial == 0:
            d[:] = d[0, 0]                             # all-equal weights: y = sum(x) * d
        y = o.matmul_f64(x, d)
        assert y.shape == (B, N)
        # every fp16 value is an integer multiple of 2^-24
        xi = [[int(Fraction(float(v)) * 2 ** 24) for v in row] for row in x]
        di = [[int(Fraction(float(v)) * 2 ** 24) for v in row] for row in d]
        for b in range(B):
            for n in range(N):
                exact = Fraction(sum(xi[b][k] * di[n][k] for k in range(K)), 2 ** 48)
                mag = sum(abs(Fraction(xi[b][k] * di[n][k], 2 ** 48)) for k in range(K))
                assert abs(Fraction(y[b, n]) - exact) <= mag * Fraction(K, 2 ** 52), (trial, b, n)
        if trial == 0:
            want = x.astype(np.float64).sum(axis=1, keepdims=True) * d[0, 0]
            assert np.allclose(y, np.repeat(want, N, axis=1), rtol=1e-12, atol=0)
        assert np.allclose(y, x.astype(np.float64) @ d.astype(np.float64).T, rtol=1e-12,
                           atol=1e-300)


ALL_CHECKS = [check_sym_worked_examples, check_sym_invariants, check_sym_scale_is_nearest,
              check_sym_bruteforce, check_f16_decode, check_f16_encode, check_worked_examples,
              check_pack_closed_forms, check_pack_bigint, check_invariants,
              check_scale_is_nearest, check_dequant_is_exact, check_rtn_bruteforce,
              check_matmul_exact, check_meta_words, check_meta_round_trip,
              check_gptq_worked_example, check_gptq_hessian_closed_form,
              check_gptq_uncoupled_is_rtn, check_gptq_other_formulations,
              check_gptq_lowers_output_error]
