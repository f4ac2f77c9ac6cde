"""Host-side checks of the arithmetic identities the GPU quantizer uses in
place of a per-weight IEEE division: the exhaustive check, every finite fp16
weight against every positive finite fp16 scale (2,015,299,584 pairs), split
over parallel processes, plus the scale quotient for every fp32 significand
and the bound that makes the rounding trick exact."""
from __future__ import annotations

import os
import re
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ALL_PAIRS = 2015299584   # finite fp16 w (63488) x positive finite fp16 s (31743)


def test_division_identities_exhaustive(tmp_path):
    exe = tmp_path / "division_identity"
    src = os.path.join(HERE, "native", "division_identity.c")
    r = subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-o", str(exe), src,
                        "-lm"], capture_output=True, text=True)
    if r.returncode != 0:
        pytest.fail(r.stderr)
    parts = max(1, min(16, len(os.sched_getaffinity(0))))

    def run(i):
        return subprocess.run([str(exe), "1", str(i), str(parts)], capture_output=True,
                              text=True, timeout=600)

    with ThreadPoolExecutor(parts) as ex:
        results = list(ex.map(run, range(parts)))
    pairs = 0
    for r in results:
        assert r.returncode == 0, r.stdout + r.stderr
        m = re.search(r"quotient identity: (\d+) pairs, 0 mismatches", r.stdout)
        assert m, r.stdout
        pairs += int(m.group(1))
        assert "scale identity: 0 mismatches" in r.stdout
    assert pairs == ALL_PAIRS
