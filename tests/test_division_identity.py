"""Host-side checks of the arithmetic identities the GPU quantizer uses in
place of a per-weight IEEE division (a reduced version of the exhaustive
check: every fp16 weight against every 61st fp16 scale)."""
from __future__ import annotations

import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


def test_division_identities(tmp_path):
    exe = tmp_path / "division_identity"
    src = os.path.join(HERE, "native", "division_identity.c")
    r = subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-o", str(exe), src,
                        "-lm"], capture_output=True, text=True)
    if r.returncode != 0:
        pytest.fail(r.stderr)
    r = subprocess.run([str(exe), "61"], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "0 mismatches" in r.stdout
