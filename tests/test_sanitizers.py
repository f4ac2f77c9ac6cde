"""The CPU oracle and the C ABI's host code under AddressSanitizer and
UndefinedBehaviorSanitizer (host code only; nothing runs on a GPU).

- The oracle is rebuilt with ``-fsanitize=address,undefined`` and every pin
  runs against that build in a child process (the sanitizer runtime is
  preloaded there, since the Python interpreter itself is not instrumented).
- Every planted mistake of ``test_oracle_mutants`` is rebuilt the same way:
  each must still be caught, by a failing pin or by a sanitizer report.
- The host half of the ABI (``abi.hip``: argument checks and status codes) is
  rebuilt with the sanitizers on its host code only and linked with the
  library's other objects; the host-validation cases run against it.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

from test_oracle_mutants import MUTANTS

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
ORACLE_SRC = os.path.join(ROOT, "oracle", "lowbit_oracle.c")
ORACLE_HDR = os.path.join(ROOT, "oracle", "lowbit_oracle.h")
RUN_PINS = os.path.join(HERE, "native", "run_pins.py")
SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all",
             "-fno-omit-frame-pointer"]
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=0",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _gcc_runtime(name: str) -> str:
    return subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True,
                          text=True).stdout.strip()


def _build_oracle(src_text: str, out_dir, name: str) -> str:
    src = os.path.join(out_dir, f"{name}.c")
    with open(src, "w") as f:
        f.write(src_text)
    hdr = os.path.join(out_dir, "lowbit_oracle.h")
    if not os.path.exists(hdr):
        with open(hdr, "w") as f:
            f.write(open(ORACLE_HDR).read())
    so = os.path.join(out_dir, f"{name}.so")
    subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
                    "-fPIC", "-shared", *SAN_FLAGS, "-o", so, src, "-lm"], check=True)
    return so


def _run_pins(so: str):
    env = dict(os.environ, LD_PRELOAD=_gcc_runtime("libasan.so"), **SAN_ENV)
    return subprocess.run([sys.executable, RUN_PINS, so], capture_output=True, text=True,
                          env=env, timeout=600)


def _sanitizer_report(r) -> bool:
    return "AddressSanitizer" in r.stderr or "runtime error:" in r.stderr


def test_oracle_pins_under_sanitizers(tmp_path):
    so = _build_oracle(open(ORACLE_SRC).read(), str(tmp_path), "oracle_san")
    r = _run_pins(so)
    assert not _sanitizer_report(r), r.stderr[-4000:]
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]
    assert "0 failed" in r.stdout


def test_planted_mistakes_under_sanitizers(tmp_path):
    text = open(ORACLE_SRC).read()

    def one(name):
        old, new = MUTANTS[name]
        assert text.count(old) == 1, name
        d = tmp_path / name
        d.mkdir()
        so = _build_oracle(text.replace(old, new), str(d), f"mutant_{name}")
        r = _run_pins(so)
        caught = r.returncode != 0 and ("FAIL " in r.stdout or _sanitizer_report(r))
        return name, caught, r

    workers = max(1, min(8, len(os.sched_getaffinity(0))))
    with ThreadPoolExecutor(workers) as ex:
        results = list(ex.map(one, sorted(MUTANTS)))
    missed = [name for name, caught, _ in results if not caught]
    assert not missed, f"planted mistakes not caught under the sanitizers: {missed}"


def _clang_asan_runtime() -> str | None:
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/*/libclang_rt.asan-x86_64.so") +
                  glob.glob("/opt/rocm/llvm/lib/clang/*/lib/*/libclang_rt.asan.so"))
    return hits[-1] if hits else None


def test_abi_host_checks_under_sanitizers(tmp_path):
    """abi.hip rebuilt with host-side ASan + UBSan (the device code is built
    as usual), linked with the library's other objects; every host-validation
    case of test_abi_host must return its status with no sanitizer report."""
    from weight_only_bit_rtn_amd import build as lib_build
    rt = _clang_asan_runtime()
    if rt is None:
        pytest.skip("no clang AddressSanitizer runtime in this ROCm install")
    objs = []
    for src in lib_build.SOURCES:
        obj = os.path.join(lib_build._obj_dir(), os.path.splitext(src)[0] + ".o")
        if src != "abi.hip" and not os.path.exists(obj):
            obj = lib_build._compile(src)
        objs.append(obj)
    san_obj = str(tmp_path / "abi_san.o")
    host_san = []
    for flag in ("-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all"):
        host_san += ["-Xarch_host", flag]
    cmd = [lib_build.HIPCC, *lib_build.FLAGS, *host_san, "-c",
           os.path.join(lib_build.CSRC, "abi.hip"), "-o", san_obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    objs = [san_obj if o.endswith(os.sep + "abi.o") else o for o in objs]
    so = str(tmp_path / "liblowbit_san.so")
    # the sanitizer runtime is linked as a plain shared library (it is also
    # preloaded into the child process)
    r = subprocess.run([lib_build.HIPCC, f"--offload-arch={lib_build.ARCH}", "-shared", "-fPIC",
                        "-o", so, *objs, rt], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, LD_PRELOAD=rt, **SAN_ENV)
    r = subprocess.run([sys.executable, os.path.join(HERE, "native", "run_abi_checks.py"), so],
                       capture_output=True, text=True, env=env, timeout=600)
    assert not _sanitizer_report(r), r.stderr[-4000:]
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]
    assert "0 wrong" in r.stdout
