"""Child process of the sanitizer tests: load one build of liblowbit (a path)
and run every host-validation case of test_abi_host against it.  These calls
fail validation (or are empty problems) before any HIP call, so no GPU is
needed.  Prints a summary line; exit status 1 when some status is wrong."""
from __future__ import annotations

import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
TESTS = os.path.dirname(HERE)
ROOT = os.path.dirname(TESTS)
for p in (ROOT, TESTS):
    if p not in sys.path:
        sys.path.insert(0, p)

import weight_only_bit_rtn_amd as lw  # noqa: E402
from test_abi_host import HOST_VALIDATION_CASES, expected_status  # noqa: E402


def main() -> int:
    lw.load_library(sys.argv[1])
    wrong = 0
    for i, (call, status) in enumerate(HOST_VALIDATION_CASES):
        got = call(lw)
        if got != expected_status(lw, status):
            wrong += 1
            print(f"case {i}: got {got}, want {status}", flush=True)
    for st in (0, -1, -2, -3, -4, 17):
        assert lw.status_string(st)
    print(f"abi checks: {len(HOST_VALIDATION_CASES)} cases, {wrong} wrong", flush=True)
    return 1 if wrong else 0


if __name__ == "__main__":
    sys.exit(main())
