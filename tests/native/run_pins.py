"""Child process of the sanitizer tests: run every oracle pin against one
build of the oracle (a path to its shared library) and print one line per
pin, then a summary line.  Exit status 0 when every pin passes, 1 when some
pin fails; a sanitizer report ends the process with its own status."""
from __future__ import annotations

import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
TESTS = os.path.dirname(HERE)
ROOT = os.path.dirname(TESTS)
for p in (ROOT, TESTS):
    if p not in sys.path:
        sys.path.insert(0, p)

import pins  # noqa: E402
from oracle import Oracle  # noqa: E402


def main() -> int:
    lib = Oracle(sys.argv[1])
    failed = []
    for check in pins.ALL_CHECKS:
        try:
            check(lib)
            print(f"pass {check.__name__}", flush=True)
        except AssertionError:
            failed.append(check.__name__)
            print(f"FAIL {check.__name__}", flush=True)
    print(f"pins: {len(pins.ALL_CHECKS) - len(failed)} passed, {len(failed)} failed", flush=True)
    return 1 if failed else 0


if __name__ == "__main__":
    sys.exit(main())
