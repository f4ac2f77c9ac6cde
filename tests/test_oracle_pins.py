"""The CPU oracle against its pins (no GPU needed)."""
import pytest

import pins


@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=lambda c: c.__name__)
def test_oracle_pin(oracle_lib, check):
    check(oracle_lib)


def test_oracle_rejects_bad_arguments(oracle_lib):
    import numpy as np
    w = np.zeros((2, 32), np.float16)
    with pytest.raises(ValueError):
        oracle_lib.quantize_rtn(w, 5, 0)          # unsupported width
    with pytest.raises(ValueError):
        oracle_lib.quantize_rtn(w, 4, 12)         # group size does not divide K
    with pytest.raises(ValueError):
        oracle_lib.pack(np.zeros((1, 4), np.uint8), 3)   # 12 bits is not whole words
