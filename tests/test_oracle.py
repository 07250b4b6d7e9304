"""The fp64 oracle against its pins (CPU only)."""
import pytest

import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(orc, pin):
    pin(orc)


def test_oracle_rejects_bad_arguments(orc):
    import numpy as np

    q = np.zeros((4, 2, 8))
    k = np.zeros((4, 1, 8))
    with pytest.raises(ValueError):
        orc.attention(q, k, k, [0, 4], ("window", 0), 1.0)
    with pytest.raises(ValueError):
        orc.attention(q, k, k, [0, 3], "causal", 1.0)
    with pytest.raises(ValueError):
        orc.attention(q, np.zeros((4, 3, 8)), np.zeros((4, 3, 8)), [0, 4], "causal", 1.0)
    with pytest.raises(ValueError):
        orc.attention(q, k, k, [0, 3, 2, 4], "causal", 1.0)
    with pytest.raises(ValueError):
        orc.attention_rows(q, k, k, [0, 4], "causal", 1.0, [4], [0])
