"""The CPU oracle against its pins (values printed on the pages, the dense-mask
brute force, closed forms and invariants).  No GPU needed."""
import pytest

from tests import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(orc, pin):
    pin(orc)


def test_bf16_rounding_matches_torch():
    import numpy as np
    import torch
    from sliding_window_attention_tiled_amd.inputs import to_bf16_bits
    rng = np.random.Generator(np.random.PCG64(0))
    x = np.concatenate([
        rng.standard_normal(100000, dtype=np.float32),
        rng.standard_normal(1000, dtype=np.float32) * 1e30,
        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3.4e38, -3.4e38, 1e-40, np.inf, -np.inf],
                 np.float32),
    ])
    # ties: 1 + 2^-8 is exactly half-way between two bf16 values
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(to_bf16_bits(x), ref)
