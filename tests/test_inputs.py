"""The seeded input generator: rounding, exact widening, determinism."""
import numpy as np
import pytest
import torch

import fa_inputs


def test_bf16_rounding_matches_torch_on_all_high_halves_and_ties():
    hi = np.arange(0, 1 << 16, dtype=np.uint32)
    lows = np.array([0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF], dtype=np.uint32)
    u = (hi[:, None] << 16 | lows[None, :]).ravel()
    x = u.view(np.float32)
    x = x[np.isfinite(x)]
    # values that round up past the largest finite bf16 become inf in both; skip them
    ours = fa_inputs._f32_to_bf16_bits(x.copy())
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_widen_is_exact_round_trip(dtype):
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    w = fa_inputs.widen(bits, dtype)
    finite = np.isfinite(w)
    back = fa_inputs.narrow(w[finite], dtype)
    assert np.array_equal(back, bits[finite])
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float16
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(tdt).to(torch.float64).numpy()
    assert np.array_equal(w[finite], ref[finite])


def test_generator_is_deterministic_and_streams_differ():
    a = fa_inputs.normal_bits(1000, "bf16", 7, 0)
    b = fa_inputs.normal_bits(1000, "bf16", 7, 0)
    c = fa_inputs.normal_bits(1000, "bf16", 7, 1)
    assert np.array_equal(a, b)
    assert not np.array_equal(a, c)


def test_samples_look_standard_normal():
    x = fa_inputs.widen(fa_inputs.normal_bits(200_000, "f16", 11, 2), "f16")
    assert abs(x.mean()) < 0.01
    assert abs(x.std() - 1) < 0.01
