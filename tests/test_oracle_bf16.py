"""Pins of the bfloat16 rounding against torch's own cast and closed forms."""
import numpy as np
import torch

from oracle.bf16 import bf16_bits_to_f64, f32_to_bf16_bits, round_f64_to_bf16


def _torch_bits(x32):
    t = torch.from_numpy(x32).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def test_halfway_and_neighbours_match_torch_exhaustively():
    hi = np.arange(1 << 16, dtype=np.uint32) << np.uint32(16)
    lows = np.array([0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF], dtype=np.uint32)
    bits = (hi[:, None] | lows[None, :]).ravel()
    x32 = bits.view(np.float32)
    mine = f32_to_bf16_bits(x32)
    ref = _torch_bits(x32)
    nan = np.isnan(x32)
    assert np.array_equal(mine[~nan], ref[~nan])
    assert np.all(np.isnan(bf16_bits_to_f64(mine[nan])))


def test_ties_go_to_even():
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7 -> even (1.0);
    # 1 + 3 * 2^-8 is halfway between 1 + 2^-7 and 1 + 2^-6 -> even (1 + 2^-6).
    x = np.array([1 + 2.0**-8, 1 + 3 * 2.0**-8], dtype=np.float32)
    got = bf16_bits_to_f64(f32_to_bf16_bits(x))
    assert got.tolist() == [1.0, 1 + 2.0**-6]


def test_two_step_chain_rounds_through_float32():
    # Just above a bf16 halfway point in float64, but the float32 rounding lands
    # exactly on the halfway point, which then ties to even: the chain gives 1.0
    # where a single float64 -> bf16 rounding would give 1 + 2^-7.
    x = 1 + 2.0**-8 + 2.0**-30
    assert round_f64_to_bf16(np.array([x]))[0] == 1.0
    assert round_f64_to_bf16(np.array([1 + 2.0**-8 + 2.0**-20]))[0] == 1 + 2.0**-7


def test_widening_is_exact():
    r = np.random.default_rng(0).standard_normal(1000).astype(np.float32)
    b = f32_to_bf16_bits(r)
    w = bf16_bits_to_f64(b)
    assert np.array_equal(w, torch.from_numpy(r).to(torch.bfloat16).double().numpy())
