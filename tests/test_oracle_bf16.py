"""Pins for oracle.bf16 against torch's CPU bfloat16 cast (a library routine)."""

import numpy as np
import torch

from oracle.bf16 import bf16_to_f32, f32_to_bf16


def _torch_bits(x_f32):
    t = torch.from_numpy(np.ascontiguousarray(x_f32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _check(u32):
    x = np.asarray(u32, dtype=np.uint32).view(np.float32)
    ours = f32_to_bf16(x)
    ref = _torch_bits(x)
    nan = np.isnan(x)
    assert (ours[~nan] == ref[~nan]).all()
    # NaN stays NaN (payload not compared), with its sign
    got = bf16_to_f32(ours[nan])
    assert np.isnan(got).all()
    assert (np.signbit(got) == np.signbit(x[nan])).all()


def test_edge_classes():
    pats = [0x00000000, 0x80000000,             # +-0
            0x3F800000, 0xBF800000,             # +-1
            0x3F808000,                         # tie, lower even -> down
            0x3F818000,                         # tie, lower odd -> up
            0x3F808001, 0x3F807FFF,             # just above / below a tie
            0x7F7FFFFF, 0xFF7FFFFF,             # max finite fp32 -> inf
            0x7F7F7FFF,                         # stays max finite bf16
            0x7F7F8000,                         # tie at the top -> inf
            0x7F800000, 0xFF800000,             # +-inf
            0x7FC00000, 0xFFC00000, 0x7F800001, 0x7FA50000,   # NaNs
            0x00000001, 0x80000001, 0x00008000, 0x00018000,   # denormals, ties
            0x007FFFFF, 0x00800000, 0x0080FFFF]
    _check(pats)


def test_random_patterns():
    """10^8 random 32-bit patterns, in chunks of 2^24."""
    rng = np.random.default_rng(7)
    left = 100_000_000
    while left > 0:
        n = min(left, 1 << 24)
        _check(rng.integers(0, 2**32, size=n, dtype=np.uint64).astype(np.uint32))
        left -= n


def test_all_low_halves_of_some_exponents():
    # every rounding-relevant low half for a few leading halves
    low = np.arange(0, 1 << 16, dtype=np.uint32)
    for hi in (0x3F80, 0x3F81, 0x0000, 0x0001, 0x7F7F, 0xC2F7, 0x8080):
        _check((np.uint32(hi) << np.uint32(16)) | low)


def test_widening_is_exact():
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    wide = bf16_to_f32(bits)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(wide), nan)
    assert np.array_equal(wide[~nan].view(np.uint32), ref[~nan].view(np.uint32))
    # and round trip is the identity on every non-NaN pattern
    assert (f32_to_bf16(wide)[~nan] == bits[~nan]).all()
