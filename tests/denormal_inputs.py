"""Seeded AdamW inputs that live in the subnormal range of fp32 and bf16, for
the tests that check the update keeps subnormals instead of flushing them to
zero. No arithmetic of the method is done here.

  * "moments": subnormal gradients (bf16 patterns 0x0001-0x007F of either sign,
    or fp32 subnormals), subnormal m and v, a normal master weight; clipping
    on (coefficient about 1/2), so the scaled gradient is subnormal too;
  * "decay": zero gradient and moments, a subnormal master weight, a weight
    decay large enough (lr * wd = 0.05) to move subnormals by many units.
"""

import numpy as np

from oracle import step as O

TINY = 2.0 ** -149          # the smallest fp32 subnormal


def subnormal_f32(rng, n, kmax=1 << 23, signed=True):
    """n fp32 subnormals k * 2^-149, 1 <= k < kmax."""
    k = rng.integers(1, kmax, n).astype(np.float64)
    s = rng.choice([-1.0, 1.0], n) if signed else 1.0
    return (s * k * TINY).astype(np.float32)


def subnormal_bf16_bits(rng, n):
    """n bf16 subnormal patterns: magnitude 0x0001-0x007F, random sign."""
    mag = rng.integers(1, 0x80, n).astype(np.uint16)
    return mag | (rng.integers(0, 2, n).astype(np.uint16) << 15)


def case(kind, n, seed, f32grad=False):
    """(grad, master, m, v, ohp, step, partials): grad is bf16 bits, or fp32
    with ``f32grad``; partials is the per-rank sums of squares fed to the
    clip."""
    rng = np.random.default_rng(seed)
    if kind == "moments":
        grad = subnormal_f32(rng, n) if f32grad else subnormal_bf16_bits(rng, n)
        master = (rng.standard_normal(n) * 0.02).astype(np.float32)
        m = subnormal_f32(rng, n, kmax=1 << 20)
        v = subnormal_f32(rng, n, kmax=1 << 20, signed=False)
        ohp = O.AdamWHParams(max_norm=1.0)
        parts = np.array([1.5, 2.5])               # global norm 2: coefficient ~1/2
        return grad, master, m, v, ohp, 3, parts
    if kind == "decay":
        grad = np.zeros(n, np.float32) if f32grad else np.zeros(n, np.uint16)
        master = subnormal_f32(rng, n)
        zeros = np.zeros(n, np.float32)
        ohp = O.AdamWHParams(lr=0.1, weight_decay=0.5, max_norm=0.0)
        return grad, master, zeros, zeros.copy(), ohp, 1, np.zeros(1)
    raise ValueError(kind)


def check_against_oracle(got, want, old_m, old_v):
    """got/want: (master, m, v, param bits). Subnormal results agree with the
    oracle to within 2 units of 2^-149 (a flush to zero is millions of units
    off), every nonzero oracle value stays nonzero, and the bf16 parameter is
    within 1 bf16 ulp of the oracle's."""
    from tolerance import assert_bf16_close, assert_bf16_param, assert_f32_state, ulp_f32
    names = ("master", "m", "v")
    for i, name in enumerate(names):
        g, w = np.asarray(got[i], np.float32), np.asarray(want[i], np.float32)
        assert_f32_state(g, w, name, (None, old_m, old_v)[i])
        sub = np.abs(w) < np.float32(2.0 ** -126)
        d = ulp_f32(g[sub], w[sub])
        assert d.size == 0 or int(d.max()) <= 2, f"{name}: {int(d.max())} subnormal units off"
        lost = (w != 0) & (g == 0)
        assert not lost.any(), f"{name}: {int(lost.sum())} nonzero values flushed to zero"
    assert_bf16_close(got[3], want[3], "param", 1)
    assert_bf16_param(got[3], want[3], want[0], "param", got[0])
    lost = (np.asarray(want[3]) & 0x7FFF != 0) & (np.asarray(got[3]) & 0x7FFF == 0)
    assert not lost.any(), "param: nonzero bf16 values flushed to zero"
