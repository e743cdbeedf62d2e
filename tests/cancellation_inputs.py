"""Update inputs whose new master lands near zero by cancellation.

The bf16 parameter is the rounding of the new fp32 master. When the decayed
master p(1 - lr*wd) and the step (lr/(1-beta1^t)) * m'/denominator nearly
cancel, the new master is tiny and an fp32 evaluation of the step keeps few of
its bits; the update recomputes such elements in fp64. These inputs put a
tenth of the masters at cancellation points, within relative distances spread
over 1e-9 .. 1e-3, so both sides of the update's threshold are exercised.

``deep`` marks the elements whose exact new master is below 2^-14 of the
magnitudes it is formed from (``size``, the sum of the absolute values of the
decayed master and of the two terms of the step's first moment, scaled as in
the step): those are certainly recomputed in fp64, and their stored fp32
values must equal the oracle's bit for bit (the oracle takes the same fp64
steps in the same order). Elsewhere the fp32 evaluation is accurate to
2^-21 of ``size``, which near such cancellations can exceed the absolute
1e-8 of the fp32 agreement rule (a master of 1e-3 formed from two terms of
0.02 carries fp32 rounding of the terms, ~1e-9 each); the tests of these
inputs check that bound instead.
"""

import numpy as np

from fsdp_sharded_mixed_zero_amd import synth

LR, BETA1, BETA2, EPS, WD = 1e-3, 0.9, 0.999, 1e-8, 0.01


def planted(n, seed, kind):
    """(grad_bits, master, m, v, step, G, deep, size) for ``n`` elements; ``kind``
    0: warm state at step 1000; 1: early steps; 2: spiky gradients (1% x100);
    3: values spread over several decades."""
    rng = np.random.default_rng([seed, kind])
    if kind == 0:
        g = rng.standard_normal(n) * 1e-3
        m = rng.standard_normal(n) * 1e-4
        v = np.abs(rng.standard_normal(n) * 1e-8)
        step, G = 1000, 7.6e3
    elif kind == 1:
        g = rng.standard_normal(n) * 1e-3
        m = rng.standard_normal(n) * 1e-5
        v = np.abs(rng.standard_normal(n) * 1e-10)
        step, G = 2, 1.5e3
    elif kind == 2:
        g = rng.standard_normal(n) * 1e-4
        g[rng.random(n) < 0.01] *= 100
        m = rng.standard_normal(n) * 1e-6
        v = np.abs(rng.standard_normal(n) * 1e-12)
        step, G = 5, 6.8e3
    else:
        g = rng.standard_normal(n) * 10.0 ** rng.uniform(-6, -1, n)
        m = rng.standard_normal(n) * 10.0 ** rng.uniform(-7, -2, n)
        v = np.abs(rng.standard_normal(n)) * 10.0 ** rng.uniform(-14, -4, n)
        step, G = 77, 3.0
    g_bits = synth.to_bf16_bits(g.astype(np.float32))
    m = m.astype(np.float32)
    v = v.astype(np.float32)
    p = (rng.standard_normal(n) * 0.02).astype(np.float32)

    def parts(p):
        c = min(1.0, 1.0 / (np.sqrt(G) + 1e-6))
        gh = c * (g_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        m1 = BETA1 * m.astype(np.float64) + (1 - BETA1) * gh
        v1 = BETA2 * v.astype(np.float64) + (1 - BETA2) * gh * gh
        s = LR / (1 - BETA1 ** step)
        d = np.sqrt(v1) / np.sqrt(1 - BETA2 ** step) + EPS
        pd = p.astype(np.float64) * (1 - LR * WD)
        size = np.abs(pd) + s * (np.abs(BETA1 * m.astype(np.float64)) + np.abs((1 - BETA1) * gh)) / d
        return pd - s * m1 / d, s * m1 / d, size

    _, stepterm, _ = parts(p)
    pick = rng.random(n) < 0.1
    rel = rng.standard_normal(pick.sum()) * 10.0 ** rng.uniform(-9, -3, pick.sum())
    p[pick] = (stepterm[pick] / (1 - LR * WD) * (1 + rel)).astype(np.float32)
    new, _, size = parts(p)
    deep = np.abs(new) < 2.0 ** -14 * size
    return g_bits, p, m, v, step, G, deep, size
