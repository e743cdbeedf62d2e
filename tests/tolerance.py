"""Agreement rules between the HIP path and the oracle.

  * layout, offsets, packed/unpacked bf16 bytes: bit-exact;
  * fp32 master, m, v: |gpu - oracle| <= 1e-8 + 1e-6 * |oracle|;
  * bf16 parameters: at most 1 bf16 ulp apart (ordered-integer distance),
    everywhere, near-zero masters included; and each GPU parameter is
    exactly the round-to-nearest-even bf16 of the GPU's own fp32 master
    (torch's cast);
  * global norm: |sqrt(G_gpu) - sqrt(G_oracle)| <= 1e-5 * sqrt(G_oracle).

The fp32 rule's absolute term (1e-8) exceeds typical v values (~1e-9 to 1e-12),
so fp32 state is also bounded in ulps of |old| + |new| (see assert_f32_state).
"""

import numpy as np


RTOL_F32 = 1e-6
ATOL_F32 = 1e-8
MAX_SCALED_ULP = 16
RTOL_NORM = 1e-5


def ordered_f32(x):
    i = np.asarray(x, dtype=np.float32).view(np.int32).astype(np.int64)
    return np.where(i < 0, -(2**31) - i, i)


def ordered_bf16(bits):
    i = np.asarray(bits, dtype=np.uint16).view(np.int16).astype(np.int64)
    return np.where(i < 0, -(2**15) - i, i)


def ulp_f32(a, b):
    return np.abs(ordered_f32(a) - ordered_f32(b))


def assert_f32_state(got, want, name, old=None, max_scaled_ulp=MAX_SCALED_ULP):
    """The stated rule, plus (when the pre-step values ``old`` are given) a
    bound in fp32 ulps of |old| + |new|. Use it for the moments: for
    m' = b1*m + (1-b1)*g both terms are bounded by |m| + |m'|, and v' is a sum
    of non-negative terms, so the bound holds where m' cancels to almost zero
    and where the stated rule's absolute term is vacuous (v ~ 1e-12). The
    master weight's update also carries m's absolute error, scaled by
    lr / denominator, so only the stated rule applies to it.
    Returns the worst error in those ulps."""
    got = np.asarray(got, np.float32)
    want = np.asarray(want, np.float32)
    assert got.shape == want.shape, name
    assert not np.isnan(want).any(), f"{name}: oracle produced NaN"
    err = np.abs(got.astype(np.float64) - want.astype(np.float64))
    bound = ATOL_F32 + RTOL_F32 * np.abs(want.astype(np.float64))
    bad = err > bound
    assert not bad.any(), (f"{name}: {bad.sum()} of {bad.size} outside rel {RTOL_F32}/abs {ATOL_F32}; "
                           f"first at {np.flatnonzero(bad)[:5]}")
    if old is None or got.size == 0:
        return 0.0
    scale = (np.abs(np.asarray(old, np.float64)) + np.abs(want.astype(np.float64))).astype(np.float32)
    spacing = np.spacing(scale).astype(np.float64)
    scaled = np.where(err > 0, err / spacing, 0.0)
    worst = float(scaled.max())
    assert worst <= max_scaled_ulp, (f"{name}: {worst:.1f} ulp of |old|+|new| at "
                                     f"{np.flatnonzero(scaled > max_scaled_ulp)[:5]}")
    return worst


def assert_bf16_close(got_bits, want_bits, name, max_ulp=1):
    d = np.abs(ordered_bf16(got_bits) - ordered_bf16(want_bits))
    worst = int(d.max()) if d.size else 0
    assert worst <= max_ulp, f"{name}: {worst} bf16 ulp apart at {np.flatnonzero(d > max_ulp)[:5]}"
    return worst


def assert_bf16_param(got_bits, want_bits, want_master, name, got_master=None):
    """bf16 parameters against the oracle's: at most 1 bf16 ulp apart at every
    element (``want_master``, the oracle's fp32 master, is named in the
    failure message), and, when ``got_master`` is given, each parameter is the
    round-to-nearest-even bf16 of its own fp32 master. Returns the largest
    distance."""
    ow = ordered_bf16(want_bits)
    d = np.abs(ordered_bf16(got_bits) - ow)
    bad = d > 1
    if bad.any():
        k = np.flatnonzero(bad)[:5]
        raise AssertionError(f"{name}: {int(d.max())} bf16 ulp apart at {k} "
                             f"(oracle masters {np.asarray(want_master, np.float32)[k]})")
    if got_master is not None:
        import torch
        cast = torch.from_numpy(np.ascontiguousarray(got_master, np.float32)).to(torch.bfloat16)
        cast = cast.view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(np.asarray(got_bits, np.uint16), cast), f"{name}: not the bf16 of its master"
    return int(d.max()) if d.size else 0


def assert_norm_close(g_gpu, g_oracle, name="norm"):
    a, b = np.sqrt(float(g_gpu)), np.sqrt(float(g_oracle))
    assert abs(a - b) <= RTOL_NORM * b, f"{name}: sqrt(G) {a!r} vs oracle {b!r}"
    return abs(a - b) / b if b else 0.0
