"""Pins for oracle.step: brute force, exact rational sums, the AdamW first-step
closed form, torch.optim.AdamW and torch.nn.utils.clip_grad_norm_ in float64,
and sharding invariance."""

import math
from fractions import Fraction

import numpy as np
import pytest
import torch

from fsdp_sharded_mixed_zero_amd import synth
from oracle import step as S
from oracle.bf16 import bf16_to_f32, f32_to_bf16
from oracle.layout import build_layout


def _rand_bits(rng, n, scale=1e-2):
    return synth.to_bf16_bits((rng.standard_normal(n) * scale).astype(np.float32))


# ------------------------------------------------------------- pack/unpack

def test_pack_unpack_brute_force():
    rng = np.random.default_rng(5)
    for trial in range(60):
        t = int(rng.integers(1, 9))
        sizes = [int(x) for x in rng.integers(0, 40, size=t)]
        sizes[0] += 1
        n_d = int(rng.integers(1, 6))
        align = int(rng.choice([1, 4, 8]))
        tensors = [rng.integers(0, 2**16, size=n, dtype=np.uint64).astype(np.uint16) for n in sizes]
        flat = np.concatenate(tensors)
        lay0 = build_layout(sizes, n_d, 0, align)
        padded = np.zeros(lay0.padded, np.uint16)
        padded[:flat.size] = flat
        for rank in range(n_d):
            lay = build_layout(sizes, n_d, rank, align)
            expect = padded[rank * lay.shard:(rank + 1) * lay.shard]
            got = S.pack(lay, tensors)
            assert np.array_equal(got, expect)
            # any sub-range packs to the same elements
            b = int(rng.integers(0, lay.shard + 1))
            c = int(rng.integers(0, lay.shard - b + 1))
            assert np.array_equal(S.pack(lay, tensors, b, c), expect[b:b + c])
            # unpack writes exactly the rank's elements and nothing else
            new_shard = rng.integers(0, 2**16, size=lay.shard, dtype=np.uint64).astype(np.uint16)
            out = S.unpack(lay, new_shard, tensors)
            new_flat = padded.copy()
            new_flat[rank * lay.shard:(rank + 1) * lay.shard] = new_shard
            want = np.split(new_flat[:flat.size], np.cumsum(sizes)[:-1])
            assert all(np.array_equal(a, w) for a, w in zip(out, want))
            # round trip
            back = S.unpack(lay, got, tensors)
            assert all(np.array_equal(a, w) for a, w in zip(back, tensors))
            # partial unpack only touches its range
            part = S.unpack(lay, new_shard[b:b + c], tensors, b, c)
            ref_flat = padded.copy()
            ref_flat[rank * lay.shard + b:rank * lay.shard + b + c] = new_shard[b:b + c]
            want = np.split(ref_flat[:flat.size], np.cumsum(sizes)[:-1])
            assert all(np.array_equal(a, w) for a, w in zip(part, want))


def test_pack_rejects_bad_ranges():
    lay = build_layout([10, 6], 2, 0, 1)
    t = [np.zeros(10, np.uint16), np.zeros(6, np.uint16)]
    for b, c in [(-1, 2), (0, 9), (7, 2)]:
        with pytest.raises(ValueError):
            S.pack(lay, t, b, c)


# ---------------------------------------------------------- sum of squares

def _exact_sq(bits):
    vals = bf16_to_f32(bits).astype(np.float64)
    return sum((Fraction(float(x)) ** 2 for x in vals), Fraction(0))


def test_sqnorm_against_exact_rational_sum():
    rng = np.random.default_rng(11)
    for n in (0, 1, 7, 1000, 5000):
        bits = _rand_bits(rng, n, scale=3.0)
        exact = _exact_sq(bits)
        got = S.sqnorm(bits)
        assert abs(Fraction(got) - exact) <= Fraction(2 * n + 1) * Fraction(2.0 ** -52) * exact + 0


def test_sqnorm_special_cases():
    assert S.sqnorm(np.full(12345, 0x3F80, np.uint16)) == 12345.0       # all ones
    assert S.sqnorm(np.full(4, 0xC000, np.uint16)) == 16.0             # all -2
    assert S.sqnorm(np.zeros(9, np.uint16)) == 0.0
    # extreme exponents: squares beyond fp32 range are still exact in fp64
    big = f32_to_bf16(np.array([3.0e38], np.float32))
    assert S.sqnorm(big) == float(bf16_to_f32(big)[0]) ** 2
    tiny = np.array([0x0001], np.uint16)                                 # smallest denormal
    assert S.sqnorm(tiny) == float(bf16_to_f32(tiny)[0]) ** 2 > 0
    assert math.isinf(S.sqnorm(np.array([0x7F80], np.uint16)))
    assert math.isnan(S.sqnorm(np.array([0x7FC0], np.uint16)))


def test_sqnorm_is_additive_over_ranks():
    rng = np.random.default_rng(3)
    sizes = [300, 11, 977, 64]
    tensors = [_rand_bits(rng, n) for n in sizes]
    whole = S.sqnorm(np.concatenate(tensors))
    for n_d in (1, 2, 3, 7):
        parts = [S.sqnorm(S.pack(build_layout(sizes, n_d, r, 1), tensors)) for r in range(n_d)]
        assert S.global_sqnorm(parts) == pytest.approx(whole, rel=1e-14)
    # with integer-valued squares the sums are exact in any order
    ints = [np.full(n, 0x4040, np.uint16) for n in sizes]        # all 3.0
    parts = [S.sqnorm(S.pack(build_layout(sizes, 4, r, 8), ints)) for r in range(4)]
    assert S.global_sqnorm(parts) == 9.0 * sum(sizes)


# -------------------------------------------------------------------- clip

def test_clip_matches_torch_clip_grad_norm():
    rng = np.random.default_rng(17)
    for max_norm, scale in [(1.0, 1e-3), (1.0, 0.5), (0.3, 1.0), (5.0, 10.0), (1.0, 0.0)]:
        sizes = [37, 1000, 5, 256]
        grads = [_rand_bits(rng, n, scale) for n in sizes]
        G = S.global_sqnorm([S.sqnorm(g) for g in grads])
        c = S.clip_coef(G, max_norm)
        params = [torch.nn.Parameter(torch.zeros(n, dtype=torch.float64)) for n in sizes]
        for p, g in zip(params, grads):
            p.grad = torch.from_numpy(bf16_to_f32(g).astype(np.float64))
        total = torch.nn.utils.clip_grad_norm_(params, max_norm)
        assert math.sqrt(G) == pytest.approx(float(total), rel=1e-13, abs=0)
        for p, g in zip(params, grads):
            want = p.grad.numpy()
            got = c * bf16_to_f32(g).astype(np.float64)
            assert np.allclose(got, want, rtol=1e-13, atol=0)


def test_clip_special_cases():
    assert S.clip_coef(4.0, 0.0) == 1.0            # off
    assert S.clip_coef(4.0, -1.0) == 1.0
    assert S.clip_coef(0.0, 1.0) == 1.0            # zero gradient never scales up
    assert S.clip_coef(1e-12, 1.0) == 1.0
    assert S.clip_coef(4.0, 1.0) == pytest.approx(1.0 / (2.0 + 1e-6), rel=1e-15)
    assert S.clip_coef(math.inf, 1.0) == 0.0
    assert math.isnan(S.clip_coef(math.nan, 1.0))


# ------------------------------------------------------------------- AdamW

def test_first_step_closed_form():
    # m0 = v0 = 0, step 1, no decay: bias correction undoes (1-beta1) and
    # (1-beta2), leaving an update of lr * g / (|g| + eps)
    rng = np.random.default_rng(23)
    g = rng.standard_normal(5000) * 10.0 ** rng.uniform(-9, 1, size=5000)
    zeros = np.zeros_like(g)
    for hp in [S.AdamWHParams(weight_decay=0.0),
               S.AdamWHParams(lr=3e-4, beta1=0.8, beta2=0.95, eps=1e-6, weight_decay=0.0)]:
        p1, m1, v1 = S.adamw_f64(zeros, zeros, zeros, g, 1, hp)
        assert np.allclose(-p1, hp.lr * g / (np.abs(g) + hp.eps), rtol=1e-12, atol=0)
        assert np.allclose(m1, (1 - hp.beta1) * g, rtol=1e-15, atol=0)
        assert np.allclose(v1, (1 - hp.beta2) * g * g, rtol=1e-15, atol=0)
        # far above eps the step is lr * sign(g)
        big = np.abs(g) > 1e5 * hp.eps
        assert np.allclose(-p1[big], hp.lr * np.sign(g[big]), rtol=1e-5, atol=0)
    # with decoupled weight decay the parameter also shrinks by lr*lambda*p
    p = rng.standard_normal(5000)
    hp = S.AdamWHParams(weight_decay=0.1)
    p1, _, _ = S.adamw_f64(p, zeros, zeros, g, 1, hp)
    want = p - hp.lr * hp.weight_decay * p - hp.lr * g / (np.abs(g) + hp.eps)
    assert np.allclose(p1, want, rtol=0, atol=4 * np.finfo(np.float64).eps * np.abs(p).max())


def test_adamw_matches_torch_over_ten_steps():
    rng = np.random.default_rng(29)
    sizes = [1000, 3, 517]
    for hp in [S.AdamWHParams(), S.AdamWHParams(lr=2e-3, beta1=0.85, beta2=0.99, eps=1e-7,
                                               weight_decay=0.05, max_norm=0.5)]:
        p0 = [rng.standard_normal(n) * 0.02 for n in sizes]
        params = [torch.nn.Parameter(torch.from_numpy(x.copy())) for x in p0]
        opt = torch.optim.AdamW(params, lr=hp.lr, betas=(hp.beta1, hp.beta2), eps=hp.eps,
                                weight_decay=hp.weight_decay, foreach=False)
        ours_p = np.concatenate(p0)
        ours_m = np.zeros_like(ours_p)
        ours_v = np.zeros_like(ours_p)
        for t in range(1, 11):
            grads = [rng.standard_normal(n) * 10.0 ** rng.uniform(-4, 0) for n in sizes]
            for p, g in zip(params, grads):
                p.grad = torch.from_numpy(g.copy())
            torch.nn.utils.clip_grad_norm_(params, hp.max_norm)
            opt.step()
            g = np.concatenate(grads)
            c = S.clip_coef(float(np.dot(g, g)), hp.max_norm)
            ours_p, ours_m, ours_v = S.adamw_f64(ours_p, ours_m, ours_v, c * g, t, hp)
            ref = np.concatenate([p.detach().numpy() for p in params])
            assert np.allclose(ours_p, ref, rtol=1e-12, atol=1e-15), t
            ref_m = np.concatenate([opt.state[p]["exp_avg"].numpy() for p in params])
            ref_v = np.concatenate([opt.state[p]["exp_avg_sq"].numpy() for p in params])
            assert np.allclose(ours_m, ref_m, rtol=1e-12, atol=1e-18)
            assert np.allclose(ours_v, ref_v, rtol=1e-12, atol=1e-24)


def test_adamw_step_stores_fp32_and_casts_stored_master():
    rng = np.random.default_rng(31)
    n = 3000
    bits = _rand_bits(rng, n, 1e-3)
    master = (rng.standard_normal(n) * 0.02).astype(np.float32)
    m = (rng.standard_normal(n) * 1e-4).astype(np.float32)
    v = np.abs(rng.standard_normal(n) * 1e-8).astype(np.float32)
    hp = S.AdamWHParams()
    c = 0.37
    p1, m1, v1, b1 = S.adamw_step(bits, master, m, v, 7, hp, c)
    g_hat = c * bf16_to_f32(bits).astype(np.float64)
    rp, rm, rv = S.adamw_f64(master, m, v, g_hat, 7, hp)
    assert np.array_equal(p1, rp.astype(np.float32))
    assert np.array_equal(m1, rm.astype(np.float32))
    assert np.array_equal(v1, rv.astype(np.float32))
    ref_b = torch.from_numpy(p1).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(b1, ref_b)


def test_padding_stays_zero():
    hp = S.AdamWHParams()
    z = np.zeros(16, np.float32)
    p1, m1, v1, b1 = S.adamw_step(np.zeros(16, np.uint16), z, z, z, 1, hp, 0.5)
    assert not p1.any() and not m1.any() and not v1.any() and not b1.any()


def test_sharded_update_equals_unsharded():
    """N_d ranks each updating their own shard with the shared global norm give
    exactly the N_d = 1 update, element for element."""
    # gradients large enough that the global norm exceeds max_norm
    wl = synth.Workload("t", (1000, 333, 4096, 17), n_d=1, rank=0, align=8,
                        grad_std=0.05, m_std=1e-4, v_std=1e-8)
    grads = synth.host_tensor_grads(wl, step=1)
    hp = S.AdamWHParams()
    full = build_layout(wl.sizes, 1, 0, 8)
    for n_d in (2, 3, 5):
        lays = [build_layout(wl.sizes, n_d, r, 8) for r in range(n_d)]
        padded = lays[0].padded
        master, m, v = synth.host_flat_state(wl, lays[0].psi, padded)
        shards = [S.pack(l, grads) for l in lays]
        G = S.global_sqnorm([S.sqnorm(s) for s in shards])
        c = S.clip_coef(G, hp.max_norm)
        assert c < 1.0
        outs = []
        for l, g in zip(lays, shards):
            sl = slice(l.shard_begin, l.shard_begin + l.shard)
            outs.append(S.adamw_step(g, master[sl], m[sl], v[sl], 3, hp, c))
        # unsharded reference over the same padded flat buffer
        g_full = np.zeros(padded, np.uint16)
        g_full[:full.psi] = S.pack(full, grads)[:full.psi]
        ref = S.adamw_step(g_full, master, m, v, 3, hp, c)
        for k in range(4):
            assert np.array_equal(np.concatenate([o[k] for o in outs]), ref[k])
        # and per-rank clipping with the local norm would differ (the silent
        # divergence the shard-aware rule prevents)
        local = [S.clip_coef(S.sqnorm(s), hp.max_norm) for s in shards]
        assert any(abs(x - c) > 1e-3 for x in local)


# ------------------------------------------------ fp32 gradient accumulation

def test_accumulate_matches_torch_fp32_add():
    rng = np.random.default_rng(41)
    n = 200_000
    # accumulators and gradients spanning wide exponent gaps both ways
    acc = (rng.standard_normal(n) * 10.0 ** rng.uniform(-30, 10, n)).astype(np.float32)
    g = _rand_bits(rng, n, 1.0)
    g = np.where(rng.random(n) < 0.5, g,
                 synth.to_bf16_bits((rng.standard_normal(n) * 10.0 ** rng.uniform(-30, 10, n))
                                    .astype(np.float32)))
    ours = S.accumulate(acc, g, first=False)
    ref = (torch.from_numpy(acc) + torch.from_numpy(g.view(np.int16).copy()).view(torch.bfloat16).float())
    assert np.array_equal(ours.view(np.uint32), ref.numpy().view(np.uint32))
    # first micro-batch: exactly the widened gradient
    first = S.accumulate(np.full(n, np.nan, np.float32), g, first=True)
    assert np.array_equal(first, bf16_to_f32(g))


def test_accumulate_exact_small_integers():
    ones = np.full(100, 0x3F80, np.uint16)       # 1.0
    acc = S.accumulate(None, ones, first=True)
    for _ in range(9):
        acc = S.accumulate(acc, ones, first=False)
    assert (acc == 10.0).all()


def test_sqnorm_f32_exact():
    rng = np.random.default_rng(43)
    x = (rng.standard_normal(3000) * 7.0).astype(np.float32)
    exact = sum((Fraction(float(v)) ** 2 for v in x), Fraction(0))
    assert abs(Fraction(S.sqnorm_f32(x)) - exact) <= Fraction(6001) * Fraction(2.0 ** -52) * exact
    assert S.sqnorm_f32(np.full(777, 3.0, np.float32)) == 9.0 * 777
    big = np.array([3.0e38, -3.0e38], np.float32)               # squares beyond fp32 range
    assert S.sqnorm_f32(big) == 2 * float(np.float32(3.0e38)) ** 2
    assert S.sqnorm_f32(np.zeros(0, np.float32)) == 0.0


def test_adamw_f32grad_agrees_with_bf16_path():
    rng = np.random.default_rng(47)
    n = 5000
    bits = _rand_bits(rng, n, 1e-3)
    master = (rng.standard_normal(n) * 0.02).astype(np.float32)
    m = (rng.standard_normal(n) * 1e-4).astype(np.float32)
    v = np.abs(rng.standard_normal(n) * 1e-8).astype(np.float32)
    hp = S.AdamWHParams()
    a = S.adamw_step(bits, master, m, v, 4, hp, 0.3)
    b = S.adamw_step_f32grad(bf16_to_f32(bits), master, m, v, 4, hp, 0.3)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    # a gradient that is not bf16-representable is used as is, not rounded
    g = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    p1, m1, _, _ = S.adamw_step_f32grad(g, master, np.zeros(n, np.float32), np.zeros(n, np.float32),
                                        1, S.AdamWHParams(weight_decay=0.0, max_norm=0.0), 1.0)
    assert np.array_equal(m1, (0.1 * g.astype(np.float64)).astype(np.float32))


# ------------------------------------------------------- argument checking

INVALID_HPARAMS = [dict(lr=-1e-3), dict(lr=float("nan")), dict(eps=-1e-8), dict(eps=float("nan")),
                   dict(beta1=-0.1), dict(beta1=1.0), dict(beta2=1.0), dict(beta2=1.5), dict(beta2=float("nan")),
                   dict(weight_decay=-0.01), dict(weight_decay=float("nan"))]
EDGE_HPARAMS = [dict(lr=0.0), dict(eps=0.0), dict(beta1=0.0), dict(beta2=0.0), dict(weight_decay=0.0),
                dict(lr=float("inf"))]


def _torch_adamw(kw):
    p = torch.nn.Parameter(torch.zeros(3, dtype=torch.float64))
    return torch.optim.AdamW([p], lr=kw.get("lr", 1e-3), betas=(kw.get("beta1", 0.9), kw.get("beta2", 0.999)),
                             eps=kw.get("eps", 1e-8), weight_decay=kw.get("weight_decay", 0.01))


@pytest.mark.parametrize("kw", INVALID_HPARAMS)
def test_hparams_refused_as_torch_refuses_them(kw):
    with pytest.raises(ValueError):
        _torch_adamw(kw)
    with pytest.raises(ValueError):
        S.AdamWHParams(**kw)


@pytest.mark.parametrize("kw", EDGE_HPARAMS)
def test_hparams_accepted_as_torch_accepts_them(kw):
    _torch_adamw(kw)
    S.AdamWHParams(**kw)


OWN_INVALID = [dict(clip_eps=-1e-6), dict(clip_eps=float("nan")), dict(max_norm=float("nan"))]


@pytest.mark.parametrize("kw", OWN_INVALID)
def test_clip_arguments_refused(kw):
    """The clip arguments (not torch.optim.AdamW's): clip_eps below 0 and a
    NaN max_norm are refused; max_norm <= 0 or infinite is allowed."""
    with pytest.raises(ValueError):
        S.AdamWHParams(**kw)
    for ok in (dict(clip_eps=0.0), dict(max_norm=0.0), dict(max_norm=-1.0), dict(max_norm=float("inf"))):
        S.AdamWHParams(**ok)
