"""Seeded random layouts through the C ABI against the oracle. Each trial
draws a tensor list (empty, small and large tensors), N_d, rank, alignment, a
shard range, tensor pointers off their natural alignment and AdamW
hyperparameters, then checks:

  * the fused pack + sum of squares: packed bytes bit-exact, the sum within
    1e-12 relative, everything outside the range untouched;
  * the update with the unpack fused (bf16 or fp32 gradient): fp32 state and
    bf16 parameters within the stated tolerances, each tensor element that
    the layout maps into the range equal to its parameter-shard element, and
    every byte outside the range, padding around the tensors included,
    untouched."""

import numpy as np
import pytest

from fsdp_sharded_mixed_zero_amd import synth, zero
from oracle import step as O
from oracle.layout import build_layout
from state_tiles import from_tiles, to_tiles
from tolerance import assert_bf16_param, assert_f32_state
from devbits import u16

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = torch.device("cuda")
PAD = 5                      # sentinel elements around every tensor buffer


def draw(rng):
    T = int(rng.integers(1, 41))
    u = rng.random(T)
    sizes = np.where(u < 0.15, 0,
                     np.where(u < 0.55, rng.integers(1, 100, T),
                              np.where(u < 0.95, rng.integers(100, 20_000, T), rng.integers(20_000, 300_000, T))))
    sizes = [int(x) for x in sizes]
    if sum(sizes) == 0:
        sizes[int(rng.integers(0, T))] = int(rng.integers(1, 5000))
    n_d = int(rng.integers(1, 3)) if rng.random() < 0.35 else int(rng.integers(1, 17))   # few ranks: many segments
    align = int(rng.choice([1, 2, 8, 64, 128]))
    rank = int(rng.integers(0, n_d))
    return sizes, n_d, rank, align


def hyper(rng):
    betas = [(0.9, 0.999), (0.8, 0.95)][int(rng.integers(0, 2))]
    return O.AdamWHParams(lr=float(rng.choice([1e-3, 3e-4])), beta1=betas[0], beta2=betas[1],
                          eps=float(rng.choice([1e-8, 1e-6])), weight_decay=float(rng.choice([0.0, 0.01, 0.1])),
                          max_norm=float(rng.choice([0.0, 1.0, 1e-3])))


def device_tensors(host, offsets):
    """Each host uint16 array in a device buffer with PAD sentinels on both
    sides, starting `offset` further elements in; returns (views, buffers)."""
    views, bufs = [], []
    for x, off in zip(host, offsets):
        buf = torch.full((len(x) + off + 2 * PAD,), synth.SENTINEL, dtype=torch.int16, device=DEV)
        if len(x):
            buf[PAD + off:PAD + off + len(x)] = torch.from_numpy(x.view(np.int16)).to(DEV)
        views.append(buf[PAD + off:PAD + off + len(x)].view(torch.bfloat16))
        bufs.append(buf)
    return views, bufs


def shard_positions(lay, shard_bits, sizes, b, c):
    """Per tensor: the sentinel everywhere except the elements the layout
    maps to shard range [b, b+c), which hold those shard elements (a
    consistency check of the GPU's tensors against its own shard)."""
    out = [np.full(n, synth.SENTINEL, np.uint16) for n in sizes]
    for seg in lay.segments:
        lo, hi = max(seg.dst_off, b), min(seg.dst_off + seg.length, b + c)
        if lo < hi:
            s0 = seg.src_off + (lo - seg.dst_off)
            out[seg.tensor][s0:s0 + (hi - lo)] = shard_bits[lo:hi]
    return out


def one_trial(rng, trial):
    sizes, n_d, rank, align = draw(rng)
    lay = build_layout(sizes, n_d, rank, align)
    S = lay.shard
    if rng.random() < 0.4:
        b, c = 0, S
    else:
        b = int(rng.integers(0, S + 1))
        c = int(rng.integers(0, S - b + 1))
    f32grad = rng.random() < 0.3
    ohp = hyper(rng)
    step = int(rng.choice([1, 2, 10, 1000]))
    print(f"trial {trial}: {len(sizes)} tensors, psi {sum(sizes)}, n_d {n_d}, rank {rank}, align {align}, "
          f"S {S}, range [{b}, +{c}), f32grad {f32grad}, step {step}, {ohp}", flush=True)
    h = zero.zero_layout(sizes, n_d, rank, align)

    # pack with the sum of squares
    grads = [synth.to_bf16_bits((rng.standard_normal(n) * 1e-3).astype(np.float32)) for n in sizes]
    offsets = [int(x) for x in rng.integers(0, 4, len(sizes))]
    d_grads, _ = device_tensors(grads, offsets)
    shard = torch.full((S,), synth.SENTINEL, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    ws = torch.empty(zero.zero_pack_sqnorm_workspace_bytes(h, b, c) // 8, dtype=torch.float64, device=DEV)
    out = torch.full((1,), 123.0, dtype=torch.float64, device=DEV)
    zero.zero_pack_grads_sqnorm(h, d_grads, shard, b, c, out, False, ws)
    torch.cuda.synchronize()
    packed = O.pack(lay, grads, b, c)
    got = u16(shard)
    assert np.array_equal(got[b:b + c], packed), trial
    assert (got[:b] == synth.SENTINEL).all() and (got[b + c:] == synth.SENTINEL).all(), trial
    want_sq = O.sqnorm(packed)
    got_sq = float(out.cpu()[0])
    assert abs(got_sq - want_sq) <= 1e-12 * want_sq, (trial, got_sq, want_sq)

    # the update with the unpack fused
    master = (rng.standard_normal(S) * 0.02).astype(np.float32)
    m = (rng.standard_normal(S) * 1e-4).astype(np.float32)
    v = np.abs(rng.standard_normal(S) * 1e-8).astype(np.float32)
    parts = np.abs(rng.standard_normal(n_d)) * max(want_sq, 1e-6)
    parts[rank] = want_sq                  # the same partial sums for both sides, the oracle's own
    d_state = torch.from_numpy(to_tiles(master, m, v)).to(DEV)
    d_param = torch.full((S,), synth.SENTINEL, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    sent = [np.full(n, synth.SENTINEL, np.uint16) for n in sizes]
    p_offsets = [int(x) for x in rng.integers(0, 4, len(sizes))]
    d_params, p_bufs = device_tensors(sent, p_offsets)
    hp = zero.hparams(lr=ohp.lr, beta1=ohp.beta1, beta2=ohp.beta2, eps=ohp.eps, weight_decay=ohp.weight_decay,
                      max_norm=ohp.max_norm, clip_eps=ohp.clip_eps, step=step)
    d_parts = torch.from_numpy(parts).to(DEV)
    coef = O.clip_coef(O.global_sqnorm(parts), ohp.max_norm, ohp.clip_eps)
    sl = slice(b, b + c)
    if f32grad:
        g32 = (rng.standard_normal(S) * 1e-3).astype(np.float32)
        zero.zero_adamw_step_f32grad_unpack(torch.from_numpy(g32).to(DEV), d_state, d_param, S, b, c, hp, d_parts,
                                            n_d, h, d_params)
        want = O.adamw_step_f32grad(g32[sl], master[sl], m[sl], v[sl], step, ohp, coef)
    else:
        zero.zero_adamw_step_unpack(shard, d_state, d_param, S, b, c, hp, d_parts, n_d, h, d_params)
        want = O.adamw_step(packed, master[sl], m[sl], v[sl], step, ohp, coef)
    torch.cuda.synchronize()
    g_master, g_m, g_v = from_tiles(d_state.cpu().numpy(), S)
    g_param = u16(d_param)
    assert_f32_state(g_master[sl], want[0], f"master (trial {trial})")
    assert_f32_state(g_m[sl], want[1], f"m (trial {trial})", m[sl])
    assert_f32_state(g_v[sl], want[2], f"v (trial {trial})", v[sl])
    assert_bf16_param(g_param[sl], want[3], want[0], f"param (trial {trial})", g_master[sl])
    out_of_range = np.ones(S, bool)
    out_of_range[sl] = False
    assert np.array_equal(g_master[out_of_range], master[out_of_range]), trial
    assert np.array_equal(g_m[out_of_range], m[out_of_range]) and np.array_equal(g_v[out_of_range], v[out_of_range])
    assert (g_param[out_of_range] == synth.SENTINEL).all(), trial
    placed = shard_positions(lay, g_param, sizes, b, c)
    for i, (buf, off, wt) in enumerate(zip(p_bufs, p_offsets, placed)):
        whole = u16(buf)
        assert np.array_equal(whole[PAD + off:PAD + off + sizes[i]], wt), (trial, i)
        assert (whole[:PAD + off] == synth.SENTINEL).all() and (whole[PAD + off + sizes[i]:] == synth.SENTINEL).all()


@pytest.mark.parametrize("seed", range(16))
def test_random_layouts(seed):
    rng = np.random.default_rng(1000 + seed)
    for k in range(10):
        one_trial(rng, f"{seed}.{k}")
