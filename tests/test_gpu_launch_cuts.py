"""Ranges longer than one AdamW launch (about 2^27 elements): the update is
cut into equal launches (whole tiles), and the fused update also cuts a
tensor piece there and continues it in the next launch. Each entry point over
long ranges must give the bits of the same update run as sub-ranges that each
fit one launch (nothing skipped, nothing updated twice), and the elements
around every cut must match the oracle."""

import numpy as np
import pytest

from fsdp_sharded_mixed_zero_amd import synth, zero
from oracle import step as O
from oracle.layout import build_layout
from state_tiles import TILE
from tolerance import assert_bf16_param, assert_f32_state

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = torch.device("cuda")
CUT = zero.ZERO_ADAMW_LAUNCH_ELEMS    # a range longer than this takes several launches


def cuts(b, c):
    """Where the library cuts [b, b + c) into launches (the fewest launches
    of at most CUT elements, equal lengths rounded up to whole tiles)."""
    k = -(-c // CUT)
    chunk = -(-(-(-c // k)) // TILE) * TILE
    return [b + j * chunk for j in range(1, k) if b + j * chunk < b + c]


def fused_cuts(lay, b, c, max_pieces=zero.ZERO_PIECES_PER_LAUNCH):
    """Where the fused update cuts [b, b + c): the same launch length, and a
    launch in which more than 64 tensor pieces start ends at its 64th."""
    starts = sorted(max(g.dst_off, b) for g in lay.segments
                    if g.dst_off < b + c and g.dst_off + g.length > b)
    k = -(-c // CUT)
    chunk = -(-(-(-c // k)) // TILE) * TILE
    out, r0, e = [], b, b + c
    while r0 < e:
        r1 = min(e, r0 + chunk)
        inside = [x for x in starts if r0 <= x < r1] if starts and starts[0] <= r0 else []
        if len(inside) > max_pieces:
            r1 = inside[max_pieces]
        if r1 < e:
            out.append(r1)
        r0 = r1
    return out


def make_state(S, f32grad, seed):
    gen = torch.Generator(device=DEV).manual_seed(seed)
    gdt = torch.float32 if f32grad else torch.bfloat16
    grad = (torch.randn(S, device=DEV, generator=gen) * 1e-3).to(gdt)
    master = torch.randn(S, device=DEV, generator=gen) * 0.02
    m = torch.randn(S, device=DEV, generator=gen) * 1e-4
    v = (torch.randn(S, device=DEV, generator=gen) * 1e-8).abs_()
    state = torch.empty(3 * S, dtype=torch.float32, device=DEV)
    zero.zero_state_import(master, m, v, state, S)
    return grad, state


def small_ranges(b, c, step=CUT // 4):
    """[b, b + c) as sub-ranges that each lie inside one launch."""
    out = []
    e = b + c
    while b < e:
        n = min(e, (b // step + 1) * step) - b
        out.append((b, n))
        b += n
    return out


def oracle_sample(grad, state0, S, idx, step, ohp, coef, f32grad):
    """The oracle's update of the elements idx (the update is elementwise)."""
    idx = np.asarray(idx, np.int64)
    t, j = idx // TILE, idx % TILE
    L = np.minimum(TILE, S - t * TILE)
    base = 3 * t * TILE + j
    pos = torch.from_numpy(np.concatenate([base, base + L, base + 2 * L])).to(DEV)
    vals = state0[pos].cpu().numpy()
    n = idx.size
    p, m, v = vals[:n], vals[n:2 * n], vals[2 * n:]
    gi = torch.from_numpy(idx).to(DEV)
    if f32grad:
        g = grad[gi].cpu().numpy()
        return O.adamw_step_f32grad(g, p, m, v, step, ohp, coef), (base, L)
    g = grad[gi].view(torch.int16).cpu().numpy().view(np.uint16)
    return O.adamw_step(g, p, m, v, step, ohp, coef), (base, L)


def around_cuts(b, c, width=300):
    e = b + c
    pts = set(range(b, min(e, b + width))) | set(range(max(b, e - width), e))
    for x in cuts(b, c):
        pts |= set(range(max(b, x - width), min(e, x + width)))
    return sorted(pts)


@pytest.mark.parametrize("f32grad", [False, True], ids=["bf16-grad", "f32-grad"])
def test_update_across_launch_cuts(f32grad):
    S = 2 * CUT + 3 * TILE + 5           # three launches, a compact last tile
    grad, state0 = make_state(S, f32grad, seed=5)
    ohp = O.AdamWHParams(max_norm=1.0)
    parts = torch.tensor([2.0, 3.0], dtype=torch.float64, device=DEV)
    coef = O.clip_coef(O.global_sqnorm([2.0, 3.0]), ohp.max_norm, ohp.clip_eps)
    fn = zero.zero_adamw_step_f32grad if f32grad else zero.zero_adamw_step
    hp = zero.hparams(max_norm=1.0, step=4)
    for b, c in ((0, S), (CUT - 7, CUT + 100), (3, S - 9)):
        assert cuts(b, c)
        state, param = state0.clone(), torch.zeros(S, dtype=torch.bfloat16, device=DEV)
        fn(grad, state, param, S, b, c, hp, parts, 2)
        r_state, r_param = state0.clone(), torch.zeros(S, dtype=torch.bfloat16, device=DEV)
        for rb, rc in small_ranges(b, c):
            fn(grad, r_state, r_param, S, rb, rc, hp, parts, 2)
        torch.cuda.synchronize()
        assert torch.equal(state.view(torch.int32), r_state.view(torch.int32)), (b, c)
        assert torch.equal(param.view(torch.int16), r_param.view(torch.int16)), (b, c)
        idx = around_cuts(b, c)
        want, (base, L) = oracle_sample(grad, state0, S, idx, 4, ohp, coef, f32grad)
        pos = torch.from_numpy(np.concatenate([base, base + L, base + 2 * L])).to(DEV)
        got = state[pos].cpu().numpy()
        n = len(idx)
        assert_f32_state(got[:n], want[0], "master")
        assert_f32_state(got[n:2 * n], want[1], "m")
        assert_f32_state(got[2 * n:], want[2], "v")
        g_param = param[torch.from_numpy(np.asarray(idx)).to(DEV)].view(torch.int16).cpu().numpy().view(np.uint16)
        assert_bf16_param(g_param, want[3], want[0], "param", got[:n])
        # nothing outside the range moved
        if b > 0:
            assert torch.equal(state[:3 * TILE * (b // TILE)].view(torch.int32),
                               state0[:3 * TILE * (b // TILE)].view(torch.int32))
            assert not param[:b].view(torch.int16).any()
        if b + c < S:
            assert not param[b + c:].view(torch.int16).any()


@pytest.mark.parametrize("f32grad", [False, True], ids=["bf16-grad", "f32-grad"])
def test_fused_update_across_launch_cuts(f32grad):
    """Two ranks of a layout of 2.7e8 elements: on rank 0 the first launch
    fills its 64-piece table (ending early); on both a tensor piece runs
    across a launch cut; rank 1's shard ends in padding."""
    sizes = [37] * 100 + [CUT - 37 * 100 - 1001, 5003, 3, CUT - 4000, 77_777, 3 * TILE]
    n_d, align = 2, 128
    for rank in (0, 1):
        lay = build_layout(sizes, n_d, rank, align)
        S = lay.shard
        assert S > CUT
        h = zero.zero_layout(sizes, n_d, rank, align)
        grad, state0 = make_state(S, f32grad, seed=9 + rank)
        parts = torch.tensor([7.0], dtype=torch.float64, device=DEV)
        hp = zero.hparams(max_norm=1.0, step=2)
        fused = zero.zero_adamw_step_f32grad_unpack if f32grad else zero.zero_adamw_step_unpack
        plain = zero.zero_adamw_step_f32grad if f32grad else zero.zero_adamw_step
        for b, c in [(0, S), (3, S - 3), (1000, S - 2000), (CUT - 5, 20)]:
            at = fused_cuts(lay, b, c)
            spans = [x for x in at for g in lay.segments if g.dst_off < x < g.dst_off + g.length]
            assert c <= CUT or spans, (rank, b, c, at)      # a piece continues in the next launch
            outs = []
            for mode in ("fused", "separate"):
                state = state0.clone()
                param = torch.full((S,), synth.SENTINEL, dtype=torch.int16, device=DEV).view(torch.bfloat16)
                tensors = [torch.full((n,), synth.SENTINEL, dtype=torch.int16, device=DEV).view(torch.bfloat16)
                           for n in sizes]
                if mode == "fused":
                    fused(grad, state, param, S, b, c, hp, parts, 1, h, tensors)
                else:
                    for rb, rc in small_ranges(b, c):
                        plain(grad, state, param, S, rb, rc, hp, parts, 1)
                    zero.zero_unpack_params(h, param, tensors, b, c)
                outs.append((state, param, tensors))
            torch.cuda.synchronize()
            (s0, p0, t0), (s1, p1, t1) = outs
            assert torch.equal(s0.view(torch.int32), s1.view(torch.int32)), (rank, b, c)
            assert torch.equal(p0.view(torch.int16), p1.view(torch.int16)), (rank, b, c)
            for i, (x, y) in enumerate(zip(t0, t1)):
                assert torch.equal(x.view(torch.int16), y.view(torch.int16)), (rank, b, c, i)
            del outs, s0, s1


def test_element_path_across_launch_cuts():
    """A gradient pointer off its vector alignment sends every launch down the
    element path; over a range of three launches it must give the vector
    path's bits, for the update and for the update with the unpack fused."""
    S = 2 * CUT + 3 * TILE + 5
    grad, state0 = make_state(S, False, seed=9)
    shifted = torch.empty(S + 1, dtype=torch.bfloat16, device=DEV)[1:]
    shifted.copy_(grad)
    assert shifted.data_ptr() % 8 == 2
    parts = torch.tensor([2.0, 3.0], dtype=torch.float64, device=DEV)
    hp = zero.hparams(max_norm=1.0, step=4)
    lay = zero.zero_layout([S], 1, 0, 1)
    outs = []
    for g in (grad, shifted):
        print(f"[element path] gradient at {g.data_ptr() % 16} mod 16", flush=True)
        state, param = state0.clone(), torch.zeros(S, dtype=torch.bfloat16, device=DEV)
        zero.zero_adamw_step(g, state, param, S, 0, S, hp, parts, 2)
        f_state, f_param = state0.clone(), torch.zeros(S, dtype=torch.bfloat16, device=DEV)
        tensor = torch.zeros(S, dtype=torch.bfloat16, device=DEV)
        zero.zero_adamw_step_unpack(g, f_state, f_param, S, 0, S, hp, parts, 2, lay, [tensor])
        torch.cuda.synchronize()
        outs.append((state, param, f_state, f_param, tensor))
    for a, b in zip(*outs):
        assert torch.equal(a.view(torch.int32 if a.dtype == torch.float32 else torch.int16),
                           b.view(torch.int32 if b.dtype == torch.float32 else torch.int16))
    assert torch.equal(outs[0][1].view(torch.int16), outs[0][4].view(torch.int16))
