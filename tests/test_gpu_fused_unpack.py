"""The update with the unpack fused (zero_adamw_step_unpack and its fp32-
gradient twin) against the two calls it replaces, zero_adamw_step followed
by zero_unpack_params over the same range: the fp32 state, the bf16 shard and
every byte of every tensor (sentinels outside the rank's segments included)
must be bit-identical. Ragged layouts on every rank, sub-ranges, padding,
tensors whose pointers are not 8-byte congruent with the shard (scalar
stores), misaligned shard pointers (the element path) and ranges of more
than 64 pieces (several launches)."""

import numpy as np
import pytest

from fsdp_sharded_mixed_zero_amd import synth, zero
from oracle.layout import build_layout

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = torch.device("cuda")

LAYOUTS = [
    # (sizes, n_d, align)
    ([3, 100_001, 7, 65_541, 0, 250_000, 13], 3, 1),
    ([3, 100_001, 7, 65_541, 0, 250_000, 13], 3, 128),
    ([1_000_003, 5, 77_777], 2, 8),
    ([8] * 9 + [123_457], 5, 1),
    ([37] * 150 + [5000], 1, 128),            # more than 64 pieces in one range
    ([1], 4, 1),                               # ranks made of padding only
]


def sentinel(n, offset=0):
    """n bf16 sentinels; with offset > 0 the tensor starts `offset` elements
    into a larger buffer (pointer not 8-byte aligned when offset is odd)."""
    buf = torch.full((n + offset + 8,), synth.SENTINEL, dtype=torch.int16, device=DEV)
    return buf[offset:offset + n].view(torch.bfloat16)


def bits(t):
    return t.view(torch.int16).cpu().numpy()


def run_pair(sizes, n_d, rank, align, b, c, f32grad, tensor_offset, shard_offset, rng):
    lay = build_layout(sizes, n_d, rank, align)
    h = zero.zero_layout(sizes, n_d, rank, align)
    S = lay.shard
    n_ranks = 3
    parts = torch.tensor(rng.random(n_ranks) * 4.0, dtype=torch.float64, device=DEV)
    hp = zero.hparams(max_norm=1.0, step=5)
    gdt = torch.float32 if f32grad else torch.bfloat16
    grad = (torch.randn(S + shard_offset, device=DEV) * 1e-2).to(gdt)[shard_offset:]
    master = torch.randn(S, device=DEV) * 0.02
    m = torch.randn(S, device=DEV) * 1e-4
    v = torch.rand(S, device=DEV) * 1e-8
    state0 = torch.empty(3 * S, dtype=torch.float32, device=DEV)
    if S:
        zero.zero_state_import(master, m, v, state0, S)
    outs = []
    for fused in (False, True):
        state = state0.clone()
        param = sentinel(S, shard_offset)
        tensors = [sentinel(n, tensor_offset) for n in sizes]
        if fused:
            fn = zero.zero_adamw_step_f32grad_unpack if f32grad else zero.zero_adamw_step_unpack
            fn(grad, state, param, S, b, c, hp, parts, n_ranks, h, tensors)
        else:
            fn = zero.zero_adamw_step_f32grad if f32grad else zero.zero_adamw_step
            fn(grad, state, param, S, b, c, hp, parts, n_ranks)
            zero.zero_unpack_params(h, param, tensors, b, c)
        torch.cuda.synchronize()
        outs.append((state.view(torch.int32).cpu().numpy(), bits(param), [bits(t) for t in tensors]))
    (s0, p0, t0), (s1, p1, t1) = outs
    assert np.array_equal(s0, s1), (sizes, rank, b, c)
    assert np.array_equal(p0, p1), (sizes, rank, b, c)
    for i, (x, y) in enumerate(zip(t0, t1)):
        assert np.array_equal(x, y), (sizes, rank, b, c, i)


@pytest.mark.parametrize("f32grad", [False, True], ids=["bf16-grad", "f32-grad"])
@pytest.mark.parametrize("sizes,n_d,align", LAYOUTS)
def test_fused_unpack_equals_update_then_unpack(sizes, n_d, align, f32grad):
    rng = np.random.default_rng(sum(sizes) + n_d + align + f32grad)
    for rank in range(n_d):
        S = build_layout(sizes, n_d, rank, align).shard
        ranges = [(0, S), (0, 0)]
        for _ in range(3):
            b = int(rng.integers(0, S + 1))
            ranges.append((b, int(rng.integers(0, S - b + 1))))
        for b, c in ranges:
            run_pair(sizes, n_d, rank, align, b, c, f32grad, 0, 0, rng)


@pytest.mark.parametrize("tensor_offset,shard_offset", [(1, 0), (2, 0), (0, 1), (3, 3)])
def test_fused_unpack_misaligned(tensor_offset, shard_offset):
    """Tensor pointers not 8-byte congruent with the shard take scalar stores;
    a shard pointer off the vector alignment takes the element path."""
    rng = np.random.default_rng(tensor_offset * 10 + shard_offset)
    sizes = [3, 100_001, 7, 65_541, 250_000, 13]
    for rank in range(2):
        S = build_layout(sizes, 2, rank, 1).shard
        for b, c in ((0, S), (5, S - 11)):
            for f32grad in (False, True):
                run_pair(sizes, 2, rank, 1, b, c, f32grad, tensor_offset, shard_offset, rng)


def test_fused_unpack_rejects_bad_layout_arguments():
    sizes = [100, 28]
    h = zero.zero_layout(sizes, 1, 0, 1)
    S = 128
    g = torch.zeros(S, dtype=torch.bfloat16, device=DEV)
    st = torch.zeros(3 * S, dtype=torch.float32, device=DEV)
    p = torch.zeros(S, dtype=torch.bfloat16, device=DEV)
    hp = zero.hparams(max_norm=0.0, step=1)
    tensors = [sentinel(n) for n in sizes]
    with pytest.raises(zero.ZeroError):
        zero.zero_adamw_step_unpack(g, st, p, S - 1, 0, 8, hp, None, 0, h, tensors)
    with pytest.raises(zero.ZeroError):        # a tensor the range needs is missing
        zero.zero_adamw_step_unpack(g, st, p, S, 0, 8, hp, None, 0, h, [None, tensors[1]])
