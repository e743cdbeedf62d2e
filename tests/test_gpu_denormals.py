"""Subnormal inputs through the HIP path: the update keeps subnormal
gradients, moments, master weights and bf16 parameters (no flush to zero),
agreeing with the oracle; the update with the unpack fused and the host
update give the same bits as the GPU update; the packed sum of squares of
subnormal bf16 gradients is exact."""

import numpy as np
import pytest

import denormal_inputs as D
from fsdp_sharded_mixed_zero_amd import zero
from oracle import step as O
from oracle.layout import build_layout
from state_tiles import TILE, from_tiles, to_tiles
from devbits import hp_of, u16

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = torch.device("cuda")


def dev_grad(grad):
    if grad.dtype == np.float32:
        return torch.from_numpy(grad.copy()).to(DEV)
    return torch.from_numpy(grad.view(np.int16).copy()).to(DEV).view(torch.bfloat16)


@pytest.mark.parametrize("f32grad", [False, True], ids=["bf16-grad", "f32-grad"])
@pytest.mark.parametrize("kind", ["moments", "decay"])
def test_update_keeps_subnormals(kind, f32grad):
    n = 3 * TILE + 7
    grad, master, m, v, ohp, step, parts = D.case(kind, n, seed=7, f32grad=f32grad)
    hp = hp_of(ohp, step)
    d_parts = torch.from_numpy(parts).to(DEV)
    state0 = torch.from_numpy(to_tiles(master, m, v)).to(DEV)

    state = state0.clone()
    param = torch.empty(n, dtype=torch.bfloat16, device=DEV)
    fn = zero.zero_adamw_step_f32grad if f32grad else zero.zero_adamw_step
    fn(dev_grad(grad), state, param, n, 0, n, hp, d_parts, parts.size)

    # the same update with the unpack fused, into a one-tensor layout
    lay = zero.zero_layout([n], 1, 0, 1)
    f_state = state0.clone()
    f_param = torch.empty(n, dtype=torch.bfloat16, device=DEV)
    tensor = torch.empty(n, dtype=torch.bfloat16, device=DEV)
    fn = zero.zero_adamw_step_f32grad_unpack if f32grad else zero.zero_adamw_step_unpack
    fn(dev_grad(grad), f_state, f_param, n, 0, n, hp, d_parts, parts.size, lay, [tensor])
    torch.cuda.synchronize()

    got_state = state.cpu().numpy()
    got_param = u16(param)
    assert np.array_equal(f_state.cpu().numpy().view(np.uint32), got_state.view(np.uint32))
    assert np.array_equal(u16(f_param), got_param) and np.array_equal(u16(tensor), got_param)

    coef = O.clip_coef(O.global_sqnorm(parts), ohp.max_norm, ohp.clip_eps)
    if f32grad:
        want = O.adamw_step_f32grad(grad, master, m, v, step, ohp, coef)
    else:
        want = O.adamw_step(grad, master, m, v, step, ohp, coef)
    D.check_against_oracle((*from_tiles(got_state, n), got_param), want, m, v)

    if not f32grad:     # the host update (ZeRO-Offload) gives the GPU's bits
        h_state = to_tiles(master, m, v)
        h_param = np.zeros(n, np.uint16)
        zero.zero_cpu_adamw_step(grad, h_state, h_param, n, 0, n, hp, parts, parts.size, 2)
        assert np.array_equal(h_state.view(np.uint32), got_state.view(np.uint32))
        assert np.array_equal(h_param, got_param)


def test_packed_sum_of_squares_of_subnormals_is_exact():
    """Every square of a bf16 subnormal k * 2^-133 (k < 128) is k^2 * 2^-266,
    and sums of fewer than 2^39 of them are exact in fp64: the GPU's sum must
    equal the oracle's in every bit, whatever the order."""
    sizes = [1000, 3, 70_001, 5]
    rng = np.random.default_rng(3)
    grads = [D.subnormal_bf16_bits(rng, s) for s in sizes]
    d_grads = [torch.from_numpy(g.view(np.int16)).to(DEV).view(torch.bfloat16) for g in grads]
    for rank in range(2):
        lay = build_layout(sizes, 2, rank, 8)
        h = zero.zero_layout(sizes, 2, rank, 8)
        S = lay.shard
        out = torch.zeros(1, dtype=torch.float64, device=DEV)
        ws = torch.empty(max(zero.zero_pack_sqnorm_workspace_bytes(h, 0, S) // 8, 1), dtype=torch.float64,
                         device=DEV)
        shard = torch.empty(S, dtype=torch.bfloat16, device=DEV)
        zero.zero_pack_grads_sqnorm(h, d_grads, shard, 0, S, out, False, ws)
        torch.cuda.synchronize()
        want_shard = O.pack(lay, grads)
        assert np.array_equal(u16(shard), want_shard)
        want = O.sqnorm(want_shard)
        assert want > 0 and float(out.cpu()[0]) == want
