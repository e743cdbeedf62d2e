"""Element offsets beyond 2^31 inside one tensor: a single bf16 tensor of
2^31 + 12,345 elements (4.3 GB) is the whole model at N_d = 1, and short
ranges near and past element 2^31 go through pack, unpack and the update with
the unpack fused. Values are a known pattern (element i holds i mod 2^16), so
every element of a range is checked against its index; sentinels around each
range must stay."""

import numpy as np
import pytest

from fsdp_sharded_mixed_zero_amd import synth, zero
from oracle.layout import build_layout
from devbits import u16

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = torch.device("cuda")
N = (1 << 31) + 12_345
RANGES = [((1 << 31) - 100, 1000), ((1 << 31) + 7, 4099), (N - 1000, 1000), (3, 8)]


def pattern(lo, hi):
    return (np.arange(lo, hi, dtype=np.int64) & 0xFFFF).astype(np.uint16)


@pytest.fixture(scope="module")
def big():
    lay = build_layout([N], 1, 0, 1)
    assert lay.shard == N and len(lay.segments) == 1
    tensor = torch.empty(N, dtype=torch.int16, device=DEV)
    step = 1 << 28
    for lo in range(0, N, step):                     # element i holds i mod 2^16
        hi = min(N, lo + step)
        tensor[lo:hi] = (torch.arange(lo, hi, dtype=torch.int64, device=DEV) & 0xFFFF).to(torch.int32).to(
            torch.int16)
    yield zero.zero_layout([N], 1, 0, 1), tensor
    del tensor
    torch.cuda.empty_cache()


def test_pack_and_unpack_past_element_2_31(big):
    h, tensor = big
    shard = torch.full((N,), synth.SENTINEL, dtype=torch.int16, device=DEV)
    back = torch.full((N,), synth.SENTINEL, dtype=torch.int16, device=DEV)
    for b, c in RANGES:
        print(f"[large offsets] pack/unpack [{b}, +{c})", flush=True)
        zero.zero_pack_grads(h, [tensor], shard, b, c)
        zero.zero_unpack_params(h, shard, [back], b, c)
    torch.cuda.synchronize()
    for b, c in RANGES:
        lo, hi = max(0, b - 16), min(N, b + c + 16)
        want = pattern(b, b + c)
        for buf in (shard, back):
            got = u16(buf[lo:hi])
            assert np.array_equal(got[b - lo:b - lo + c], want), (b, c)
            inside = np.zeros(hi - lo, bool)
            for b2, c2 in RANGES:                    # neighbours of other ranges may be written
                inside[max(0, b2 - lo):max(0, min(hi, b2 + c2) - lo)] = True
            assert (got[~inside] == synth.SENTINEL).all(), (b, c)
    del shard, back


def test_fused_update_past_element_2_31(big):
    """The update with the unpack fused over the same ranges, against the
    plain update followed by unpack (bit-exact), with the state initialised
    only on the ranges it reads."""
    h, tensor = big
    grad = tensor.view(torch.bfloat16)               # the pattern as gradients: finite bf16 values
    state0 = torch.zeros(3 * N, dtype=torch.float32, device=DEV)
    hp = zero.hparams(max_norm=0.0, step=3)
    outs = []
    for fused in (True, False):
        state = state0.clone()
        param = torch.full((N,), synth.SENTINEL, dtype=torch.int16, device=DEV)
        dst = torch.full((N,), synth.SENTINEL, dtype=torch.int16, device=DEV)
        for b, c in RANGES:
            print(f"[large offsets] {'fused' if fused else 'separate'} update [{b}, +{c})", flush=True)
            if fused:
                zero.zero_adamw_step_unpack(grad, state, param, N, b, c, hp, None, 0, h, [dst])
            else:
                zero.zero_adamw_step(grad, state, param, N, b, c, hp, None, 0)
                zero.zero_unpack_params(h, param, [dst], b, c)
        torch.cuda.synchronize()
        outs.append([(u16(param[b:b + c]), u16(dst[max(0, b - 16):b + c + 16]),
                      state[3 * ((b // 8192) * 8192):3 * (((b + c - 1) // 8192 + 1) * 8192)].view(torch.int32).cpu())
                     for b, c in RANGES])
        del state, param, dst
        torch.cuda.empty_cache()
    for (p0, d0, s0), (p1, d1, s1), (b, c) in zip(outs[0], outs[1], RANGES):
        assert np.array_equal(p0, p1) and np.array_equal(d0, d1) and torch.equal(s0, s1), (b, c)
        assert (p0 != synth.SENTINEL).any(), (b, c)
