"""Pack, pack + sum of squares and unpack at sizes where the copy kernels
split one call into several launches: a single bf16 tensor of 2^35 + 2^20
elements (68.7 GB) is the whole model at N_d = 1, so its range is cut into
three pieces (2^34, 2^34 and 2^20 elements). The plain copy takes one launch
per piece (a piece of 2^34 elements fills the 2^23 blocks of 256 lanes a
launch may hold); the copy with the sum of squares takes two launches (the
first two pieces fill 2^22 blocks of 512 lanes, the third goes alone), and
its final sum adds over 4 million block partials.

Element i holds the bf16 value 1 + (i mod 128)/128, so every square and every
partial sum is a multiple of 2^-14 below 2^39: any order of fp64 additions
gives the exact sum, which a closed form states. Sampled ranges around the
piece cuts, the launch cut, 2^31, 2^32 and the ends are checked element by
element."""

from fractions import Fraction

import numpy as np
import pytest

from fsdp_sharded_mixed_zero_amd import synth, zero
from devbits import u16

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = torch.device("cuda")
N = (1 << 35) + (1 << 20)
PIECE = 1 << 34
W = 4096
# around 2^31, 2^32, the first piece cut, the second (also the launch cut of
# the copy with the sum of squares), the end, and two other places
STARTS = [0, (1 << 31) - W // 2, (1 << 32) - W // 2, PIECE - W // 2, 2 * PIECE - W // 2 - 3 * W,
          2 * PIECE - W // 2, N - W, 12_345_678_901]


def pattern(lo, hi):
    return (0x3F80 + (np.arange(lo, hi, dtype=np.int64) & 127)).astype(np.uint16)


def other(lo, hi):
    return (0x4000 + (np.arange(lo, hi, dtype=np.int64) & 63)).astype(np.uint16)


def put(t, lo, bits):
    t[lo:lo + len(bits)] = torch.from_numpy(bits.view(np.int16).copy()).to(DEV)


def exact_sum():
    """Sum over i < N of (1 + (i mod 128)/128)^2, exactly (N is a multiple of 128)."""
    cycle = sum(Fraction(128 + k, 128) ** 2 for k in range(128))
    total = cycle * (N // 128)
    assert total.denominator <= 1 << 14 and total < 1 << 39
    return float(total)


@pytest.fixture(scope="module")
def big():
    torch.cuda.empty_cache()
    free, _ = torch.cuda.mem_get_info()
    if free < 2 * 2 * N + (4 << 30):
        pytest.skip(f"needs {2 * 2 * N / 2**30:.0f} GiB of free device memory, {free / 2**30:.0f} GiB free")
    tensor = torch.empty(N, dtype=torch.int16, device=DEV)
    step = 1 << 28
    for lo in range(0, N, step):
        hi = min(N, lo + step)
        tensor[lo:hi] = ((torch.arange(lo, hi, dtype=torch.int64, device=DEV) & 127) + 0x3F80).to(torch.int16)
    shard = torch.empty(N, dtype=torch.int16, device=DEV)
    yield zero.zero_layout([N], 1, 0, 1), tensor, shard
    del tensor, shard
    torch.cuda.empty_cache()


def test_pack_with_sum_of_squares_in_two_launches(big):
    h, tensor, shard = big
    for s in STARTS:
        put(shard, s, np.full(W, synth.SENTINEL, np.uint16))
    ws = torch.empty(zero.zero_pack_sqnorm_workspace_bytes(h, 0, N) // 8, dtype=torch.float64, device=DEV)
    out = torch.full((1,), -1.0, dtype=torch.float64, device=DEV)
    print(f"[max sizes] pack + sum of squares of {N} elements", flush=True)
    zero.zero_pack_grads_sqnorm(h, [tensor], shard, 0, N, out, False, ws)
    torch.cuda.synchronize()
    for s in STARTS:
        assert np.array_equal(u16(shard[s:s + W]), pattern(s, s + W)), s
    assert float(out.cpu()[0]) == exact_sum()
    del ws


def test_plain_pack_one_launch_per_piece(big):
    h, tensor, shard = big
    for s in STARTS:
        put(shard, s, np.full(W, synth.SENTINEL, np.uint16))
    print(f"[max sizes] pack of {N} elements", flush=True)
    zero.zero_pack_grads(h, [tensor], shard, 0, N)
    torch.cuda.synchronize()
    for s in STARTS:
        assert np.array_equal(u16(shard[s:s + W]), pattern(s, s + W)), s


def test_unpack_one_launch_per_piece(big):
    """The shard holds the pattern except on the sampled ranges, which hold
    other values; after the unpack the tensor must hold the same."""
    h, tensor, shard = big
    zero.zero_pack_grads(h, [tensor], shard, 0, N)
    for s in STARTS:
        put(shard, s + 16, other(s + 16, s + W - 16))
    print(f"[max sizes] unpack of {N} elements", flush=True)
    zero.zero_unpack_params(h, shard, [tensor], 0, N)
    torch.cuda.synchronize()
    for s in STARTS:
        want = pattern(s, s + W)
        want[16:W - 16] = other(s + 16, s + W - 16)
        assert np.array_equal(u16(tensor[s:s + W]), want), s
