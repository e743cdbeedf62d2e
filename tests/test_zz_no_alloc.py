"""zero_pack_grads_sqnorm_noalloc (block partial sums in the library's static
device array) against zero_pack_grads_sqnorm (partial sums in a workspace),
through the C ABI: packed bytes and sums bit-identical, on calls in a row
whose later ranges are smaller (the array keeps the previous call's
contents), and the refusal of a range that needs more partial sums than the
array holds."""

import numpy as np
import pytest

from fsdp_sharded_mixed_zero_amd import synth, zero

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda"


def _both(lay, grads, S, begin, count, accumulate, start):
    """The two calls on the same inputs; returns (shard, sum) of each."""
    out = []
    for noalloc in (False, True):
        shard = torch.full((S,), synth.SENTINEL, dtype=torch.int16, device=DEV).view(torch.bfloat16)
        acc = torch.full((1,), start, dtype=torch.float64, device=DEV)
        if noalloc:
            zero.zero_pack_grads_sqnorm_noalloc(lay, grads, shard, begin, count, acc, accumulate)
        else:
            ws = torch.empty(max(1, zero.zero_pack_sqnorm_workspace_bytes(lay, begin, count) // 8),
                             dtype=torch.float64, device=DEV)
            zero.zero_pack_grads_sqnorm(lay, grads, shard, begin, count, acc, accumulate, ws)
        torch.cuda.synchronize()
        out.append((shard.view(torch.int16).cpu().numpy(), acc.cpu().numpy().view(np.uint64)))
    return out


def test_noalloc_matches_workspace_call():
    """The GPT-2 1.5B shard of rank 32 of 64 (24.3 M elements, 13 segments):
    the whole shard, then a smaller sub-range, then a short accumulating
    range, then a range of padding only on the last rank."""
    wl = synth.WORKLOADS["gpt2-1.5b"]
    for rank, ranges in ((wl.rank, [(0, None, False), (1_000_003, 7_777_777, False), (5, 4099, True)]),
                         (wl.n_d - 1, [(None, None, False)])):
        lay = zero.zero_layout(wl.sizes, wl.n_d, rank, wl.align)
        S = lay.info["shard"]
        grads = [None] * len(wl.sizes)
        for i in sorted({s[0] for s in lay.segments}):
            grads[i] = synth.device_grad_(torch.empty(wl.sizes[i], dtype=torch.bfloat16, device=DEV), wl, 1, salt=i)
        for begin, count, accumulate in ranges:
            if begin is None:                                  # the padding at the end of the last shard
                begin = lay.info["pad_begin"]
                count = S - begin
                assert count > 0
            if count is None:
                count = S - begin
            print(f"[noalloc] rank {rank} range [{begin}, +{count}) accumulate={accumulate}", flush=True)
            (sh_a, g_a), (sh_b, g_b) = _both(lay, grads, S, begin, count, accumulate, 2.5)
            assert np.array_equal(sh_a, sh_b)
            assert np.array_equal(g_a, g_b), (g_a, g_b)
            assert (sh_b[:begin] == synth.SENTINEL).all() and (sh_b[begin + count:] == synth.SENTINEL).all()


def test_noalloc_largest_range_and_refusal():
    """One tensor of 2^31 elements: a range of the largest length the array
    covers in one piece (2,147,475,456 elements) matches the workspace call;
    the whole tensor needs one partial sum too many and is refused before
    anything runs."""
    n = 1 << 31
    most = (zero.ZERO_NOALLOC_PARTIALS - 1) * 8192
    lay = zero.zero_layout([n], 1, 0, 1)
    grad = torch.empty(n, dtype=torch.bfloat16, device=DEV)
    grad[:1 << 24].copy_(torch.randn(1 << 24, device=DEV, generator=torch.Generator(DEV).manual_seed(3)))
    grad[1 << 24:].fill_(1.5)
    assert zero.zero_pack_sqnorm_workspace_bytes(lay, 0, most) == 8 * zero.ZERO_NOALLOC_PARTIALS
    print("[noalloc] largest range", flush=True)
    shard = torch.empty(n, dtype=torch.bfloat16, device=DEV)
    out = []
    for noalloc in (False, True):
        acc = torch.zeros(1, dtype=torch.float64, device=DEV)
        if noalloc:
            zero.zero_pack_grads_sqnorm_noalloc(lay, [grad], shard, 0, most, acc, False)
        else:
            ws = torch.empty(zero.ZERO_NOALLOC_PARTIALS, dtype=torch.float64, device=DEV)
            zero.zero_pack_grads_sqnorm(lay, [grad], shard, 0, most, acc, False, ws)
        torch.cuda.synchronize()
        out.append(acc.cpu().numpy().view(np.uint64))
        assert torch.equal(shard[:most].view(torch.int16), grad[:most].view(torch.int16))
    assert np.array_equal(out[0], out[1])
    with pytest.raises(zero.ZeroError, match="static scratch holds"):
        zero.zero_pack_grads_sqnorm_noalloc(lay, [grad], shard, 0, n, torch.zeros(1, dtype=torch.float64,
                                                                                   device=DEV), False)
