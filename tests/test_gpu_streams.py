"""Concurrent steps on two streams: the library keeps no device-side state of
its own (every buffer is the caller's), so two ranks' shards stepped at the
same time on two streams of one GPU must give the bits of the same steps run
one after another."""

import pytest

from fsdp_sharded_mixed_zero_amd import synth
from fsdp_sharded_mixed_zero_amd.rank import RankShard

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def bits(t):
    return t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32)


def test_two_streams_equal_sequential_steps():
    names = ("gpt2-1.5b", "tiny")
    concurrent = [RankShard(synth.WORKLOADS[n]) for n in names]
    sequential = [RankShard(synth.WORKLOADS[n]) for n in names]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    for k in range(3):
        print(f"[streams] step {k}", flush=True)
        for rs, st in zip(concurrent, streams):        # both enqueued before either finishes
            with torch.cuda.stream(st):
                rs.step(rs.wl.step + k)
        for rs in sequential:
            rs.step(rs.wl.step + k)
            torch.cuda.synchronize()
        torch.cuda.synchronize()
        for name, a, b in zip(names, concurrent, sequential):
            for buf in ("state", "param_shard", "grad_shard", "rank_sq"):
                x, y = getattr(a, buf), getattr(b, buf)
                same = torch.equal(x.view(torch.int64), y.view(torch.int64)) if x.dtype == torch.float64 else \
                    torch.equal(bits(x), bits(y))
                assert same, (name, k, buf)
            for i in a.touched:
                assert torch.equal(bits(a.params[i]), bits(b.params[i])), (name, k, i)
