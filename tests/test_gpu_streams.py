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
    """The tensor's bits as integers of its element size."""
    return t.view({2: torch.int16, 4: torch.int32, 8: torch.int64}[t.element_size()])


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
                assert torch.equal(bits(getattr(a, buf)), bits(getattr(b, buf))), (name, k, buf)
            for i in a.touched:
                assert torch.equal(bits(a.params[i]), bits(b.params[i])), (name, k, i)


def test_bucketed_step_on_one_or_two_streams():
    """A bucketed step (each bucket's sum of squares in its own slot, one
    fixed-order combine, the buckets dealt out to the streams) gives the same
    bits on one stream and on two, over several steps."""
    wl = synth.WORKLOADS["gpt2-1.5b"]
    one = RankShard(wl, bucket=5_000_000, streams=1)
    two = RankShard(wl, bucket=5_000_000, streams=2)
    assert one.bucketed and two.bucketed and one.n_streams == 1 and two.n_streams == 2
    for k in range(3):
        print(f"[buckets] step {k}", flush=True)
        one.step(wl.step + k)
        two.step(wl.step + k)
        torch.cuda.synchronize()
        for buf in ("state", "param_shard", "grad_shard", "bucket_sq", "rank_sq"):
            assert torch.equal(bits(getattr(one, buf)), bits(getattr(two, buf))), (k, buf)
        for i in one.touched:
            assert torch.equal(bits(one.params[i]), bits(two.params[i])), (k, i)


def test_step_on_a_given_stream_times_its_own_launches():
    """A step handed a stream (a torch stream or its raw handle) runs there
    and records its timing events there: each phase's interval covers its
    kernels (the GPT-2 shard's update moves 0.73 GB, so it takes tens of
    microseconds at least), and the results equal a step on the current
    stream bit for bit."""
    wl = synth.WORKLOADS["gpt2-1.5b"]
    side, ref = RankShard(wl), RankShard(wl)
    st = torch.cuda.Stream()
    torch.cuda.synchronize()
    for k, handle in enumerate((st, st.cuda_stream)):
        print(f"[given stream] step {k}", flush=True)
        timing = {}
        side.step(wl.step + k, stream=handle, timing=timing)
        ref.step(wl.step + k)
        torch.cuda.synchronize()
        for phase in ("pack_sqnorm", "adamw"):
            (e0, e1), = timing[phase]
            assert e0.elapsed_time(e1) * 1e3 > (50.0 if phase == "adamw" else 5.0), (phase, e0.elapsed_time(e1))
        for buf in ("state", "param_shard", "grad_shard", "rank_sq"):
            assert torch.equal(bits(getattr(side, buf)), bits(getattr(ref, buf))), (k, buf)
