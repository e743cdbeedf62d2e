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


def test_bucket_sums_equal_the_per_bucket_call():
    """The bucketed step's sums of squares (each bucket's block partials in its
    own slice, one row-sum launch) equal, bit for bit, zero_pack_grads_sqnorm
    called bucket by bucket; the packed shard is the same too."""
    from fsdp_sharded_mixed_zero_amd import zero

    wl = synth.WORKLOADS["gpt2-1.5b"]
    rs = RankShard(wl, bucket=3_000_017, streams=2)
    assert rs.bucketed
    own = torch.zeros(1, dtype=torch.float64, device="cuda")
    rs.pack_norm_buckets(own, torch.cuda.current_stream())
    torch.cuda.synchronize()
    shard = rs.grad_shard.clone()
    per_call = torch.zeros(len(rs.pieces()), dtype=torch.float64, device="cuda")
    for k, (b, n) in enumerate(rs.pieces()):
        zero.zero_pack_grads_sqnorm(rs.layout, rs.grad_ptrs, rs.grad_shard, b, n, per_call[k:k + 1], False,
                                    rs.workspace)
    torch.cuda.synchronize()
    assert torch.equal(bits(per_call), bits(rs.bucket_sq))
    assert torch.equal(bits(shard), bits(rs.grad_shard))
    again = torch.zeros(1, dtype=torch.float64, device="cuda")
    zero.zero_sum_partials(per_call, len(rs.pieces()), again)
    assert torch.equal(bits(again), bits(own))


def test_partial_rows_equal_sum_partials():
    """zero_sum_partials_rows over 400 rows of random lengths (0 to 20000,
    three launches of at most 192 rows) equals zero_sum_partials on each row
    bit for bit, plain and accumulating; and the calls refuse what they
    should."""
    from fsdp_sharded_mixed_zero_amd import zero

    g = torch.Generator(device="cuda").manual_seed(5)
    lens = torch.randint(0, 20001, (400,), generator=g, device="cuda").tolist()
    lens[3] = 0
    begins = [sum(lens[:r]) + 7 * r for r in range(400)]             # gaps between the rows
    data = torch.randn(begins[-1] + lens[-1] + 5, dtype=torch.float64, device="cuda", generator=g) ** 2
    out = torch.full((400,), 0.5, dtype=torch.float64, device="cuda")
    zero.zero_sum_partials_rows(data, begins, lens, out, accumulate=False)
    acc = torch.full((400,), 0.5, dtype=torch.float64, device="cuda")
    zero.zero_sum_partials_rows(data, begins, lens, acc, accumulate=True)
    want = torch.zeros(400, dtype=torch.float64, device="cuda")
    want_acc = torch.full((400,), 0.5, dtype=torch.float64, device="cuda")
    for r in range(400):
        zero.zero_sum_partials(data[begins[r]:], lens[r], want[r:r + 1])
        zero.zero_sum_partials(data[begins[r]:], lens[r], want_acc[r:r + 1], accumulate=True)
    torch.cuda.synchronize()
    assert torch.equal(bits(out), bits(want))
    assert torch.equal(bits(acc), bits(want_acc))
    assert float(out[3]) == 0.0
    with pytest.raises(zero.ZeroError):
        zero.zero_sum_partials_rows(data, [0, -1], [1, 1], out)
    lay = zero.zero_layout([1000], 1, 0, 1)
    grad = torch.zeros(1000, dtype=torch.bfloat16, device="cuda")
    shard = torch.empty_like(grad)
    with pytest.raises(zero.ZeroError, match="room for"):
        zero.zero_pack_grads_sqnorm_partials(lay, [grad], shard, 0, 1000, out, 8)
