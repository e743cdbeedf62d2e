"""The step captured in a HIP graph: the entry points allocate nothing and
record no memset, so a caller can capture a step (fused pack + sum of squares,
then the update with the unpack fused) and replay it. Two identical shards
run side by side, one eagerly and one by graph replay; between replays the
gradients of both are refilled by eager work and the device is synchronised,
and after every replay each buffer of the graph's shard must equal the eager
one bit for bit. The step count is a kernel argument, so both use the step
the graph was captured with. The step with the state as three arrays (the
three-array update, then the unpack) is captured the same way."""

import pytest

from fsdp_sharded_mixed_zero_amd import synth
from fsdp_sharded_mixed_zero_amd.rank import RankShard

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def same(a, b):
    if a.dtype in (torch.bfloat16, torch.float16):
        return torch.equal(a.view(torch.int16), b.view(torch.int16))
    if a.dtype == torch.float32:
        return torch.equal(a.view(torch.int32), b.view(torch.int32))
    return torch.equal(a.view(torch.int64), b.view(torch.int64))


@pytest.mark.parametrize("name,arrays", [("tiny", False), ("gpt2-1.5b", False), ("tiny", True),
                                         ("gpt2-1.5b", True)],
                         ids=["tiny", "gpt2-1.5b", "tiny-state-arrays", "gpt2-1.5b-state-arrays"])
def test_graph_replays_equal_eager_steps(name, arrays):
    wl = synth.WORKLOADS[name]
    eager, graphed = RankShard(wl, state_arrays=arrays), RankShard(wl, state_arrays=arrays)
    torch.cuda.synchronize()
    t = wl.step
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):                 # warm-up outside capture, as torch advises
        eager.step(t)
        graphed.step(t)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        graphed.step(t)
    torch.cuda.synchronize()
    # the capture ran nothing: bring the eager shard to the same point
    for rep in range(4):
        print(f"[graph {name}] replay {rep}", flush=True)
        eager.fill_grads(wl.step + 10 + rep)          # eager work between replays, read by the graph
        graphed.fill_grads(wl.step + 10 + rep)
        torch.cuda.synchronize()
        eager.step(t)
        g.replay()
        torch.cuda.synchronize()
        if arrays:
            for k in ("master", "m", "v"):
                assert same(getattr(graphed, k), getattr(eager, k)), (name, rep, k)
        else:
            assert same(graphed.state, eager.state), (name, rep)
        assert same(graphed.param_shard, eager.param_shard), (name, rep)
        assert same(graphed.grad_shard, eager.grad_shard), (name, rep)
        assert same(graphed.rank_sq, eager.rank_sq), (name, rep)
        for i in graphed.touched:
            assert same(graphed.params[i], eager.params[i]), (name, rep, i)
