"""A sharded checkpoint of one rank's optimizer state, resumed: each rank
saves only its own shard of the fp32 master, m and v ("別再複製本可分片的東西：
ZeRO 與 FSDP", on sharded checkpoints). Ten steps straight through must equal,
bit for bit, five steps, a save of the shard (zero_state_export to three
arrays, written to .npy files), a fresh state buffer filled with garbage, a
load (zero_state_import), and five more steps: the state, the bf16 parameter
shard and the per-tensor parameters. Each step draws fresh gradients. With
the state held as three arrays (master, m, v: the pages' own form), the
shard is saved as those arrays and the rank's arrays are replaced by the
loaded ones."""

import numpy as np
import pytest

from fsdp_sharded_mixed_zero_amd import zero

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _run(rs, steps, t0):
    for t in range(t0, t0 + steps):
        rs.fill_grads(t)
        rs.step(t)
    torch.cuda.synchronize()


@pytest.mark.parametrize("name", ["tiny", "gpt2-1.5b"])
def test_resume_from_sharded_checkpoint(name, tmp_path):
    from fsdp_sharded_mixed_zero_amd import synth
    from fsdp_sharded_mixed_zero_amd.rank import RankShard

    wl = synth.WORKLOADS[name]
    print(f"\n[checkpoint {name}]", flush=True)
    straight = RankShard(wl)
    _run(straight, 10, wl.step)

    resumed = RankShard(wl)
    _run(resumed, 5, wl.step)
    S = resumed.shard
    saved = [torch.empty(S, dtype=torch.float32, device="cuda") for _ in range(3)]
    zero.zero_state_export(resumed.state, *saved, S)
    torch.cuda.synchronize()
    for k, x in enumerate(saved):
        np.save(tmp_path / f"rank{resumed.rank}_state{k}.npy", x.cpu().numpy())
    del saved
    resumed.state = torch.full((3 * S,), float("nan"), dtype=torch.float32, device="cuda")
    loaded = [torch.from_numpy(np.load(tmp_path / f"rank{resumed.rank}_state{k}.npy")).to("cuda")
              for k in range(3)]
    zero.zero_state_import(*loaded, resumed.state, S)
    _run(resumed, 5, wl.step + 5)

    assert torch.equal(straight.state.view(torch.int32), resumed.state.view(torch.int32))
    assert torch.equal(straight.param_shard.view(torch.int16), resumed.param_shard.view(torch.int16))
    for a, b in zip(straight.params, resumed.params):
        if a is not None:
            assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    print(f"[checkpoint {name}] ten steps == five + save/load + five, bit for bit", flush=True)


@pytest.mark.parametrize("name", ["tiny", "gpt2-1.5b"])
def test_resume_three_state_arrays(name, tmp_path):
    from fsdp_sharded_mixed_zero_amd import synth
    from fsdp_sharded_mixed_zero_amd.rank import RankShard

    wl = synth.WORKLOADS[name]
    print(f"\n[checkpoint {name}, three state arrays]", flush=True)
    straight = RankShard(wl, state_arrays=True)
    _run(straight, 10, wl.step)

    resumed = RankShard(wl, state_arrays=True)
    _run(resumed, 5, wl.step)
    names = ("master", "m", "v")
    for k in names:
        np.save(tmp_path / f"rank{resumed.rank}_{k}.npy", getattr(resumed, k).cpu().numpy())
        setattr(resumed, k, None)
    torch.cuda.empty_cache()
    for k in names:
        setattr(resumed, k, torch.from_numpy(np.load(tmp_path / f"rank{resumed.rank}_{k}.npy")).to("cuda"))
    _run(resumed, 5, wl.step + 5)

    for k in names:
        assert torch.equal(getattr(straight, k).view(torch.int32), getattr(resumed, k).view(torch.int32)), k
    assert torch.equal(straight.param_shard.view(torch.int16), resumed.param_shard.view(torch.int16))
    for a, b in zip(straight.params, resumed.params):
        if a is not None:
            assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    print(f"[checkpoint {name}, three state arrays] ten steps == five + save/load + five, bit for bit", flush=True)
