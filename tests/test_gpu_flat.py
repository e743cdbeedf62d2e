"""The ZeRO-1 flat-buffer form on the GPU: gradients and parameters are views
into two flat buffers and the shard is the rank's slice of each, so the step
is the sum of squares and AdamW only (no pack, no unpack). It must equal the
packed step with the separate norm bit for bit (same values reduced in the
same order), padding included, and write nothing outside the rank's slice."""

import numpy as np
import pytest

from fsdp_sharded_mixed_zero_amd import synth
from devbits import u16

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,rank", [("tiny", 1), ("tiny", 3), ("gpt2-1.5b", 63), ("gpt-7.5b", 1), ("llama-7b", 3)])
def test_flat_equals_packed(name, rank):
    from fsdp_sharded_mixed_zero_amd.rank import RankShard

    wl = synth.WORKLOADS[name]
    print(f"\n[flat {name} rank {rank}]", flush=True)
    packed = RankShard(wl, rank=rank, fused_norm=False)
    flat = RankShard(wl, rank=rank, flat=True)
    lo, S = flat.info["shard_begin"], flat.shard
    if name == "gpt2-1.5b":
        assert flat.real < S                              # the last rank holds the padding
    for t in (wl.step, wl.step + 1):
        packed.step(t)
        flat.step(t)
        torch.cuda.synchronize()
        assert float(packed.rank_sq[rank].cpu()) == float(flat.rank_sq[rank].cpu())
        assert np.array_equal(u16(packed.param_shard), u16(flat.param_shard)), t
        assert torch.equal(packed.state.view(torch.int32), flat.state.view(torch.int32)), t
        for a, b in zip(packed.params, flat.params):
            if a is not None:
                assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    sentinel = torch.tensor(synth.SENTINEL, dtype=torch.int16, device=flat.param_flat.device)
    whole = flat.param_flat.view(torch.int16)
    assert bool((whole[:lo] == sentinel).all()) and bool((whole[lo + S:] == sentinel).all())
    print(f"[flat {name} rank {rank}] bit-identical to the packed step; nothing written outside the slice",
          flush=True)
    del packed, flat
    torch.cuda.empty_cache()
