"""The binding example in README.md, run as written on a small ragged model
(the shard cuts through tensors and ends in padding), against the oracle:
the packed shard bit for bit, the sum of squares, the fp32 state and bf16
parameters within the stated tolerances, and the per-tensor parameters
equal to the parameter shard on the rank's segments and untouched
elsewhere."""

import os
import re

import numpy as np
import pytest

from fsdp_sharded_mixed_zero_amd import synth
from oracle import step as O
from oracle.layout import build_layout
from state_tiles import from_tiles
from tolerance import assert_bf16_param, assert_f32_state, assert_norm_close

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

README = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "README.md")


def readme_example():
    text = open(README, encoding="utf-8").read()
    blocks = re.findall(r"```python\n(.*?)```", text, re.S)
    assert len(blocks) == 1, "README holds one python example"
    return blocks[0]


def test_readme_example_runs_and_matches_the_oracle():
    sizes, n_d, rank = [5000, 37, 70_000, 12_345, 0, 9], 3, 2
    lay = build_layout(sizes, n_d, rank, 128)
    assert lay.pad_end > lay.pad_begin and len(lay.segments) > 1
    S = lay.shard
    rng = np.random.default_rng(5)
    host_grads = [synth.to_bf16_bits((rng.standard_normal(n) * 1e-3).astype(np.float32)) for n in sizes]
    master = (rng.standard_normal(S) * 0.02).astype(np.float32)
    m = (rng.standard_normal(S) * 1e-4).astype(np.float32)
    v = np.abs(rng.standard_normal(S) * 1e-8).astype(np.float32)
    dev = torch.device("cuda")
    env = {
        "sizes": sizes, "n_d": n_d, "rank": rank,
        "grads": [torch.from_numpy(g.view(np.int16).copy()).to(dev).view(torch.bfloat16) for g in host_grads],
        "params": [torch.full((n,), synth.SENTINEL, dtype=torch.int16, device=dev).view(torch.bfloat16)
                   for n in sizes],
        "master": torch.from_numpy(master).to(dev), "m": torch.from_numpy(m).to(dev),
        "v": torch.from_numpy(v).to(dev),
    }
    print("[readme] running the example", flush=True)
    exec(readme_example(), env)
    torch.cuda.synchronize()

    packed = O.pack(lay, host_grads)
    got_shard = env["grad_shard"].view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got_shard, packed)
    sq = O.sqnorm(packed)
    got_sq = env["rank_sq"].cpu().numpy()
    assert_norm_close(got_sq[rank], sq)
    assert not got_sq[np.arange(n_d) != rank].any()        # the other ranks' entries were never filled
    # the oracle's coefficient from its own partial (the example's update read the GPU's)
    coef = O.clip_coef(O.global_sqnorm([sq if r == rank else 0.0 for r in range(n_d)]), 1.0)
    want = O.adamw_step(packed, master, m, v, 1, O.AdamWHParams(lr=1e-3, weight_decay=0.01, max_norm=1.0), coef)
    g_master, g_m, g_v = from_tiles(env["state"].cpu().numpy(), S)
    assert_f32_state(g_master, want[0], "master")
    assert_f32_state(g_m, want[1], "m", m)
    assert_f32_state(g_v, want[2], "v", v)
    g_param = env["param_shard"].view(torch.int16).cpu().numpy().view(np.uint16)
    assert_bf16_param(g_param, want[3], want[0], "param", g_master)
    # each tensor element the rank owns holds its shard element; the rest keep the sentinel
    placed = [np.full(n, synth.SENTINEL, np.uint16) for n in sizes]
    for seg in lay.segments:
        placed[seg.tensor][seg.src_off:seg.src_off + seg.length] = g_param[seg.dst_off:seg.dst_off + seg.length]
    for i, t in enumerate(env["params"]):
        assert np.array_equal(t.view(torch.int16).cpu().numpy().view(np.uint16), placed[i]), i
