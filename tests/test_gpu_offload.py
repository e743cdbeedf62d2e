"""ZeRO-Offload on the GPU: the offloaded step (GPU pack + norm, PCIe
copies through pinned staging slots, AdamW on the host cores, GPU unpack)
against the oracle, and against the all-GPU step with the same inputs and
buckets, which it must equal bit for bit (same fp32 operation sequence)."""

import numpy as np
import pytest

from fsdp_sharded_mixed_zero_amd import synth, zero
from oracle import step as O
from oracle.layout import build_layout
from state_tiles import from_tiles, to_tiles
from tolerance import assert_bf16_param, assert_f32_state, assert_norm_close
from devbits import u16

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,bucket", [("tiny", 65_536), ("tiny", 100_003), ("gpt2-1.5b", 1 << 22),
                                         ("gpt-7.5b", 1 << 24)])
def test_offload_equals_gpu_step(name, bucket):
    from fsdp_sharded_mixed_zero_amd.rank import OffloadRank, RankShard

    wl = synth.WORKLOADS[name]
    print(f"\n[offload {name}] bucket {bucket}", flush=True)
    gpu = RankShard(wl, bucket=bucket)
    off = OffloadRank(wl, bucket=bucket, slots=3)
    assert off.pieces() == gpu.pieces()
    assert off.state is None                        # no optimizer state left on the device
    for t in (wl.step, wl.step + 1):
        gpu.step(t)
        off.step(t)
        torch.cuda.synchronize()
        assert float(gpu.rank_sq[gpu.rank].cpu()) == float(off.rank_sq[off.rank].cpu())
        assert np.array_equal(u16(gpu.param_shard), u16(off.param_shard)), t
        assert np.array_equal(gpu.state.cpu().numpy().view(np.uint32), off.h_state.view(np.uint32)), t
        for a, b in zip(gpu.params, off.params):
            if a is not None:
                assert np.array_equal(u16(a), u16(b))
    print(f"[offload {name}] {len(off.pieces())} buckets; bit-identical to the GPU step", flush=True)
    del gpu, off
    torch.cuda.empty_cache()


def test_offload_tiny_against_oracle():
    """The tiny workload's rank 1, offloaded, for three steps against the
    oracle (other ranks' partial sums as inputs, as in the benchmark)."""
    from fsdp_sharded_mixed_zero_amd.rank import OffloadRank

    wl = synth.WORKLOADS["tiny"]
    lay = build_layout(wl.sizes, wl.n_d, wl.rank, wl.align)
    S = lay.shard
    off = OffloadRank(wl, bucket=50_000, fill=False)
    captured = {}
    off.fill_state(on_chunk=lambda lo, hi, p, m, v: captured.update(
        master=p.cpu().numpy(), m=m.cpu().numpy(), v=v.cpu().numpy()))
    off.move_state_to_host()
    off.fill_grads(wl.step)
    off.fill_other_ranks()
    others = off.rank_sq.cpu().numpy().copy()
    grads = [None if g is None else u16(g) for g in off.grads]
    o_master, o_m, o_v = captured["master"], captured["m"], captured["v"]
    ohp = O.AdamWHParams(lr=wl.lr, beta1=wl.beta1, beta2=wl.beta2, eps=wl.eps,
                         weight_decay=wl.weight_decay, max_norm=wl.max_norm)
    for t in range(1, 4):
        off.step(t)
        torch.cuda.synchronize()
        g_bits = O.pack(lay, grads)
        own = O.sqnorm(g_bits)
        assert_norm_close(float(off.rank_sq[off.rank].cpu()), own, "partial")
        partials = others.copy()
        partials[off.rank] = own
        coef = O.clip_coef(O.global_sqnorm(partials), wl.max_norm)
        old_m, old_v = o_m, o_v
        o_master, o_m, o_v, o_param = O.adamw_step(g_bits, o_master, o_m, o_v, t, ohp, coef)
        h_master, h_m, h_v = from_tiles(off.h_state, S)
        assert_f32_state(h_master, o_master, f"master {t}")
        assert_f32_state(h_m, o_m, f"m {t}", np.maximum(np.abs(old_m), np.abs(o_m)), 16 * t)
        assert_f32_state(h_v, o_v, f"v {t}", np.maximum(np.abs(old_v), np.abs(o_v)), 16 * t)
        assert_bf16_param(u16(off.param_shard), o_param, o_master, f"param {t}", h_master)


@pytest.mark.parametrize("n_ranks", [1, 64, 65, 1000, 5000])
def test_clip_sum_order_gpu_equals_host(n_ranks):
    """The ranks' partial sums are added in the same fixed order on the GPU
    and on the host (rank order up to 64 ranks, 64 strided lane sums beyond), so the
    two updates agree bit for bit; partials spanning nine decades make the
    order matter. Both also match the oracle, which adds in rank order."""
    n = 100_003
    rng = np.random.default_rng(n_ranks)
    bits = synth.to_bf16_bits((rng.standard_normal(n) * 1e-3).astype(np.float32))
    master = (rng.standard_normal(n) * 0.02).astype(np.float32)
    m = (rng.standard_normal(n) * 1e-4).astype(np.float32)
    v = np.abs(rng.standard_normal(n) * 1e-8).astype(np.float32)
    parts = rng.random(n_ranks) * 10.0 ** rng.integers(-6, 3, n_ranks).astype(np.float64)
    parts *= 9.0 / parts.sum()                    # global norm ~3: clipping is on
    hp = zero.hparams(max_norm=1.0, step=3)
    dev = torch.device("cuda")
    d_g = torch.from_numpy(bits.view(np.int16)).to(dev)
    d_state = torch.from_numpy(to_tiles(master, m, v)).to(dev)
    d_param = torch.empty(n, dtype=torch.int16, device=dev)
    d_parts = torch.from_numpy(parts).to(dev)
    zero.zero_adamw_step(d_g, d_state, d_param, n, 0, n, hp, d_parts, n_ranks)
    h_state = to_tiles(master, m, v)
    h_param = np.zeros(n, np.uint16)
    zero.zero_cpu_adamw_step(bits, h_state, h_param, n, 0, n, hp, parts, n_ranks, 4)
    torch.cuda.synchronize()
    assert np.array_equal(d_state.cpu().numpy().view(np.uint32), h_state.view(np.uint32))
    assert np.array_equal(d_param.cpu().numpy().view(np.uint16), h_param)
    coef = O.clip_coef(O.global_sqnorm(parts), 1.0)
    assert coef < 1.0
    want = O.adamw_step(bits, master, m, v, 3, O.AdamWHParams(max_norm=1.0), coef)
    g_master, g_m, g_v = from_tiles(h_state, n)
    assert_f32_state(g_master, want[0], "master")
    assert_f32_state(g_m, want[1], "m", m)
    assert_f32_state(g_v, want[2], "v", v)
    assert_bf16_param(h_param, want[3], want[0], "param", g_master)
