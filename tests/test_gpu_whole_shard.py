"""Every element of a full-size shard against the oracle, in the launch
configuration the benchmark times (RankShard.step: pack with the sum of
squares fused, then the update with the unpack fused):

  * the GPT-2 1.5B shard of rank 32 of 64 (24.3 M elements, 13 segments) and
    the 7.5B shard of rank 1 of 64 (119.4 M elements, 13 segments);
  * the ZeRO-1 flat-buffer form (sum of squares, then the update, on the
    rank's slice of flat buffers) on the GPT-2 shard of rank 63 (padding at
    its end) and the 7.5B shard of rank 1, against the oracle directly.

Checked: the packed gradient shard bit for bit; the rank's sum of squares;
the other ranks' partial sums the library computed from the model's generated
gradients, against torch's sums (every rank) and the oracle's (two ranks);
the fp32 master, m and v and the bf16 parameter shard at every element; and
the per-tensor parameters: every element the shard owns holds its bf16
parameter, every other element keeps its sentinel.
"""

import concurrent.futures as cf

import numpy as np
import pytest

from fsdp_sharded_mixed_zero_amd import synth
from oracle import step as O
from oracle.layout import build_layout
from other_ranks import check_library_partials, oracle_rank_partial, torch_rank_partials
from state_tiles import from_tiles
from tolerance import assert_bf16_param, assert_f32_state, assert_norm_close
from devbits import u16

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

PIECE = 1 << 23


def oracle_update(grad_bits, master, m, v, step, ohp, coef):
    """O.adamw_step over the whole shard, in pieces on host threads (the
    pieces are independent given the coefficient)."""
    n = grad_bits.size
    out = [np.empty(n, np.float32) for _ in range(3)] + [np.empty(n, np.uint16)]

    def one(lo):
        hi = min(n, lo + PIECE)
        res = O.adamw_step(grad_bits[lo:hi], master[lo:hi], m[lo:hi], v[lo:hi], step, ohp, coef)
        for o, r in zip(out, res):
            o[lo:hi] = r

    with cf.ThreadPoolExecutor(max_workers=8) as ex:
        list(ex.map(one, range(0, n, PIECE)))
    return out


WHOLE = [("gpt2-1.5b", 32, False), ("gpt-7.5b", 1, False), ("gpt2-1.5b", 63, True), ("gpt-7.5b", 1, True)]


@pytest.mark.parametrize("name,rank,flat", WHOLE, ids=[f"{n}-rank{r}{'-flat' if f else ''}" for n, r, f in WHOLE])
def test_whole_shard(name, rank, flat):
    from fsdp_sharded_mixed_zero_amd.rank import RankShard

    wl = synth.WORKLOADS[name]
    lay = build_layout(wl.sizes, wl.n_d, rank, wl.align)
    S = lay.shard
    print(f"\n[whole {name} rank {rank}{' flat' if flat else ''}] shard {S}, {len(lay.segments)} segments",
          flush=True)
    rs = RankShard(wl, rank=rank, fill=False, flat=flat)
    assert rs.shard == S
    chunks = []
    rs.fill_state(on_chunk=lambda lo, hi, p, m, v: chunks.append(
        (lo, p.cpu().numpy(), m.cpu().numpy(), v.cpu().numpy())))
    chunks.sort(key=lambda c: c[0])
    master, m, v = (np.concatenate([c[k] for c in chunks]) for k in (1, 2, 3))
    rs.fill_grads(wl.step)
    rs.fill_other_ranks()
    lib_others = rs.rank_sq.cpu().numpy().copy()
    others = torch_rank_partials(wl, S, wl.step, rank)
    check_library_partials(lib_others, others, rank)
    for r in ((rank - 1) % wl.n_d, (rank + 1) % wl.n_d):
        want_r = oracle_rank_partial(wl, r, wl.step)
        assert_norm_close(lib_others[r], want_r, f"rank {r} partial")
        assert_norm_close(others[r], want_r, f"rank {r} partial (torch)")
    grads = [None if t is None else u16(t) for t in rs.grads]
    params_before = [None if t is None else u16(t) for t in rs.params]
    torch.cuda.synchronize()

    rs.step(wl.step)
    torch.cuda.synchronize()
    print(f"[whole {name} rank {rank}] step done", flush=True)

    o_grad = O.pack(lay, grads)
    assert np.array_equal(u16(rs.grad_shard), o_grad), "gradient shard (packed, or the flat buffer's slice)"
    own = O.sqnorm(o_grad)
    rel = assert_norm_close(float(rs.rank_sq[rank].cpu()), own, "partial")
    partials = others.copy()
    partials[rank] = own
    coef = O.clip_coef(O.global_sqnorm(partials), wl.max_norm)
    ohp = O.AdamWHParams(lr=wl.lr, beta1=wl.beta1, beta2=wl.beta2, eps=wl.eps,
                         weight_decay=wl.weight_decay, max_norm=wl.max_norm)
    want = oracle_update(o_grad, master, m, v, wl.step, ohp, coef)
    g_master, g_m, g_v = from_tiles(rs.state.cpu().numpy(), S)
    g_param = u16(rs.param_shard)
    assert_f32_state(g_master, want[0], "master")
    um = assert_f32_state(g_m, want[1], "m", m)
    uv = assert_f32_state(g_v, want[2], "v", v)
    worst = assert_bf16_param(g_param, want[3], want[0], "param", g_master)
    same = int((g_param == want[3]).sum())

    # the per-tensor parameters: the shard's values at its tensor positions
    expect = O.unpack(lay, g_param, params_before)
    for i, t in enumerate(rs.params):
        if t is not None:
            assert np.array_equal(u16(t), expect[i]), f"tensor {i}"
    print(f"[whole {name} rank {rank}] every element checked: sqrt(G) rel {rel:.1e}, clip {coef:.6g}, "
          f"m/v within {um:.1f}/{uv:.1f} ulp of |old|+|new|, bf16 params {same} of {S} identical to the "
          f"oracle's (the rest 1 ulp: {worst <= 1})", flush=True)
    del rs
    torch.cuda.empty_cache()
