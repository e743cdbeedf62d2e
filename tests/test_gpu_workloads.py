"""Parity at the workloads' full sizes, in the launch configuration the
benchmark times (RankShard.step: whole shard, or 5e7-element buckets for the
70B shard). The oracle checks element by element a window across every
tensor seam in the shard, every bucket seam and every seam between update
launches, plus random ranges (every element of the GPT-2 and 7.5B shards is
checked in test_gpu_whole_shard.py); the rank's whole-shard sum of squares is
recomputed by the oracle over the full shard, packed by the oracle from the
per-tensor gradients. The other ranks' partial sums come from the model's
generated gradients: the library's (RankShard.fill_other_ranks) are checked
against torch's, and the oracle's global norm takes torch's.

Per workload:
  * pack: sampled shard ranges equal the oracle's pack of the same ranges of
    the per-tensor gradients (bit-exact);
  * sum of squares: the rank's partial equals the oracle's over the whole
    shard (sqrt within 1e-5, and reported), bit-identical when repeated;
  * AdamW: sampled ranges of the tiled state and the bf16 shard equal the
    oracle's update of the same ranges (inputs captured before the step from
    the input generator, the global norm from the oracle's partial plus the
    same other-rank inputs);
  * unpack: the sampled ranges land at the oracle layout's tensor positions,
    and tensor bytes outside the rank's segments keep their sentinel.
"""

import concurrent.futures as cf

import numpy as np
import pytest

from fsdp_sharded_mixed_zero_amd import synth, zero
from oracle import step as O
from oracle.layout import build_layout
from state_tiles import state_range
from tolerance import assert_bf16_param, assert_f32_state, assert_norm_close
from devbits import u16

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

SAMPLE = 1 << 16


class DeviceTensor:
    """Slices of a device bf16 tensor fetched on demand, for the oracle's pack."""

    def __init__(self, t):
        self.t = t

    def __getitem__(self, sl):
        return u16(self.t[sl])


SEAM = 4096                # elements of a window across a seam


def update_launch_seams(S, bucket):
    """Where the update's launches meet inside a call (ranges longer than
    ZERO_ADAMW_LAUNCH_ELEMS are cut into equal launches of whole state
    tiles)."""
    out = []
    for b0 in (range(0, S, bucket) if bucket else [0]):
        n = min(bucket, S - b0) if bucket else S
        k = -(-n // zero.ZERO_ADAMW_LAUNCH_ELEMS)
        chunk = -(-(-(-n // k)) // zero.ZERO_STATE_TILE) * zero.ZERO_STATE_TILE
        out += [b0 + j for j in range(chunk, n, chunk)]
    return out


def sample_ranges(lay, wl, rng, bucket=None):
    """Random windows of SAMPLE elements, the shard's ends, and a SEAM-element
    window (at an odd offset) across every tensor seam, bucket seam and
    update-launch seam."""
    S = lay.shard
    bucket = wl.bucket if bucket is None else bucket
    c = min(SAMPLE, S)
    wins = {(0, c), (S - c, c)}
    for _ in range(4):
        wins.add((int(rng.integers(0, S - c + 1)), c))
    w = min(SEAM, S)
    seams = [seg.dst_off for seg in lay.segments[1:]]
    if bucket:
        seams += list(range(bucket, S, bucket))
    seams += update_launch_seams(S, bucket)
    for x in seams:
        wins.add((min(max(0, x - w // 2 - 3), S - w), w))
    # merge overlapping windows (a range is compared as one piece)
    out = []
    for b, n in sorted(wins):
        if out and b <= out[-1][0] + out[-1][1]:
            lo = out[-1][0]
            out[-1] = (lo, max(out[-1][0] + out[-1][1], b + n) - lo)
        else:
            out.append((b, n))
    return out


_TORCH_OTHERS = {}


def other_partials(wl, S, rank):
    """torch's partial sums of the other ranks (computed once per workload)."""
    from other_ranks import torch_rank_partials
    key = (wl.name, rank, wl.step)
    if key not in _TORCH_OTHERS:
        _TORCH_OTHERS[key] = torch_rank_partials(wl, S, wl.step, rank)
    return _TORCH_OTHERS[key]


def oracle_partial(lay, tensors, S):
    """The oracle's sum of squares of the rank's whole shard: the oracle packs
    it from the per-tensor gradients (the inputs, fetched in pieces) and sums
    each piece's squares; the pieces' sums are added in order."""
    piece = 1 << 27
    bounds = [(lo, min(S, lo + piece)) for lo in range(0, S, piece)]

    def one(b):
        return O.sqnorm(O.pack(lay, tensors, b[0], b[1] - b[0]))

    with cf.ThreadPoolExecutor(max_workers=8) as ex:
        parts = list(ex.map(one, bounds))
    total = 0.0
    for p in parts:
        total += p
    return total


# (workload, fused norm, bucket, fused unpack): bucket None keeps the
# workload's own bucketing. The 70B shard in one piece is updated in 65
# launches of equal length (at most 2^27 elements each); the fused pack then
# covers 8.6e9 elements in two launches (91 pieces, 64 per launch) and its
# final sum adds ~1e6 block partials. The 7B shard's 1.68e9 elements take 13
# update launches.
FULL_SIZE = ([(n, f, None, True) for n in ("gpt2-1.5b", "gpt-7.5b", "llama-7b", "llama-70b") for f in (True, False)]
             + [("llama-70b", True, 0, True)]
             + [(n, True, None, False) for n in ("gpt2-1.5b", "gpt-7.5b", "llama-7b", "llama-70b")])


@pytest.mark.parametrize("name,fused_norm,bucket,fused_unpack", FULL_SIZE,
                         ids=[f"{n}-{'fused' if f else 'separate'}-norm{'-one-piece' if b == 0 else ''}"
                              f"{'' if u else '-separate-unpack'}" for n, f, b, u in FULL_SIZE])
def test_workload_full_size(name, fused_norm, bucket, fused_unpack):
    import dataclasses

    from fsdp_sharded_mixed_zero_amd.rank import RankShard

    wl = synth.WORKLOADS[name]
    if bucket is not None:
        wl = dataclasses.replace(wl, bucket=bucket)
    lay = build_layout(wl.sizes, wl.n_d, wl.rank, wl.align)
    S = lay.shard
    rng = np.random.default_rng(len(wl.sizes))
    ranges = sample_ranges(lay, wl, rng)
    print(f"\n[{name}] shard {S}, {len(lay.segments)} segments, bucket {wl.bucket}, "
          f"{len(ranges)} sampled ranges, fused norm {fused_norm}", flush=True)

    rs = RankShard(wl, fill=False, fused_norm=fused_norm, fused_unpack=fused_unpack)
    assert rs.shard == S
    assert rs.segments == [(s.tensor, s.src_off, s.dst_off, s.length) for s in lay.segments]
    before = {}

    def capture(lo, hi, master, m, v):
        for b, c in ranges:
            a, z = max(b, lo), min(b + c, hi)
            if a < z:
                before.setdefault(b, []).append((a, master[a - lo:z - lo].cpu().numpy(),
                                                 m[a - lo:z - lo].cpu().numpy(),
                                                 v[a - lo:z - lo].cpu().numpy()))

    rs.fill_state(on_chunk=capture)
    rs.fill_grads(wl.step)
    rs.fill_other_ranks()
    from other_ranks import check_library_partials
    others = other_partials(wl, S, rs.rank)
    check_library_partials(rs.rank_sq.cpu().numpy(), others, rs.rank)
    lazy = [None if t is None else DeviceTensor(t) for t in rs.grads]
    grads_before = {b: O.pack(lay, lazy, b, c) for b, c in ranges}
    torch.cuda.synchronize()

    rs.step(wl.step)
    torch.cuda.synchronize()
    print(f"[{name}] step done", flush=True)

    # pack: bit-exact on the sampled ranges
    for b, c in ranges:
        assert np.array_equal(u16(rs.grad_shard[b:b + c]), grads_before[b]), (name, b)

    # sum of squares over the whole shard
    got = float(rs.rank_sq[rs.rank].cpu())
    want = oracle_partial(lay, lazy, S)
    rel = assert_norm_close(got, want, f"{name} partial")
    print(f"[{name}] partial sum of squares: relative error of sqrt {rel:.2e}", flush=True)
    again = torch.zeros(1, dtype=torch.float64, device="cuda")
    if rs.bucketed:                                      # bucket slots, then the fixed-order combine
        rs.pack_norm_buckets(again, torch.cuda.current_stream())
    else:
        for k, (b, n) in enumerate(rs.pieces()):
            if fused_norm:
                zero.zero_pack_grads_sqnorm(rs.layout, rs.grads, rs.grad_shard, b, n, again, k > 0,
                                            rs.workspace)
            else:
                zero.zero_shard_sqnorm(rs.grad_shard[b:], n, again, k > 0, rs.workspace)
    assert float(again.cpu()) == got                     # bit-identical repeat

    # AdamW on the sampled ranges
    partials = others.copy()
    partials[rs.rank] = want
    coef = O.clip_coef(O.global_sqnorm(partials), wl.max_norm)
    ohp = O.AdamWHParams(lr=wl.lr, beta1=wl.beta1, beta2=wl.beta2, eps=wl.eps,
                         weight_decay=wl.weight_decay, max_norm=wl.max_norm)
    flat_state = rs.state
    for b, c in ranges:
        pieces = sorted(before[b], key=lambda x: x[0])
        master = np.concatenate([p[1] for p in pieces])
        m = np.concatenate([p[2] for p in pieces])
        v = np.concatenate([p[3] for p in pieces])
        assert master.size == c
        o_master, o_m, o_v, o_param = O.adamw_step(grads_before[b], master, m, v, wl.step, ohp, coef)
        g_master, g_m, g_v = state_range(lambda a, z: flat_state[a:z].cpu().numpy(), S, b, c)
        assert_f32_state(g_master, o_master, f"{name} master @{b}")
        assert_f32_state(g_m, o_m, f"{name} m @{b}", m)
        assert_f32_state(g_v, o_v, f"{name} v @{b}", v)
        assert_bf16_param(u16(rs.param_shard[b:b + c]), o_param, o_master, f"{name} param @{b}", g_master)
        # unpack: the range lands where the oracle layout maps it
        for seg in lay.segments:
            lo, hi = max(seg.dst_off, b), min(seg.dst_off + seg.length, b + c)
            if lo < hi:
                s0 = seg.src_off + (lo - seg.dst_off)
                placed = u16(rs.params[seg.tensor][s0:s0 + (hi - lo)])
                assert np.array_equal(placed, u16(rs.param_shard[lo:hi])), (name, seg.tensor, lo)

    # tensor bytes outside the rank's segments keep the sentinel
    for seg in (lay.segments[0], lay.segments[-1]):
        t = rs.params[seg.tensor]
        inside = seg.length
        outside = int((t.view(torch.int16) == synth.SENTINEL).sum())
        assert outside == t.numel() - inside + int(
            (t.view(torch.int16)[seg.src_off:seg.src_off + seg.length] == synth.SENTINEL).sum())
    print(f"[{name}] clip coefficient {coef:.6g}; checks passed", flush=True)
    del rs
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name,micro", [("gpt2-1.5b", 3), ("gpt-7.5b", 4)])
def test_workload_grad_accumulation(name, micro):
    """fp32 gradient accumulation over several micro-batches at full size:
    the whole accumulator bit-exact with the oracle's, the fp32 norm against
    the oracle's, AdamW on sampled ranges."""
    from fsdp_sharded_mixed_zero_amd.rank import RankShard

    wl = synth.WORKLOADS[name]
    lay = build_layout(wl.sizes, wl.n_d, wl.rank, wl.align)
    S = lay.shard
    rng = np.random.default_rng(7 + len(wl.sizes))
    ranges = sample_ranges(lay, wl, rng)
    print(f"\n[{name} x{micro}] shard {S}, fp32 accumulation over {micro} micro-batches", flush=True)
    rs = RankShard(wl, fill=False, accum_steps=micro)
    before = {}

    def capture(lo, hi, master, m, v):
        for b, c in ranges:
            a, z = max(b, lo), min(b + c, hi)
            if a < z:
                before.setdefault(b, []).append((a, master[a - lo:z - lo].cpu().numpy(),
                                                 m[a - lo:z - lo].cpu().numpy(),
                                                 v[a - lo:z - lo].cpu().numpy()))

    rs.fill_state(on_chunk=capture)
    rs.fill_other_ranks()
    from other_ranks import check_library_partials
    others = other_partials(wl, S, rs.rank)
    check_library_partials(rs.rank_sq.cpu().numpy(), others, rs.rank)
    lazy = [None if t is None else DeviceTensor(t) for t in rs.grads]
    o_acc = [None]

    def before_micro(mb):
        rs.fill_grads(100 + mb)                       # a different gradient per micro-batch
        torch.cuda.synchronize()
        o_acc[0] = O.accumulate(o_acc[0], O.pack(lay, lazy, 0, S), first=(mb == 0))

    rs.step(wl.step, before_micro=before_micro)
    torch.cuda.synchronize()
    acc = o_acc[0]
    assert np.array_equal(rs.acc.cpu().numpy().view(np.uint32), acc.view(np.uint32))
    got = float(rs.rank_sq[rs.rank].cpu())
    want = O.sqnorm_f32(acc)
    rel = assert_norm_close(got, want, f"{name} fp32 partial")
    print(f"[{name} x{micro}] accumulator bit-exact; partial relative error {rel:.2e}", flush=True)
    partials = others.copy()
    partials[rs.rank] = want
    coef = O.clip_coef(O.global_sqnorm(partials), wl.max_norm)
    ohp = O.AdamWHParams(lr=wl.lr, beta1=wl.beta1, beta2=wl.beta2, eps=wl.eps,
                         weight_decay=wl.weight_decay, max_norm=wl.max_norm)
    for b, c in ranges:
        pieces = sorted(before[b], key=lambda x: x[0])
        master = np.concatenate([p[1] for p in pieces])
        m = np.concatenate([p[2] for p in pieces])
        v = np.concatenate([p[3] for p in pieces])
        o_master, o_m, o_v, o_param = O.adamw_step_f32grad(acc[b:b + c], master, m, v, wl.step, ohp, coef)
        g_master, g_m, g_v = state_range(lambda a, z: rs.state[a:z].cpu().numpy(), S, b, c)
        assert_f32_state(g_master, o_master, f"{name} master @{b}")
        assert_f32_state(g_m, o_m, f"{name} m @{b}", m)
        assert_f32_state(g_v, o_v, f"{name} v @{b}", v)
        assert_bf16_param(u16(rs.param_shard[b:b + c]), o_param, o_master, f"{name} param @{b}", g_master)
    print(f"[{name} x{micro}] clip coefficient {coef:.6g}; checks passed", flush=True)
    del rs
    torch.cuda.empty_cache()
