"""One data-parallel rank's shard held in device memory, and the local step
run through the C ABI: pack -> sum of squares -> clip + AdamW + bf16 cast ->
unpack.

The step is the rank-local part of a ZeRO-2/3 training step ("第 5 课：ZeRO 与
FSDP" section 3; notes on the ZeRO paper, sections 4.1-4.3). The collectives
around it (reduce-scatter of gradients before, all-gather of parameters
after, and the exchange of the ranks' partial sums of squares) are not run:
on one GPU, the other ranks' partial sums are inputs in ``rank_sq``.

Buffers are allocated once, as contiguous blocks ("ZeRO: Memory
Optimizations..." notes, section 3.2.3): per-tensor bf16 gradients and
parameters of every tensor the shard touches (whole tensors, as a model would
hold them), the flat bf16 gradient and parameter shards, the fp32 state
(master, m, v: one 12 B/element buffer in the library's tiled layout), the
ranks' partial sums and the sum-of-squares workspace. With ``bucket`` > 0
the shard is processed in pieces of that many elements, a constant-size
working set (notes, section 5.2). By default the unpack is fused into the
update (zero_adamw_step_unpack: AdamW also stores each bf16 parameter at its
tensor position); ``fused_unpack=False`` runs it as its own pass. With
``accum_steps`` = K > 1 the step runs K micro-batches of pack + fp32
accumulation, then the norm and AdamW on the fp32 accumulator ("第 5 课：ZeRO
与 FSDP" section 2, fp32 gradient accumulation, 4 extra bytes per shard
element).

With ``state_arrays=True`` the fp32 master, m and v are three separate
arrays, the form the pages hold the state in ("第 5 课：ZeRO 与 FSDP" section
2), updated by zero_adamw_step_arrays, with the unpack as its own pass.

With ``flat=True`` the rank holds the ZeRO-1 form (notes on the ZeRO paper,
section 4.1): the whole gradient and parameter sets live in two flat,
padded buffers, every tensor is a view into them, and the shard is the rank's
slice of each. The step then reads the gradient slice in place (no pack) and
AdamW writes the bf16 parameters straight into the flat parameter buffer (no
unpack): sum of squares -> clip + AdamW + bf16 cast.
"""

from __future__ import annotations

import torch

from . import synth, zero


def other_rank_slices(sizes, shard, rank):
    """For each tensor that reaches a shard other than ``rank``'s: (tensor
    index, [(other rank, first element, end element) of the tensor's part in
    that rank's shard]), in tensor order. RankShard.fill_other_ranks makes one
    zero_shard_sqnorm call per part."""
    out, off = [], 0
    for i, n in enumerate(sizes):
        if n > 0:
            r0, r1 = off // shard, (off + n - 1) // shard
            parts = [(r, max(off, r * shard) - off, min(off + n, (r + 1) * shard) - off)
                     for r in range(r0, r1 + 1) if r != rank]
            if parts:
                out.append((i, parts))
        off += n
    return out


class RankShard:
    def __init__(self, wl: synth.Workload, rank: int | None = None, device="cuda",
                 fill: bool = True, bucket: int | None = None, fused_norm: bool = True,
                 accum_steps: int = 1, flat: bool = False, fused_unpack: bool = True, streams: int = 2,
                 state_arrays: bool = False):
        self.wl = wl
        self.rank = wl.rank if rank is None else rank
        self.device = torch.device(device)
        self.layout = zero.zero_layout(wl.sizes, wl.n_d, self.rank, wl.align)
        self.info = self.layout.info
        self.segments = self.layout.segments
        S = self.info["shard"]
        self.shard = S
        self.real = S - (self.info["pad_end"] - self.info["pad_begin"])
        self.bucket = wl.bucket if bucket is None else bucket
        self.touched = sorted({s[0] for s in self.segments})
        n_t = len(wl.sizes)
        self.grads = [None] * n_t
        self.params = [None] * n_t
        dev = self.device
        self.flat = flat
        if state_arrays and (flat or accum_steps > 1):
            raise ValueError("three state arrays are used with the packed step without accumulation only")
        self.state_arrays = state_arrays
        if flat:
            if accum_steps > 1:
                raise ValueError("flat buffers are not combined with gradient accumulation here")
            P, lo = self.info["padded"], self.info["shard_begin"]
            self.grad_flat = torch.empty(P, dtype=torch.bfloat16, device=dev)
            self.grad_flat[self.info["psi"]:].zero_()          # padding reads as zero gradients
            self.param_flat = torch.full((P,), synth.SENTINEL, dtype=torch.int16,
                                         device=dev).view(torch.bfloat16)
            off = 0
            for i, n in enumerate(wl.sizes):
                if i in self.touched:
                    self.grads[i] = self.grad_flat[off:off + n]
                    self.params[i] = self.param_flat[off:off + n]
                off += n
            self.grad_shard = self.grad_flat[lo:lo + S]
            self.param_shard = self.param_flat[lo:lo + S]
        else:
            for i in self.touched:
                self.grads[i] = torch.empty(wl.sizes[i], dtype=torch.bfloat16, device=dev)
                self.params[i] = torch.full((wl.sizes[i],), synth.SENTINEL, dtype=torch.int16,
                                            device=dev).view(torch.bfloat16)
            self.grad_shard = torch.empty(S, dtype=torch.bfloat16, device=dev)
            self.param_shard = torch.empty(S, dtype=torch.bfloat16, device=dev)
        self.grad_ptrs = zero.pointer_array(self.grads)
        self.param_ptrs = zero.pointer_array(self.params)
        if state_arrays:
            self.state = None
            self.master, self.m, self.v = (torch.empty(S, dtype=torch.float32, device=dev) for _ in range(3))
        else:
            self.state = torch.empty(3 * S, dtype=torch.float32, device=dev)
        self.rank_sq = torch.zeros(wl.n_d, dtype=torch.float64, device=dev)
        self.fused_norm = fused_norm
        self.fused_unpack = fused_unpack and not flat and not state_arrays
        self.accum_steps = accum_steps
        self.acc = torch.empty(S, dtype=torch.float32, device=dev) if accum_steps > 1 else None
        ws = max(max(zero.zero_sqnorm_workspace_bytes(n),
                     zero.zero_pack_sqnorm_workspace_bytes(self.layout, b, n)) for b, n in self.pieces())
        self.workspace = torch.empty((ws + 7) // 8, dtype=torch.float64, device=dev)
        # buckets of the default step: each bucket's sum of squares in its own
        # slot, combined once (zero_sum_partials), and the buckets dealt out
        # to `streams` streams in turn
        n_pieces = len(self.pieces())
        self.bucketed = n_pieces > 1 and not flat and accum_steps == 1 and fused_norm
        self.bucket_sq = torch.zeros(n_pieces, dtype=torch.float64, device=dev) if n_pieces > 1 else None
        if self.bucketed:
            # each bucket's block partial sums in its own slice of one buffer
            caps = [zero.zero_pack_sqnorm_workspace_bytes(self.layout, b, n) // 8 for b, n in self.pieces()]
            self.part_off = [sum(caps[:k]) for k in range(n_pieces)]
            self.part_cap = caps
            self.bucket_partials = torch.empty(sum(caps), dtype=torch.float64, device=dev)
        self.n_streams = max(1, int(streams)) if self.bucketed else 1
        self.streams = [torch.cuda.Stream(device=dev) for _ in range(self.n_streams)] if self.n_streams > 1 else []
        if fill:
            self.fill_state()
            self.fill_grads(wl.step)
            self.fill_other_ranks()

    # ------------------------------------------------------------ inputs
    STATE_CHUNK = 1 << 26     # elements per generation chunk (a multiple of the state tile)

    def fill_state(self, on_chunk=None):
        """Draw master ~ N(0, master_std), m ~ N(0, m_std), v ~ |N(0, v_std)|
        (zeros where the std is 0 and on padding) chunk by chunk as three
        separate arrays, and import each chunk into the tiled state buffer
        (with ``state_arrays``, draw them straight into the three arrays).
        ``on_chunk(lo, hi, master, m, v)`` sees each chunk's separate arrays
        before the import."""
        wl, real, S = self.wl, self.real, self.shard
        assert self.STATE_CHUNK % zero.ZERO_STATE_TILE == 0
        for k, lo in enumerate(range(0, S, self.STATE_CHUNK)):
            hi = min(S, lo + self.STATE_CHUNK)
            n = hi - lo
            bufs = []
            for buf_id, std, absval in ((synth.MASTER, wl.master_std, False),
                                        (synth.EXP_AVG, wl.m_std, False),
                                        (synth.EXP_AVG_SQ, wl.v_std, True)):
                if self.state_arrays:
                    x = {synth.MASTER: self.master, synth.EXP_AVG: self.m, synth.EXP_AVG_SQ: self.v}[buf_id][lo:hi]
                    x.zero_()
                else:
                    x = torch.zeros(n, dtype=torch.float32, device=self.device)
                r = max(0, min(n, real - lo))
                if std > 0 and r > 0:
                    synth.device_normal_(x[:r], std, wl.seed, buf_id, abs_value=absval,
                                         salt=(self.rank << 12) + k)
                bufs.append(x)
            if on_chunk is not None:
                on_chunk(lo, hi, *bufs)
            if not self.state_arrays:
                zero.zero_state_import(*bufs, self.state[3 * lo:], n)
        torch.cuda.synchronize()

    def fill_grads(self, step):
        for i in self.touched:
            synth.device_grad_(self.grads[i], self.wl, step, salt=i)

    def fill_other_ranks(self, step=None):
        """The other ranks' partial sums of squares, each from its own slice of
        the model's gradients: every tensor that reaches another rank's shard
        is drawn on the device exactly as this rank draws its own tensors
        (synth.device_grad_, stream pieces by tensor index, gradients of
        ``step``, by default the workload's), and the sum of squares of each
        other rank's part of it is added into that rank's slot with
        zero_shard_sqnorm, in tensor order. Padding adds nothing. This rank's
        slot is left at 0 (the step computes it). The slots stand for what the
        all-reduce of the ranks' partial sums would deliver ("ZeRO-3 核心流程",
        pitfall 1: the clip norm covers every rank's slice). Set-up work, not
        part of a step: it draws the whole model's gradients once."""
        wl = self.wl
        step = wl.step if step is None else step
        self.rank_sq.zero_()
        slices = other_rank_slices(wl.sizes, self.shard, self.rank)
        if not slices:
            torch.cuda.synchronize(self.device)
            return
        longest = max(wl.sizes[i] for i, _ in slices)
        buf = torch.empty(longest, dtype=torch.bfloat16, device=self.device)
        ws = torch.empty((zero.zero_sqnorm_workspace_bytes(longest) + 7) // 8, dtype=torch.float64,
                         device=self.device)
        for i, parts in slices:
            g = synth.device_grad_(buf[:wl.sizes[i]], wl, step, salt=i)
            for r, a, b in parts:
                zero.zero_shard_sqnorm(g[a:], b - a, self.rank_sq[r:r + 1], True, ws)
        torch.cuda.synchronize(self.device)

    # --------------------------------------------------------------- step
    def hparams(self, step):
        wl = self.wl
        return zero.hparams(lr=wl.lr, beta1=wl.beta1, beta2=wl.beta2, eps=wl.eps,
                            weight_decay=wl.weight_decay, max_norm=wl.max_norm, step=step)

    def pieces(self):
        if self.bucket <= 0:
            return [(0, self.shard)]
        return [(b, min(self.bucket, self.shard - b)) for b in range(0, self.shard, self.bucket)]

    def step(self, step, stream=None, timing=None, events=None, before_micro=None, phases=None):
        """One local step on ``stream`` (a torch stream or a raw handle; by
        default the current stream). ``timing``: optional dict; each phase
        ("pack_sqnorm" or "pack" and "sqnorm", "adamw", "unpack") gets a list
        of (start, end) CUDA events recorded around its launches on that stream, taken
        from the iterator ``events`` (pre-created, so timing adds no event
        creation to the step); ``phases`` limits the timed phases (each event
        record costs GPU time between launches). A bucketed default step times
        each phase as a whole (its buckets overlap on several streams).
        ``before_micro(mb)`` runs before each micro-batch when accumulating (to
        refill the gradients)."""
        hp = self.hparams(step)
        own = self.rank_sq[self.rank:self.rank + 1]
        pieces = self.pieces()
        if self.bucketed:
            self._step_buckets(hp, own, pieces, torch.cuda.current_stream() if stream is None else stream,
                               timing, events, phases)
            return
        if stream is None:
            stream = torch.cuda.current_stream()
        on = torch.cuda.ExternalStream(stream) if isinstance(stream, int) else stream   # events go here
        stream = on.cuda_stream

        def mark(phase, fn):
            if timing is None or (phases is not None and phase not in phases):
                fn()
                return
            e0 = next(events) if events is not None else torch.cuda.Event(enable_timing=True)
            e1 = next(events) if events is not None else torch.cuda.Event(enable_timing=True)
            e0.record(on)
            fn()
            e1.record(on)
            timing.setdefault(phase, []).append((e0, e1))

        if self.accum_steps > 1:
            self._step_accumulated(hp, own, pieces, stream, mark, before_micro)
            return
        if self.flat:
            self._step_flat(hp, own, pieces, stream, mark)
            return
        for k, (b, n) in enumerate(pieces):
            if self.fused_norm:
                mark("pack_sqnorm", lambda: zero.zero_pack_grads_sqnorm(
                    self.layout, self.grad_ptrs, self.grad_shard, b, n, own, k > 0, self.workspace,
                    stream=stream))
                continue
            mark("pack", lambda: zero.zero_pack_grads(self.layout, self.grad_ptrs, self.grad_shard, b, n,
                                                      stream))
            mark("sqnorm", lambda: zero.zero_shard_sqnorm(self.grad_shard[b:], n, own, k > 0,
                                                          self.workspace, stream=stream))
        for b, n in pieces:
            if self.fused_unpack:
                mark("adamw", lambda: zero.zero_adamw_step_unpack(
                    self.grad_shard, self.state, self.param_shard, self.shard, b, n, hp, self.rank_sq,
                    self.wl.n_d, self.layout, self.param_ptrs, stream))
                continue
            mark("adamw", lambda: self._adamw(b, n, hp, stream))
            mark("unpack", lambda: zero.zero_unpack_params(self.layout, self.param_shard, self.param_ptrs,
                                                          b, n, stream))

    def _adamw(self, b, n, hp, stream):
        """The update of shard elements [b, b+n) without the unpack: over the
        tiled state, or over the three state arrays (offset pointers)."""
        if self.state_arrays:
            # addresses read at each call: the arrays may be rebound (a restored checkpoint)
            zero.zero_adamw_step_arrays(self.grad_shard.data_ptr() + 2 * b, self.master.data_ptr() + 4 * b,
                                        self.m.data_ptr() + 4 * b, self.v.data_ptr() + 4 * b,
                                        self.param_shard.data_ptr() + 2 * b, n, hp, self.rank_sq, self.wl.n_d,
                                        stream)
            return
        zero.zero_adamw_step(self.grad_shard, self.state, self.param_shard, self.shard, b, n, hp, self.rank_sq,
                             self.wl.n_d, stream)

    def pack_norm_buckets(self, own, stream):
        """Pack + sum of squares of every bucket on the step's streams in turn,
        each bucket's block partial sums in its own slice of bucket_partials;
        then, on ``stream`` once all are done, one launch reduces every slice
        into the bucket's slot (zero_sum_partials_rows) and ``own`` = the slots
        added in a fixed order. Each bucket's sum is the one
        zero_pack_grads_sqnorm would give, and the result does not depend on
        the number of streams."""
        pieces = self.pieces()
        main = torch.cuda.ExternalStream(stream) if isinstance(stream, int) else stream
        for st in self.streams:
            st.wait_stream(main)
        counts = []
        for k, (b, n) in enumerate(pieces):
            st = self.streams[k % self.n_streams].cuda_stream if self.streams else main.cuda_stream
            counts.append(zero.zero_pack_grads_sqnorm_partials(
                self.layout, self.grad_ptrs, self.grad_shard, b, n, self.bucket_partials[self.part_off[k]:],
                8 * self.part_cap[k], stream=st))
        for st in self.streams:
            main.wait_stream(st)
        zero.zero_sum_partials_rows(self.bucket_partials, self.part_off, counts, self.bucket_sq, False,
                                    stream=main.cuda_stream)
        zero.zero_sum_partials(self.bucket_sq, len(pieces), own, False, stream=main.cuda_stream)

    def _step_buckets(self, hp, own, pieces, stream, timing, events, phases):
        """The default step over buckets: the packs on the streams in turn and
        the combine, then the updates with the unpack fused on the streams in
        turn (or the updates, then the unpacks). With timing, one event pair
        spans each phase on the calling stream (the buckets of a phase overlap
        on the streams)."""
        main = torch.cuda.ExternalStream(stream) if isinstance(stream, int) else stream

        def timed(phase, fn):
            if timing is None or (phases is not None and phase not in phases):
                fn()
                return
            e0 = next(events) if events is not None else torch.cuda.Event(enable_timing=True)
            e1 = next(events) if events is not None else torch.cuda.Event(enable_timing=True)
            e0.record(main)
            fn()
            e1.record(main)
            timing.setdefault(phase, []).append((e0, e1))

        def on_streams(call):
            for st in self.streams:
                st.wait_stream(main)
            for k, (b, n) in enumerate(pieces):
                call(b, n, self.streams[k % self.n_streams].cuda_stream if self.streams else main.cuda_stream)
            for st in self.streams:
                main.wait_stream(st)

        timed("pack_sqnorm", lambda: self.pack_norm_buckets(own, main))
        if self.fused_unpack:
            timed("adamw", lambda: on_streams(lambda b, n, st: zero.zero_adamw_step_unpack(
                self.grad_shard, self.state, self.param_shard, self.shard, b, n, hp, self.rank_sq, self.wl.n_d,
                self.layout, self.param_ptrs, st)))
        else:
            timed("adamw", lambda: on_streams(lambda b, n, st: self._adamw(b, n, hp, st)))
            timed("unpack", lambda: on_streams(lambda b, n, st: zero.zero_unpack_params(
                self.layout, self.param_shard, self.param_ptrs, b, n, st)))

    def _step_flat(self, hp, own, pieces, stream, mark):
        for k, (b, n) in enumerate(pieces):
            mark("sqnorm", lambda: zero.zero_shard_sqnorm(self.grad_shard[b:], n, own, k > 0, self.workspace,
                                                          stream=stream))
        for b, n in pieces:
            mark("adamw", lambda: zero.zero_adamw_step(
                self.grad_shard, self.state, self.param_shard, self.shard, b, n, hp, self.rank_sq,
                self.wl.n_d, stream))

    def _step_accumulated(self, hp, own, pieces, stream, mark, before_micro):
        for mb in range(self.accum_steps):
            if before_micro is not None:
                before_micro(mb)
            for b, n in pieces:
                mark("pack", lambda: zero.zero_pack_grads(self.layout, self.grad_ptrs, self.grad_shard, b, n,
                                                          stream))
                mark("accumulate", lambda: zero.zero_accumulate_grads(self.grad_shard[b:], self.acc[b:], n,
                                                                      mb == 0, stream))
        for k, (b, n) in enumerate(pieces):
            mark("sqnorm", lambda: zero.zero_shard_sqnorm_f32(self.acc[b:], n, own, k > 0, self.workspace,
                                                              stream=stream))
        for b, n in pieces:
            if self.fused_unpack:
                mark("adamw", lambda: zero.zero_adamw_step_f32grad_unpack(
                    self.acc, self.state, self.param_shard, self.shard, b, n, hp, self.rank_sq,
                    self.wl.n_d, self.layout, self.param_ptrs, stream))
                continue
            mark("adamw", lambda: zero.zero_adamw_step_f32grad(
                self.acc, self.state, self.param_shard, self.shard, b, n, hp, self.rank_sq,
                self.wl.n_d, stream))
            mark("unpack", lambda: zero.zero_unpack_params(self.layout, self.param_shard, self.param_ptrs,
                                                          b, n, stream))

    def bytes_per_step(self):
        """Algorithmic HBM bytes of one step: pack 4, sum of squares 2 (0 when
        fused into pack), AdamW 28 and unpack 4 bytes per shard element (pack
        writes only 2 on padding, unpack moves nothing there). Accumulating K
        micro-batches: K packs, accumulation 6 then 10 bytes per element, an
        fp32 norm (4) and AdamW on fp32 gradients (30). Flat buffers: the sum
        of squares (2) and AdamW (28) only. With the unpack fused into AdamW,
        AdamW also writes 2 bytes per real element to the tensors and there is
        no unpack pass."""
        if self.flat:
            return {"sqnorm": 2 * self.shard, "adamw": 28 * self.shard}
        pad = self.shard - self.real
        pack = 4 * self.real + 2 * pad
        if self.accum_steps > 1:
            K, S = self.accum_steps, self.shard
            # accumulate: 2 + 4 bytes for the first micro-batch, 2 + 4 + 4 after
            out = {"pack": K * pack, "accumulate": 6 * S + (K - 1) * 10 * S, "sqnorm": 4 * S,
                   "adamw": 30 * S}
        else:
            out = {"adamw": 28 * self.shard}
            if self.fused_norm:
                out["pack_sqnorm"] = pack
            else:
                out.update(pack=pack, sqnorm=2 * self.shard)
        if self.fused_unpack:
            out["adamw"] += 2 * self.real
        else:
            out["unpack"] = 4 * self.real
        return out


class OffloadRank(RankShard):
    """ZeRO-Offload (the mlqm.cn article's ZeRO-Offload section): the fp32
    optimizer state lives in host memory and the host cores run AdamW; the GPU
    keeps the bf16 gradient and parameter shards and runs pack + norm and
    unpack. Per bucket, the gradient slice goes device->host into a pinned
    staging slot, the host updates it (zero_cpu_adamw_step), and the bf16
    parameters come back host->device before the GPU unpacks them. A ring of
    ``slots`` staging buffers and two copy streams let the PCIe copies of one
    bucket overlap the host update of another.

    Shards without buckets are staged in pieces of ``bucket`` elements, ramping
    up from 1/8 of that size at the start and down again at the end: the
    first download and the last upload are the parts nothing overlaps. Pack
    and the norm keep the uniform ``pieces()``, so the norm's accumulation
    order (and every result) is that of the all-GPU step. The views, events
    and slots of every staged piece are made once, so the host thread, which
    also runs a share of the update, spends little time between updates."""

    def __init__(self, wl: synth.Workload, rank: int | None = None, device="cuda", fill: bool = True,
                 bucket: int = 1 << 24, slots: int = 3, threads: int | None = None):
        import numpy as np
        import os

        super().__init__(wl, rank, device, fill=fill, bucket=wl.bucket or bucket, fused_norm=True,
                         fused_unpack=False)
        S = self.shard
        self.h_state = np.empty(3 * S, np.float32)
        if fill:
            self.move_state_to_host()
        self.threads = threads if threads is not None else int(
            os.environ.get("ZERO_CPU_THREADS", os.environ.get("OMP_NUM_THREADS", "0")) or 0)
        staged = self.transfer_pieces()
        piece = max(n for _, n in staged)
        self.stage_g = [torch.empty(piece, dtype=torch.int16, pin_memory=True) for _ in range(slots)]
        self.stage_p = [torch.empty(piece, dtype=torch.int16, pin_memory=True) for _ in range(slots)]
        self.h_rank_sq = torch.zeros(wl.n_d, dtype=torch.float64, pin_memory=True)
        self.d2h = torch.cuda.Stream(device=self.device)
        self.h2d = torch.cuda.Stream(device=self.device)
        self.host_seconds = 0.0
        g16, p16 = self.grad_shard.view(torch.int16), self.param_shard.view(torch.int16)
        # per staged piece: begin, count, device gradient and parameter views,
        # staging views, and the events marking its download and upload
        self.plan = [(b, n, g16[b:b + n], p16[b:b + n], self.stage_g[i % slots][:n], self.stage_p[i % slots][:n],
                      torch.cuda.Event(), torch.cuda.Event()) for i, (b, n) in enumerate(staged)]
        self.packed = torch.cuda.Event()
        self.sums_ready = torch.cuda.Event()

    def transfer_pieces(self):
        """The (begin, count) pieces staged through host memory."""
        pieces = self.pieces()
        if self.wl.bucket or len(pieces) < 4:
            return pieces
        B = self.bucket
        ramp = [B >> 3, B >> 2, B >> 1]
        mid = self.shard - 2 * sum(ramp)
        sizes = ramp + [B] * (mid // B) + ([mid % B] if mid % B else []) + ramp[::-1]
        out, b = [], 0
        for n in sizes:
            out.append((b, n))
            b += n
        return out

    def move_state_to_host(self, piece=1 << 26):
        """Copy the device state (drawn by fill_state) into host memory and
        free it on the device: from here on the GPU holds no optimizer state.
        With fill=False, call fill_state() and then this."""
        for lo in range(0, 3 * self.shard, piece):
            hi = min(3 * self.shard, lo + piece)
            self.h_state[lo:hi] = self.state[lo:hi].cpu().numpy()
        self.state = None
        torch.cuda.empty_cache()

    def step(self, step, stream=None, timing=None, events=None, before_micro=None, phases=None):
        import time

        hp = self.hparams(step)
        cs = torch.cuda.current_stream()
        stream = cs.cuda_stream
        own = self.rank_sq[self.rank:self.rank + 1]
        if self.bucketed:          # the same buckets and combine as the all-GPU step
            self.pack_norm_buckets(own, cs)
        else:
            zero.zero_pack_grads_sqnorm(self.layout, self.grad_ptrs, self.grad_shard, 0, self.shard, own, False,
                                        self.workspace, stream=stream)
        self.packed.record(cs)
        self.d2h.wait_event(self.packed)
        plan, R = self.plan, len(self.stage_g)
        with torch.cuda.stream(self.d2h):
            self.h_rank_sq.copy_(self.rank_sq, non_blocking=True)
            self.sums_ready.record(self.d2h)
            for _, _, g_dev, _, g_stage, _, got, _ in plan[:R]:
                g_stage.copy_(g_dev, non_blocking=True)
                got.record(self.d2h)
        self.sums_ready.synchronize()
        for i, (b, n, _, p_dev, g_stage, p_stage, got, sent) in enumerate(plan):
            got.synchronize()
            if i >= R:
                plan[i - R][7].synchronize()      # the staging slot's previous upload has left
            t0 = time.perf_counter()
            zero.zero_cpu_adamw_step(g_stage, self.h_state, p_stage, self.shard, b, n, hp, self.h_rank_sq,
                                     self.wl.n_d, self.threads)
            self.host_seconds += time.perf_counter() - t0
            with torch.cuda.stream(self.h2d):
                p_dev.copy_(p_stage, non_blocking=True)
                sent.record(self.h2d)
            if i + R < len(plan):                 # the next download into the slot just read
                nxt = plan[i + R]
                with torch.cuda.stream(self.d2h):
                    nxt[4].copy_(nxt[2], non_blocking=True)
                    nxt[6].record(self.d2h)
            cs.wait_event(sent)
            zero.zero_unpack_params(self.layout, self.param_shard, self.param_ptrs, b, n, stream)
        for entry in plan[-R:]:
            entry[7].synchronize()                # staging slots free for the next step

    def pcie_bytes_per_step(self):
        """Bytes the step moves over PCIe: the bf16 gradients down, the bf16
        parameters up, the partial sums."""
        return 2 * self.shard + 2 * self.shard + 8 * self.wl.n_d
