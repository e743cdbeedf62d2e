"""Partitioner oracle: per-tensor size list -> flat buffer -> one rank's shard.

Sources (pages, not code):
  * "ZeRO: Memory Optimizations Toward Training Trillion Parameter Models"
    (notes), section 2.2 (temporary buffers) and section 5.2 (C_B): the tensors
    are flattened and fused into one contiguous buffer.
  * Same notes, section 4.1 (P_os): with data-parallel degree N_d, the state is
    split into N_d equal parts and rank i owns part i.
  * "第 5 课：ZeRO 与 FSDP", section 2: each rank keeps a 1/N_d slice.

Readings where the pages are silent: tensors are concatenated in list order
with no gaps between them; the flat buffer is padded at the tail only, up to
P = ceil(Psi / (N_d*A)) * N_d*A elements, so every rank owns S = P / N_d
elements and every shard starts on a multiple of A elements; zero-size
tensors own no elements and produce no segment.
"""

from __future__ import annotations

from dataclasses import dataclass, field


class LayoutError(ValueError):
    """Invalid partitioner arguments."""


@dataclass(frozen=True)
class Segment:
    """One run of consecutive elements of tensor ``tensor`` that lands in the
    rank's shard: tensor elements [src_off, src_off+length) map to shard
    elements [dst_off, dst_off+length)."""

    tensor: int
    src_off: int
    dst_off: int
    length: int


@dataclass(frozen=True)
class Layout:
    sizes: tuple
    n_d: int
    rank: int
    align: int
    offsets: tuple          # flat offset of each tensor
    psi: int                # real elements (sum of sizes)
    padded: int             # P
    shard: int              # S
    shard_begin: int        # r * S, flat coordinates
    segments: tuple = field(default_factory=tuple)
    pad_begin: int = 0      # shard coordinates; [pad_begin, pad_end) is padding
    pad_end: int = 0

    @property
    def real_elems(self) -> int:
        return self.shard - (self.pad_end - self.pad_begin)


def build_layout(sizes, n_d: int, rank: int, align: int = 128) -> Layout:
    """Flatten ``sizes`` in order, pad the tail, and cut out rank ``rank``'s
    1/N_d slice."""
    sizes = tuple(int(s) for s in sizes)
    if n_d <= 0:
        raise LayoutError("n_d must be positive")
    if not 0 <= rank < n_d:
        raise LayoutError("rank must lie in [0, n_d)")
    if align <= 0:
        raise LayoutError("align must be positive")
    if any(s < 0 for s in sizes):
        raise LayoutError("tensor sizes must be non-negative")

    offsets = []
    running = 0
    for s in sizes:
        offsets.append(running)
        running += s
    psi = running
    if psi == 0:
        raise LayoutError("the model has no parameters")

    quantum = n_d * align
    padded = -(-psi // quantum) * quantum
    shard = padded // n_d
    lo_rank = rank * shard
    hi_rank = lo_rank + shard

    segments = []
    for i, (off, n) in enumerate(zip(offsets, sizes)):
        lo = max(off, lo_rank)
        hi = min(off + n, hi_rank)
        if lo < hi:
            segments.append(Segment(i, lo - off, lo - lo_rank, hi - lo))

    pad_lo = max(psi, lo_rank)
    if pad_lo < hi_rank:
        pad_begin, pad_end = pad_lo - lo_rank, shard
    else:
        pad_begin = pad_end = shard

    return Layout(sizes, n_d, rank, align, tuple(offsets), psi, padded, shard,
                  lo_rank, tuple(segments), pad_begin, pad_end)


def buckets(begin: int, count: int, bucket: int):
    """Split the shard range [begin, begin+count) into consecutive pieces of at
    most ``bucket`` elements (constant-size buffers, notes section 5.2)."""
    if bucket <= 0:
        raise LayoutError("bucket must be positive")
    out = []
    pos = begin
    end = begin + count
    while pos < end:
        n = min(bucket, end - pos)
        out.append((pos, n))
        pos += n
    return out
