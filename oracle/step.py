"""One rank's local optimizer step: pack, sum of squares, clip, AdamW, bf16
cast, unpack. Plain numpy, float64 arithmetic.

Sources (pages, not code):
  * "第 5 课：ZeRO 与 FSDP", section 3 (ZeRO-1/2 step 2): each rank updates its
    own 1/N_d slice of the fp32 optimizer state and master weights with its own
    gradient slice and converts the result to BF16 in place; the all-gather
    then reassembles the full parameters. Section 2: K = 12 bytes of state per
    parameter (fp32 master, m, v). Section 3 (ZeRO-3): the optimizer update
    needs no communication.
  * "ZeRO: Memory Optimizations Toward Training Trillion Parameter Models"
    (notes): section 2.2 (tensors are flattened and fused into a contiguous
    buffer for the gradient norm), section 3.2.3 (tensors are copied into
    pre-allocated contiguous blocks as they are produced), section 4.1 (rank i
    reads only its slice of the gradient and updates only its slice; an
    all-gather then restores the full 16-bit parameters).
  * "ZeRO-3 核心流程：把参数也切开的那一档", pitfall 1: gradient clipping must
    use the norm over all ranks' slices, not each rank's own.

Readings where the pages are silent (the pages print no optimizer equations,
no clipping formula and no rounding mode):
  * AdamW as PyTorch's ``torch.optim.AdamW`` computes it (decoupled weight
    decay scaled by lr, bias-corrected moments, eps added outside the square
    root), applied to every element of the flat shard.
  * Clipping as ``torch.nn.utils.clip_grad_norm_`` computes it, on the global
    L2 norm: c = max_norm / (norm + clip_eps), kept only when below 1; a
    max_norm <= 0 turns clipping off. c scales the gradient before the
    moments. A NaN norm gives a NaN coefficient (it is not clamped to 1).
  * The global sum of squares is the sum of the per-rank partial sums taken in
    rank order.
  * m, v and the master weight are stored as fp32 (round to nearest even)
    after every step; the bf16 parameter is the bf16 rounding of the stored
    fp32 master.
"""

from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

from .bf16 import bf16_to_f32, f32_to_bf16

CHUNK = 1 << 22   # elements per piece: temporaries stay a constant size


@dataclass(frozen=True)
class AdamWHParams:
    """Hyperparameters, refused as ``torch.optim.AdamW`` refuses them (lr,
    eps and weight_decay below 0, a beta outside [0, 1); NaN fails every
    check), and clip_eps below 0 or a NaN max_norm. A max_norm <= 0 turns
    clipping off."""
    lr: float = 1e-3
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    weight_decay: float = 0.01
    max_norm: float = 1.0
    clip_eps: float = 1e-6

    def __post_init__(self):
        if not self.lr >= 0.0:
            raise ValueError(f"invalid learning rate {self.lr}")
        if not self.eps >= 0.0:
            raise ValueError(f"invalid eps {self.eps}")
        for name in ("beta1", "beta2"):
            b = getattr(self, name)
            if not 0.0 <= b < 1.0:
                raise ValueError(f"{name} {b} outside [0, 1)")
        if not self.weight_decay >= 0.0:
            raise ValueError(f"invalid weight decay {self.weight_decay}")
        if not self.clip_eps >= 0.0:
            raise ValueError(f"invalid clip_eps {self.clip_eps}")
        if math.isnan(self.max_norm):
            raise ValueError("max_norm is NaN")


# ---------------------------------------------------------------- pack/unpack

def pack(layout, tensors, begin: int = 0, count: int | None = None) -> np.ndarray:
    """Shard elements [begin, begin+count) gathered from the per-tensor bf16
    gradients. Padding elements are 0. ``tensors[i]`` is tensor i's full
    uint16 array (or None when no segment of the range touches it)."""
    if count is None:
        count = layout.shard - begin
    if begin < 0 or count < 0 or begin + count > layout.shard:
        raise ValueError("range outside the shard")
    out = np.zeros(count, dtype=np.uint16)
    end = begin + count
    for seg in layout.segments:
        lo = max(seg.dst_off, begin)
        hi = min(seg.dst_off + seg.length, end)
        if lo >= hi:
            continue
        s0 = seg.src_off + (lo - seg.dst_off)
        out[lo - begin:hi - begin] = np.asarray(tensors[seg.tensor][s0:s0 + (hi - lo)],
                                                dtype=np.uint16)
    return out


def unpack(layout, shard_bits, tensors, begin: int = 0, count: int | None = None):
    """Copies of ``tensors`` with the elements that shard range
    [begin, begin+count) owns overwritten from ``shard_bits`` (which holds that
    range). Padding goes nowhere; nothing else changes."""
    if count is None:
        count = layout.shard - begin
    if begin < 0 or count < 0 or begin + count > layout.shard:
        raise ValueError("range outside the shard")
    shard_bits = np.asarray(shard_bits, dtype=np.uint16)
    out = [None if t is None else np.array(t, dtype=np.uint16, copy=True) for t in tensors]
    end = begin + count
    for seg in layout.segments:
        lo = max(seg.dst_off, begin)
        hi = min(seg.dst_off + seg.length, end)
        if lo >= hi:
            continue
        d0 = seg.src_off + (lo - seg.dst_off)
        out[seg.tensor][d0:d0 + (hi - lo)] = shard_bits[lo - begin:hi - begin]
    return out


# ------------------------------------------------------------ sum of squares

def sqnorm(grad_bits) -> float:
    """Sum of squares of a bf16 gradient range, in float64. Each square of a
    bf16 value is exact in float64."""
    g = np.asarray(grad_bits, dtype=np.uint16).reshape(-1)
    total = 0.0
    for lo in range(0, g.size, CHUNK):
        x = bf16_to_f32(g[lo:lo + CHUNK]).astype(np.float64)
        total += float(np.dot(x, x))
    return total


def global_sqnorm(rank_partials) -> float:
    """Global sum of squares from the ranks' partial sums, added in rank
    order (the value an all-reduce of the partials stands for)."""
    total = 0.0
    for p in rank_partials:
        total += float(p)
    return total


def clip_coef(global_sq: float, max_norm: float, clip_eps: float = 1e-6) -> float:
    """Clip coefficient from the global sum of squares."""
    if max_norm <= 0:
        return 1.0
    ratio = max_norm / (math.sqrt(global_sq) + clip_eps)
    return 1.0 if ratio >= 1.0 else ratio


# ------------------------------------------------ fp32 gradient accumulation
#
# "第 5 课：ZeRO 与 FSDP", section 2 (note on fp32 gradient accumulation):
# with ZeRO-2/3 each rank keeps an fp32 accumulator for its own gradient slice
# (4 Psi / N_d extra bytes); every micro-batch's 16-bit gradient slice is added
# into it, and the optimizer step then reads fp32 gradients.

def accumulate(acc, grad_bits, first: bool):
    """acc + g for one micro-batch, stored as fp32 (round to nearest even);
    ``first`` starts from zero. The fp64 sum is exact whenever the fp32 result
    can differ from acc, so rounding it once to fp32 is the correctly rounded
    fp32 sum."""
    g = bf16_to_f32(grad_bits).astype(np.float64)
    base = 0.0 if first else np.asarray(acc, dtype=np.float32).astype(np.float64)
    return (base + g).astype(np.float32)


def sqnorm_f32(grad):
    """Sum of squares of an fp32 gradient range in fp64 (each square exact)."""
    x = np.asarray(grad, dtype=np.float32).reshape(-1)
    total = 0.0
    for lo in range(0, x.size, CHUNK):
        y = x[lo:lo + CHUNK].astype(np.float64)
        total += float(np.dot(y, y))
    return total


# ---------------------------------------------------------------------- AdamW

def adamw_f64(p, m, v, g_hat, step: int, hp: AdamWHParams):
    """One AdamW update in float64 (no storage rounding). ``g_hat`` is the
    already clipped gradient. Returns (p', m', v')."""
    if step < 1:
        raise ValueError("step counts from 1")
    p = np.asarray(p, dtype=np.float64)
    m = np.asarray(m, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    g = np.asarray(g_hat, dtype=np.float64)
    m_new = hp.beta1 * m + (1.0 - hp.beta1) * g
    v_new = hp.beta2 * v + (1.0 - hp.beta2) * (g * g)
    bias1 = 1.0 - hp.beta1 ** step
    bias2 = 1.0 - hp.beta2 ** step
    denom = np.sqrt(v_new) / math.sqrt(bias2) + hp.eps
    p_new = p * (1.0 - hp.lr * hp.weight_decay) - (hp.lr / bias1) * (m_new / denom)
    return p_new, m_new, v_new


def adamw_step(grad_bits, master, m, v, step: int, hp: AdamWHParams, coef: float):
    """The rank's fused update over its shard range: scale the bf16 gradient by
    the clip coefficient, update master/m/v (stored back as fp32) and produce
    the bf16 parameter shard. Returns (master', m', v', param_bits)."""
    g = bf16_to_f32(np.asarray(grad_bits, dtype=np.uint16).reshape(-1))
    return adamw_step_f32grad(g, master, m, v, step, hp, coef)


def adamw_step_f32grad(grad, master, m, v, step: int, hp: AdamWHParams, coef: float):
    """adamw_step for an fp32 gradient (the fp32-accumulated one)."""
    g_f32 = np.asarray(grad, dtype=np.float32).reshape(-1)
    master = np.asarray(master, dtype=np.float32).reshape(-1)
    m = np.asarray(m, dtype=np.float32).reshape(-1)
    v = np.asarray(v, dtype=np.float32).reshape(-1)
    n = g_f32.size
    if not (master.size == m.size == v.size == n):
        raise ValueError("shard arrays differ in length")
    out_p = np.empty(n, dtype=np.float32)
    out_m = np.empty(n, dtype=np.float32)
    out_v = np.empty(n, dtype=np.float32)
    out_b = np.empty(n, dtype=np.uint16)
    for lo in range(0, n, CHUNK):
        hi = min(n, lo + CHUNK)
        g_hat = coef * g_f32[lo:hi].astype(np.float64)
        p1, m1, v1 = adamw_f64(master[lo:hi], m[lo:hi], v[lo:hi], g_hat, step, hp)
        out_p[lo:hi] = p1.astype(np.float32)
        out_m[lo:hi] = m1.astype(np.float32)
        out_v[lo:hi] = v1.astype(np.float32)
        out_b[lo:hi] = f32_to_bf16(out_p[lo:hi])
    return out_p, out_m, out_v, out_b
