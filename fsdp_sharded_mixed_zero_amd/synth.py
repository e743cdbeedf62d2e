"""Seeded synthetic inputs and the workload shapes.

This module holds no arithmetic of the method itself: it lists the per-tensor
parameter sizes of the transformer shapes the pages discuss and draws random
inputs for them. Both the HIP path's tests/benchmark and the oracle's tests
take their inputs from here.

Workloads (model sizes named on the pages; the pages give no tensor lists, so
the lists below are the usual GPT-2 and Llama layouts):
  * GPT-2 1.5B: notes on the ZeRO paper, section 2.1 (model states of a 1.5B
    GPT-2); 48 layers, d = 1600, vocab 50257, context 1024.
  * Llama-style 7B: "第 5 课：ZeRO 与 FSDP", worked 7B example; 32 layers,
    d = 4096, ffn 11008, vocab 32000.
  * GPT-style 7.5B: "ZeRO-3 核心流程", section 1 (7.5B model on 64 cards);
    72 layers, d = 2944; vocab 50257 and context 1024 are taken from GPT-2.
  * Llama-style 70B: "第 5 课：ZeRO 与 FSDP", section 1 (70B model); 80 layers,
    d = 8192, ffn 28672, 64 heads with 8 KV heads, vocab 32000.

Random streams: numpy ``default_rng([seed, buffer, step, piece])`` on the
host and ``torch.Generator`` seeded from the same four numbers on the device.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

# buffer ids of the random streams
GRAD, MASTER, EXP_AVG, EXP_AVG_SQ, MASK = 0, 1, 2, 3, 4

# bf16 pattern used to fill tensor bytes that lie outside the rank's shard:
# a NaN with a recognisable payload, so a stray read or write shows up.
SENTINEL = 0x7FA5


# ------------------------------------------------------------ tensor lists

def tiny_sizes():
    return [131072] * 8


def gpt_sizes(layers, d, vocab=50257, ctx=1024):
    """GPT-2 style: token and position embeddings, per block LN/attention/MLP
    weights and biases, final LN; the LM head shares the token embedding."""
    sizes = [vocab * d, ctx * d]
    for _ in range(layers):
        sizes += [d, d,                  # ln1 weight, bias
                  d * 3 * d, 3 * d,      # fused qkv weight, bias
                  d * d, d,              # attention output proj
                  d, d,                  # ln2 weight, bias
                  d * 4 * d, 4 * d,      # MLP up
                  4 * d * d, d]          # MLP down
    sizes += [d, d]                      # final LN
    return sizes


def llama_sizes(layers, d, ffn, vocab=32000, heads=32, kv_heads=32):
    """Llama style: embedding, per block RMSNorm/q/k/v/o and gated MLP, final
    norm, untied LM head."""
    hd = d // heads
    sizes = [vocab * d]
    for _ in range(layers):
        sizes += [d,                     # attention norm
                  d * d,                 # q
                  d * kv_heads * hd,     # k
                  d * kv_heads * hd,     # v
                  d * d,                 # o
                  d,                     # MLP norm
                  d * ffn, d * ffn,      # gate, up
                  ffn * d]               # down
    sizes += [d, vocab * d]              # final norm, LM head
    return sizes


@dataclass(frozen=True)
class Workload:
    name: str
    sizes: tuple
    n_d: int
    rank: int
    align: int = 128
    grad_std: float = 1e-3
    spike_frac: float = 0.0       # fraction of gradient entries scaled up
    spike_scale: float = 1.0
    master_std: float = 0.02
    m_std: float = 0.0            # 0: zeros
    v_std: float = 0.0            # v ~ |N(0, v_std)|, 0: zeros
    step: int = 1
    steps: int = 1
    bucket: int = 0               # 0: whole shard in one piece
    lr: float = 1e-3
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    weight_decay: float = 0.01
    max_norm: float = 1.0
    seed: int = 0
    notes: dict = field(default_factory=dict, compare=False)

    def grad_sq_mean(self):
        """Expected square of one gradient entry (the benchmark's CPU baseline
        takes the other ranks' share of the norm of its timing sample from
        it)."""
        s2 = self.grad_std ** 2
        return (1 - self.spike_frac) * s2 + self.spike_frac * s2 * self.spike_scale ** 2


WORKLOADS = {
    "tiny": Workload("tiny", tuple(tiny_sizes()), n_d=4, rank=1, steps=10),
    "gpt2-1.5b": Workload("gpt2-1.5b", tuple(gpt_sizes(48, 1600)), n_d=64, rank=32,
                          steps=3),
    "llama-7b": Workload("llama-7b", tuple(llama_sizes(32, 4096, 11008)), n_d=4, rank=1,
                         grad_std=1e-4, spike_frac=0.01, spike_scale=100.0),
    "gpt-7.5b": Workload("gpt-7.5b", tuple(gpt_sizes(72, 2944)), n_d=64, rank=1,
                         m_std=1e-4, v_std=1e-8, step=1000),
    "llama-70b": Workload("llama-70b",
                          tuple(llama_sizes(80, 8192, 28672, heads=64, kv_heads=8)),
                          n_d=8, rank=1, bucket=50_000_000),
}


# ------------------------------------------------------------ host streams

def host_rng(seed, buffer, step=0, piece=0):
    return np.random.default_rng([int(seed), int(buffer), int(step), int(piece)])


def to_bf16_bits(x_f32: np.ndarray) -> np.ndarray:
    """bf16 bit patterns of float32 samples, rounded by torch's CPU cast (a
    library conversion, used only to make inputs)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x_f32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def host_normal(n, std, seed, buffer, step=0, piece=0) -> np.ndarray:
    r = host_rng(seed, buffer, step, piece)
    return (r.standard_normal(n, dtype=np.float32) * np.float32(std)).astype(np.float32)


def host_grad_f32(n, wl: Workload, step, piece) -> np.ndarray:
    g = host_normal(n, wl.grad_std, wl.seed, GRAD, step, piece)
    if wl.spike_frac > 0:
        mask = host_rng(wl.seed, MASK, step, piece).random(n) < wl.spike_frac
        g[mask] *= np.float32(wl.spike_scale)
    return g


def host_tensor_grads(wl: Workload, step, tensors=None):
    """Full bf16 gradient of each listed tensor (default: all), tensor i drawn
    from stream piece i."""
    idx = range(len(wl.sizes)) if tensors is None else tensors
    out = [None] * len(wl.sizes)
    for i in idx:
        out[i] = to_bf16_bits(host_grad_f32(wl.sizes[i], wl, step, i))
    return out


def host_flat_state(wl: Workload, psi, padded):
    """fp32 master, m, v over the whole padded flat buffer (small workloads
    only). Padding entries are 0."""
    master = np.zeros(padded, np.float32)
    master[:psi] = host_normal(psi, wl.master_std, wl.seed, MASTER)
    m = np.zeros(padded, np.float32)
    v = np.zeros(padded, np.float32)
    if wl.m_std > 0:
        m[:psi] = host_normal(psi, wl.m_std, wl.seed, EXP_AVG)
    if wl.v_std > 0:
        v[:psi] = np.abs(host_normal(psi, wl.v_std, wl.seed, EXP_AVG_SQ))
    return master, m, v


def host_shard_state(wl: Workload, begin, count, real, piece=0):
    """fp32 master, m, v for ``count`` shard elements drawn as their own
    streams (for large shards); the first ``real`` are parameters, the rest
    padding (0)."""
    master = np.zeros(count, np.float32)
    master[:real] = host_normal(real, wl.master_std, wl.seed, MASTER, 0, piece)
    m = np.zeros(count, np.float32)
    v = np.zeros(count, np.float32)
    if wl.m_std > 0:
        m[:real] = host_normal(real, wl.m_std, wl.seed, EXP_AVG, 0, piece)
    if wl.v_std > 0:
        v[:real] = np.abs(host_normal(real, wl.v_std, wl.seed, EXP_AVG_SQ, 0, piece))
    return master, m, v


# ---------------------------------------------------------- device streams

def _device_gen(seed, buffer, step, piece, device):
    import torch
    key = ((int(seed) * 1_000_003 + int(buffer)) * 1_000_033 + int(step)) * 1_000_037 + int(piece)
    g = torch.Generator(device=device)
    g.manual_seed(key & ((1 << 63) - 1))
    return g


DEVICE_PIECE = 1 << 26


def device_normal_(out, std, seed, buffer, step=0, abs_value=False, salt=0):
    """Fill a float32 or bfloat16 CUDA tensor with N(0, std) samples (|N| when
    ``abs_value``), drawn in pieces of 2^26 elements, piece k from stream
    (seed, buffer, step, salt * 2^20 + k)."""
    import torch
    flat = out.view(-1)
    for k, lo in enumerate(range(0, flat.numel(), DEVICE_PIECE)):
        hi = min(flat.numel(), lo + DEVICE_PIECE)
        gen = _device_gen(seed, buffer, step, (salt << 20) + k, out.device)
        x = torch.randn(hi - lo, generator=gen, device=out.device, dtype=torch.float32)
        x.mul_(std)
        if abs_value:
            x.abs_()
        flat[lo:hi].copy_(x)
    return out


def device_grad_(out_bf16, wl: Workload, step, salt=0):
    """Fill a bfloat16 CUDA tensor with the workload's gradient distribution
    (rounded to bf16 by torch's cast), piece k from stream
    (seed, GRAD, step, salt * 2^20 + k)."""
    import torch
    flat = out_bf16.view(-1)
    for k, lo in enumerate(range(0, flat.numel(), DEVICE_PIECE)):
        hi = min(flat.numel(), lo + DEVICE_PIECE)
        piece = (salt << 20) + k
        gen = _device_gen(wl.seed, GRAD, step, piece, out_bf16.device)
        x = torch.randn(hi - lo, generator=gen, device=out_bf16.device, dtype=torch.float32)
        x.mul_(wl.grad_std)
        if wl.spike_frac > 0:
            mgen = _device_gen(wl.seed, MASK, step, piece, out_bf16.device)
            u = torch.rand(hi - lo, generator=mgen, device=out_bf16.device)
            x = torch.where(u < wl.spike_frac, x * wl.spike_scale, x)
        flat[lo:hi].copy_(x)
    return out_bf16
