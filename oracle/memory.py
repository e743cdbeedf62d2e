"""Per-rank memory and communication accounting of ZeRO stages 0-3.

Sources (pages, not code):
  * "第 5 课：ZeRO 与 FSDP", section 2 (per-rank model-state bytes for each
    stage, and the fp32 gradient-accumulation note) and section 3 (per-step
    communication: 2 Psi for stages 0-2, 3 Psi for stage 3).
  * "ZeRO: Memory Optimizations Toward Training Trillion Parameter Models"
    (notes), section 2.1 (16-bit parameters 2 Psi, 16-bit gradients 2 Psi,
    fp32 master/momentum/variance K Psi with K = 12) and section 6
    (communication volume).
  * "別再複製本可分片的東西：ZeRO 與 FSDP", section on the three ZeRO stages.

Model states are three components: 16-bit parameters (2 B/param), 16-bit
gradients (2 B/param) and optimizer state (K B/param). Stage s partitions over
the N_d ranks the optimizer state when s >= 1, the gradients when s >= 2 and
the parameters when s >= 3; everything else stays replicated.
"""

from __future__ import annotations

PARAM_BYTES = 2
GRAD_BYTES = 2
ADAM_K = 12
FP32_ACCUM_BYTES = 4


def _check(psi, n_d, stage):
    if psi <= 0 or n_d <= 0:
        raise ValueError("parameter count and data-parallel degree must be positive")
    if stage not in (0, 1, 2, 3):
        raise ValueError("ZeRO stage must be 0, 1, 2 or 3")


def _partitioned(stage):
    """Which of (params, grads, optimizer) a stage splits across ranks."""
    return (stage >= 3, stage >= 2, stage >= 1)


def model_state_bytes(psi, n_d, stage, k=ADAM_K, fp32_grad_accum=False):
    """Bytes of model state one rank holds, using the pages' Psi/N_d
    (fractional) split. Returns a float."""
    _check(psi, n_d, stage)
    total = 0.0
    for bytes_per, split in zip((PARAM_BYTES, GRAD_BYTES, k), _partitioned(stage)):
        total += bytes_per * psi / (n_d if split else 1)
    if fp32_grad_accum:
        # the fp32 accumulation buffer follows the gradients: replicated up to
        # stage 1, partitioned from stage 2 on
        grads_split = _partitioned(stage)[1]
        total += FP32_ACCUM_BYTES * psi / (n_d if grads_split else 1)
    return total


def model_state_bytes_layout(psi, shard, stage, k=ADAM_K, fp32_grad_accum=False):
    """Same accounting on a generated layout: a partitioned component costs
    its bytes times the rank's padded shard S instead of Psi / N_d. Integer."""
    if psi <= 0 or shard <= 0:
        raise ValueError("parameter count and shard size must be positive")
    if stage not in (0, 1, 2, 3):
        raise ValueError("ZeRO stage must be 0, 1, 2 or 3")
    total = 0
    for bytes_per, split in zip((PARAM_BYTES, GRAD_BYTES, k), _partitioned(stage)):
        total += bytes_per * (shard if split else psi)
    if fp32_grad_accum:
        total += FP32_ACCUM_BYTES * (shard if _partitioned(stage)[1] else psi)
    return total


def comm_values_pages(psi, stage):
    """Values each rank moves per step in the pages' approximation: one
    all-reduce (= reduce-scatter + all-gather, 2 Psi) for stages 0-2; forward
    all-gather + backward all-gather + reduce-scatter (3 Psi) for stage 3."""
    _check(psi, 1, stage)
    return 3 * psi if stage == 3 else 2 * psi


def comm_values_exact(shard, n_d, stage):
    """Values one rank sends per step with ring collectives on a padded layout:
    each reduce-scatter or all-gather moves (N_d - 1) shards. Stages 0-2 make
    two such passes (an all-reduce is a reduce-scatter then an all-gather),
    stage 3 three."""
    if shard <= 0 or n_d <= 0:
        raise ValueError("shard size and data-parallel degree must be positive")
    if stage not in (0, 1, 2, 3):
        raise ValueError("ZeRO stage must be 0, 1, 2 or 3")
    passes = 3 if stage == 3 else 2
    return passes * (n_d - 1) * shard
