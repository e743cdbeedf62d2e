"""Oracle: a plain, slow CPU reference for one data-parallel rank's share of a
ZeRO/FSDP mixed-precision training step.

TEST INFRASTRUCTURE ONLY. Nothing on the product path (the HIP library under
``fsdp_sharded_mixed_zero_amd/`` and its Python binding) imports, links or
executes anything here. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may use this package.

The oracle shares no code, tables or constants with the HIP path. All floating
point arithmetic is done in float64 (numpy); state that the method keeps in
fp32 between steps is rounded to fp32 once per step, exactly where the method
stores it.

Modules
-------
``layout``  flat offsets, padding, rank shards and segments of a per-tensor
            size list (the partitioner).
``memory``  per-rank byte and communication accounting of ZeRO stages 0-3.
``bf16``    fp32 <-> bfloat16 conversion with round-to-nearest-even.
``step``    pack, sum of squares, clip coefficient, AdamW, bf16 cast, unpack.

Pins
----
Every function here is checked by ``tests/test_oracle_*.py`` against something
other than itself: printed numbers on the pages, brute force on tiny inputs,
exact rational arithmetic, closed forms, and library routines
(``torch.optim.AdamW``, ``torch.nn.utils.clip_grad_norm_``, torch's bf16
cast). No function is "parity unpinned".
"""

from . import bf16, layout, memory, step  # noqa: F401
