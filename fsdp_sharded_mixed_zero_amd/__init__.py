"""MI355X-native data-parallel hot path of ZeRO/FSDP: one rank's share of a
sharded mixed-precision training step, run by hand-written gfx950 kernels
behind a C ABI (``libzero_mi355x.so``).

Importing the package does not load the library; the first call through
``fsdp_sharded_mixed_zero_amd.zero`` does, and raises if it is not built.
"""
