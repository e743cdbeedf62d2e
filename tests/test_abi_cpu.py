"""The C ABI on the host: the library loads and exports every declared symbol,
the host partitioner equals the oracle's layout bit for bit, and invalid
arguments are rejected before anything is enqueued. No call here reaches a
kernel launch, so these tests need no GPU."""

import ctypes
import os
import re

import numpy as np
import pytest

from fsdp_sharded_mixed_zero_amd import synth, zero
from oracle import memory
from oracle.layout import LayoutError, build_layout

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "zero.h")

pytestmark = pytest.mark.skipif(not os.path.exists(zero.LIB_PATH),
                                reason="libzero_mi355x.so not built (run __graft_entry__.build())")


def _declared_functions():
    text = open(HEADER, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(zero_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = _declared_functions()
    assert len(names) == 25, names
    lib = zero.library()
    for name in names:
        assert hasattr(lib, name), name
    # and the binding covers the same names
    for name in names:
        assert callable(getattr(zero, name)), name


def _compare(sizes, n_d, rank, align):
    ref = build_layout(sizes, n_d, rank, align)
    lay = zero.zero_layout(sizes, n_d, rank, align)
    info = lay.info
    assert info["psi"] == ref.psi
    assert info["padded"] == ref.padded
    assert info["shard"] == ref.shard
    assert info["shard_begin"] == ref.shard_begin
    assert (info["pad_begin"], info["pad_end"]) == (ref.pad_begin, ref.pad_end)
    assert info["n_tensors"] == len(sizes) and info["n_d"] == n_d and info["rank"] == rank
    segs = lay.segments
    assert segs == [(s.tensor, s.src_off, s.dst_off, s.length) for s in ref.segments]
    assert info["n_segments"] == len(segs)
    for stage in range(4):
        assert info["bytes_stage"][stage] == memory.model_state_bytes_layout(ref.psi, ref.shard, stage)
        assert info["bytes_stage_fp32acc"][stage] == memory.model_state_bytes_layout(
            ref.psi, ref.shard, stage, fp32_grad_accum=True)
        assert info["comm_pages"][stage] == memory.comm_values_pages(ref.psi, stage)
        assert info["comm_exact"][stage] == memory.comm_values_exact(ref.shard, n_d, stage)


def test_layout_matches_oracle_random():
    rng = np.random.default_rng(99)
    for _ in range(200):
        t = int(rng.integers(1, 30))
        sizes = [int(x) for x in rng.integers(0, 1000, size=t)]
        if rng.random() < 0.3:
            sizes[int(rng.integers(0, t))] = 0
        if sum(sizes) == 0:
            sizes[0] = 5
        n_d = int(rng.integers(1, 17))
        align = int(rng.choice([1, 2, 3, 8, 128]))
        for rank in {0, n_d - 1, int(rng.integers(0, n_d))}:
            _compare(sizes, n_d, rank, align)


def test_layout_matches_oracle_many_ranks():
    """Large data-parallel degrees and alignments: shards shorter than a
    tensor, ranks made wholly of padding, alignment beyond the model size."""
    rng = np.random.default_rng(100)
    for _ in range(100):
        t = int(rng.integers(1, 50))
        sizes = [int(x) for x in rng.integers(0, 1_000_000, size=t)]
        if sum(sizes) == 0:
            sizes[0] = 7
        n_d = int(rng.choice([int(rng.integers(1, 64)), int(rng.integers(64, 5000))]))
        align = int(rng.choice([1, 64, 256, 4096, 1 << 20]))
        for rank in {0, n_d - 1, int(rng.integers(0, n_d)), n_d // 2}:
            _compare(sizes, n_d, rank, align)


@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_layout_matches_oracle_workloads(name):
    wl = synth.WORKLOADS[name]
    for rank in sorted({0, wl.rank, wl.n_d - 1}):
        _compare(list(wl.sizes), wl.n_d, rank, wl.align)


def test_layout_rejects_what_the_oracle_rejects():
    for sizes, n_d, rank, align in [([1, 2], 0, 0, 1), ([1, 2], 2, 2, 1), ([1, 2], 2, -1, 1),
                                    ([1, -2], 2, 0, 1), ([0, 0], 2, 0, 1), ([4], 2, 0, 0)]:
        with pytest.raises(LayoutError):
            build_layout(sizes, n_d, rank, align)
        with pytest.raises(zero.ZeroError) as err:
            zero.zero_layout(sizes, n_d, rank, align)
        assert err.value.code == zero.ZERO_EINVAL
        assert zero.zero_last_error()


def test_layout_rejects_overflow_and_empty_list():
    with pytest.raises(zero.ZeroError):
        zero.zero_layout([2**62, 2**62], 1, 0, 1)
    with pytest.raises(zero.ZeroError):
        zero.zero_layout([2**61], 1, 0, 1)   # byte report would overflow
    lib = zero.library()
    h = ctypes.c_void_p()
    arr = (ctypes.c_int64 * 1)(5)
    assert lib.zero_layout(arr, 0, 1, 0, 1, ctypes.byref(h)) == zero.ZERO_EINVAL
    assert lib.zero_layout(None, 1, 1, 0, 1, ctypes.byref(h)) == zero.ZERO_EINVAL
    assert lib.zero_layout(arr, 1, 1, 0, 1, None) == zero.ZERO_EINVAL


def test_device_calls_reject_bad_arguments_on_the_host():
    lib = zero.library()
    lay = zero.zero_layout([100, 28], 2, 1, 8)
    ptrs = (ctypes.c_void_p * 2)(None, None)
    # range errors and NULLs are caught before any launch
    assert lib.zero_pack_grads(lay.handle, ptrs, None, 0, 4, None) == zero.ZERO_EINVAL
    assert lib.zero_pack_grads(None, ptrs, None, 0, 4, None) == zero.ZERO_EINVAL
    assert lib.zero_unpack_params(lay.handle, None, ptrs, 0, 4, None) == zero.ZERO_EINVAL
    assert lib.zero_shard_sqnorm(None, -1, None, 0, None, 0, None) == zero.ZERO_EINVAL
    assert lib.zero_shard_sqnorm(None, 5, None, 0, None, 0, None) == zero.ZERO_EINVAL
    hp = zero.hparams(step=0)
    assert lib.zero_adamw_step(None, None, None, 8, 0, 8, ctypes.byref(hp), None, 1,
                               None) == zero.ZERO_EINVAL
    hp = zero.hparams(step=1)
    for n_state, begin, count in [(8, 0, -1), (8, -1, 2), (8, 4, 5), (-1, 0, 0), (8, 9, 0)]:
        assert lib.zero_adamw_step(None, None, None, n_state, begin, count, ctypes.byref(hp), None, 1,
                                   None) == zero.ZERO_EINVAL
    # clipping on without partial sums
    assert lib.zero_adamw_step(None, None, None, 8, 0, 8, ctypes.byref(hp), None, 0,
                               None) == zero.ZERO_EINVAL
    # NULL buffers with work to do
    assert lib.zero_adamw_step(None, None, None, 8, 0, 8, ctypes.byref(hp), None, 0,
                               None) == zero.ZERO_EINVAL
    assert lib.zero_adamw_step(None, None, None, 8, 0, 8, None, None, 1, None) == zero.ZERO_EINVAL
    assert "zero_adamw_step" in zero.zero_last_error()
    assert lib.zero_state_import(None, None, None, None, -1, None) == zero.ZERO_EINVAL
    assert lib.zero_pack_grads_sqnorm(lay.handle, ptrs, None, 0, 4, None, 0, None, 0, None) == zero.ZERO_EINVAL
    assert lib.zero_pack_sqnorm_workspace_bytes(None, 0, 4) == 0
    assert lib.zero_pack_sqnorm_workspace_bytes(lay.handle, 0, 10**6) == 0     # range outside
    assert lib.zero_pack_sqnorm_workspace_bytes(lay.handle, 0, 64) >= 8
    assert lib.zero_accumulate_grads(None, None, -1, 0, None) == zero.ZERO_EINVAL
    assert lib.zero_accumulate_grads(None, None, 4, 0, None) == zero.ZERO_EINVAL
    assert lib.zero_shard_sqnorm_f32(None, 4, None, 0, None, 0, None) == zero.ZERO_EINVAL
    assert lib.zero_sum_partials(None, -1, None, 0, None) == zero.ZERO_EINVAL
    assert lib.zero_sum_partials(None, 3, ctypes.c_void_p(8), 0, None) == zero.ZERO_EINVAL   # NULL partials
    assert lib.zero_sum_partials(ctypes.c_void_p(8), 3, None, 0, None) == zero.ZERO_EINVAL   # NULL output
    assert lib.zero_sum_partials(ctypes.c_void_p(12), 3, ctypes.c_void_p(8), 0, None) == zero.ZERO_EINVAL
    assert lib.zero_adamw_step_f32grad(None, None, None, 8, 0, 8, ctypes.byref(hp), None, 1,
                                       None) == zero.ZERO_EINVAL
    assert lib.zero_state_export(None, None, None, None, 5, None) == zero.ZERO_EINVAL
    # the update with the unpack fused: layout handle and shard size checked first
    lay = zero.zero_layout([100, 28], 1, 0, 1)
    arr = (ctypes.c_void_p * 2)()
    for fn in (lib.zero_adamw_step_unpack, lib.zero_adamw_step_f32grad_unpack):
        assert fn(None, None, None, 128, 0, 8, ctypes.byref(hp), None, 1, None, arr, None) == zero.ZERO_EINVAL
        assert fn(None, None, None, 100, 0, 8, ctypes.byref(hp), None, 1, lay.handle, arr,
                  None) == zero.ZERO_EINVAL
        assert "shard" in zero.zero_last_error()
        assert fn(None, None, None, 128, 0, 8, ctypes.byref(hp), None, 1, lay.handle, arr,
                  None) == zero.ZERO_EINVAL                      # NULL buffers with work to do
        off = zero.hparams(max_norm=0.0, step=1)
        assert fn(None, None, None, 128, 3, 0, ctypes.byref(off), None, 0, lay.handle, arr, None) == zero.ZERO_OK


def test_device_calls_reject_invalid_hyperparameters():
    """What torch.optim.AdamW refuses (and clip_eps below 0 or a NaN
    max_norm) the GPU updates refuse on the host, before anything is
    launched."""
    from test_oracle_step import EDGE_HPARAMS, INVALID_HPARAMS, OWN_INVALID

    lib = zero.library()
    n = 8
    fake = ctypes.c_void_p(1 << 20)                  # never dereferenced: the checks fail first
    lay = zero.zero_layout([n], 1, 0, 1)
    ptrs = zero.pointer_array([None])
    for kw in INVALID_HPARAMS + OWN_INVALID:
        hp = zero.hparams(**kw)
        for fn in (lib.zero_adamw_step, lib.zero_adamw_step_f32grad):
            assert fn(fake, fake, fake, n, 0, n, ctypes.byref(hp), fake, 1, None) == zero.ZERO_EINVAL, kw
        for fn in (lib.zero_adamw_step_unpack, lib.zero_adamw_step_f32grad_unpack):
            assert fn(fake, fake, fake, n, 0, n, ctypes.byref(hp), fake, 1, lay.handle, ptrs,
                      None) == zero.ZERO_EINVAL, kw
        assert zero.zero_last_error()
    for kw in EDGE_HPARAMS:                          # accepted (an empty range launches nothing)
        hp = zero.hparams(**kw)
        assert lib.zero_adamw_step(fake, fake, fake, n, 0, 0, ctypes.byref(hp), fake, 1, None) == zero.ZERO_OK


def test_cpu_update_refuses_invalid_hyperparameters():
    """The host update applies the same checks."""
    from test_oracle_step import EDGE_HPARAMS, INVALID_HPARAMS, OWN_INVALID

    lib = zero.library()
    n = 8
    h_grad = (ctypes.c_uint16 * n)()
    h_state = (ctypes.c_float * (3 * n))()
    h_param = (ctypes.c_uint16 * n)()
    parts = (ctypes.c_double * 1)(1.0)
    for kw in INVALID_HPARAMS + OWN_INVALID:
        hp = zero.hparams(**kw)
        assert lib.zero_cpu_adamw_step(h_grad, h_state, h_param, n, 0, n, ctypes.byref(hp), parts, 1,
                                       1) == zero.ZERO_EINVAL, kw
        assert zero.zero_last_error()
    for kw in EDGE_HPARAMS:
        hp = zero.hparams(**kw)
        assert lib.zero_cpu_adamw_step(h_grad, h_state, h_param, n, 0, n, ctypes.byref(hp), parts, 1,
                                       1) == zero.ZERO_OK, kw


def test_empty_ranges_return_before_any_launch():
    """An update over an empty range is a no-op that returns OK on the host
    (no launch, no division by its length), at the start, inside and at the
    end of the state, with clipping on and off."""
    lib = zero.library()
    lay = zero.zero_layout([100, 28], 1, 0, 1)
    arr = (ctypes.c_void_p * 2)()
    parts = ctypes.c_void_p(8)            # never read: nothing is launched
    for hp, sq, n_ranks in ((zero.hparams(max_norm=0.0, step=1), None, 0),
                            (zero.hparams(max_norm=1.0, step=3), parts, 4)):
        for begin in (0, 5, 128):
            for fn in (lib.zero_adamw_step, lib.zero_adamw_step_f32grad):
                assert fn(None, None, None, 128, begin, 0, ctypes.byref(hp), sq, n_ranks, None) == zero.ZERO_OK
            for fn in (lib.zero_adamw_step_unpack, lib.zero_adamw_step_f32grad_unpack):
                assert fn(None, None, None, 128, begin, 0, ctypes.byref(hp), sq, n_ranks, lay.handle, arr,
                          None) == zero.ZERO_OK


def test_state_tile_constant_matches_header():
    from state_tiles import TILE
    assert TILE == zero.ZERO_STATE_TILE


def test_binding_constants_match_the_header():
    text = open(HEADER, encoding="utf-8").read()
    defines = {m.group(1): eval(m.group(2), {})
               for m in re.finditer(r"#define (ZERO_[A-Z0-9_]+)[ \t]+([^/\n]+)", text)}
    for name in ("ZERO_OK", "ZERO_EINVAL", "ZERO_EHIP", "ZERO_ENOMEM", "ZERO_STATE_TILE",
                 "ZERO_PIECES_PER_LAUNCH", "ZERO_ADAMW_LAUNCH_ELEMS"):
        assert getattr(zero, name) == defines[name], name


def test_state_tile_helper_follows_the_stated_layout():
    # element e of an n-element state: master at 3kT + j, m at 3kT + L + j,
    # v at 3kT + 2L + j (k = e // T, j = e % T, L = min(T, n - kT))
    from state_tiles import TILE, from_tiles, to_tiles
    for n in (1, 5, TILE, TILE + 3, 2 * TILE + 7):
        master = np.arange(n, dtype=np.float32)
        st = to_tiles(master, master + 0.25, master + 0.5)
        for e in {0, n - 1, n // 2, min(n - 1, TILE), min(n - 1, TILE - 1)}:
            k, j = divmod(e, TILE)
            L = min(TILE, n - k * TILE)
            base = 3 * k * TILE
            assert st[base + j] == e and st[base + L + j] == e + 0.25 and st[base + 2 * L + j] == e + 0.5
        back = from_tiles(st, n)
        assert np.array_equal(back[0], master) and np.array_equal(back[2], master + 0.5)


def test_workspace_size_is_bounded():
    sizes = [zero.zero_sqnorm_workspace_bytes(n) for n in (0, 1, 8, 10**6, 10**9, 10**11)]
    assert all(8 <= s <= 8 * 65536 for s in sizes)
    assert sizes == sorted(sizes)


def test_segments_query_with_small_capacity():
    lay = zero.zero_layout([10, 10, 10], 1, 0, 1)
    lib = zero.library()
    n = ctypes.c_int64()
    segs = (zero.zero_segment * 1)()
    assert lib.zero_layout_segments(lay.handle, segs, 1, ctypes.byref(n)) == 0
    assert n.value == 3 and segs[0].len == 10
    assert lib.zero_layout_segments(lay.handle, None, 2, ctypes.byref(n)) == zero.ZERO_EINVAL


def test_binding_refuses_short_pointer_arrays():
    """The library reads one pointer per tensor of the layout: the binding
    refuses a shorter array before calling it."""
    lay = zero.zero_layout([100, 28, 5], 1, 0, 1)
    hp = zero.hparams(step=1)
    short = [None, None]
    for call in (lambda: zero.zero_pack_grads(lay, short, 0, 0, 8),
                 lambda: zero.zero_unpack_params(lay, 0, short, 0, 8),
                 lambda: zero.zero_pack_grads_sqnorm(lay, short, 0, 0, 8, 0, False, 0, 8),
                 lambda: zero.zero_adamw_step_unpack(0, 0, 0, 133, 0, 8, hp, 0, 1, lay, short),
                 lambda: zero.zero_adamw_step_f32grad_unpack(0, 0, 0, 133, 0, 8, hp, 0, 1, lay,
                                                             (ctypes.c_void_p * 2)())):
        with pytest.raises(ValueError):
            call()


def test_binding_refuses_strided_host_buffers():
    """The host update reads consecutive elements: a strided numpy array or
    CPU tensor is refused before the call."""
    torch = pytest.importorskip("torch")
    hp = zero.hparams(step=1)
    state = np.zeros(3 * 8, np.float32)
    for bad in (np.zeros(16, np.uint16)[::2], torch.zeros(16, dtype=torch.int16)[::2]):
        with pytest.raises(ValueError):
            zero.zero_cpu_adamw_step(bad, state, np.zeros(8, np.uint16), 8, 0, 8, hp, np.ones(1), 1)


def test_binding_refuses_memory_on_the_wrong_side():
    """Host buffers given to a device entry point (and device buffers given to
    the host update) are refused by the binding before anything runs."""
    torch = pytest.importorskip("torch")
    import numpy as np

    x = torch.zeros(24, dtype=torch.float32)        # large enough for every buffer below
    hp = zero.hparams(step=1)
    with pytest.raises(TypeError):
        zero.zero_adamw_step(x, x, x, 8, 0, 8, hp, None, 0)
    with pytest.raises(TypeError):
        zero.zero_accumulate_grads(np.zeros(8, np.uint16), x, 8, True)
    with pytest.raises(TypeError):
        zero.zero_state_import(x, x, x, x, 8)


def test_binding_refuses_short_buffers():
    """A tensor or array smaller than the bytes a call reaches in it is
    refused before the call (a kernel would run past its end)."""
    torch = pytest.importorskip("torch")
    hp = zero.hparams(step=1, max_norm=0.0)
    n = 100
    with pytest.raises(ValueError, match="state"):
        zero.zero_cpu_adamw_step(np.zeros(n, np.uint16), np.zeros(3 * n - 1, np.float32), np.zeros(n, np.uint16),
                                 n, 0, n, hp, None, 0)
    with pytest.raises(ValueError, match="parameters"):
        zero.zero_cpu_adamw_step(np.zeros(n, np.uint16), np.zeros(3 * n, np.float32), np.zeros(n - 1, np.uint16),
                                 n, 0, n, hp, None, 0)
    with pytest.raises(ValueError, match="rank sums"):
        zero.zero_cpu_adamw_step(np.zeros(n, np.uint16), np.zeros(3 * n, np.float32), np.zeros(n, np.uint16),
                                 n, 0, n, zero.hparams(step=1), np.ones(3), 4)
    # a bf16 tensor where the fp32 state belongs: half the bytes
    with pytest.raises(ValueError, match="state"):
        zero.zero_cpu_adamw_step(np.zeros(n, np.uint16), torch.zeros(3 * n, dtype=torch.bfloat16),
                                 np.zeros(n, np.uint16), n, 0, n, hp, None, 0)
    lay = zero.zero_layout([100, 28], 1, 0, 1)
    with pytest.raises(ValueError, match="tensor 1"):
        zero.zero_pack_grads(lay, [torch.zeros(100, dtype=torch.int16), torch.zeros(27, dtype=torch.int16)], 0, 0,
                             8)
    # an empty range reaches nothing
    zero.zero_cpu_adamw_step(np.zeros(0, np.uint16), np.zeros(0, np.float32), np.zeros(0, np.uint16), n, 5, 0,
                             hp, None, 0)


def test_last_error_is_per_thread():
    """zero_last_error() reports the calling thread's own last failure: two
    threads fail in different ways at the same time, and a third that
    succeeds sees an empty message."""
    import threading

    lib = zero.library()
    barrier = threading.Barrier(3)
    seen = {}

    def fail_layout():
        h = ctypes.c_void_p()
        arr = (ctypes.c_int64 * 2)(4, 4)
        barrier.wait()
        for _ in range(200):
            assert lib.zero_layout(arr, 2, 0, 0, 1, ctypes.byref(h)) == zero.ZERO_EINVAL   # n_d = 0
        seen["layout"] = zero.zero_last_error()

    def fail_update():
        hp = zero.hparams(step=0)
        g, st, p = (ctypes.c_uint16 * 8)(), (ctypes.c_float * 24)(), (ctypes.c_uint16 * 8)()
        barrier.wait()
        for _ in range(200):
            assert lib.zero_cpu_adamw_step(g, st, p, 8, 0, 8, ctypes.byref(hp), None, 0, 1) == zero.ZERO_EINVAL
        seen["update"] = zero.zero_last_error()

    def succeed():
        barrier.wait()
        for _ in range(200):
            zero.zero_layout([8, 8], 2, 1, 1)
        seen["ok"] = zero.zero_last_error()

    threads = [threading.Thread(target=f) for f in (fail_layout, fail_update, succeed)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert "zero_layout" in seen["layout"] and "zero_cpu_adamw_step" not in seen["layout"]
    assert "zero_cpu_adamw_step" in seen["update"] and "zero_layout" not in seen["update"]
    assert seen["ok"] == ""
