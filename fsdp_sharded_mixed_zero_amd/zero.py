"""Python binding of libzero_mi355x.so: the C ABI declared in include/zero.h,
same names, argument marshalling only.

Device buffers may be passed as torch tensors (their ``data_ptr()`` is used,
so a slice passes its offset) or as integer addresses. ``stream`` defaults to
torch's current stream on the current device. Every step of the computation
runs in the library's kernels; nothing here computes on the data. A missing
library raises ``ZeroLibraryMissing`` at the first call.
"""

from __future__ import annotations

import ctypes
import os

from .build import LIB_PATH

ZERO_OK = 0
ZERO_EINVAL = -1
ZERO_EHIP = -3
ZERO_ENOMEM = -4
ZERO_STATE_TILE = 8192      # elements per tile of the fp32 state buffer (include/zero.h)
ZERO_PIECES_PER_LAUNCH = 64            # tensor pieces one launch carries (include/zero.h)
ZERO_ADAMW_LAUNCH_ELEMS = 1 << 27      # longer update ranges take several launches
ZERO_NOALLOC_PARTIALS = 1 << 18        # partial sums the static scratch of the no-allocation call holds


class ZeroError(RuntimeError):
    def __init__(self, func, code, message):
        super().__init__(f"{func} failed ({code}): {message}")
        self.code = code


class ZeroLibraryMissing(RuntimeError):
    pass


class zero_segment(ctypes.Structure):
    _fields_ = [("tensor", ctypes.c_int64), ("src_off", ctypes.c_int64),
                ("dst_off", ctypes.c_int64), ("len", ctypes.c_int64)]


class zero_layout_info(ctypes.Structure):
    _fields_ = [("n_tensors", ctypes.c_int64), ("n_d", ctypes.c_int64), ("rank", ctypes.c_int64),
                ("align", ctypes.c_int64), ("psi", ctypes.c_int64), ("padded", ctypes.c_int64),
                ("shard", ctypes.c_int64), ("shard_begin", ctypes.c_int64),
                ("n_segments", ctypes.c_int64), ("pad_begin", ctypes.c_int64),
                ("pad_end", ctypes.c_int64), ("bytes_stage", ctypes.c_int64 * 4),
                ("bytes_stage_fp32acc", ctypes.c_int64 * 4), ("comm_pages", ctypes.c_int64 * 4),
                ("comm_exact", ctypes.c_int64 * 4)]

    def as_dict(self):
        out = {}
        for name, _ in self._fields_:
            val = getattr(self, name)
            out[name] = list(val) if isinstance(val, ctypes.Array) else int(val)
        return out


class zero_adamw_hparams(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_double), ("beta1", ctypes.c_double), ("beta2", ctypes.c_double),
                ("eps", ctypes.c_double), ("weight_decay", ctypes.c_double),
                ("max_norm", ctypes.c_double), ("clip_eps", ctypes.c_double),
                ("step", ctypes.c_int64)]


_VP = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32

_SIGNATURES = {
    "zero_layout": (ctypes.c_int, [ctypes.POINTER(_I64), _I32, _I32, _I32, _I64, ctypes.POINTER(_VP)]),
    "zero_layout_query": (ctypes.c_int, [_VP, ctypes.POINTER(zero_layout_info)]),
    "zero_layout_segments": (ctypes.c_int, [_VP, ctypes.POINTER(zero_segment), _I64, ctypes.POINTER(_I64)]),
    "zero_layout_free": (None, [_VP]),
    "zero_pack_grads": (ctypes.c_int, [_VP, ctypes.POINTER(_VP), _VP, _I64, _I64, _VP]),
    "zero_sqnorm_workspace_bytes": (ctypes.c_size_t, [_I64]),
    "zero_pack_sqnorm_workspace_bytes": (ctypes.c_size_t, [_VP, _I64, _I64]),
    "zero_pack_grads_sqnorm": (ctypes.c_int, [_VP, ctypes.POINTER(_VP), _VP, _I64, _I64, _VP, _I32, _VP,
                                              ctypes.c_size_t, _VP]),
    "zero_pack_grads_sqnorm_noalloc": (ctypes.c_int, [_VP, ctypes.POINTER(_VP), _VP, _I64, _I64, _VP, _I32, _VP]),
    "zero_shard_sqnorm": (ctypes.c_int, [_VP, _I64, _VP, _I32, _VP, ctypes.c_size_t, _VP]),
    "zero_sum_partials": (ctypes.c_int, [_VP, _I64, _VP, _I32, _VP]),
    "zero_pack_grads_sqnorm_partials": (ctypes.c_int, [_VP, ctypes.POINTER(_VP), _VP, _I64, _I64, _VP,
                                                       ctypes.c_size_t, ctypes.POINTER(_I64), _VP]),
    "zero_sum_partials_rows": (ctypes.c_int, [_VP, ctypes.POINTER(_I64), ctypes.POINTER(_I64), _I64, _VP, _I32,
                                              _VP]),
    "zero_adamw_step": (ctypes.c_int, [_VP, _VP, _VP, _I64, _I64, _I64,
                                       ctypes.POINTER(zero_adamw_hparams), _VP, _I32, _VP]),
    "zero_adamw_step_f32grad": (ctypes.c_int, [_VP, _VP, _VP, _I64, _I64, _I64,
                                               ctypes.POINTER(zero_adamw_hparams), _VP, _I32, _VP]),
    "zero_adamw_step_unpack": (ctypes.c_int, [_VP, _VP, _VP, _I64, _I64, _I64,
                                              ctypes.POINTER(zero_adamw_hparams), _VP, _I32, _VP,
                                              ctypes.POINTER(_VP), _VP]),
    "zero_adamw_step_f32grad_unpack": (ctypes.c_int, [_VP, _VP, _VP, _I64, _I64, _I64,
                                                      ctypes.POINTER(zero_adamw_hparams), _VP, _I32, _VP,
                                                      ctypes.POINTER(_VP), _VP]),
    "zero_adamw_step_arrays": (ctypes.c_int, [_VP, _VP, _VP, _VP, _VP, _I64,
                                              ctypes.POINTER(zero_adamw_hparams), _VP, _I32, _VP]),
    "zero_accumulate_grads": (ctypes.c_int, [_VP, _VP, _I64, _I32, _VP]),
    "zero_cpu_adamw_step": (ctypes.c_int, [_VP, _VP, _VP, _I64, _I64, _I64,
                                           ctypes.POINTER(zero_adamw_hparams), _VP, _I32, _I32]),
    "zero_shard_sqnorm_f32": (ctypes.c_int, [_VP, _I64, _VP, _I32, _VP, ctypes.c_size_t, _VP]),
    "zero_state_import": (ctypes.c_int, [_VP, _VP, _VP, _VP, _I64, _VP]),
    "zero_state_export": (ctypes.c_int, [_VP, _VP, _VP, _VP, _I64, _VP]),
    "zero_unpack_params": (ctypes.c_int, [_VP, _VP, ctypes.POINTER(_VP), _I64, _I64, _VP]),
    "zero_last_error": (ctypes.c_char_p, []),
}

_lib = None


def library(path: str | None = None):
    """Load (once) and return the ctypes handle of libzero_mi355x.so."""
    global _lib
    if _lib is not None:
        return _lib
    path = path or os.environ.get("ZERO_MI355X_LIB", LIB_PATH)
    if not os.path.exists(path):
        raise ZeroLibraryMissing(
            f"{path} is not built; run `python -m fsdp_sharded_mixed_zero_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def zero_last_error() -> str:
    return library().zero_last_error().decode(errors="replace")


def _check(func, rc):
    if rc != ZERO_OK:
        raise ZeroError(func, rc, zero_last_error())


def _ptr(x):
    """Device address of a torch tensor (or an integer address). A host
    tensor or array is refused here: a kernel would read a host address."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if not getattr(x, "is_cuda", False):
        raise TypeError(f"device memory expected, got {type(x).__name__}"
                        f"{' on ' + str(x.device) if hasattr(x, 'device') else ''}")
    if not x.is_contiguous():
        raise ValueError("a contiguous tensor is expected: the library reads consecutive elements")
    return x.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _ptr_array(items):
    if isinstance(items, ctypes.Array):
        return items
    arr = (_VP * len(items))()
    for i, t in enumerate(items):
        arr[i] = _ptr(t)
    return arr


def pointer_array(tensors):
    """A reusable host array of device pointers (tensor_grads/tensor_params
    arguments); None entries stay NULL."""
    return _ptr_array(tensors)


def _tensor_array(layout, items):
    """The per-tensor pointer array of a call on `layout`. The library reads
    one pointer per tensor of the layout, so a shorter array is refused here
    (it would be read past its end)."""
    if not isinstance(items, ctypes.Array):
        for i, t in enumerate(items):
            if i < len(layout.sizes):
                _need(t, 2 * layout.sizes[i], f"tensor {i}")
    arr = _ptr_array(items)
    if len(arr) < layout.n_tensors:
        raise ValueError(f"{len(arr)} tensor pointers for a layout of {layout.n_tensors} tensors")
    return arr


def _need(x, nbytes: int, what: str):
    """Refuse a tensor or array smaller than the bytes the call reaches in it
    (a kernel would read or write past its end). Raw addresses are the
    caller's to size."""
    if x is None or isinstance(x, int) or not hasattr(x, "nbytes"):
        return
    if int(x.nbytes) < nbytes:
        raise ValueError(f"{what}: {int(x.nbytes)} bytes given, the call reaches {nbytes}")


def _need_update(grad, gsize, state, param, n_state, begin, count, rank_sqnorms, n_ranks):
    if count <= 0:
        return
    _need(grad, gsize * (begin + count), "gradient")
    _need(state, 12 * n_state, "state")
    _need(param, 2 * (begin + count), "parameter shard")
    if n_ranks > 0:
        _need(rank_sqnorms, 8 * n_ranks, "rank sums of squares")


class Layout:
    """Owner of a zero_layout_t handle (and of the size list it was made from)."""

    def __init__(self, handle: int, n_tensors: int, sizes=()):
        self.handle = handle
        self.n_tensors = n_tensors
        self.sizes = tuple(sizes)

    def close(self):
        if self.handle:
            library().zero_layout_free(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def info(self) -> dict:
        return zero_layout_query(self)

    @property
    def segments(self):
        return zero_layout_segments(self)


def zero_layout(sizes, n_d: int, rank: int, align_elems: int = 128) -> Layout:
    sizes = [int(s) for s in sizes]
    arr = (_I64 * max(1, len(sizes)))(*sizes)
    h = _VP()
    _check("zero_layout", library().zero_layout(arr, len(sizes), n_d, rank, align_elems, ctypes.byref(h)))
    return Layout(h.value, len(sizes), sizes)


def zero_layout_free(layout: Layout) -> None:
    layout.close()


def zero_layout_query(layout: Layout) -> dict:
    info = zero_layout_info()
    _check("zero_layout_query", library().zero_layout_query(layout.handle, ctypes.byref(info)))
    return info.as_dict()


def zero_layout_segments(layout: Layout):
    n = _I64()
    _check("zero_layout_segments", library().zero_layout_segments(layout.handle, None, 0, ctypes.byref(n)))
    segs = (zero_segment * max(1, n.value))()
    _check("zero_layout_segments",
           library().zero_layout_segments(layout.handle, segs, n.value, ctypes.byref(n)))
    return [(s.tensor, s.src_off, s.dst_off, s.len) for s in segs[:n.value]]


def zero_pack_grads(layout: Layout, tensor_grads, grad_shard, begin: int, count: int, stream=None):
    arr = _tensor_array(layout, tensor_grads)
    if count > 0:
        _need(grad_shard, 2 * (begin + count), "gradient shard")
    _check("zero_pack_grads", library().zero_pack_grads(
        layout.handle, arr, _ptr(grad_shard), begin, count, _stream(stream)))


def zero_pack_sqnorm_workspace_bytes(layout: Layout, begin: int, count: int) -> int:
    return int(library().zero_pack_sqnorm_workspace_bytes(layout.handle, begin, count))


def zero_pack_grads_sqnorm(layout: Layout, tensor_grads, grad_shard, begin: int, count: int, out,
                           accumulate: bool, workspace, ws_bytes: int | None = None, stream=None):
    arr = _tensor_array(layout, tensor_grads)
    if count > 0:
        _need(grad_shard, 2 * (begin + count), "gradient shard")
    _need(out, 8, "output")
    if ws_bytes is None:
        ws_bytes = workspace.numel() * workspace.element_size()
    _check("zero_pack_grads_sqnorm", library().zero_pack_grads_sqnorm(
        layout.handle, arr, _ptr(grad_shard), begin, count, _ptr(out), 1 if accumulate else 0,
        _ptr(workspace), ws_bytes, _stream(stream)))


def zero_pack_grads_sqnorm_noalloc(layout: Layout, tensor_grads, grad_shard, begin: int, count: int, out,
                                   accumulate: bool, stream=None):
    arr = _tensor_array(layout, tensor_grads)
    if count > 0:
        _need(grad_shard, 2 * (begin + count), "gradient shard")
    _need(out, 8, "output")
    _check("zero_pack_grads_sqnorm_noalloc", library().zero_pack_grads_sqnorm_noalloc(
        layout.handle, arr, _ptr(grad_shard), begin, count, _ptr(out), 1 if accumulate else 0, _stream(stream)))


def zero_unpack_params(layout: Layout, param_shard, tensor_params, begin: int, count: int, stream=None):
    arr = _tensor_array(layout, tensor_params)
    if count > 0:
        _need(param_shard, 2 * (begin + count), "parameter shard")
    _check("zero_unpack_params", library().zero_unpack_params(
        layout.handle, _ptr(param_shard), arr, begin, count, _stream(stream)))


def zero_sqnorm_workspace_bytes(count: int) -> int:
    return int(library().zero_sqnorm_workspace_bytes(count))


def zero_shard_sqnorm(grad, count: int, out, accumulate: bool, workspace, ws_bytes: int | None = None,
                      stream=None):
    if count > 0:
        _need(grad, 2 * count, "gradient")
    _need(out, 8, "output")
    if ws_bytes is None:
        ws_bytes = workspace.numel() * workspace.element_size()
    _check("zero_shard_sqnorm", library().zero_shard_sqnorm(
        _ptr(grad), count, _ptr(out), 1 if accumulate else 0, _ptr(workspace), ws_bytes,
        _stream(stream)))


def zero_sum_partials(partials, n: int, out, accumulate: bool = False, stream=None):
    if n > 0:
        _need(partials, 8 * n, "partial sums")
    _need(out, 8, "output")
    _check("zero_sum_partials", library().zero_sum_partials(
        _ptr(partials), n, _ptr(out), 1 if accumulate else 0, _stream(stream)))


def zero_pack_grads_sqnorm_partials(layout: Layout, tensor_grads, grad_shard, begin: int, count: int, partials,
                                    cap_bytes: int | None = None, stream=None) -> int:
    """Returns the number of partial sums written."""
    arr = _tensor_array(layout, tensor_grads)
    if count > 0:
        _need(grad_shard, 2 * (begin + count), "gradient shard")
    if cap_bytes is None:
        cap_bytes = partials.numel() * partials.element_size()
    n = ctypes.c_int64(0)
    _check("zero_pack_grads_sqnorm_partials", library().zero_pack_grads_sqnorm_partials(
        layout.handle, arr, _ptr(grad_shard), begin, count, _ptr(partials), cap_bytes, ctypes.byref(n),
        _stream(stream)))
    return int(n.value)


def zero_sum_partials_rows(partials, row_begin, row_len, out, accumulate: bool = False, stream=None):
    n = len(row_begin)
    if len(row_len) != n:
        raise ValueError("row_begin and row_len differ in length")
    if n > 0:
        _need(partials, 8 * max(b + c for b, c in zip(row_begin, row_len)), "partial sums")
        _need(out, 8 * n, "output")
    begins = (ctypes.c_int64 * n)(*row_begin)
    lens = (ctypes.c_int64 * n)(*row_len)
    _check("zero_sum_partials_rows", library().zero_sum_partials_rows(
        _ptr(partials), begins, lens, n, _ptr(out), 1 if accumulate else 0, _stream(stream)))


def hparams(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, max_norm=1.0,
            clip_eps=1e-6, step=1) -> zero_adamw_hparams:
    return zero_adamw_hparams(lr, beta1, beta2, eps, weight_decay, max_norm, clip_eps, step)


def zero_adamw_step(grad, state, param, n_state: int, begin: int, count: int, hp: zero_adamw_hparams,
                    rank_sqnorms, n_ranks: int, stream=None):
    _need_update(grad, 2, state, param, n_state, begin, count, rank_sqnorms, n_ranks)
    _check("zero_adamw_step", library().zero_adamw_step(
        _ptr(grad), _ptr(state), _ptr(param), n_state, begin, count, ctypes.byref(hp),
        _ptr(rank_sqnorms), n_ranks, _stream(stream)))


def zero_adamw_step_arrays(grad, master, m, v, param, count: int, hp: zero_adamw_hparams, rank_sqnorms,
                           n_ranks: int, stream=None):
    if count > 0:
        _need(grad, 2 * count, "gradient")
        for x, what in ((master, "master"), (m, "m"), (v, "v")):
            _need(x, 4 * count, what)
        _need(param, 2 * count, "parameter shard")
        if n_ranks > 0:
            _need(rank_sqnorms, 8 * n_ranks, "rank sums of squares")
    _check("zero_adamw_step_arrays", library().zero_adamw_step_arrays(
        _ptr(grad), _ptr(master), _ptr(m), _ptr(v), _ptr(param), count, ctypes.byref(hp),
        _ptr(rank_sqnorms), n_ranks, _stream(stream)))


def zero_adamw_step_f32grad(grad, state, param, n_state: int, begin: int, count: int,
                            hp: zero_adamw_hparams, rank_sqnorms, n_ranks: int, stream=None):
    _need_update(grad, 4, state, param, n_state, begin, count, rank_sqnorms, n_ranks)
    _check("zero_adamw_step_f32grad", library().zero_adamw_step_f32grad(
        _ptr(grad), _ptr(state), _ptr(param), n_state, begin, count, ctypes.byref(hp),
        _ptr(rank_sqnorms), n_ranks, _stream(stream)))


def zero_adamw_step_unpack(grad, state, param, n_state: int, begin: int, count: int, hp: zero_adamw_hparams,
                           rank_sqnorms, n_ranks: int, layout: Layout, tensor_params, stream=None):
    arr = _tensor_array(layout, tensor_params)
    _need_update(grad, 2, state, param, n_state, begin, count, rank_sqnorms, n_ranks)
    _check("zero_adamw_step_unpack", library().zero_adamw_step_unpack(
        _ptr(grad), _ptr(state), _ptr(param), n_state, begin, count, ctypes.byref(hp),
        _ptr(rank_sqnorms), n_ranks, layout.handle, arr, _stream(stream)))


def zero_adamw_step_f32grad_unpack(grad, state, param, n_state: int, begin: int, count: int,
                                   hp: zero_adamw_hparams, rank_sqnorms, n_ranks: int, layout: Layout,
                                   tensor_params, stream=None):
    arr = _tensor_array(layout, tensor_params)
    _need_update(grad, 4, state, param, n_state, begin, count, rank_sqnorms, n_ranks)
    _check("zero_adamw_step_f32grad_unpack", library().zero_adamw_step_f32grad_unpack(
        _ptr(grad), _ptr(state), _ptr(param), n_state, begin, count, ctypes.byref(hp),
        _ptr(rank_sqnorms), n_ranks, layout.handle, arr, _stream(stream)))


def _host_ptr(x):
    """Address of a host buffer: a CPU torch tensor, a numpy array or an int.
    A device tensor is refused: the host update would read a device address."""
    if x is None or isinstance(x, int):
        return x
    if hasattr(x, "ctypes"):
        if not x.flags["C_CONTIGUOUS"]:
            raise ValueError("a contiguous array is expected: the library reads consecutive elements")
        return x.ctypes.data
    if getattr(x, "is_cuda", False):
        raise TypeError("host memory expected, got a device tensor")
    if not x.is_contiguous():
        raise ValueError("a contiguous tensor is expected: the library reads consecutive elements")
    return x.data_ptr()


def zero_cpu_adamw_step(grad, state, param, n_state: int, begin: int, count: int, hp: zero_adamw_hparams,
                        rank_sqnorms, n_ranks: int, n_threads: int = 0):
    """Host memory throughout (numpy arrays or CPU tensors). The gradient and
    parameter buffers hold the range only (element begin first)."""
    if count > 0:
        _need(grad, 2 * count, "gradient")
        _need(state, 12 * n_state, "state")
        _need(param, 2 * count, "parameters")
        if n_ranks > 0:
            _need(rank_sqnorms, 8 * n_ranks, "rank sums of squares")
    _check("zero_cpu_adamw_step", library().zero_cpu_adamw_step(
        _host_ptr(grad), _host_ptr(state), _host_ptr(param), n_state, begin, count, ctypes.byref(hp),
        _host_ptr(rank_sqnorms), n_ranks, n_threads))


def zero_accumulate_grads(grad, acc, count: int, first: bool, stream=None):
    if count > 0:
        _need(grad, 2 * count, "gradient")
        _need(acc, 4 * count, "accumulator")
    _check("zero_accumulate_grads", library().zero_accumulate_grads(
        _ptr(grad), _ptr(acc), count, 1 if first else 0, _stream(stream)))


def zero_shard_sqnorm_f32(grad, count: int, out, accumulate: bool, workspace, ws_bytes: int | None = None,
                          stream=None):
    if count > 0:
        _need(grad, 4 * count, "gradient")
    _need(out, 8, "output")
    if ws_bytes is None:
        ws_bytes = workspace.numel() * workspace.element_size()
    _check("zero_shard_sqnorm_f32", library().zero_shard_sqnorm_f32(
        _ptr(grad), count, _ptr(out), 1 if accumulate else 0, _ptr(workspace), ws_bytes,
        _stream(stream)))


def zero_state_import(master, m, v, state, n: int, stream=None):
    for x, what in ((master, "master"), (m, "m"), (v, "v")):
        _need(x, 4 * n, what)
    _need(state, 12 * n, "state")
    _check("zero_state_import", library().zero_state_import(
        _ptr(master), _ptr(m), _ptr(v), _ptr(state), n, _stream(stream)))


def zero_state_export(state, master, m, v, n: int, stream=None):
    for x, what in ((master, "master"), (m, "m"), (v, "v")):
        _need(x, 4 * n, what)
    _need(state, 12 * n, "state")
    _check("zero_state_export", library().zero_state_export(
        _ptr(state), _ptr(master), _ptr(m), _ptr(v), n, _stream(stream)))
