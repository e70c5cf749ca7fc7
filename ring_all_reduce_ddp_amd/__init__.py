"""Python binding of libddp_ring.so: the bucketed ring all-reduce of DDP
gradients over N virtual ranks on one MI355X.

The functions have the names of the C entry points in include/ddp_ring.h and
only marshal arguments: torch tensors become device pointers, dtypes become
DDP_FP32 / DDP_BF16, and the stream defaults to torch's current stream. Every
step of the computation runs in the library's HIP kernels; there is no other
code path. The library is loaded on first use; every call fails with an
ImportError naming the build command if it has not been built
(python -m ring_all_reduce_ddp_amd.build).

PyTorch is used for device memory and streams only. It is imported before the
library is loaded so that both use the single HIP runtime that torch ships.
"""

import ctypes
import os
import sys

import torch  # noqa: F401  (loads the HIP runtime the library binds to)

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libddp_ring.so")

DDP_OK = 0
DDP_EINVAL = -1
DDP_EHIP = -2
DDP_ENORESOURCE = -3
DDP_ETIMEOUT = -4
DDP_ENOMEM = -5
DDP_FP32 = 0
DDP_BF16 = 1
DDP_RS = 0
DDP_AG = 1
DDP_MAX_RANKS = 64
VARIANTS = {"fused": 0, "steps": 1, "persistent": 2, "view": 3}

_STATUS_NAMES = {DDP_EINVAL: "DDP_EINVAL", DDP_EHIP: "DDP_EHIP", DDP_ENORESOURCE: "DDP_ENORESOURCE",
                 DDP_ETIMEOUT: "DDP_ETIMEOUT", DDP_ENOMEM: "DDP_ENOMEM"}


class DDPError(RuntimeError):
    """A non-zero status from the library, with ddp_last_error()'s message."""

    def __init__(self, status, message):
        super().__init__(f"{_STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m ring_all_reduce_ddp_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
    pp = ctypes.POINTER(ctypes.c_void_p)
    sig = {
        "ddp_last_error": (ctypes.c_char_p, []),
        "ddp_bucket_plan": (ctypes.c_int, [ctypes.POINTER(i64), i32, i32, i64, i64, i32,
                                           ctypes.POINTER(vp)]),
        "ddp_bucket_plan_ex": (ctypes.c_int, [ctypes.POINTER(i64), i32, i32, i32, i64, i64, i32,
                                              ctypes.POINTER(vp)]),
        "ddp_plan_free": (None, [vp]),
        "ddp_plan_num_buckets": (ctypes.c_int, [vp, ctypes.POINTER(i32)]),
        "ddp_plan_bucket": (ctypes.c_int, [vp, i32, ctypes.POINTER(i64), ctypes.POINTER(i32)]),
        "ddp_plan_member": (ctypes.c_int, [vp, i32, i32, ctypes.POINTER(i32), ctypes.POINTER(i64),
                                           ctypes.POINTER(i64)]),
        "ddp_plan_grad_arena": (ctypes.c_int, [vp, ctypes.POINTER(i64), ctypes.POINTER(i64)]),
        "ddp_plan_arena_map": (ctypes.c_int, [vp, vp, i64]),
        "bucket_pack": (ctypes.c_int, [vp, i32, pp, pp, i32, vp]),
        "bucket_unpack_scale": (ctypes.c_int, [vp, i32, pp, pp, i32, f32, vp]),
        "ring_allreduce_step": (ctypes.c_int, [pp, i32, i64, i32, i32, i32, vp]),
        "ring_allreduce_persistent": (ctypes.c_int, [pp, i32, i64, i32, i32, vp]),
        "ring_allreduce_persistent_ex": (ctypes.c_int, [pp, i32, i64, i32, i32, i32, i64, ctypes.c_uint32, vp]),
        "ring_allreduce_persistent_noalloc": (ctypes.c_int, [pp, i32, i64, i32, i32, vp]),
        "ddp_persistent_test_hook": (ctypes.c_int, [ctypes.c_uint32, i64]),
        "ddp_persistent_grid": (ctypes.c_int, [i32, i64, i32, ctypes.POINTER(i32), ctypes.POINTER(i32)]),
        "ddp_persistent_status": (ctypes.c_int, [vp]),
        "ring_allreduce_fused": (ctypes.c_int, [pp, i32, i64, i32, vp]),
        "bucket_allreduce_view": (ctypes.c_int, [vp, i32, pp, i32, f32, vp]),
        "ring_reduce_scatter_fused": (ctypes.c_int, [pp, pp, i32, i64, i32, f32, vp]),
        "ddp_sync": (ctypes.c_int, [vp, pp, pp, i32, i32, f32, vp]),
        "ddp_reducer_create": (ctypes.c_int, [vp, pp, pp, i32, i32, f32, i64, vp, ctypes.POINTER(vp)]),
        "ddp_reducer_free": (None, [vp]),
        "ddp_reducer_prepare": (ctypes.c_int, [vp]),
        "ddp_reducer_mark_ready": (ctypes.c_int, [vp, i32, vp]),
        "ddp_reducer_finalize": (ctypes.c_int, [vp, vp]),
        "ddp_synthetic_backward": (ctypes.c_int, [pp, pp, i32, i64, i32, i32, i32, vp]),
        "ddp_synthetic_backward_pass": (ctypes.c_int, [vp, pp, pp, i32, i32, i32, vp, vp]),
        "ddp_count_mismatches": (ctypes.c_int, [pp, i32, i64, i32, vp, vp]),
        "ddp_copy_probe": (ctypes.c_int, [vp, vp, i64, vp]),
        "ddp_device_alloc": (ctypes.c_int, [i64, i32, ctypes.POINTER(vp)]),
        "ddp_device_free": (ctypes.c_int, [vp]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


_lib = None


def _get_lib():
    global _lib
    if _lib is None:
        _lib = _load()
    return _lib


def __getattr__(name):
    # `ring_all_reduce_ddp_amd.lib` is the ctypes handle, loaded on first access.
    if name == "lib":
        return _get_lib()
    raise AttributeError(f"module {__name__!r} has no attribute {name!r}")


def _check(status):
    if status != DDP_OK:
        msg = _get_lib().ddp_last_error()
        raise DDPError(status, msg.decode() if msg else "")


# ---------------------------------------------------------------- marshalling helpers

_TORCH_DTYPES = {torch.float32: DDP_FP32, torch.bfloat16: DDP_BF16}
_NAMED_DTYPES = {"fp32": DDP_FP32, "bf16": DDP_BF16, DDP_FP32: DDP_FP32, DDP_BF16: DDP_BF16}


def dtype_code(dtype):
    if dtype in _TORCH_DTYPES:
        return _TORCH_DTYPES[dtype]
    if dtype in _NAMED_DTYPES:
        return _NAMED_DTYPES[dtype]
    raise ValueError(f"unsupported dtype {dtype!r}")


def _ptr(x):
    if isinstance(x, torch.Tensor):
        return x.data_ptr()
    return int(x)


def _ptr_array(xs):
    return (ctypes.c_void_p * len(xs))(*[_ptr(x) for x in xs])


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _ring_args(bufs, count, dtype):
    """(pointer array, N, count, dtype code) from tensors or raw pointers."""
    n = len(bufs)
    if isinstance(bufs[0], torch.Tensor):
        t0 = bufs[0]
        if dtype is None:
            dtype = t0.dtype
        if count is None:
            count = t0.numel()
        for t in bufs:
            if not t.is_contiguous() or t.numel() < count or t.dtype != t0.dtype:
                raise ValueError("rank buffers must be contiguous tensors of one dtype holding count elements")
    if count is None or dtype is None:
        raise ValueError("count and dtype are required for raw pointers")
    return _ptr_array(bufs), n, int(count), dtype_code(dtype)


# ---------------------------------------------------------------- planner

class Plan:
    """A bucket plan (see ddp_bucket_plan). Owns the library's handle."""

    def __init__(self, handle, n_params, dtype, world_size):
        self._h = handle
        self.n_params = n_params
        self.dtype = dtype
        self.comm_dtype = dtype
        self.world_size = world_size

    @property
    def handle(self):
        return self._h

    def free(self):
        if self._h:
            _get_lib().ddp_plan_free(self._h)
            self._h = None

    def __del__(self, _finalizing=sys.is_finalizing):
        # Never while the interpreter shuts down: freeing a plan's device
        # tables calls into the HIP runtime, which may already be going away
        # (the process's memory is returned anyway). The check is bound at
        # definition: module globals such as `sys` may already be None here.
        if _finalizing():
            return
        try:
            self.free()
        except Exception:
            pass

    @property
    def num_buckets(self):
        n = ctypes.c_int32()
        _check(_get_lib().ddp_plan_num_buckets(self._h, ctypes.byref(n)))
        return n.value

    def bucket(self, b):
        """(padded_numel, [(param_index, offset, numel), ...]) of bucket b."""
        padded, nm = ctypes.c_int64(), ctypes.c_int32()
        _check(_get_lib().ddp_plan_bucket(self._h, b, ctypes.byref(padded), ctypes.byref(nm)))
        members = []
        for i in range(nm.value):
            p, off, m = ctypes.c_int32(), ctypes.c_int64(), ctypes.c_int64()
            _check(_get_lib().ddp_plan_member(self._h, b, i, ctypes.byref(p), ctypes.byref(off), ctypes.byref(m)))
            members.append((p.value, off.value, m.value))
        return padded.value, members

    def buckets(self):
        """All buckets as dicts {"members": [...], "padded_numel": int}."""
        out = []
        for b in range(self.num_buckets):
            padded, members = self.bucket(b)
            out.append({"members": members, "padded_numel": padded})
        return out

    def arena_map(self):
        """The in-place sync's per-vector arena map, as a numpy uint16 array."""
        import numpy as np
        n, _ = self.grad_arena()
        v = 16 // (4 if self.dtype == DDP_FP32 else 2)
        out = np.empty(n // v, dtype=np.uint16)
        _check(_get_lib().ddp_plan_arena_map(self._h, out.ctypes.data_as(ctypes.c_void_p), len(out)))
        return out

    def grad_arena(self):
        """(arena_numel, [offset of parameter p in elements])."""
        n = ctypes.c_int64()
        offs = (ctypes.c_int64 * max(self.n_params, 1))()
        _check(_get_lib().ddp_plan_grad_arena(self._h, ctypes.byref(n), offs))
        return n.value, list(offs[:self.n_params])


def ddp_bucket_plan(param_numels, dtype="fp32", cap_bytes=25 * 1024 * 1024,
                    first_bucket_bytes=1024 * 1024, world_size=1):
    numels = (ctypes.c_int64 * max(len(param_numels), 1))(*[int(m) for m in param_numels])
    h = ctypes.c_void_p()
    _check(_get_lib().ddp_bucket_plan(numels, len(param_numels), dtype_code(dtype), int(cap_bytes),
                                      int(first_bucket_bytes), int(world_size), ctypes.byref(h)))
    return Plan(h.value, len(param_numels), dtype_code(dtype), int(world_size))


def ddp_bucket_plan_ex(param_numels, grad_dtype="fp32", comm_dtype="bf16", cap_bytes=25 * 1024 * 1024,
                       first_bucket_bytes=1024 * 1024, world_size=1):
    numels = (ctypes.c_int64 * max(len(param_numels), 1))(*[int(m) for m in param_numels])
    h = ctypes.c_void_p()
    _check(_get_lib().ddp_bucket_plan_ex(numels, len(param_numels), dtype_code(grad_dtype),
                                         dtype_code(comm_dtype), int(cap_bytes), int(first_bucket_bytes),
                                         int(world_size), ctypes.byref(h)))
    plan = Plan(h.value, len(param_numels), dtype_code(grad_dtype), int(world_size))
    plan.comm_dtype = dtype_code(comm_dtype)
    return plan


# ---------------------------------------------------------------- kernels

def bucket_pack(plan, b, grad_arenas, bucket_bufs, stream=None):
    _check(_get_lib().bucket_pack(plan.handle, b, _ptr_array(grad_arenas), _ptr_array(bucket_bufs),
                           len(bucket_bufs), _stream(stream)))


def bucket_unpack_scale(plan, b, bucket_bufs, grad_arenas, scale, stream=None):
    _check(_get_lib().bucket_unpack_scale(plan.handle, b, _ptr_array(bucket_bufs), _ptr_array(grad_arenas),
                                   len(bucket_bufs), float(scale), _stream(stream)))


def ring_allreduce_step(bufs, step, phase, count=None, dtype=None, stream=None):
    ptrs, n, count, dt = _ring_args(bufs, count, dtype)
    _check(_get_lib().ring_allreduce_step(ptrs, n, count, dt, int(step), int(phase), _stream(stream)))


def ring_allreduce_stepwise(bufs, count=None, dtype=None, stream=None):
    """The whole all-reduce as 2(N-1) ring_allreduce_step launches, in order."""
    n = len(bufs)
    for phase in (DDP_RS, DDP_AG):
        for s in range(n - 1):
            ring_allreduce_step(bufs, s, phase, count, dtype, stream)


def ring_allreduce_persistent(bufs, n_steps=None, count=None, dtype=None, stream=None):
    ptrs, n, count, dt = _ring_args(bufs, count, dtype)
    if n_steps is None:
        n_steps = 2 * (n - 1)
    _check(_get_lib().ring_allreduce_persistent(ptrs, n, count, dt, int(n_steps), _stream(stream)))


def ring_allreduce_persistent_ex(bufs, n_steps=None, max_blocks=0, timeout_us=10_000_000,
                                 extra_arrivals=0, count=None, dtype=None, stream=None):
    ptrs, n, count, dt = _ring_args(bufs, count, dtype)
    if n_steps is None:
        n_steps = 2 * (n - 1)
    _check(_get_lib().ring_allreduce_persistent_ex(ptrs, n, count, dt, int(n_steps), int(max_blocks),
                                            int(timeout_us), int(extra_arrivals), _stream(stream)))


def ring_allreduce_persistent_noalloc(bufs, n_steps=None, count=None, dtype=None, stream=None):
    """ring_allreduce_persistent with its barrier words in the library's fixed
    device array instead of an allocation (calls on one GPU must not overlap)."""
    ptrs, n, count, dt = _ring_args(bufs, count, dtype)
    if n_steps is None:
        n_steps = 2 * (n - 1)
    _check(_get_lib().ring_allreduce_persistent_noalloc(ptrs, n, count, dt, int(n_steps), _stream(stream)))


def ddp_persistent_test_hook(extra_arrivals=0, timeout_us=0):
    """Tests of the time-out path only: later default persistent launches
    expect extra_arrivals more blocks and give up after timeout_us (0 resets)."""
    _check(_get_lib().ddp_persistent_test_hook(int(extra_arrivals), int(timeout_us)))


def ddp_persistent_grid(n, count, dtype="fp32"):
    """(grid, compute units) the persistent launch would use."""
    g, cu = ctypes.c_int32(), ctypes.c_int32()
    _check(_get_lib().ddp_persistent_grid(int(n), int(count), dtype_code(dtype), ctypes.byref(g), ctypes.byref(cu)))
    return g.value, cu.value


def ddp_persistent_status(stream=None):
    _check(_get_lib().ddp_persistent_status(_stream(stream)))


def ring_allreduce_fused(bufs, count=None, dtype=None, stream=None):
    ptrs, n, count, dt = _ring_args(bufs, count, dtype)
    _check(_get_lib().ring_allreduce_fused(ptrs, n, count, dt, _stream(stream)))


def bucket_allreduce_view(plan, b, grad_arenas, scale, stream=None):
    _check(_get_lib().bucket_allreduce_view(plan.handle, b, _ptr_array(grad_arenas), len(grad_arenas),
                                     float(scale), _stream(stream)))


def ring_reduce_scatter_fused(bufs, shards, scale=1.0, count=None, dtype=None, stream=None):
    """shards[c] receives chunk c of the ring sum (times scale); None for an
    empty chunk."""
    ptrs, n, count, dt = _ring_args(bufs, count, dtype)
    sh = (ctypes.c_void_p * n)(*[None if x is None else _ptr(x) for x in shards])
    _check(_get_lib().ring_reduce_scatter_fused(ptrs, sh, n, count, dt, float(scale), _stream(stream)))


def ddp_sync(plan, grad_arenas, bucket_bufs=None, *, scale, variant="fused", stream=None):
    """bucket_bufs: list over buckets of lists over ranks (or a flat list,
    bucket-major); None for the "view" variant, which uses no bucket buffers.
    scale: the fp32 multiplier of the copy back, chosen by the caller (1/N
    for DDP's mean)."""
    n = len(grad_arenas)
    if bucket_bufs is None:
        bufs = None
    else:
        flat = [x for row in bucket_bufs for x in row] if isinstance(bucket_bufs[0], (list, tuple)) \
            else list(bucket_bufs)
        bufs = _ptr_array(flat)
    _check(_get_lib().ddp_sync(plan.handle, _ptr_array(grad_arenas), bufs, n, VARIANTS[variant], float(scale),
                        _stream(stream)))


class Reducer:
    """Launches each bucket's sync as soon as its last gradient is marked
    ready, on `comm_stream` (see ddp_reducer_* in include/ddp_ring.h).
    bucket_bufs: list over buckets of lists over ranks; None for "view".
    scale: the fp32 multiplier of each bucket's copy back (1/N for DDP's
    mean), chosen by the caller."""

    def __init__(self, plan, grad_arenas, bucket_bufs=None, *, scale, variant="view", comm_stream=None,
                 comm_max_blocks=0):
        n = len(grad_arenas)
        self.plan = plan   # the plan must outlive the reducer
        if bucket_bufs is None:
            bufs = None
        else:
            flat = [x for row in bucket_bufs for x in row] if isinstance(bucket_bufs[0], (list, tuple)) \
                else list(bucket_bufs)
            bufs = _ptr_array(flat)
        h = ctypes.c_void_p()
        _check(_get_lib().ddp_reducer_create(plan.handle, _ptr_array(grad_arenas), bufs, n, VARIANTS[variant],
                                             float(scale), int(comm_max_blocks),
                                             _stream(comm_stream), ctypes.byref(h)))
        self._h = h.value

    def prepare(self):
        _check(_get_lib().ddp_reducer_prepare(self._h))

    def mark_ready(self, param, stream=None):
        _check(_get_lib().ddp_reducer_mark_ready(self._h, int(param), _stream(stream)))

    def finalize(self, stream=None):
        _check(_get_lib().ddp_reducer_finalize(self._h, _stream(stream)))

    def free(self):
        if self._h:
            _get_lib().ddp_reducer_free(self._h)
            self._h = None

    def __del__(self, _finalizing=sys.is_finalizing):
        if _finalizing():   # as for Plan: no HIP calls during shutdown
            return
        try:
            self.free()
        except Exception:
            pass


def ddp_synthetic_backward(srcs, dsts, work, lds_kib=0, numel=None, dtype=None, stream=None):
    """dsts[r][:numel] = srcs[r][:numel] after `work` FMAs per element (a
    stand-in for the backward kernels that produce gradients)."""
    ptrs, n, numel, dt = _ring_args(srcs, numel, dtype)
    _check(_get_lib().ddp_synthetic_backward(ptrs, _ptr_array(dsts), n, numel, dt, int(work), int(lds_kib),
                                             _stream(stream)))


def ddp_synthetic_backward_pass(plan, src_arenas, grad_arenas, work, reducer=None, lds_kib=0, stream=None):
    """One synthetic backward over the plan's parameters in reverse order,
    marking each gradient ready on `reducer` (if given) as it is produced."""
    _check(_get_lib().ddp_synthetic_backward_pass(plan.handle, _ptr_array(src_arenas), _ptr_array(grad_arenas),
                                                  len(grad_arenas), int(work), int(lds_kib),
                                                  None if reducer is None else reducer._h, _stream(stream)))


def ddp_count_mismatches(bufs, out, count=None, dtype=None, stream=None):
    """Enqueues the count into `out` (a device int64/uint64 tensor of one element)."""
    ptrs, n, count, dt = _ring_args(bufs, count, dtype)
    _check(_get_lib().ddp_count_mismatches(ptrs, n, count, dt, ctypes.c_void_p(_ptr(out)), _stream(stream)))


DDP_ALLOC_CONTIGUOUS = 1

_TORCH_TYPESTR = {torch.float32: "<f4", torch.bfloat16: "<V2", torch.uint8: "|u1"}


class DeviceBuffer:
    """Device memory from ddp_device_alloc, owned by this object (freed by
    free() or when it is collected). `ptr` is the device address; tensor()
    gives a torch view of it (the buffer must outlive the view)."""

    def __init__(self, ptr, nbytes, contiguous):
        self.ptr = ptr
        self.nbytes = nbytes
        self.contiguous = contiguous

    def tensor(self, dtype=torch.float32, numel=None, offset_bytes=0):
        """A 1-D tensor of `numel` elements at ptr + offset_bytes (no copy)."""
        esize = torch.empty((), dtype=dtype).element_size()
        if numel is None:
            numel = (self.nbytes - offset_bytes) // esize
        if self.ptr is None or offset_bytes < 0 or offset_bytes % esize or offset_bytes + numel * esize > self.nbytes:
            raise ValueError("the view does not fit in the buffer")
        # bfloat16 has no array-interface type string: view the bytes, then reinterpret
        view_dtype = dtype if dtype in (torch.float32, torch.uint8) else torch.uint8
        n = numel if view_dtype is dtype else numel * esize

        class _Iface:
            __cuda_array_interface__ = {"shape": (n,), "typestr": _TORCH_TYPESTR[view_dtype],
                                        "data": (self.ptr + offset_bytes, False), "version": 2}
        t = torch.as_tensor(_Iface(), device=torch.device("cuda", torch.cuda.current_device()))
        return t if view_dtype is dtype else t.view(dtype)

    def free(self):
        if self.ptr is not None:
            _check(_get_lib().ddp_device_free(ctypes.c_void_p(self.ptr)))
            self.ptr = None

    def __del__(self, _finalizing=sys.is_finalizing):
        if _finalizing():
            return
        try:
            self.free()
        except Exception:
            pass


def device_alloc(nbytes, contiguous=True):
    """nbytes of device memory on the current device (ddp_device_alloc);
    contiguous=True asks for physically contiguous memory."""
    p = ctypes.c_void_p()
    _check(_get_lib().ddp_device_alloc(int(nbytes), DDP_ALLOC_CONTIGUOUS if contiguous else 0, ctypes.byref(p)))
    return DeviceBuffer(p.value, int(nbytes), bool(contiguous))


def ddp_copy_probe(dst, src, nbytes=None, stream=None):
    if nbytes is None:
        nbytes = src.numel() * src.element_size()
    _check(_get_lib().ddp_copy_probe(ctypes.c_void_p(_ptr(dst)), ctypes.c_void_p(_ptr(src)), int(nbytes),
                              _stream(stream)))
