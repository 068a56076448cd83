"""Python binding of libzero.so, the MI355X ZeRO sharded optimizer step.

Argument marshalling only: every entry point here forwards to the C function
of the same name declared in ``include/zero.h``; all step arithmetic runs in
the library's HIP kernels.  torch tensors supply device memory (``data_ptr``)
and streams (``torch.cuda.current_stream().cuda_stream``).  There is no CPU
fallback: importing this package raises if the built library is missing.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Sequence

import numpy as np

# torch carries its own HIP runtime (SONAME libamdhip64.so.7, the same as
# ROCm's).  Loading torch first makes libzero.so's dependency resolve to that
# already-loaded runtime; loading libzero.so first would map a second HIP
# runtime into the process, and whichever initialises second sees no device.
import torch  # noqa: F401  (must precede the CDLL below)

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libzero.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python fsdp_sharded_optimizer_flat_amd/_build.py` "
        "(there is no CPU fallback for the sharded step)")

_lib = C.CDLL(LIB_PATH)

# -- constants mirrored from zero.h -------------------------------------------
ZERO_OK, ZERO_EINVAL, ZERO_ERANGE, ZERO_EALIGN, ZERO_ENOSPC, ZERO_EHIP = 0, -1, -2, -3, -4, -5
ZERO_EIO, ZERO_ECORRUPT = -6, -7
ZERO_F32, ZERO_BF16 = 0, 1
ZERO_GLOBAL, ZERO_LOCAL = 0, 1
ZERO_MAX_RANKS = 256
ZERO_LAYOUT_MAGIC = 0x5A45524F
ZERO_ABI_VERSION = 2
ZERO_NOALLOC_SCRATCH_BYTES = 16 << 20
ZERO_CAP_STEP, ZERO_CAP_STEP1, ZERO_CAP_NORM = 0, 1, 2

i32, i64, f32, f64, vp, sz = C.c_int32, C.c_int64, C.c_float, C.c_double, C.c_void_p, C.c_size_t


class ZeroUnit(C.Structure):
    _fields_ = [("numel", i64), ("padded", i64), ("shard", i64), ("offset", i64),
                ("local_offset", i64), ("granule", i64)]


class ZeroLayoutHeader(C.Structure):
    _fields_ = [("magic", C.c_uint32), ("n_ranks", i32), ("n_units", i32), ("reserved", i32),
                ("numel", i64), ("padded", i64), ("shard", i64)]


class ZeroAdamwScalars(C.Structure):
    _fields_ = [("t", i32), ("lr", f32), ("b1", f32), ("b2", f32), ("eps", f32), ("wd", f32),
                ("one_minus_b1", f32), ("one_minus_b2", f32), ("pow1", f32), ("pow2", f32),
                ("bc1", f32), ("bc2", f32), ("step_size", f32), ("decay", f32),
                ("clip_coef", f32)]

    def as_dict(self):
        return {k: getattr(self, k) for k, _ in self._fields_}


class ZeroOverlapOut(C.Structure):
    _fields_ = [("gather_bytes", f64), ("gather_s", f64), ("compute_flops", f64),
                ("compute_s", f64), ("ratio", f64), ("hidden", i32), ("reserved", i32)]

    def as_dict(self):
        return {k: getattr(self, k) for k, _ in self._fields_ if k != "reserved"}


class ZeroLedgerOut(C.Structure):
    _fields_ = [("params_bytes", f64), ("grads_bytes", f64), ("optim_bytes", f64),
                ("model_state_bytes", f64), ("comm_elements", f64),
                ("comm_elements_ring", f64), ("optimizer_floats_per_rank", f64)]

    def as_dict(self):
        return {k: getattr(self, k) for k, _ in self._fields_}


class ZeroFootprintOut(C.Structure):
    _fields_ = [("grads_bytes", f64), ("state_bytes", f64), ("out_bytes", f64), ("g_bytes", f64),
                ("total_bytes", f64)]

    def as_dict(self):
        return {k: getattr(self, k) for k, _ in self._fields_}


class ZeroCkptInfo(C.Structure):
    _fields_ = [("format", i32), ("abi", i32), ("n_ranks", i32), ("n_units", i32), ("rank", i32),
                ("step", i32), ("numel", i64), ("shard", i64)]

    def as_dict(self):
        return {k: getattr(self, k) for k, _ in self._fields_}


def _sig(name, res, *args):
    fn = getattr(_lib, name)
    fn.restype = res
    fn.argtypes = list(args)
    return fn


_zero_layout_bytes = _sig("zero_layout_bytes", sz, i32)
_zero_pack = _sig("zero_pack", i32, i32, i32, vp, vp, sz, C.POINTER(sz))
_zero_pack_rows = _sig("zero_pack_rows", i32, i32, i32, vp, vp, vp, sz, C.POINTER(sz))
_zero_reshard = _sig("zero_reshard", i32, vp, vp, vp, i32, vp, i32, vp)
_zero_reshard_host = _sig("zero_reshard_host", i32, vp, vp, vp, i32, vp, i32)
_zero_reshard_traffic = _sig("zero_reshard_traffic", i32, vp, vp, i32, i32, C.POINTER(f64),
                             C.POINTER(i64))
_zero_global_index = _sig("zero_global_index", i32, vp, i32, i64, C.POINTER(i64))
_zero_owner = _sig("zero_owner", i32, vp, i64, C.POINTER(i32), C.POINTER(i64))
_zero_pack_copy = _sig("zero_pack_copy", i32, vp, i32, i32, vp, vp, vp, i32, vp, i32, vp)
_zero_unpack_copy = _sig("zero_unpack_copy", i32, vp, i32, vp, i32, i32, vp, vp, vp, i32, vp)
_zero_adamw_scalars_for = _sig("zero_adamw_scalars_for", i32, i32, f32, f32, f32, f32, f32, f32,
                               C.POINTER(ZeroAdamwScalars))
_zero_adamw_scalars_next = _sig("zero_adamw_scalars_next", i32, C.POINTER(ZeroAdamwScalars),
                                C.POINTER(ZeroAdamwScalars))
_zero_step = _sig("zero_step", i32, vp, i32, vp, i32, i32, i32, f32, vp, vp, vp, i32, vp, i32,
                  C.POINTER(ZeroAdamwScalars), vp)
_zero_step_staged = _sig("zero_step_staged", i32, vp, i32, vp, i32, i32, i32, f32, vp, vp, vp, i32, vp,
                         i32, C.POINTER(ZeroAdamwScalars), vp, sz, vp)
_zero_step_units = _sig("zero_step_units", i32, vp, i32, i32, i32, vp, i32, i32, i32, f32, vp, vp, vp,
                        i32, vp, i32, C.POINTER(ZeroAdamwScalars), vp, sz, vp)
_zero_step_staged_workspace_bytes = _sig("zero_step_staged_workspace_bytes", i32, vp, i32, i32,
                                         C.POINTER(sz))
_zero_step_device_clip = _sig("zero_step_device_clip", i32, vp, i32, vp, i32, i32, i32, f32, vp, vp,
                              vp, i32, vp, i32, C.POINTER(ZeroAdamwScalars), vp, vp)
_zero_clip_coef_async = _sig("zero_clip_coef_async", i32, vp, f64, vp, vp)
_zero_clip_coef_ranks = _sig("zero_clip_coef_ranks", i32, vp, i32, f64, C.POINTER(f32),
                             C.POINTER(f64))
_zero_clip_coef_ranks_async = _sig("zero_clip_coef_ranks_async", i32, vp, i32, f64, vp, vp, vp)
_zero_overlap = _sig("zero_overlap", i32, f64, i32, f64, f64, f64, C.POINTER(ZeroOverlapOut))
_zero_step_host = _sig("zero_step_host", i32, vp, i32, vp, i32, i32, i32, f32, vp, vp, vp, i32, vp,
                       i32, C.POINTER(ZeroAdamwScalars), i32)
_zero_offload_step = _sig("zero_offload_step", i32, vp, i32, vp, vp, vp, vp, vp, vp, vp, i64,
                          C.POINTER(ZeroAdamwScalars), i32, vp, vp)
_zero_gradnorm_workspace_bytes = _sig("zero_gradnorm_workspace_bytes", i32, vp, i32,
                                      C.POINTER(sz))
_zero_gradnorm = _sig("zero_gradnorm", i32, vp, i32, vp, i32, i32, i32, f32, vp, i32, vp, sz,
                      C.POINTER(f64), vp)
_zero_gradnorm_async = _sig("zero_gradnorm_async", i32, vp, i32, vp, i32, i32, i32, f32, vp, i32, vp,
                            sz, vp, vp)
_zero_gradnorm_async_noalloc = _sig("zero_gradnorm_async_noalloc", i32, vp, i32, vp, i32, i32, i32,
                                    f32, vp, i32, vp, vp)
_zero_clip_coef = _sig("zero_clip_coef", i32, f64, f64, C.POINTER(f32))
_zero_ledger = _sig("zero_ledger", i32, f64, i32, i32, i32, C.POINTER(ZeroLedgerOut))
_zero_sim_footprint = _sig("zero_sim_footprint", i32, vp, i32, i32, i32, i32, i32, i32, i32,
                          C.POINTER(ZeroFootprintOut))
_zero_gather_buffer_bytes = _sig("zero_gather_buffer_bytes", i32, vp, i32, C.POINTER(f64))
_zero_arena_plan = _sig("zero_arena_plan", i32, i32, vp, vp, C.POINTER(i64))
_zero_step_traffic = _sig("zero_step_traffic", i32, vp, i32, i32, i32, i32, C.POINTER(f64),
                          C.POINTER(i64))
_zero_gradnorm_traffic = _sig("zero_gradnorm_traffic", i32, vp, i32, i32, i32, i32,
                              C.POINTER(f64), C.POINTER(i64))
_zero_ckpt_save = _sig("zero_ckpt_save", i32, C.c_char_p, vp, i32, i32, vp, vp, vp)
_zero_ckpt_inspect = _sig("zero_ckpt_inspect", i32, C.c_char_p, i32, C.POINTER(ZeroCkptInfo), vp, sz,
                          C.POINTER(sz))
_zero_ckpt_load = _sig("zero_ckpt_load", i32, vp, i32, vp, i32, i32, C.POINTER(i32), vp, vp, vp)
_zero_set_waves_per_cu = _sig("zero_set_waves_per_cu", i32, i32, i32)
_zero_get_waves_per_cu = _sig("zero_get_waves_per_cu", i32, i32, i32, C.POINTER(i32))
_zero_get_waves_per_cu_for = _sig("zero_get_waves_per_cu_for", i32, i32, i32, i32, i32, C.POINTER(i32))
_zero_strerror = _sig("zero_strerror", C.c_char_p, i32)
_zero_last_hip_error = _sig("zero_last_hip_error", C.c_char_p)
_zero_abi_version = _sig("zero_abi_version", i32)

EXPORTED = ["zero_layout_bytes", "zero_pack", "zero_pack_rows", "zero_reshard",
            "zero_reshard_host", "zero_reshard_traffic", "zero_global_index", "zero_owner", "zero_pack_copy",
            "zero_unpack_copy", "zero_adamw_scalars_for", "zero_adamw_scalars_next", "zero_step",
            "zero_step_staged", "zero_step_staged_workspace_bytes", "zero_step_units",
            "zero_step_host", "zero_offload_step", "zero_step_device_clip",
            "zero_clip_coef_async", "zero_clip_coef_ranks", "zero_clip_coef_ranks_async",
            "zero_overlap",
            "zero_gradnorm_workspace_bytes", "zero_gradnorm", "zero_gradnorm_async",
            "zero_gradnorm_async_noalloc",
            "zero_clip_coef", "zero_ledger", "zero_sim_footprint",
            "zero_gather_buffer_bytes", "zero_arena_plan", "zero_step_traffic",
            "zero_gradnorm_traffic", "zero_ckpt_save", "zero_ckpt_inspect", "zero_ckpt_load",
            "zero_set_waves_per_cu", "zero_get_waves_per_cu", "zero_get_waves_per_cu_for",
            "zero_strerror", "zero_last_hip_error", "zero_abi_version"]


class ZeroError(RuntimeError):
    def __init__(self, status: int, where: str):
        msg = _zero_strerror(status).decode()
        if status == ZERO_EHIP:
            msg += ": " + _zero_last_hip_error().decode()
        super().__init__(f"{where}: {msg} ({status})")
        self.status = status


def _check(status: int, where: str):
    if status != ZERO_OK:
        raise ZeroError(status, where)


# -- tensor marshalling ---------------------------------------------------------

def _torch():
    import torch
    return torch


def _dev_ptr(t, what: str) -> int:
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{what} must be a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{what} must be a device tensor (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    return t.data_ptr()


def _grad_dtype(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return ZERO_BF16
    if t.dtype == torch.float32:
        return ZERO_F32
    raise TypeError(f"gradient dtype must be bfloat16 or float32, got {t.dtype}")


def _f32_ptr(t, what):
    torch = _torch()
    if t.dtype != torch.float32:
        raise TypeError(f"{what} must be float32")
    return _dev_ptr(t, what)


def _bf16_ptr(t, what):
    torch = _torch()
    if t.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise TypeError(f"{what} must hold bf16 bits (bfloat16, int16 or uint16)")
    return _dev_ptr(t, what)


def _stream(stream):
    if stream is None:
        return _torch().cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _numel(t) -> int:
    return int(t.numel()) if hasattr(t, "numel") and callable(t.numel) else int(np.asarray(t).size)


def _need(t, n: int, what: str):
    """Refuse a buffer with fewer elements than the call reads or writes: the
    library sees only pointers, so a short buffer would be overrun."""
    if t is not None and _numel(t) < n:
        raise ValueError(f"{what} holds {_numel(t)} elements; the call needs {n}")


def _extent(layout, index: int) -> int:
    """Elements of a buffer in the given index space: P^ (GLOBAL) or S (LOCAL)."""
    return int(layout.padded) if index == ZERO_GLOBAL else int(layout.shard)


def _need_step(layout, grads, grad_index, master, exp_avg, exp_avg_sq, state_index, out,
               out_index):
    ge, se = _extent(layout, grad_index), _extent(layout, state_index)
    for g in grads:
        _need(g, ge, "grad")
    for t, what in ((master, "master"), (exp_avg, "exp_avg"), (exp_avg_sq, "exp_avg_sq")):
        _need(t, se, what)
    _need(out, _extent(layout, out_index), "out")


# -- layout -------------------------------------------------------------------------

class Layout:
    """A filled ``zero_layout`` in host memory (the library's own copy)."""

    def __init__(self, buf: C.Array):
        self._buf = buf
        self.header = ZeroLayoutHeader.from_buffer(buf)
        n = self.header.n_units
        self.units = (ZeroUnit * n).from_buffer(buf, C.sizeof(ZeroLayoutHeader))

    @property
    def ptr(self) -> int:
        return C.addressof(self._buf)

    n_ranks = property(lambda s: s.header.n_ranks)
    n_units = property(lambda s: s.header.n_units)
    numel = property(lambda s: s.header.numel)
    padded = property(lambda s: s.header.padded)
    shard = property(lambda s: s.header.shard)

    def unit_table(self) -> np.ndarray:
        """(U, 5) int64: numel, padded, shard, offset, local_offset."""
        return np.array([[u.numel, u.padded, u.shard, u.offset, u.local_offset]
                         for u in self.units], dtype=np.int64).reshape(-1, 5)

    def unit_granules(self) -> np.ndarray:
        """(U,) int64: each unit's granule (1 for the flat layout)."""
        return np.array([u.granule for u in self.units], dtype=np.int64)


def zero_layout_bytes(n_units: int) -> int:
    return int(_zero_layout_bytes(n_units))


def zero_pack(n_ranks: int, unit_numel: Sequence[int]) -> Layout:
    numel = np.ascontiguousarray(unit_numel, dtype=np.int64)
    need = sz()
    _check(_zero_pack(n_ranks, len(numel), numel.ctypes.data if len(numel) else None, None, 0,
                      C.byref(need)), "zero_pack")
    buf = (C.c_char * need.value)()
    _check(_zero_pack(n_ranks, len(numel), numel.ctypes.data if len(numel) else None,
                      C.addressof(buf), need.value, None), "zero_pack")
    return Layout(buf)


def zero_pack_rows(n_ranks: int, unit_numel: Sequence[int], unit_granule: Sequence[int]) -> Layout:
    """Row-aligned layout: unit u pads to a multiple of n_ranks * granule[u]."""
    numel = np.ascontiguousarray(unit_numel, dtype=np.int64)
    gran = np.ascontiguousarray(unit_granule, dtype=np.int64)
    if len(gran) != len(numel):
        raise ValueError("one granule per unit")
    args = (n_ranks, len(numel), numel.ctypes.data if len(numel) else None,
            gran.ctypes.data if len(gran) else None)
    need = sz()
    _check(_zero_pack_rows(*args, None, 0, C.byref(need)), "zero_pack_rows")
    buf = (C.c_char * need.value)()
    _check(_zero_pack_rows(*args, C.addressof(buf), need.value, None), "zero_pack_rows")
    return Layout(buf)


def zero_pack_params(n_ranks: int, shapes, *, rows: bool) -> Layout:
    """One unit per parameter shape: the row-aligned (FSDP2, dim-0) layout
    when ``rows``, else per-parameter flat units."""
    numel = [int(np.prod(s)) for s in shapes]
    if not rows:
        return zero_pack(n_ranks, numel)
    return zero_pack_rows(n_ranks, numel, [int(np.prod(s[1:])) if len(s) > 1 else 1 for s in shapes])


def zero_global_index(layout: Layout, rank: int, k: int) -> int:
    j = i64()
    _check(_zero_global_index(layout.ptr, rank, k, C.byref(j)), "zero_global_index")
    return j.value


def zero_owner(layout: Layout, j: int):
    r, k = i32(), i64()
    _check(_zero_owner(layout.ptr, j, C.byref(r), C.byref(k)), "zero_owner")
    return r.value, k.value


def _param_arrays(params, units):
    torch = _torch()
    n = len(params)
    ptrs = (vp * max(n, 1))(*[_dev_ptr(p, "param") for p in params])
    numel = np.ascontiguousarray([p.numel() for p in params], dtype=np.int64)
    unit = np.ascontiguousarray(units, dtype=np.int32)
    if len(unit) != n:
        raise ValueError("one unit id per parameter")
    dt = {torch.float32: ZERO_F32, torch.bfloat16: ZERO_BF16}
    dts = {dt.get(p.dtype, -1) for p in params}
    if len(dts) > 1 or -1 in dts:
        raise TypeError("parameters must all be float32 or all bfloat16")
    return ptrs, numel, unit, (dts.pop() if dts else ZERO_F32)


def _flat_dtype(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return ZERO_F32
    if t.dtype in (torch.bfloat16, torch.int16, torch.uint16):
        return ZERO_BF16
    raise TypeError("flat buffer must be float32 or bf16")


def zero_pack_copy(layout: Layout, rank: int, params, units, dst, stream=None):
    ptrs, numel, unit, sdt = _param_arrays(params, units)
    _need(dst, layout.padded if rank < 0 else layout.shard, "dst")
    _check(_zero_pack_copy(layout.ptr, rank, len(params), C.addressof(ptrs), numel.ctypes.data,
                           unit.ctypes.data, sdt, _dev_ptr(dst, "dst"), _flat_dtype(dst),
                           _stream(stream)), "zero_pack_copy")


def zero_unpack_copy(layout: Layout, rank: int, src, params, units, stream=None):
    ptrs, numel, unit, ddt = _param_arrays(params, units)
    _need(src, layout.padded if rank < 0 else layout.shard, "src")
    _check(_zero_unpack_copy(layout.ptr, rank, _dev_ptr(src, "src"), _flat_dtype(src),
                             len(params), C.addressof(ptrs), numel.ctypes.data, unit.ctypes.data,
                             ddt, _stream(stream)), "zero_unpack_copy")


def _reshard_dtype(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return ZERO_F32
    if t.dtype in (torch.bfloat16, torch.int16, torch.uint16):
        return ZERO_BF16
    raise TypeError("reshard buffers must be float32 or 16-bit (bf16 bits)")


def reshard_pointer_array(src):
    """The sources of zero_reshard marshalled once: ``(array, dtype)`` for
    ``src_ptrs=`` in loops that reshard the same buffers repeatedly."""
    dts = {_reshard_dtype(t) for t in src}
    if len(dts) > 1:
        raise TypeError("sources must share one element type")
    arr = (vp * max(len(src), 1))(*[_dev_ptr(t, "src") for t in src])
    return _prepared((arr, (dts.pop() if dts else None), len(src)), src)


def zero_reshard(src_layout: Layout, src, dst_layout: Layout, dst_rank: int, dst, stream=None, *,
                 src_ptrs=None):
    """Fill device tensor ``dst`` with rank dst_rank's local shard under
    dst_layout, from the device tensors ``src`` (one local shard per rank of
    src_layout).  Asynchronous on ``stream``.  ``src_ptrs`` (from
    :func:`reshard_pointer_array`) skips re-marshalling ``src``."""
    arr, sdt, ns = src_ptrs if src_ptrs is not None else reshard_pointer_array(src)
    if ns != src_layout.n_ranks:
        raise ValueError("one source shard per rank of the source layout")
    if src_ptrs is None:
        for t in src:
            _need(t, src_layout.shard, "src")
    _need_prepared(src_ptrs, src_layout.shard, "src")
    _need(dst, dst_layout.shard, "dst")
    dt = _reshard_dtype(dst)
    if sdt is not None and sdt != dt:
        raise TypeError("sources and destination must share one element type")
    _check(_zero_reshard(src_layout.ptr, C.addressof(arr), dst_layout.ptr, dst_rank,
                         _dev_ptr(dst, "dst"), dt, _stream(stream)), "zero_reshard")


def zero_reshard_host(src_layout: Layout, src, dst_layout: Layout, dst_rank: int, dst):
    """zero_reshard on host buffers (numpy arrays or CPU tensors); synchronous."""
    if len(src) != src_layout.n_ranks:
        raise ValueError("one source shard per rank of the source layout")
    for t in src:
        _need(t, src_layout.shard, "src")
    _need(dst, dst_layout.shard, "dst")
    sp = [_host_ptr(t, "src", "grad") for t in src]
    dp, dk = _host_ptr(dst, "dst", "grad")
    if any(k != dk for _, k in sp):
        raise TypeError("sources and destination must share one element type")
    arr = (vp * max(len(sp), 1))(*[p for p, _ in sp])
    _check(_zero_reshard_host(src_layout.ptr, C.addressof(arr), dst_layout.ptr, dst_rank, dp,
                              ZERO_F32 if dk == "f32" else ZERO_BF16), "zero_reshard_host")


def zero_reshard_traffic(src_layout: Layout, dst_layout: Layout, dst_rank: int, dtype: int):
    b, e = f64(), i64()
    _check(_zero_reshard_traffic(src_layout.ptr, dst_layout.ptr, dst_rank, dtype, C.byref(b),
                                 C.byref(e)), "zero_reshard_traffic")
    return b.value, e.value


# -- scalars ------------------------------------------------------------------------------

def zero_adamw_scalars_for(t: int, lr: float, b1: float, b2: float, eps: float, wd: float,
                           clip_coef: float = 1.0) -> ZeroAdamwScalars:
    s = ZeroAdamwScalars()
    _check(_zero_adamw_scalars_for(t, lr, b1, b2, eps, wd, clip_coef, C.byref(s)),
           "zero_adamw_scalars_for")
    return s


def zero_adamw_scalars_next(prev: ZeroAdamwScalars) -> ZeroAdamwScalars:
    s = ZeroAdamwScalars()
    _check(_zero_adamw_scalars_next(C.byref(prev), C.byref(s)), "zero_adamw_scalars_next")
    return s


def zero_clip_coef(sumsq: float, max_norm: float) -> float:
    c = f32()
    _check(_zero_clip_coef(sumsq, max_norm, C.byref(c)), "zero_clip_coef")
    return c.value


# -- the step and the norm -------------------------------------------------------------

class _Prepared(tuple):
    """Marshalled buffer pointers; ``min_numel`` is the smallest buffer's
    element count, so calls taking them still refuse short buffers."""
    min_numel = 0


def _prepared(items, buffers):
    p = _Prepared(items)
    p.min_numel = min((_numel(b) for b in buffers), default=0)
    return p


def _grad_ptrs(grads):
    if len(grads) < 1:
        raise ValueError("at least one gradient buffer")
    gdt = {_grad_dtype(g) for g in grads}
    if len(gdt) != 1:
        raise TypeError("all gradient buffers must share one dtype")
    arr = (vp * len(grads))(*[_dev_ptr(g, "grad") for g in grads])
    return _prepared((arr, gdt.pop()), grads)


def _need_prepared(prepared, n: int, what: str):
    if prepared is not None and getattr(prepared, "min_numel", n) < n:
        raise ValueError(f"a {what} buffer holds {prepared.min_numel} elements; the call needs {n}")


def zero_step(layout: Layout, rank: int, grads, grad_index: int, divisor: float,
              master, exp_avg, exp_avg_sq, state_index: int, out, out_index: int,
              scalars: ZeroAdamwScalars, stream=None, *, grad_ptrs=None):
    """Enqueue the fused step.  ``grads``: list of device tensors (bf16 or
    fp32), summed in list order.  ``grad_ptrs`` (a prepared ``(array, dtype)``
    from :func:`grad_pointer_array`) skips re-marshalling in timed loops."""
    arr, gdt = grad_ptrs if grad_ptrs is not None else _grad_ptrs(grads)
    _need_step(layout, grads if grad_ptrs is None else (), grad_index, master, exp_avg, exp_avg_sq,
               state_index, out, out_index)
    _need_prepared(grad_ptrs, _extent(layout, grad_index), "grad")
    _check(_zero_step(layout.ptr, rank, C.addressof(arr), len(arr), gdt, grad_index, divisor,
                      _f32_ptr(master, "master"), _f32_ptr(exp_avg, "exp_avg"),
                      _f32_ptr(exp_avg_sq, "exp_avg_sq"), state_index,
                      _bf16_ptr(out, "out") if out is not None else None, out_index,
                      C.byref(scalars), _stream(stream)), "zero_step")


def zero_step_staged(layout: Layout, rank: int, grads, grad_index: int, divisor: float,
                     master, exp_avg, exp_avg_sq, state_index: int, out, out_index: int,
                     scalars: ZeroAdamwScalars, workspace, stream=None, *, grad_ptrs=None):
    """Enqueue the staged step (zero_step's result, two kernels per chunk
    through ``workspace``, a device tensor; None where the fused step runs:
    up to 32 bf16 or 24 fp32 gradients)."""
    arr, gdt = grad_ptrs if grad_ptrs is not None else _grad_ptrs(grads)
    _need_step(layout, grads if grad_ptrs is None else (), grad_index, master, exp_avg, exp_avg_sq,
               state_index, out, out_index)
    _need_prepared(grad_ptrs, _extent(layout, grad_index), "grad")
    wp = _dev_ptr(workspace, "workspace") if workspace is not None else None
    wb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(_zero_step_staged(layout.ptr, rank, C.addressof(arr), len(arr), gdt, grad_index, divisor,
                             _f32_ptr(master, "master"), _f32_ptr(exp_avg, "exp_avg"),
                             _f32_ptr(exp_avg_sq, "exp_avg_sq"), state_index,
                             _bf16_ptr(out, "out") if out is not None else None, out_index,
                             C.byref(scalars), wp, wb, _stream(stream)), "zero_step_staged")


def unit_range_extent(layout: Layout, unit_begin: int, unit_end: int, index: int) -> int:
    """Elements of a gradient bucket holding units [unit_begin, unit_end) in an
    index space (padded sizes for GLOBAL, shard sizes for LOCAL)."""
    col = 1 if index == ZERO_GLOBAL else 2
    t = layout.unit_table()
    return int(t[unit_begin:unit_end, col].sum()) if unit_end > unit_begin else 0


def zero_step_units(layout: Layout, rank: int, unit_begin: int, unit_end: int, grads,
                    grad_index: int, divisor: float, master, exp_avg, exp_avg_sq,
                    state_index: int, out, out_index: int, scalars: ZeroAdamwScalars,
                    workspace=None, stream=None, *, grad_ptrs=None):
    """Enqueue the step of units [unit_begin, unit_end) from gradient buckets
    that hold only those units (see zero.h); state and out are the whole
    buffers.  ``workspace`` (device tensor) selects the staged path above 32
    bf16 or 24 fp32 gradients."""
    arr, gdt = grad_ptrs if grad_ptrs is not None else _grad_ptrs(grads)
    if not (0 <= unit_begin <= unit_end <= layout.n_units):
        raise ValueError("unit range outside the layout")
    ge = unit_range_extent(layout, unit_begin, unit_end, grad_index)
    if grad_ptrs is None:
        for g in grads:
            _need(g, ge, "grad")
    _need_prepared(grad_ptrs, ge, "grad")
    _need_step(layout, (), grad_index, master, exp_avg, exp_avg_sq, state_index, out, out_index)
    wp = _dev_ptr(workspace, "workspace") if workspace is not None else None
    wb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(_zero_step_units(layout.ptr, rank, unit_begin, unit_end, C.addressof(arr), len(arr), gdt,
                            grad_index, divisor, _f32_ptr(master, "master"),
                            _f32_ptr(exp_avg, "exp_avg"), _f32_ptr(exp_avg_sq, "exp_avg_sq"),
                            state_index, _bf16_ptr(out, "out") if out is not None else None,
                            out_index, C.byref(scalars), wp, wb, _stream(stream)), "zero_step_units")


def zero_step_staged_workspace_bytes(layout: Layout, rank: int, n_grads: int) -> int:
    b = sz()
    _check(_zero_step_staged_workspace_bytes(layout.ptr, rank, n_grads, C.byref(b)),
           "zero_step_staged_workspace_bytes")
    return b.value


def _host_ptr(a, what: str, kind: str):
    """Address of a host buffer: a numpy array or a CPU torch tensor
    (C-contiguous).  kind: 'f32', 'bf16' (uint16 / int16 / bfloat16 bits) or
    'grad' (either)."""
    torch = _torch()
    if isinstance(a, torch.Tensor):
        if a.is_cuda:
            raise ValueError(f"{what} must be in host memory")
        if not a.is_contiguous():
            raise ValueError(f"{what} must be contiguous")
        dt = {torch.float32: "f32", torch.bfloat16: "bf16", torch.int16: "bf16",
              torch.uint16: "bf16"}.get(a.dtype)
        ptr = a.data_ptr()
    else:
        if not isinstance(a, np.ndarray) or not a.flags["C_CONTIGUOUS"]:
            raise ValueError(f"{what} must be a C-contiguous numpy array or CPU tensor")
        dt = {np.dtype(np.float32): "f32", np.dtype(np.uint16): "bf16",
              np.dtype(np.int16): "bf16"}.get(a.dtype)
        ptr = a.ctypes.data
    if dt is None or (kind != "grad" and dt != kind):
        raise TypeError(f"{what}: unexpected dtype")
    return ptr, dt


def zero_step_host(layout: Layout, rank: int, grads, grad_index: int, divisor: float,
                   master, exp_avg, exp_avg_sq, state_index: int, out, out_index: int,
                   scalars: ZeroAdamwScalars, n_threads: int = 0):
    """The step on host cores (ZeRO-Offload): same arguments as zero_step on
    host buffers (numpy arrays or CPU tensors); synchronous."""
    if len(grads) < 1:
        raise ValueError("at least one gradient buffer")
    _need_step(layout, grads, grad_index, master, exp_avg, exp_avg_sq, state_index, out, out_index)
    gp = [_host_ptr(g, "grad", "grad") for g in grads]
    kinds = {k for _, k in gp}
    if len(kinds) != 1:
        raise TypeError("all gradient buffers must share one dtype")
    gdt = ZERO_BF16 if kinds.pop() == "bf16" else ZERO_F32
    arr = (vp * len(gp))(*[p for p, _ in gp])
    _check(_zero_step_host(layout.ptr, rank, C.addressof(arr), len(gp), gdt, grad_index, divisor,
                           _host_ptr(master, "master", "f32")[0],
                           _host_ptr(exp_avg, "exp_avg", "f32")[0],
                           _host_ptr(exp_avg_sq, "exp_avg_sq", "f32")[0], state_index,
                           _host_ptr(out, "out", "bf16")[0] if out is not None else None,
                           out_index, C.byref(scalars), n_threads), "zero_step_host")


def zero_offload_step(layout: Layout, rank: int, d_grad, h_grad_stage, master, exp_avg,
                      exp_avg_sq, h_out_stage, d_out, chunk: int, scalars: ZeroAdamwScalars,
                      n_threads: int = 0, stream_down=None, stream_up=None):
    """The pipelined offload step: d_grad / d_out are device tensors, the
    staging slots pinned CPU tensors (2 * chunk elements each), the state CPU
    tensors or numpy arrays.  Synchronous."""
    torch = _torch()
    for t, what in ((h_grad_stage, "h_grad_stage"), (h_out_stage, "h_out_stage")):
        if not (isinstance(t, torch.Tensor) and t.is_pinned()):
            raise ValueError(f"{what} must be a pinned CPU tensor")
        if t.numel() < 2 * chunk:
            raise ValueError(f"{what} needs 2 * chunk elements")
    for t, what in ((d_grad, "d_grad"), (master, "master"), (exp_avg, "exp_avg"),
                    (exp_avg_sq, "exp_avg_sq"), (d_out, "d_out")):
        _need(t, layout.shard, what)
    _check(_zero_offload_step(layout.ptr, rank, _f32_ptr(d_grad, "d_grad"),
                              _host_ptr(h_grad_stage, "h_grad_stage", "f32")[0],
                              _host_ptr(master, "master", "f32")[0],
                              _host_ptr(exp_avg, "exp_avg", "f32")[0],
                              _host_ptr(exp_avg_sq, "exp_avg_sq", "f32")[0],
                              _host_ptr(h_out_stage, "h_out_stage", "bf16")[0],
                              _bf16_ptr(d_out, "d_out"), chunk, C.byref(scalars), n_threads,
                              _stream(stream_down), _stream(stream_up)), "zero_offload_step")


def zero_step_device_clip(layout: Layout, rank: int, grads, grad_index: int, divisor: float,
                          master, exp_avg, exp_avg_sq, state_index: int, out, out_index: int,
                          scalars: ZeroAdamwScalars, clip_coef_dev, stream=None, *, grad_ptrs=None):
    """zero_step with the clip multiplier read from the float32 device tensor
    ``clip_coef_dev`` (e.g. filled by zero_clip_coef_async)."""
    arr, gdt = grad_ptrs if grad_ptrs is not None else _grad_ptrs(grads)
    _need_step(layout, grads if grad_ptrs is None else (), grad_index, master, exp_avg, exp_avg_sq,
               state_index, out, out_index)
    _need_prepared(grad_ptrs, _extent(layout, grad_index), "grad")
    _need(clip_coef_dev, 1, "clip_coef_dev")
    _check(_zero_step_device_clip(layout.ptr, rank, C.addressof(arr), len(arr), gdt, grad_index,
                                  divisor, _f32_ptr(master, "master"), _f32_ptr(exp_avg, "exp_avg"),
                                  _f32_ptr(exp_avg_sq, "exp_avg_sq"), state_index,
                                  _bf16_ptr(out, "out") if out is not None else None, out_index,
                                  C.byref(scalars), _f32_ptr(clip_coef_dev, "clip_coef_dev"),
                                  _stream(stream)), "zero_step_device_clip")


def zero_clip_coef_ranks(rank_sums, max_norm: float):
    """(coef, total): the rank-ordered binary64 total of the ranks' sums of
    squares and its clip coefficient (host)."""
    arr = np.ascontiguousarray(rank_sums, dtype=np.float64)
    c, t = f32(), f64()
    _check(_zero_clip_coef_ranks(arr.ctypes.data if arr.size else None, arr.size, max_norm,
                                 C.byref(c), C.byref(t)), "zero_clip_coef_ranks")
    return c.value, t.value


def zero_clip_coef_ranks_async(rank_sums_dev, max_norm: float, coef_dev, total_dev=None,
                               stream=None):
    """The same on the device: float64 tensor of the N sums in, float32
    coefficient (and optionally the float64 total) out."""
    torch = _torch()
    if rank_sums_dev.dtype != torch.float64 or (total_dev is not None and total_dev.dtype != torch.float64):
        raise TypeError("rank sums and total must be float64")
    _need(coef_dev, 1, "coef_dev")
    _need(total_dev, 1, "total_dev")
    _check(_zero_clip_coef_ranks_async(_dev_ptr(rank_sums_dev, "rank_sums_dev"),
                                       rank_sums_dev.numel(), max_norm,
                                       _f32_ptr(coef_dev, "coef_dev"),
                                       _dev_ptr(total_dev, "total_dev") if total_dev is not None else None,
                                       _stream(stream)), "zero_clip_coef_ranks_async")


def zero_clip_coef_async(sumsq_dev, max_norm: float, coef_dev, stream=None):
    """The clip coefficient on the device: float64 tensor in, float32 out."""
    torch = _torch()
    if sumsq_dev.dtype != torch.float64:
        raise TypeError("sumsq_dev must be float64")
    _need(sumsq_dev, 1, "sumsq_dev")
    _need(coef_dev, 1, "coef_dev")
    _check(_zero_clip_coef_async(_dev_ptr(sumsq_dev, "sumsq_dev"), max_norm,
                                 _f32_ptr(coef_dev, "coef_dev"), _stream(stream)),
           "zero_clip_coef_async")


def zero_overlap(psi_unit: float, n_ranks: int, busbw_bytes_per_s: float, tokens_per_gpu: float,
                 flops_per_s: float) -> dict:
    o = ZeroOverlapOut()
    _check(_zero_overlap(psi_unit, n_ranks, busbw_bytes_per_s, tokens_per_gpu, flops_per_s,
                         C.byref(o)), "zero_overlap")
    return o.as_dict()


def grad_pointer_array(grads):
    return _grad_ptrs(grads)


def _need_norm(layout, grads, grad_index, g_out, g_index):
    ge = _extent(layout, grad_index)
    for g in grads:
        _need(g, ge, "grad")
    _need(g_out, _extent(layout, g_index), "g_out")


def zero_gradnorm_workspace_bytes(layout: Layout, rank: int) -> int:
    b = sz()
    _check(_zero_gradnorm_workspace_bytes(layout.ptr, rank, C.byref(b)),
           "zero_gradnorm_workspace_bytes")
    return b.value


def zero_gradnorm(layout: Layout, rank: int, grads, grad_index: int, divisor: float,
                  g_out, g_index: int, workspace, stream=None) -> float:
    """Sum of squares (binary64) of the averaged gradient; optionally writes
    the averaged gradient (fp32) into ``g_out``.  Synchronizes the stream."""
    arr, gdt = _grad_ptrs(grads)
    _need_norm(layout, grads, grad_index, g_out, g_index)
    res = f64()
    _check(_zero_gradnorm(layout.ptr, rank, C.addressof(arr), len(arr), gdt, grad_index, divisor,
                          _f32_ptr(g_out, "g_out") if g_out is not None else None, g_index,
                          _dev_ptr(workspace, "workspace"),
                          workspace.numel() * workspace.element_size(), C.byref(res),
                          _stream(stream)), "zero_gradnorm")
    return res.value


def zero_gradnorm_async(layout: Layout, rank: int, grads, grad_index: int, divisor: float,
                        g_out, g_index: int, workspace, sumsq_dev, stream=None):
    """Enqueue the norm pass; the binary64 sum of squares lands in
    ``sumsq_dev`` (a float64 device tensor) without synchronizing."""
    torch = _torch()
    if sumsq_dev.dtype != torch.float64:
        raise TypeError("sumsq_dev must be a float64 device tensor")
    arr, gdt = _grad_ptrs(grads)
    _need_norm(layout, grads, grad_index, g_out, g_index)
    _need(sumsq_dev, 1, "sumsq_dev")
    _check(_zero_gradnorm_async(layout.ptr, rank, C.addressof(arr), len(arr), gdt, grad_index,
                                divisor, _f32_ptr(g_out, "g_out") if g_out is not None else None,
                                g_index, _dev_ptr(workspace, "workspace"),
                                workspace.numel() * workspace.element_size(),
                                _dev_ptr(sumsq_dev, "sumsq_dev"), _stream(stream)),
           "zero_gradnorm_async")


def zero_gradnorm_async_noalloc(layout: Layout, rank: int, grads, grad_index: int,
                                divisor: float, g_out, g_index: int, sumsq_dev, stream=None):
    """zero_gradnorm_async without a workspace: the partial sums live in the
    library's own device array (for callers that cannot allocate; calls on one
    GPU must not overlap)."""
    torch = _torch()
    if sumsq_dev.dtype != torch.float64:
        raise TypeError("sumsq_dev must be a float64 device tensor")
    arr, gdt = _grad_ptrs(grads)
    _need_norm(layout, grads, grad_index, g_out, g_index)
    _need(sumsq_dev, 1, "sumsq_dev")
    _check(_zero_gradnorm_async_noalloc(layout.ptr, rank, C.addressof(arr), len(arr), gdt,
                                        grad_index, divisor,
                                        _f32_ptr(g_out, "g_out") if g_out is not None else None,
                                        g_index, _dev_ptr(sumsq_dev, "sumsq_dev"), _stream(stream)),
           "zero_gradnorm_async_noalloc")


# -- ledger -------------------------------------------------------------------------------

def zero_ledger(psi: float, n_ranks: int, stage: int, grads_transient: bool = False) -> dict:
    o = ZeroLedgerOut()
    _check(_zero_ledger(psi, n_ranks, stage, int(grads_transient), C.byref(o)), "zero_ledger")
    return o.as_dict()


def zero_sim_footprint(layout: Layout, n_grads: int, grad_dtype: int, grad_index: int,
                       state_index: int, out_index: int, with_out: bool = True,
                       with_g: bool = False) -> dict:
    """Bytes the one-GPU simulation's buffers occupy (see zero.h)."""
    o = ZeroFootprintOut()
    _check(_zero_sim_footprint(layout.ptr, n_grads, grad_dtype, grad_index, state_index, out_index,
                               int(with_out), int(with_g), C.byref(o)), "zero_sim_footprint")
    return o.as_dict()


def zero_gather_buffer_bytes(layout: Layout, units_in_flight: int = 2) -> float:
    b = f64()
    _check(_zero_gather_buffer_bytes(layout.ptr, units_in_flight, C.byref(b)),
           "zero_gather_buffer_bytes")
    return b.value


def zero_arena_plan(sizes):
    """Byte offsets of buffers of the given byte sizes inside one allocation,
    and the allocation's size (see zero.h)."""
    n = len(sizes)
    b = (i64 * max(n, 1))(*[int(x) for x in sizes])
    o = (i64 * max(n, 1))()
    t = i64()
    _check(_zero_arena_plan(n, C.addressof(b), C.addressof(o), C.byref(t)), "zero_arena_plan")
    return [o[i] for i in range(n)], t.value


def zero_step_traffic(layout: Layout, rank: int, n_grads: int, grad_dtype: int,
                      with_out: bool = True):
    b, e = f64(), i64()
    _check(_zero_step_traffic(layout.ptr, rank, n_grads, grad_dtype, int(with_out), C.byref(b),
                              C.byref(e)), "zero_step_traffic")
    return b.value, e.value


def zero_gradnorm_traffic(layout: Layout, rank: int, n_grads: int, grad_dtype: int,
                          with_g_out: bool = True):
    b, e = f64(), i64()
    _check(_zero_gradnorm_traffic(layout.ptr, rank, n_grads, grad_dtype, int(with_g_out),
                                  C.byref(b), C.byref(e)), "zero_gradnorm_traffic")
    return b.value, e.value


# -- sharded checkpoint ---------------------------------------------------------------------

def _host_f32(a, what: str, n: int):
    """A C-contiguous float32 host array of at least n elements for a checkpoint
    call: numpy arrays and CPU tensors as they are, device tensors copied to
    host memory first.  Returns (keep-alive object, address)."""
    torch = _torch()
    if isinstance(a, torch.Tensor) and a.is_cuda:
        if a.dtype != torch.float32:
            raise TypeError(f"{what} must be float32")
        a = a.detach().contiguous().cpu()
    _need(a, n, what)
    return a, _host_ptr(a, what, "f32")[0]


def zero_ckpt_save(path: str, layout: Layout, rank: int, step: int, master, exp_avg, exp_avg_sq):
    """Write rank ``rank``'s shard of the optimizer state (host or device
    float32 arrays of layout.shard elements) to ``path``."""
    keep = [_host_f32(a, w, layout.shard) for a, w in ((master, "master"), (exp_avg, "exp_avg"),
                                                        (exp_avg_sq, "exp_avg_sq"))]
    _check(_zero_ckpt_save(os.fsencode(path), layout.ptr, rank, step, *[p for _, p in keep]),
           "zero_ckpt_save")


def zero_ckpt_inspect(path: str, verify: bool = True):
    """(info dict, saved Layout) of one shard file."""
    info, need = ZeroCkptInfo(), sz()
    _check(_zero_ckpt_inspect(os.fsencode(path), int(verify), C.byref(info), None, 0, C.byref(need)),
           "zero_ckpt_inspect")
    buf = (C.c_char * need.value)()
    _check(_zero_ckpt_inspect(os.fsencode(path), 0, C.byref(info), C.addressof(buf), need.value, None),
           "zero_ckpt_inspect")
    return info.as_dict(), Layout(buf)


def zero_ckpt_load(paths, layout: Layout, rank: int, verify: bool = True):
    """Rank ``rank``'s shard of ``layout`` from a checkpoint's shard files
    (paths[q] = rank q's), resharded at load time.  Returns (step, master,
    exp_avg, exp_avg_sq) as float32 numpy arrays of layout.shard elements."""
    enc = [os.fsencode(p) for p in paths]
    arr = (C.c_char_p * max(len(enc), 1))(*enc)
    out = [np.zeros(layout.shard, np.float32) for _ in range(3)]
    step = i32()
    _check(_zero_ckpt_load(C.addressof(arr), len(enc), layout.ptr, rank, int(verify), C.byref(step),
                           *[o.ctypes.data for o in out]), "zero_ckpt_load")
    return (step.value, *out)


def zero_set_waves_per_cu(kind: int, waves: int):
    """Cap resident waves per CU of a kernel family (-1: back to the default)."""
    _check(_zero_set_waves_per_cu(kind, waves), "zero_set_waves_per_cu")


def zero_get_waves_per_cu(kind: int, n_grads: int = 1) -> int:
    w = i32()
    _check(_zero_get_waves_per_cu(kind, n_grads, C.byref(w)), "zero_get_waves_per_cu")
    return w.value


def zero_get_waves_per_cu_for(kind: int, n_grads: int, grad_dtype: int = ZERO_BF16,
                              staged: bool = False) -> int:
    w = i32()
    _check(_zero_get_waves_per_cu_for(kind, n_grads, grad_dtype, int(staged), C.byref(w)),
           "zero_get_waves_per_cu_for")
    return w.value


def zero_strerror(status: int) -> str:
    return _zero_strerror(status).decode()


def zero_last_hip_error() -> str:
    return _zero_last_hip_error().decode()


def zero_abi_version() -> int:
    return int(_zero_abi_version())


def hip_runtimes_mapped() -> list[str]:
    """Paths of every HIP runtime library mapped into this process (there
    must be exactly one)."""
    paths = set()
    with open("/proc/self/maps") as f:
        for line in f:
            if "libamdhip64" in line:
                paths.add(line.split()[-1])
    return sorted(paths)


def raw_library():
    """The ctypes handle (for tests that call the C ABI with raw pointers)."""
    return _lib
