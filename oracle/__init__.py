"""Serial CPU oracle for the ZeRO sharded AdamW step -- TEST INFRASTRUCTURE.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library
(``fsdp_sharded_optimizer_flat_amd``) never imports it, and the oracle shares no
code, header, table or helper with it.

The arithmetic lives in ``oracle.c`` (plain C, one binary32 rounding per
operation, no FMA); this module only compiles it and marshals numpy arrays.
What each function follows is documented next to its C definition, citing
the pages "ZeRO and FSDP sharding" (tirogla.com), "ZeRO: Three Ledgers, Zero
Redundancy" and "Learn: ZeRO & FSDP".
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

CFLAGS = ["-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math",
          "-fno-unsafe-math-optimizations", "-shared", "-fPIC"]


def build(src: str = SRC, out: str = LIB, extra: list[str] | None = None) -> str:
    """Compile the oracle with gcc (no FMA contraction, no fast-math)."""
    cmd = ["gcc", *CFLAGS, *(extra or []), src, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


_lib = None


def load(path: str | None = None):
    """Load (building first if needed) and return the ctypes library."""
    global _lib
    if path is None and _lib is not None:
        return _lib
    p = path or LIB
    if path is None and (not os.path.exists(p) or
                         os.path.getmtime(p) < os.path.getmtime(SRC)):
        build()
    lib = C.CDLL(p)
    _declare(lib)
    if path is None:
        _lib = lib
    return lib


i32, i64, f32, f64 = C.c_int32, C.c_int64, C.c_float, C.c_double
vp = C.c_void_p


class using:
    """Context manager: route this module's functions through another build of
    the oracle (the mutation tests plant mistakes in a copy of oracle.c)."""

    def __init__(self, path: str):
        self.path = path

    def __enter__(self):
        global _lib
        self.saved = _lib
        _lib = load(self.path)
        return _lib

    def __exit__(self, *exc):
        global _lib
        _lib = self.saved
        return False


def _declare(lib):
    lib.orc_layout.argtypes = [i32, i32, vp, vp, vp, vp, vp, vp, vp]
    lib.orc_layout.restype = C.c_int
    lib.orc_global_of_local.argtypes = [i32, vp, vp, vp, i32, i64]
    lib.orc_global_of_local.restype = i64
    lib.orc_owner_of_global.argtypes = [i32, i32, vp, vp, vp, i64, vp, vp]
    lib.orc_owner_of_global.restype = C.c_int
    lib.orc_bf16.argtypes = [f32]
    lib.orc_bf16.restype = C.c_uint16
    lib.orc_bf16_array.argtypes = [vp, vp, i64]
    lib.orc_bf16_array.restype = None
    lib.orc_adamw_scalars.argtypes = [i32, f32, f32, f32, f32, vp]
    lib.orc_adamw_scalars.restype = None
    lib.orc_adamw_vector.argtypes = [i64, vp, vp, vp, vp, i32, f32, f32, f32, f32, f32]
    lib.orc_adamw_vector.restype = None
    lib.orc_zero_step_rank.argtypes = [i32, i32, vp, i32, vp, i32, i32, i32, f32, f32,
                                       vp, vp, vp, i32, vp, i32, i32, f32, f32, f32, f32, f32]
    lib.orc_zero_step_rank.restype = C.c_int
    lib.orc_zero_step_all.argtypes = [i32, i32, vp, vp, i32, i32, f32, f32,
                                      vp, vp, vp, vp, i32, f32, f32, f32, f32, f32]
    lib.orc_zero_step_all.restype = C.c_int
    lib.orc_adamw_unsharded.argtypes = [i64, vp, i32, i32, f32, f32, vp, vp, vp,
                                        i32, f32, f32, f32, f32, f32]
    lib.orc_adamw_unsharded.restype = None
    lib.orc_reduced_grad.argtypes = [i32, i32, vp, i32, vp, i32, i32, i32, f32, vp]
    lib.orc_reduced_grad.restype = C.c_int
    lib.orc_sumsq.argtypes = [vp, i64]
    lib.orc_sumsq.restype = f64
    lib.orc_clip_coef.argtypes = [f64, f64]
    lib.orc_clip_coef.restype = f32
    lib.orc_toy.argtypes = [i32, i64, i32, f32, vp, vp, vp, vp]
    lib.orc_toy.restype = C.c_int
    lib.orc_ledger_bytes.argtypes = [f64, i32, i32, i32]
    lib.orc_ledger_bytes.restype = f64
    lib.orc_sim_footprint.argtypes = [i32, i32, vp, i32, i32, i32, i32, i32]
    lib.orc_sim_footprint.restype = f64
    lib.orc_comm_elements.argtypes = [f64, i32, i32, i32]
    lib.orc_comm_elements.restype = f64
    lib.orc_layout_rows.argtypes = [i32, i32, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.orc_layout_rows.restype = C.c_int
    lib.orc_reshard.argtypes = [i32, vp, i32, vp, vp, i32, vp, i32, vp, i32, vp, i32]
    lib.orc_reshard.restype = C.c_int
    lib.orc_reshard_span.argtypes = [i32, vp, i32, vp, vp, i32, vp, i32, vp, i32, i64, i64, vp, i32]
    lib.orc_reshard_span.restype = C.c_int


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data


def _ptr_array(arrs):
    return (vp * len(arrs))(*[_ptr(a) for a in arrs])


# ----------------------------------------------------------------------------
# Default hyperparameters: the toy's (lr 0.01) and the GPT-scale runs' (3e-4);
# b1 0.9, b2 0.95, eps 1e-8, wd 0.1 in both.
# ----------------------------------------------------------------------------
HYPER = dict(lr=3e-4, b1=0.9, b2=0.95, eps=1e-8, wd=0.1)


class Layout:
    """The oracle's own layout: units padded to a multiple of n elements
    (row_len None), or to a multiple of n whole rows of row_len[u] elements."""

    def __init__(self, n: int, numel, lib=None, row_len=None):
        self.lib = lib or load()
        self.n = int(n)
        self.numel = np.ascontiguousarray(numel, dtype=np.int64)
        U = len(self.numel)
        self.row_len = None if row_len is None else np.ascontiguousarray(row_len, dtype=np.int64)
        if self.row_len is not None and len(self.row_len) != U:
            raise ValueError("one row length per unit")
        self.padded = np.zeros(max(U, 1), np.int64)
        self.shard = np.zeros(max(U, 1), np.int64)
        self.offset = np.zeros(max(U, 1), np.int64)
        self.local_offset = np.zeros(max(U, 1), np.int64)
        tp, ts = i64(), i64()
        outs = (_ptr(self.padded), _ptr(self.shard), _ptr(self.offset), _ptr(self.local_offset),
                C.byref(tp), C.byref(ts))
        if self.row_len is None:
            rc = self.lib.orc_layout(self.n, U, _ptr(self.numel) if U else None, *outs)
        else:
            rc = self.lib.orc_layout_rows(self.n, U, _ptr(self.numel) if U else None,
                                          _ptr(self.row_len) if U else None, *outs)
        if rc != 0:
            raise ValueError(f"oracle layout rc={rc}")
        self.padded, self.shard = self.padded[:U], self.shard[:U]
        self.offset, self.local_offset = self.offset[:U], self.local_offset[:U]
        self.total_padded, self.total_shard = tp.value, ts.value
        self.n_units = U

    def global_of_local(self, r: int, k: int) -> int:
        return int(self.lib.orc_global_of_local(self.n_units, _ptr(self.shard), _ptr(self.offset),
                                                _ptr(self.local_offset), r, k))

    def owner_of_global(self, j: int):
        r, k = i32(), i64()
        rc = self.lib.orc_owner_of_global(self.n, self.n_units, _ptr(self.shard), _ptr(self.offset),
                                          _ptr(self.local_offset), j, C.byref(r), C.byref(k))
        if rc != 0:
            raise ValueError(j)
        return r.value, k.value


def reshard_span(numel, n_a, src, n_b, dst_rank, k_begin, k_end, *, row_a=None, row_b=None,
                 numel_b=None) -> np.ndarray:
    """Elements k_begin <= k < k_end of what :func:`reshard` returns."""
    lib = load()
    na = np.ascontiguousarray(numel, dtype=np.int64)
    nb = na if numel_b is None else np.ascontiguousarray(numel_b, dtype=np.int64)
    src = [np.ascontiguousarray(a) for a in src]
    if len(src) != n_a or len({a.dtype for a in src}) != 1:
        raise ValueError("one source shard per rank of layout A, one dtype")
    dt = src[0].dtype
    dst = np.zeros(max(k_end - k_begin, 0), dt)
    ra = None if row_a is None else np.ascontiguousarray(row_a, dtype=np.int64)
    rb = None if row_b is None else np.ascontiguousarray(row_b, dtype=np.int64)
    keep = _ptr_array(src)
    opt = lambda a: _ptr(a) if a is not None and len(a) else None
    rc = lib.orc_reshard_span(len(na), opt(na), n_a, opt(ra), keep, len(nb), opt(nb), n_b, opt(rb),
                              dst_rank, k_begin, k_end, _ptr(dst) if len(dst) else None,
                              dt.itemsize)
    if rc != 0:
        raise ValueError(f"orc_reshard_span rc={rc}")
    return dst


def reshard(numel, n_a, src, n_b, dst_rank, *, row_a=None, row_b=None, numel_b=None) -> np.ndarray:
    """Rank dst_rank's local shard under layout B (units numel_b, default
    numel; n_b ranks; row lengths row_b or flat), built from the local shards
    src[q] of every rank q under layout A (units numel, n_a ranks, row_a).
    src: n_a arrays of one dtype (4-byte or 2-byte elements)."""
    lib = load()
    na = np.ascontiguousarray(numel, dtype=np.int64)
    nb = na if numel_b is None else np.ascontiguousarray(numel_b, dtype=np.int64)
    src = [np.ascontiguousarray(a) for a in src]
    if len(src) != n_a or len({a.dtype for a in src}) != 1:
        raise ValueError("one source shard per rank of layout A, one dtype")
    dt = src[0].dtype
    B = Layout(n_b, nb, row_len=row_b)
    dst = np.zeros(B.total_shard, dt)
    ra = None if row_a is None else np.ascontiguousarray(row_a, dtype=np.int64)
    rb = None if row_b is None else np.ascontiguousarray(row_b, dtype=np.int64)
    keep = _ptr_array(src)
    opt = lambda a: _ptr(a) if a is not None and len(a) else None
    rc = lib.orc_reshard(len(na), opt(na), n_a, opt(ra), keep, len(nb), opt(nb), n_b, opt(rb),
                         dst_rank, _ptr(dst) if len(dst) else None, dt.itemsize)
    if rc != 0:
        raise ValueError(f"orc_reshard rc={rc}")
    return dst


def bf16(x) -> np.ndarray:
    """Round-to-nearest-even bf16 bit patterns (uint16) of a float32 array."""
    lib = load()
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, np.uint16)
    lib.orc_bf16_array(_ptr(x), _ptr(out), x.size)
    return out


def bf16_to_f32(h) -> np.ndarray:
    h = np.ascontiguousarray(h, dtype=np.uint16)
    return (h.astype(np.uint32) << 16).view(np.float32)


def adamw_scalars(t, lr, b1, b2, wd) -> dict:
    lib = load()
    out = np.zeros(8, np.float32)
    lib.orc_adamw_scalars(t, lr, b1, b2, wd, _ptr(out))
    keys = ["one_minus_b1", "one_minus_b2", "pow1", "pow2", "bc1", "bc2", "lr_over_bc1", "decay"]
    return dict(zip(keys, out.tolist())) | {"_raw": out}


def adamw_vector(w, m, v, g, t, lr, b1, b2, eps, wd):
    """In-place AdamW on float32 vectors (no sharding)."""
    lib = load()
    for a in (w, m, v, g):
        assert a.dtype == np.float32 and a.flags["C_CONTIGUOUS"]
    lib.orc_adamw_vector(w.size, _ptr(w), _ptr(m), _ptr(v), _ptr(g), t, lr, b1, b2, eps, wd)


def _grad_kind(grads):
    dt = grads[0].dtype
    assert all(g.dtype == dt for g in grads)
    if dt == np.uint16:
        return 1
    assert dt == np.float32
    return 0


def zero_step_rank(n, numel, r, grads, *, grad_local, divisor, clip, master, m, v,
                   state_global, out, out_gather, t, lr, b1, b2, eps, wd):
    """One rank's sharded step, in place on master/m/v (and out if given).

    grads: list of arrays, float32 or uint16 (bf16 bits)."""
    lib = load()
    numel = np.ascontiguousarray(numel, np.int64)
    gk = _grad_kind(grads)
    ga = _ptr_array(grads)
    rc = lib.orc_zero_step_rank(n, len(numel), _ptr(numel), r, ga, len(grads), gk, int(grad_local),
                                divisor, clip, _ptr(master), _ptr(m), _ptr(v), int(state_global),
                                _ptr(out) if out is not None else None, int(out_gather),
                                t, lr, b1, b2, eps, wd)
    if rc != 0:
        raise ValueError(f"orc_zero_step_rank rc={rc}")


def zero_step_all(n, numel, grads, *, divisor, clip, master, m, v, out, t, lr, b1, b2, eps, wd):
    lib = load()
    numel = np.ascontiguousarray(numel, np.int64)
    gk = _grad_kind(grads)
    rc = lib.orc_zero_step_all(n, len(numel), _ptr(numel), _ptr_array(grads), len(grads), gk,
                               divisor, clip, _ptr(master), _ptr(m), _ptr(v),
                               _ptr(out) if out is not None else None, t, lr, b1, b2, eps, wd)
    if rc != 0:
        raise ValueError(f"orc_zero_step_all rc={rc}")


def adamw_unsharded(grads, *, divisor, clip, w, m, v, t, lr, b1, b2, eps, wd):
    lib = load()
    gk = _grad_kind(grads)
    lib.orc_adamw_unsharded(w.size, _ptr_array(grads), len(grads), gk, divisor, clip,
                            _ptr(w), _ptr(m), _ptr(v), t, lr, b1, b2, eps, wd)


def reduced_grad(n, numel, r, grads, *, grad_local, divisor) -> np.ndarray:
    lib = load()
    lay = Layout(n, numel, lib)
    numel = np.ascontiguousarray(numel, np.int64)
    out = np.zeros(lay.total_shard, np.float32)
    rc = lib.orc_reduced_grad(n, len(numel), _ptr(numel), r, _ptr_array(grads), len(grads),
                              _grad_kind(grads), int(grad_local), divisor, _ptr(out))
    if rc != 0:
        raise ValueError(rc)
    return out


def sumsq(g) -> float:
    g = np.ascontiguousarray(g, np.float32)
    return float(load().orc_sumsq(_ptr(g), g.size))


def clip_coef(sumsq_value: float, max_norm: float) -> float:
    return float(load().orc_clip_coef(sumsq_value, max_norm))


def toy(n=4, P=1000, steps=50, lr=0.01):
    """The pages' toy; returns (w_sharded, w_unsharded, bf16_out, trace)."""
    lib = load()
    ws = np.zeros(max(P, 1), np.float32)
    wu = np.zeros(max(P, 1), np.float32)
    ob = np.zeros(max(P, 1), np.uint16)
    tr = np.zeros(max(steps, 1), np.float64)
    rc = lib.orc_toy(n, P, steps, lr, _ptr(ws), _ptr(wu), _ptr(ob), _ptr(tr))
    if rc != 0:
        raise ValueError(rc)
    return ws[:P], wu[:P], ob[:P], tr[:steps]


def ledger_bytes(psi, n, stage, grads_transient=False) -> float:
    return float(load().orc_ledger_bytes(psi, n, stage, int(grads_transient)))


def comm_elements(psi, n, stage, exact_ring=False) -> float:
    return float(load().orc_comm_elements(psi, n, stage, int(exact_ring)))


def sim_footprint(n, numel, *, every_rank, n_grads, grad_bytes, with_out=True, with_g=False) -> float:
    numel = np.ascontiguousarray(numel, np.int64)
    v = float(load().orc_sim_footprint(n, len(numel), _ptr(numel) if len(numel) else None,
                                       int(every_rank), n_grads, grad_bytes, int(with_out),
                                       int(with_g)))
    if v < 0:
        raise ValueError("oracle layout failed")
    return v
