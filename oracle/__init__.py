"""CPU oracle for the fused MoE dispatch + expert GEMM (numpy front end).

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.  The arithmetic lives
in oracle.c (plain C, OpenMP over independent outer loops only); this module
only marshals numpy arrays to it.

Steps and readings (the pages print no formula; "MoE Dispatch+GEMM" is named
in "mKernel UCCL fuses NVLink/RDMA/compute into one persistent CUDA kernel",
zubnet.ai, paragraph 2):
  route()      router logits in a fixed fp32 order, top-k (logit desc, id asc),
               fp64 softmax gate over all experts
  layout()     per-local-expert counts, exclusive offsets, slots in ascending
               token order, the inverse row -> token map
  expert_rows() fp64 expert GEMM y[r] = x[row_token[r]] . W[e]^T for chosen rows
  combine()    the next step: out[t] = sum over local choices j of w[t][j] y[slot_of[t][j]]
  swiglu(), grouped_rows()  the expert FFN after the gate|up GEMM: h = silu(g) * u, then the
               down-projection z[r] = h[r] . Wd[e]^T over the same expert layout
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_i32p = ctypes.POINTER(ctypes.c_int32)
_u16p = ctypes.POINTER(ctypes.c_uint16)
_f32p = ctypes.POINTER(ctypes.c_float)
_f64p = ctypes.POINTER(ctypes.c_double)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _build
        _build.build()
    lib = ctypes.CDLL(_LIB_PATH)
    lib.oracle_logits.argtypes = [_u16p, _f32p, _f32p, ctypes.c_int, ctypes.c_int, ctypes.c_int, _f32p]
    lib.oracle_topk.argtypes = [_f32p, ctypes.c_int, ctypes.c_int, ctypes.c_int, _i32p, _f64p]
    lib.oracle_layout.argtypes = [_i32p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                  _i32p, _i32p, _i32p, _i32p]
    lib.oracle_expert_rows.argtypes = [_u16p, ctypes.c_int, _u16p, ctypes.c_int, _i32p, ctypes.c_int,
                                       _i32p, _i32p, ctypes.c_int, _f64p]
    lib.oracle_combine.argtypes = [_f64p, _i32p, ctypes.c_int, ctypes.c_int, _i32p, _f64p, ctypes.c_int,
                                   ctypes.c_int, _f64p]
    lib.oracle_swiglu.argtypes = [_u16p, ctypes.c_int, ctypes.c_int, _f64p]
    lib.oracle_grouped_rows.argtypes = [_u16p, ctypes.c_int, _u16p, ctypes.c_int, _i32p, ctypes.c_int, _i32p,
                                        ctypes.c_int, _f64p]
    lib.oracle_num_threads.argtypes = []
    for f in (lib.oracle_logits, lib.oracle_topk, lib.oracle_layout, lib.oracle_expert_rows,
              lib.oracle_combine, lib.oracle_swiglu, lib.oracle_grouped_rows, lib.oracle_num_threads):
        f.restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(a, t):
    return a.ctypes.data_as(t)


def _bits(a):
    """bf16 data as uint16 bit patterns (accepts a numpy uint16 array or a torch bf16 tensor)."""
    if isinstance(a, np.ndarray):
        assert a.dtype == np.uint16
        return np.ascontiguousarray(a)
    import torch
    assert a.dtype == torch.bfloat16
    return np.ascontiguousarray(a.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16))


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def logits(x, w_router, bias=None):
    """fp32 router logits [T,E] in the fixed segmented order (d % 8 == 0)."""
    lib = _load()
    xb = _bits(x)
    T, d = xb.shape
    wr = np.ascontiguousarray(np.asarray(w_router, dtype=np.float32))
    assert wr.shape[0] == d
    E = wr.shape[1]
    b = None if bias is None else np.ascontiguousarray(np.asarray(bias, dtype=np.float32))
    out = np.empty((T, E), dtype=np.float32)
    rc = lib.oracle_logits(_ptr(xb, _u16p), _ptr(wr, _f32p),
                           None if b is None else _ptr(b, _f32p), T, d, E, _ptr(out, _f32p))
    if rc:
        raise ValueError("oracle_logits: bad shape (d must be a positive multiple of 8)")
    return out


def topk(lg, k):
    """(ids [T,k] int32 rank order, w [T,k] fp64 softmax gate over all E)."""
    lib = _load()
    lg = np.ascontiguousarray(lg, dtype=np.float32)
    T, E = lg.shape
    ids = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float64)
    if lib.oracle_topk(_ptr(lg, _f32p), T, E, k, _ptr(ids, _i32p), _ptr(w, _f64p)):
        raise ValueError("oracle_topk: need 1 <= k <= E")
    return ids, w


def route(x, w_router, k, bias=None):
    lg = logits(x, w_router, bias)
    ids, w = topk(lg, k)
    return lg, ids, w


def layout(ids, e_begin, E_local):
    """(count [E_local], offsets [E_local+1], slot_of [T,k], row_token [R])."""
    lib = _load()
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    T, k = ids.shape
    count = np.empty(E_local, dtype=np.int32)
    offsets = np.empty(E_local + 1, dtype=np.int32)
    slot_of = np.empty((T, k), dtype=np.int32)
    row_token = np.empty(max(T * k, 1), dtype=np.int32)
    if lib.oracle_layout(_ptr(ids, _i32p), T, k, e_begin, E_local, _ptr(count, _i32p),
                         _ptr(offsets, _i32p), _ptr(slot_of, _i32p), _ptr(row_token, _i32p)):
        raise ValueError("oracle_layout: bad arguments")
    R = int(offsets[E_local])
    return count, offsets, slot_of, row_token[:R].copy()


def expert_rows(x, w_experts, offsets, row_token, rows):
    """fp64 y[q, :] for expert-buffer rows `rows` (each < R)."""
    lib = _load()
    xb = _bits(x)
    wb = _bits(w_experts)
    T, d = xb.shape
    E_local, N, d2 = wb.shape
    assert d2 == d
    offsets = np.ascontiguousarray(offsets, dtype=np.int32)
    row_token = np.ascontiguousarray(row_token, dtype=np.int32)
    if row_token.size == 0:
        row_token = np.zeros(1, dtype=np.int32)
    rows = np.ascontiguousarray(rows, dtype=np.int32)
    y = np.empty((rows.size, N), dtype=np.float64)
    if lib.oracle_expert_rows(_ptr(xb, _u16p), d, _ptr(wb, _u16p), N, _ptr(offsets, _i32p), E_local,
                              _ptr(row_token, _i32p), _ptr(rows, _i32p), rows.size, _ptr(y, _f64p)):
        raise ValueError("oracle_expert_rows: row index out of range")
    return y


def combine(y, slot_rows, slot_of, w):
    """fp64 out [T,N] = sum over local choices j (slot_of >= 0) of w[t][j] * y[row of slot_of[t][j]];
    y [n,N] holds the rows of the slots slot_rows [n] (every chosen slot must be listed)."""
    lib = _load()
    y = np.ascontiguousarray(np.asarray(y, dtype=np.float64))
    slot_rows = np.ascontiguousarray(np.asarray(slot_rows, dtype=np.int32).reshape(-1))
    slot_of = np.ascontiguousarray(np.asarray(slot_of, dtype=np.int32))
    w = np.ascontiguousarray(np.asarray(w, dtype=np.float64))
    T, k = slot_of.shape
    n, N = y.shape
    assert slot_rows.size == n and w.shape == (T, k)
    out = np.empty((T, N), dtype=np.float64)
    if y.size == 0:
        y = np.zeros((1, max(N, 1)), dtype=np.float64)
        slot_rows = np.full(1, -2, dtype=np.int32)
    if lib.oracle_combine(_ptr(y, _f64p), _ptr(slot_rows, _i32p), n, N, _ptr(slot_of, _i32p), _ptr(w, _f64p),
                          T, k, _ptr(out, _f64p)):
        raise ValueError("oracle_combine: a chosen slot has no row in y")
    return out


def swiglu(gu):
    """fp64 h [rows, F] = silu(g) * u of bf16 rows gu [rows, 2F] (g = first F columns, u = the rest)."""
    lib = _load()
    b = _bits(gu)
    rows, F2 = b.shape
    assert F2 % 2 == 0
    h = np.empty((rows, F2 // 2), dtype=np.float64)
    if lib.oracle_swiglu(_ptr(b, _u16p), rows, F2 // 2, _ptr(h, _f64p)):
        raise ValueError("oracle_swiglu: bad shape")
    return h


def grouped_rows(a, w, offsets, rows):
    """fp64 z [len(rows), N]: row r of bf16 a [R, K] times W[e]^T (bf16 w [E_local, N, K]), e the expert of r."""
    lib = _load()
    ab, wb = _bits(a), _bits(w)
    R, K = ab.shape
    E_local, N, K2 = wb.shape
    assert K2 == K
    offsets = np.ascontiguousarray(offsets, dtype=np.int32)
    rows = np.ascontiguousarray(rows, dtype=np.int32)
    z = np.empty((rows.size, N), dtype=np.float64)
    if lib.oracle_grouped_rows(_ptr(ab, _u16p), K, _ptr(wb, _u16p), N, _ptr(offsets, _i32p), E_local,
                               _ptr(rows, _i32p), rows.size, _ptr(z, _f64p)):
        raise ValueError("oracle_grouped_rows: row index out of range")
    return z


def run(x, w_router, w_experts, k, e_begin=0, bias=None, rows=None):
    """All steps.  rows=None computes every expert-buffer row."""
    lg, ids, w = route(x, w_router, k, bias)
    E_local = _bits(w_experts).shape[0]
    count, offsets, slot_of, row_token = layout(ids, e_begin, E_local)
    R = int(offsets[-1])
    if rows is None:
        rows = np.arange(R, dtype=np.int32)
    y = expert_rows(x, w_experts, offsets, row_token, rows)
    return dict(logits=lg, ids=ids, w=w, count=count, offsets=offsets, slot_of=slot_of,
                row_token=row_token, rows=np.asarray(rows, dtype=np.int32), y=y)
