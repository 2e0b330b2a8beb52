"""Python binding of libmk.so (include/mk.h): fused MoE dispatch + expert GEMM on MI355X.

Argument marshalling only: every step of the path runs in the HIP kernels of
libmk.so.  PyTorch provides device memory and the current stream.  There is no
CPU fallback: loading fails loudly when the library is missing, and the calls
require CUDA (HIP) tensors.

Names follow the C ABI: mk_route_topk, mk_dispatch_gemm,
mk_dispatch_gemm_workspace_bytes, mk_route_topk_workspace_bytes,
mk_select_tuning, mk_poll_error, mk_status_str.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmk.so")

MK_OK, MK_EINVAL, MK_EUNSUPPORTED, MK_EWORKSPACE, MK_EHIP, MK_ETIMEOUT = range(6)

_c_i32 = ctypes.c_int32
_vp = ctypes.c_void_p


class MkShape(ctypes.Structure):
    _fields_ = [("T", _c_i32), ("d", _c_i32), ("E", _c_i32), ("k", _c_i32),
                ("e_begin", _c_i32), ("E_local", _c_i32), ("N", _c_i32)]


class MkSources(ctypes.Structure):
    _fields_ = [("S", _c_i32), ("rows_per_src", _c_i32), ("x", ctypes.POINTER(_vp)),
                ("chunk_rows", _c_i32), ("chunk_ready", _vp), ("epoch", ctypes.c_uint32),
                ("sim_delay_us", _vp), ("sim_payload", ctypes.POINTER(_vp))]


class MkTuning(ctypes.Structure):
    _fields_ = [("n_mover_wg", _c_i32), ("n_compute_wg", _c_i32), ("bm", _c_i32), ("bn", _c_i32),
                ("bk", _c_i32), ("cooperative", _c_i32), ("tile_order", _c_i32), ("ev_gemm_begin", _vp),
                ("ev_gemm_end", _vp)]

TUNING_INTS = ("n_mover_wg", "n_compute_wg", "bm", "bn", "bk", "cooperative", "tile_order")
MK_MOVERS_STAGED, MK_MOVERS_NONE = -1, -2   # n_mover_wg: one launch per step; no mover role (rows read in place)
MK_ORDER_EXPERT, MK_ORDER_TAILS_LAST = 1, 2   # tile_order: row tiles expert by expert; full tiles first


def _tuning(tune: Optional[dict]):
    if not tune:
        return None
    return MkTuning(*(int(tune.get(f, 0)) for f in TUNING_INTS), tune.get("ev_gemm_begin"),
                    tune.get("ev_gemm_end"))


class MkError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {mk_status_str(status)} (status {status})")
        self.status = status


_lib = None


def load() -> ctypes.CDLL:
    """Load libmk.so (built by moe_dispatch_expert_amd/build.py); raises if it is absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python moe_dispatch_expert_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER
    lib.mk_status_str.argtypes = [_c_i32]
    lib.mk_status_str.restype = ctypes.c_char_p
    lib.mk_route_topk_workspace_bytes.argtypes = [_c_i32, _c_i32]
    lib.mk_route_topk_workspace_bytes.restype = ctypes.c_size_t
    lib.mk_route_topk.argtypes = [_vp, _vp, _vp, _c_i32, _c_i32, _c_i32, _c_i32, _vp, _vp, _vp, _vp,
                                  ctypes.c_size_t, _vp]
    lib.mk_route_topk.restype = _c_i32
    lib.mk_dispatch_gemm_workspace_bytes.argtypes = [P(MkShape), P(MkSources), P(MkTuning)]
    lib.mk_dispatch_gemm_workspace_bytes.restype = ctypes.c_size_t
    lib.mk_dispatch_gemm.argtypes = [P(MkShape), P(MkSources), _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                     _vp, _vp, ctypes.c_size_t, P(MkTuning), _vp]
    lib.mk_dispatch_gemm.restype = _c_i32
    lib.mk_dispatch_gemm_swiglu.argtypes = lib.mk_dispatch_gemm.argtypes
    lib.mk_dispatch_gemm_swiglu.restype = _c_i32
    lib.mk_dispatch_gemm_static.argtypes = [P(MkShape), P(MkSources), _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                            _vp, _vp, P(MkTuning), _vp]
    lib.mk_dispatch_gemm_static.restype = _c_i32
    lib.mk_select_tuning.argtypes = [P(MkShape), P(MkSources), P(MkTuning)]
    lib.mk_select_tuning.restype = _c_i32
    lib.mk_poll_error.argtypes = [_vp, P(_c_i32)]
    lib.mk_poll_error.restype = _c_i32
    lib.mk_dispatch_gemm_trace.argtypes = [P(MkShape), P(MkSources), P(ctypes.c_size_t), P(_c_i32), P(_c_i32),
                                           P(_c_i32)]
    lib.mk_dispatch_gemm_trace.restype = _c_i32
    lib.mk_combine.argtypes = [_vp, _c_i32, _vp, _vp, _c_i32, _c_i32, _c_i32, _vp, _vp]
    lib.mk_combine.restype = _c_i32
    lib.mk_swiglu.argtypes = [_vp, _c_i32, _c_i32, _vp, _vp]
    lib.mk_swiglu.restype = _c_i32
    lib.mk_grouped_gemm_workspace_bytes.argtypes = [_c_i32]
    lib.mk_grouped_gemm_workspace_bytes.restype = ctypes.c_size_t
    lib.mk_grouped_gemm.argtypes = [_vp, _vp, _c_i32, _vp, _c_i32, _c_i32, _vp, _vp, ctypes.c_size_t, _vp]
    lib.mk_grouped_gemm.restype = _c_i32
    lib.mk_grouped_gemm_swiglu.argtypes = [_vp, _vp, _c_i32, _vp, _c_i32, _c_i32, _vp, _vp, ctypes.c_size_t, _vp]
    lib.mk_grouped_gemm_swiglu.restype = _c_i32
    _lib = lib
    return lib


def mk_status_str(status: int) -> str:
    return load().mk_status_str(int(status)).decode()


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("libmk takes device tensors only")
    if not t.is_contiguous():
        raise ValueError("libmk takes contiguous tensors only")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check(status: int, what: str):
    if status != MK_OK:
        raise MkError(status, what)


def _shape(T, d, E, k, e_begin, E_local, N) -> MkShape:
    return MkShape(T, d, E, k, e_begin, E_local, N)


class _Sources:
    """Keeps the ctypes arrays of a mk_sources alive."""

    def __init__(self, xs: Sequence[torch.Tensor], chunk_rows=0, chunk_ready=None, epoch=0,
                 sim_delay_us=None, sim_payload=None):
        self.xs = list(xs)
        self.arr = (_vp * len(self.xs))(*[t.data_ptr() for t in self.xs])
        self.payload = None
        if sim_payload is not None:
            self.payload = (_vp * len(sim_payload))(*[t.data_ptr() for t in sim_payload])
        rows = self.xs[0].shape[0] if self.xs else 0
        self.c = MkSources(len(self.xs), rows, ctypes.cast(self.arr, ctypes.POINTER(_vp)), int(chunk_rows),
                           _ptr(chunk_ready), int(epoch) & 0xFFFFFFFF, _ptr(sim_delay_us),
                           None if self.payload is None else ctypes.cast(self.payload, ctypes.POINTER(_vp)))


def mk_route_topk_workspace_bytes(T: int, E: int) -> int:
    return int(load().mk_route_topk_workspace_bytes(T, E))


def mk_route_topk(x: torch.Tensor, w_router: torch.Tensor, k: int, bias: Optional[torch.Tensor] = None,
                  topk_ids: Optional[torch.Tensor] = None, topk_w: Optional[torch.Tensor] = None,
                  workspace: Optional[torch.Tensor] = None, stream=None, logits: Optional[torch.Tensor] = None):
    """Router logits, top-k and softmax gate (mk_route_topk).  Returns (topk_ids, topk_w).  If `logits`
    ([T, E] fp32) is given, every logit as it entered the selection is written there too."""
    lib = load()
    T, d = x.shape
    E = w_router.shape[1]
    dev = x.device
    if topk_ids is None:
        topk_ids = torch.empty(T, k, dtype=torch.int32, device=dev)
    if topk_w is None:
        topk_w = torch.empty(T, k, dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = torch.empty(mk_route_topk_workspace_bytes(T, E), dtype=torch.uint8, device=dev)
    st = lib.mk_route_topk(_ptr(x), _ptr(w_router), _ptr(bias), T, d, E, k, _ptr(topk_ids), _ptr(topk_w),
                           _ptr(logits), _ptr(workspace), workspace.numel(), _stream(stream))
    _check(st, "mk_route_topk")
    return topk_ids, topk_w


def _placeholder_sources(T, d, S, chunk_rows, xs):
    """mk_sources for the size and table queries: the given source tensors' addresses (the table reads rows
    in place only from sources inside one 4 GiB window), else S contiguous placeholder buffers."""
    S = len(xs) if xs is not None else max(S, 1)
    rows = T // S
    addrs = ([t.data_ptr() for t in xs] if xs is not None else
             [0x1000 + i * rows * d * 2 for i in range(S)])   # never dereferenced
    ptrs = (_vp * S)(*addrs)
    src = MkSources(S, rows, ctypes.cast(ptrs, ctypes.POINTER(_vp)), int(chunk_rows),
                    ctypes.c_void_p(0x1000) if chunk_rows else None, 0, None, None)
    return src, ptrs


def mk_dispatch_gemm_workspace_bytes(T, d, E, k, e_begin, E_local, N, S=1, chunk_rows=0,
                                     tune: Optional[dict] = None, xs: Optional[Sequence[torch.Tensor]] = None) -> int:
    """Workspace bytes for this shape, sources (xs: the source tensors, else S placeholders), arrival chunking and
    tuning (None = the table)."""
    shape = _shape(T, d, E, k, e_begin, E_local, N)
    src, _ptrs = _placeholder_sources(T, d, S, chunk_rows, xs)
    tu = _tuning(tune)
    return int(load().mk_dispatch_gemm_workspace_bytes(ctypes.byref(shape), ctypes.byref(src),
                                                       None if tu is None else ctypes.byref(tu)))


def mk_select_tuning(T, d, E, k, e_begin, E_local, N, S=1, chunk_rows=0,
                     xs: Optional[Sequence[torch.Tensor]] = None) -> dict:
    """The per-shape table's tuning for this shape, sources (as for mk_dispatch_gemm_workspace_bytes) and arrival
    chunking."""
    shape = _shape(T, d, E, k, e_begin, E_local, N)
    src, _ptrs = _placeholder_sources(T, d, S, chunk_rows, xs)
    out = MkTuning()
    _check(load().mk_select_tuning(ctypes.byref(shape), ctypes.byref(src), ctypes.byref(out)), "mk_select_tuning")
    return {f: getattr(out, f) for f in TUNING_INTS}


TRACE_WORDS = ("start", "routed", "barrier_a", "counted", "barrier_b", "slots", "barrier_c", "moved",
               "first_task", "done", "tasks", "wait_ticks", "xcc", "units", "copy_ticks", "release_ticks",
               "selected")


def mk_dispatch_gemm_trace(workspace: torch.Tensor, T, d, E, k, e_begin, E_local, N, S=1) -> dict:
    """The fused kernel's per-workgroup trace records (mk_dispatch_gemm_trace) as int64 arrays, plus
    ticks_per_us.  Synchronises first."""
    shape = _shape(T, d, E, k, e_begin, E_local, N)
    src = MkSources(S, T // max(S, 1), None, 0, None, 0, None, None)
    off, n_wg, words, tpu = ctypes.c_size_t(), _c_i32(), _c_i32(), _c_i32()
    _check(load().mk_dispatch_gemm_trace(ctypes.byref(shape), ctypes.byref(src), ctypes.byref(off),
                                         ctypes.byref(n_wg), ctypes.byref(words), ctypes.byref(tpu)),
           "mk_dispatch_gemm_trace")
    torch.cuda.synchronize(workspace.device)
    raw = workspace[off.value: off.value + n_wg.value * words.value * 8].view(torch.int64)
    rec = raw.view(n_wg.value, words.value).cpu().numpy()
    out = {name: rec[:, i] for i, name in enumerate(TRACE_WORDS)}
    out["ticks_per_us"] = tpu.value
    return out


def mk_poll_error(workspace: torch.Tensor):
    """(status, detail) of the device error word; clears it.  Synchronises first."""
    torch.cuda.synchronize(workspace.device)
    detail = _c_i32(0)
    st = load().mk_poll_error(_ptr(workspace), ctypes.byref(detail))
    return int(st), int(detail.value)


def mk_dispatch_gemm(x, w_experts: torch.Tensor, k: int, *, w_router: Optional[torch.Tensor] = None,
                     bias: Optional[torch.Tensor] = None, topk_ids_in: Optional[torch.Tensor] = None,
                     E: Optional[int] = None, e_begin: int = 0, workspace: Optional[torch.Tensor] = None,
                     out: Optional[dict] = None, tune: Optional[dict] = None, chunk_rows: int = 0,
                     chunk_ready: Optional[torch.Tensor] = None, epoch: int = 0,
                     sim_delay_us: Optional[torch.Tensor] = None, sim_payload=None, stream=None,
                     swiglu: bool = False) -> dict:
    """Fused dispatch + expert GEMM (mk_dispatch_gemm; with swiglu=True mk_dispatch_gemm_swiglu).

    x: [T, d] bf16 tensor, or a list of S shards [T/S, d] (token t = s*(T/S) + r).
    w_experts: [E_local, N, d] bf16.  Routing uses w_router/bias unless topk_ids_in is given.
    swiglu: w_experts holds the gate|up weights (N = 2F: F gate rows, then F up rows) and y_perm
    receives h = silu(gate) * up, [R_cap, F].
    workspace: a zero-filled uint8 tensor of mk_dispatch_gemm_workspace_bytes bytes, reused
    across calls (allocated and zero-filled here if None).
    Returns dict(y_perm, slot_of, expert_offsets, topk_ids, topk_w, row_token, workspace).
    """
    lib = load()
    xs = list(x) if isinstance(x, (list, tuple)) else [x]
    T = sum(t.shape[0] for t in xs)
    d = xs[0].shape[1]
    E_local, N, d2 = w_experts.shape
    if d2 != d:
        raise ValueError("w_experts must be [E_local, N, d]")
    if E is None:
        E = w_router.shape[1] if w_router is not None else E_local
    dev = w_experts.device
    r_cap = T * min(k, E_local)
    o = {} if out is None else dict(out)
    o.setdefault("y_perm", torch.empty(max(r_cap, 1), N // 2 if swiglu else N, dtype=torch.bfloat16, device=dev))
    o.setdefault("slot_of", torch.empty(T, k, dtype=torch.int32, device=dev))
    o.setdefault("expert_offsets", torch.empty(E_local + 1, dtype=torch.int32, device=dev))
    o.setdefault("topk_ids", torch.empty(T, k, dtype=torch.int32, device=dev))
    o.setdefault("topk_w", torch.empty(T, k, dtype=torch.float32, device=dev))
    o.setdefault("row_token", torch.empty(max(r_cap, 1), dtype=torch.int32, device=dev))
    shape = _shape(T, d, E, k, e_begin, E_local, N)
    srcs = _Sources(xs, chunk_rows, chunk_ready, epoch, sim_delay_us, sim_payload)
    tu = _tuning(tune)
    if workspace is None:
        nbytes = int(lib.mk_dispatch_gemm_workspace_bytes(ctypes.byref(shape), ctypes.byref(srcs.c),
                                                          None if tu is None else ctypes.byref(tu)))
        if nbytes == 0:
            _check(MK_EINVAL, "mk_dispatch_gemm_workspace_bytes")
        workspace = torch.zeros(nbytes, dtype=torch.uint8, device=dev)
    fn = lib.mk_dispatch_gemm_swiglu if swiglu else lib.mk_dispatch_gemm
    st = fn(ctypes.byref(shape), ctypes.byref(srcs.c), _ptr(w_router), _ptr(bias),
            _ptr(topk_ids_in), _ptr(w_experts), _ptr(o["y_perm"]), _ptr(o["slot_of"]),
            _ptr(o["expert_offsets"]), _ptr(o["topk_ids"]), _ptr(o["topk_w"]),
            _ptr(o["row_token"]), _ptr(workspace), workspace.numel(),
            None if tu is None else ctypes.byref(tu), _stream(stream))
    _check(st, "mk_dispatch_gemm_swiglu" if swiglu else "mk_dispatch_gemm")
    o["workspace"] = workspace
    o["_sources"] = srcs
    return o


def mk_dispatch_gemm_static(x: torch.Tensor, w_experts: torch.Tensor, k: int, out: dict, status: torch.Tensor, *,
                            w_router: Optional[torch.Tensor] = None, bias: Optional[torch.Tensor] = None,
                            topk_ids_in: Optional[torch.Tensor] = None, E: Optional[int] = None, e_begin: int = 0,
                            tune: Optional[dict] = None, stream=None) -> None:
    """mk_dispatch_gemm_static: the dispatch with the library's own device scratch instead of a workspace.
    Every output must be given in `out` (y_perm, slot_of, expert_offsets, and optionally topk_ids, topk_w,
    row_token); status is a device int32 tensor of at least 2 elements receiving (status, detail)."""
    lib = load()
    T, d = x.shape
    E_local, N, _ = w_experts.shape
    if E is None:
        E = w_router.shape[1] if w_router is not None else E_local
    shape = _shape(T, d, E, k, e_begin, E_local, N)
    srcs = _Sources([x])
    tu = _tuning(tune)
    st = lib.mk_dispatch_gemm_static(ctypes.byref(shape), ctypes.byref(srcs.c), _ptr(w_router), _ptr(bias),
                                     _ptr(topk_ids_in), _ptr(w_experts), _ptr(out["y_perm"]), _ptr(out["slot_of"]),
                                     _ptr(out["expert_offsets"]), _ptr(out.get("topk_ids")), _ptr(out.get("topk_w")),
                                     _ptr(out.get("row_token")), _ptr(status),
                                     None if tu is None else ctypes.byref(tu), _stream(stream))
    _check(st, "mk_dispatch_gemm_static")


def mk_combine(y_perm: torch.Tensor, slot_of: torch.Tensor, topk_w: torch.Tensor, rows: Optional[int] = None,
               out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Weighted un-permute (mk_combine): out[t] = bf16(sum over local choices j of topk_w[t, j] *
    y_perm[slot_of[t, j]]).  rows = the valid rows of y_perm (default: all of them).  Returns out [T, N]."""
    T, k = slot_of.shape
    N = y_perm.shape[1]
    if rows is None:
        rows = y_perm.shape[0]
    if out is None:
        out = torch.empty(T, N, dtype=torch.bfloat16, device=slot_of.device)
    st = load().mk_combine(_ptr(y_perm), int(rows), _ptr(slot_of), _ptr(topk_w), T, k, N, _ptr(out),
                           _stream(stream))
    _check(st, "mk_combine")
    return out


def mk_swiglu(gate_up: torch.Tensor, rows: Optional[int] = None, out: Optional[torch.Tensor] = None,
              stream=None) -> torch.Tensor:
    """h = bf16(silu(g) * u) of [g | u] rows (mk_swiglu).  Returns h [rows_total, F]."""
    R2, F2 = gate_up.shape
    F = F2 // 2
    if rows is None:
        rows = R2
    if out is None:
        out = torch.empty(R2, F, dtype=torch.bfloat16, device=gate_up.device)
    _check(load().mk_swiglu(_ptr(gate_up), int(rows), F, _ptr(out), _stream(stream)), "mk_swiglu")
    return out


def mk_grouped_gemm(a: torch.Tensor, expert_offsets: torch.Tensor, w: torch.Tensor,
                    out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                    stream=None) -> torch.Tensor:
    """y[r] = bf16(a[r] . W[e]^T) for the rows r of each expert e of the layout (mk_grouped_gemm)."""
    E_local, N, K = w.shape
    if out is None:
        out = torch.empty(a.shape[0], N, dtype=torch.bfloat16, device=a.device)
    if workspace is None:
        workspace = torch.empty(mk_grouped_gemm_workspace_bytes(E_local), dtype=torch.uint8, device=a.device)
    _check(load().mk_grouped_gemm(_ptr(a), _ptr(expert_offsets), E_local, _ptr(w), K, N, _ptr(out),
                                  _ptr(workspace), workspace.numel(), _stream(stream)), "mk_grouped_gemm")
    return out


def mk_grouped_gemm_swiglu(a: torch.Tensor, expert_offsets: torch.Tensor, w_gate_up: torch.Tensor,
                           out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                           stream=None) -> torch.Tensor:
    """h[r] = bf16(silu(g) * u) with [g | u] = bf16(a[r] . W[e]^T), W[e] = [gate; up] of 2F rows
    (mk_grouped_gemm_swiglu)."""
    E_local, two_f, K = w_gate_up.shape
    F = two_f // 2
    if out is None:
        out = torch.empty(a.shape[0], F, dtype=torch.bfloat16, device=a.device)
    if workspace is None:
        workspace = torch.empty(mk_grouped_gemm_workspace_bytes(E_local), dtype=torch.uint8, device=a.device)
    _check(load().mk_grouped_gemm_swiglu(_ptr(a), _ptr(expert_offsets), E_local, _ptr(w_gate_up), K, F,
                                         _ptr(out), _ptr(workspace), workspace.numel(), _stream(stream)),
           "mk_grouped_gemm_swiglu")
    return out


def mk_grouped_gemm_workspace_bytes(E_local: int) -> int:
    return int(load().mk_grouped_gemm_workspace_bytes(E_local))
