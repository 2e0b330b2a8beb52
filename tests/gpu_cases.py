"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI
binding, run the oracle on the same seeded inputs, compare."""
from __future__ import annotations

import numpy as np
import torch

import moe_dispatch_expert_amd as mk
import oracle
import workloads as W

# Expert outputs: |y_gpu - y_ref| <= max(REL * |y_ref|, FLOOR) per element
# (bf16 output, fp32 accumulation, fp64 reference).
Y_REL, Y_FLOOR = 1e-2, 1e-2
# Gate weights: fp32 softmax (any summation order, HIP expf) against fp64.
W_REL, W_FLOOR = 1e-4, 1e-6


def say(*a):
    print(*a, flush=True)


def source_views(x: torch.Tensor, S: int, reverse: bool = True) -> list:
    """The S row shards of x as regions of one device receive buffer (one region per peer, a spare row
    between regions; with reverse, source s sits in region S - 1 - s), so the sources are separate buffers
    whose offsets differ from their token order."""
    rows, d = x.shape[0] // S, x.shape[1]
    recv = torch.empty(S * (rows + 1), d, dtype=x.dtype, device="cuda")
    out = []
    for s in range(S):
        r = (S - 1 - s) if reverse else s
        v = recv[r * (rows + 1):r * (rows + 1) + rows]
        v.copy_(x[s * rows:(s + 1) * rows])
        out.append(v)
    return out


def to_dev(inp: dict, separate: bool = False) -> dict:
    """Device copies of the inputs; several sources as regions of one receive buffer (separate: one
    allocation each)."""
    wl = inp["wl"]
    dev = {}
    x = inp["x"]
    if wl.S > 1 and separate:
        dev["x"] = [x[s * wl.rows_per_src:(s + 1) * wl.rows_per_src].contiguous().cuda() for s in range(wl.S)]
    elif wl.S > 1:
        dev["x"] = source_views(x, wl.S)
    else:
        dev["x"] = x.cuda()
    dev["w_router"] = inp["w_router"].cuda()
    dev["bias"] = None if inp["bias"] is None else inp["bias"].cuda()
    dev["w_experts"] = inp["w_experts"].cuda()
    return dev


def oracle_route(inp: dict):
    wl = inp["wl"]
    b = None if inp["bias"] is None else inp["bias"].numpy()
    return oracle.route(inp["x"], inp["w_router"].numpy(), wl.k, b)


def sample_rows(offsets: np.ndarray, n_random: int, seed: int = 0) -> np.ndarray:
    R = int(offsets[-1])
    rows = set()
    for e in range(len(offsets) - 1):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if b > a:
            rows.update({a, b - 1, (a + b) // 2})
    rng = np.random.default_rng(seed)
    if R > 0:
        rows.update(rng.integers(0, R, size=min(n_random, R)).tolist())
    return np.array(sorted(rows), dtype=np.int32)


def assert_y_close(y_gpu: np.ndarray, y_ref: np.ndarray, what: str):
    err = np.abs(y_gpu.astype(np.float64) - y_ref)
    tol = np.maximum(Y_REL * np.abs(y_ref), Y_FLOOR)
    bad = err > tol
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} elements out of tolerance; first at "
                             f"{tuple(i)} gpu={y_gpu[tuple(i)]} ref={y_ref[tuple(i)]}")


def assert_w_close(w_gpu: np.ndarray, w_ref: np.ndarray, what: str):
    err = np.abs(w_gpu.astype(np.float64) - w_ref)
    tol = np.maximum(W_REL * np.abs(w_ref), W_FLOOR)
    assert (err <= tol).all(), f"{what}: gate weights out of tolerance, max err {err.max()}"


def check_layout(out: dict, ref_ids, wl, what: str):
    """Bit-exact layout against the oracle's layout of the same ids; returns the oracle layout."""
    count, offsets, slot_of, row_token = oracle.layout(ref_ids, wl.e_begin, wl.E_local)
    R = int(offsets[-1])
    g_off = out["expert_offsets"].cpu().numpy()
    assert np.array_equal(g_off, offsets), f"{what}: expert offsets differ"
    assert np.array_equal(out["slot_of"].cpu().numpy(), slot_of), f"{what}: slot_of differs"
    assert np.array_equal(out["row_token"][:R].cpu().numpy(), row_token), f"{what}: row_token differs"
    return count, offsets, slot_of, row_token


def full_check(inp: dict, out: dict, rows=None, check_w=True, what=""):
    """Routing, layout and sampled (or all) expert rows against the oracle."""
    wl = inp["wl"]
    _, ids, w = oracle_route(inp)
    assert np.array_equal(out["topk_ids"].cpu().numpy(), ids), f"{what}: topk ids differ"
    if check_w:
        assert_w_close(out["topk_w"].cpu().numpy(), w, what)
    count, offsets, slot_of, row_token = check_layout(out, ids, wl, what)
    R = int(offsets[-1])
    if rows is None:
        rows = np.arange(R, dtype=np.int32)
    y_ref = oracle.expert_rows(inp["x"], inp["w_experts"], offsets, row_token, rows)
    y_gpu = out["y_perm"][torch.from_numpy(rows.astype(np.int64)).cuda()].float().cpu().numpy()
    assert_y_close(y_gpu, y_ref, what)
    return dict(ids=ids, w=w, count=count, offsets=offsets, R=R)
