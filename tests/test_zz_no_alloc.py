"""The no-allocation entry point mk_dispatch_gemm_static: the dispatch with the library's own device
scratch in place of a caller's workspace.

GPU: two calls in a row through the C ABI (the second with fewer tokens, so the scratch holds the first
call's larger contents), each against mk_dispatch_gemm (the workspace entry point) on the same inputs:
routing, layout and expert rows identical, and against the CPU oracle (ids, offsets, slot maps
bit-exact; expert rows within max(1e-2 |ref|, 1e-2)).  CPU: a shape whose workspace exceeds the scratch
is refused before any device work.
"""
import ctypes

import numpy as np
import pytest
import torch

import moe_dispatch_expert_amd as mk
import workloads as W
from gpu_cases import full_check, say, to_dev

KEYS = ("y_perm", "slot_of", "expert_offsets", "topk_ids", "topk_w", "row_token")


@pytest.mark.gpu
def test_static_scratch_matches_workspace_entry_point():
    lib = mk.load()
    for T, seed in ((256, 51), (100, 52)):
        say(f"[gpu case] mk_dispatch_gemm_static tiny T={T} seed={seed}")
        wl = W.scaled(W.WORKLOADS["tiny"], T=T)
        inp = W.make_inputs(wl, seed)
        dev = to_dev(inp)
        ref = mk.mk_dispatch_gemm(dev["x"], dev["w_experts"], wl.k, w_router=dev["w_router"], E=wl.E)
        st, detail = mk.mk_poll_error(ref["workspace"])
        assert st == mk.MK_OK, (st, detail)
        r_cap = wl.T * min(wl.k, wl.E_local)
        out = {"y_perm": torch.full((r_cap, wl.N), float("nan"), dtype=torch.bfloat16, device="cuda"),
               "slot_of": torch.full((wl.T, wl.k), -9, dtype=torch.int32, device="cuda"),
               "expert_offsets": torch.full((wl.E_local + 1,), -9, dtype=torch.int32, device="cuda"),
               "topk_ids": torch.full((wl.T, wl.k), -9, dtype=torch.int32, device="cuda"),
               "topk_w": torch.full((wl.T, wl.k), -1.0, dtype=torch.float32, device="cuda"),
               "row_token": torch.full((r_cap,), -9, dtype=torch.int32, device="cuda")}
        status = torch.full((4,), -7, dtype=torch.int32, device="cuda")
        torch.cuda.synchronize()
        # through the C ABI directly
        shape = mk.MkShape(wl.T, wl.d, wl.E, wl.k, 0, wl.E_local, wl.N)
        xs = (ctypes.c_void_p * 1)(dev["x"].data_ptr())
        src = mk.MkSources(1, wl.T, ctypes.cast(xs, ctypes.POINTER(ctypes.c_void_p)), 0, None, 0, None, None)
        p = lambda t: ctypes.c_void_p(t.data_ptr())
        rc = lib.mk_dispatch_gemm_static(ctypes.byref(shape), ctypes.byref(src), p(dev["w_router"]), None, None,
                                         p(dev["w_experts"]), p(out["y_perm"]), p(out["slot_of"]),
                                         p(out["expert_offsets"]), p(out["topk_ids"]), p(out["topk_w"]),
                                         p(out["row_token"]), p(status), None,
                                         ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        assert rc == mk.MK_OK, mk.mk_status_str(rc)
        torch.cuda.synchronize()
        assert status[:2].cpu().tolist() == [mk.MK_OK, 0]
        R = int(ref["expert_offsets"][-1])
        assert int(out["expert_offsets"][-1]) == R
        for key in KEYS:
            a, b = ref[key], out[key]
            if key in ("y_perm", "row_token"):
                a, b = a[:R], b[:R]
            assert torch.equal(a, b), key
        full_check(inp, out, what=f"static scratch T={T}")


def test_static_scratch_refuses_a_workspace_beyond_it():
    """The wide expert-parallel share (8 sources, arrival flags) needs a workspace of about 134 MB (the router's
    partial sums of 16384 tokens x 256 experts): refused with MK_EWORKSPACE before any device work (no GPU needed)."""
    lib = mk.load()
    wl = W.WORKLOADS["wide_ep"]
    assert mk.mk_dispatch_gemm_workspace_bytes(wl.T, wl.d, wl.E, wl.k, 0, wl.E_local, wl.N, S=wl.S,
                                               chunk_rows=wl.chunk_rows) > (32 << 20)
    fake = ctypes.c_void_p(0x100000)
    shape = mk.MkShape(wl.T, wl.d, wl.E, wl.k, 0, wl.E_local, wl.N)
    xs = (ctypes.c_void_p * wl.S)(*[0x100000 + i * wl.rows_per_src * wl.d * 2 for i in range(wl.S)])
    src = mk.MkSources(wl.S, wl.rows_per_src, ctypes.cast(xs, ctypes.POINTER(ctypes.c_void_p)), wl.chunk_rows,
                       fake, 1, None, None)
    rc = lib.mk_dispatch_gemm_static(ctypes.byref(shape), ctypes.byref(src), None, None, fake, fake, fake, fake,
                                     fake, None, None, None, fake, None, None)
    assert rc == mk.MK_EWORKSPACE
    # a missing or misaligned status buffer is an argument error
    rc = lib.mk_dispatch_gemm_static(ctypes.byref(shape), ctypes.byref(src), None, None, fake, fake, fake, fake,
                                     fake, None, None, None, ctypes.c_void_p(0x100008), None, None)
    assert rc == mk.MK_EINVAL
