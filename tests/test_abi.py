"""The C ABI boundary without a GPU: libmk.so loads, exports every function
include/mk.h declares, its struct layouts match the Python binding, and
argument errors come back synchronously (no launch, so no device needed)."""
import ctypes
import os
import re
import subprocess

import pytest

import moe_dispatch_expert_amd as mk

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mk.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mk_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib_path = mk.LIB_PATH
    assert os.path.exists(lib_path), "build libmk.so first (moe_dispatch_expert_amd/build.py)"
    out = subprocess.run(["nm", "-D", "--defined-only", lib_path], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\bT (mk_\w+)", out))
    declared = _declared_functions()
    assert len(declared) >= 7
    missing = [f for f in declared if f not in exported]
    assert not missing, missing
    lib = mk.load()
    for f in declared:
        assert hasattr(lib, f)


def test_struct_layout_matches_binding(tmp_path):
    src = tmp_path / "layout.c"
    src.write_text(r'''
#include <stdio.h>
#include <stddef.h>
#include "mk.h"
int main(void) {
  printf("%zu %zu %zu %zu\n", sizeof(mk_shape), sizeof(mk_sources), sizeof(mk_tuning), sizeof(mk_status));
  printf("%zu %zu %zu %zu %zu %zu %zu %zu\n", offsetof(mk_sources, S), offsetof(mk_sources, rows_per_src),
         offsetof(mk_sources, x), offsetof(mk_sources, chunk_rows), offsetof(mk_sources, chunk_ready),
         offsetof(mk_sources, epoch), offsetof(mk_sources, sim_delay_us), offsetof(mk_sources, sim_payload));
  printf("%zu %zu %zu %zu %zu\n", offsetof(mk_shape, N), offsetof(mk_tuning, bk), offsetof(mk_tuning, cooperative),
         offsetof(mk_tuning, tile_order), offsetof(mk_tuning, ev_gemm_end));
  return 0;
}
''')
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)],
                   check=True)
    lines = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split("\n")
    sizes = list(map(int, lines[0].split()))
    offs = list(map(int, lines[1].split()))
    last = list(map(int, lines[2].split()))
    assert sizes == [ctypes.sizeof(mk.MkShape), ctypes.sizeof(mk.MkSources), ctypes.sizeof(mk.MkTuning), 4]
    S = mk.MkSources
    assert offs == [S.S.offset, S.rows_per_src.offset, S.x.offset, S.chunk_rows.offset, S.chunk_ready.offset,
                    S.epoch.offset, S.sim_delay_us.offset, S.sim_payload.offset]
    assert last == [mk.MkShape.N.offset, mk.MkTuning.bk.offset, mk.MkTuning.cooperative.offset,
                    mk.MkTuning.tile_order.offset, mk.MkTuning.ev_gemm_end.offset]


def test_header_compiles_as_cxx(tmp_path):
    src = tmp_path / "h.cpp"
    src.write_text('#include "mk.h"\nint main() { return mk_status_str ? 0 : 1; }\n')
    subprocess.run(["g++", "-std=c++11", "-fsyntax-only", "-I", os.path.join(ROOT, "include"), str(src)],
                   check=True)


def test_status_strings():
    assert mk.mk_status_str(mk.MK_OK) == "ok"
    assert "workspace" in mk.mk_status_str(mk.MK_EWORKSPACE)
    assert mk.mk_status_str(99) == "unknown status"


def test_argument_errors_are_synchronous():
    lib = mk.load()
    # k > E, bad d, null pointers: rejected before any HIP call
    assert lib.mk_route_topk(None, None, None, 4, 128, 8, 9, None, None, None, None, 0, None) == mk.MK_EINVAL
    assert lib.mk_route_topk(None, None, None, 4, 100, 8, 2, None, None, None, None, 0, None) == mk.MK_EINVAL
    assert lib.mk_route_topk(None, None, None, 4, 136, 8, 2, None, None, None, None, 0, None) == mk.MK_EUNSUPPORTED
    assert lib.mk_route_topk(None, None, None, 4, 128, 8, 2, None, None, None, None, 0, None) == mk.MK_EINVAL
    assert lib.mk_route_topk(None, None, None, 0, 128, 8, 2, None, None, None, None, 0, None) == mk.MK_OK


def test_workspace_bytes_and_tuning_without_gpu():
    row_buffer = (8192 + 256) * 4096 * 2
    in_place = mk.mk_dispatch_gemm_workspace_bytes(4096, 4096, 8, 2, 0, 8, 14336)
    moved = mk.mk_dispatch_gemm_workspace_bytes(4096, 4096, 8, 2, 0, 8, 14336, tune={"n_mover_wg": 64})
    staged = mk.mk_dispatch_gemm_workspace_bytes(4096, 4096, 8, 2, 0, 8, 14336,
                                                 tune={"n_mover_wg": mk.MK_MOVERS_STAGED})
    assert 0 < in_place < row_buffer                     # rows read in place: no row buffer
    assert moved == staged and moved - in_place >= row_buffer
    # up to 8 sources in one 4 GiB window, resident or arriving: rows read in place, no row buffer; more
    # sources: the table moves rows, so the row buffer is part of the default
    assert mk.mk_dispatch_gemm_workspace_bytes(4096, 4096, 8, 2, 0, 8, 14336, S=2) < row_buffer
    assert mk.mk_dispatch_gemm_workspace_bytes(4096, 4096, 8, 2, 0, 8, 14336, S=8, chunk_rows=128) < row_buffer
    assert mk.mk_dispatch_gemm_workspace_bytes(4096, 4096, 8, 2, 0, 8, 14336, S=16) >= moved
    assert mk.mk_dispatch_gemm_workspace_bytes(4096, 4096, 8, 9, 0, 8, 14336) == 0   # k > E
    assert mk.mk_dispatch_gemm_workspace_bytes(16, 128, 8, 2, 4, 8, 64) == 0         # local range past E
    # in place needs at most 8 sources; staged launches cannot wait for arrival flags
    assert mk.mk_dispatch_gemm_workspace_bytes(4096, 4096, 8, 2, 0, 8, 14336, S=16,
                                               tune={"n_mover_wg": mk.MK_MOVERS_NONE}) == 0
    assert mk.mk_dispatch_gemm_workspace_bytes(4096, 4096, 8, 2, 0, 8, 14336, S=2, chunk_rows=128,
                                               tune={"n_mover_wg": mk.MK_MOVERS_STAGED}) == 0
    # tile sizes other than the one built, negative counts and a bad cooperative flag are refused
    for bad in ({"bm": 128}, {"bk": 32}, {"n_compute_wg": -1}, {"n_mover_wg": -3}, {"cooperative": 2},
                {"tile_order": 3}, {"tile_order": -1}):
        assert mk.mk_dispatch_gemm_workspace_bytes(4096, 4096, 8, 2, 0, 8, 14336, tune=bad) == 0, bad
    t = mk.mk_select_tuning(4096, 4096, 8, 2, 0, 8, 14336)
    assert t["bm"] == 256 and t["bn"] == 256 and t["bk"] == 64 and t["n_mover_wg"] == mk.MK_MOVERS_NONE
    assert mk.mk_select_tuning(16384, 7168, 256, 8, 0, 32, 2048, S=8, chunk_rows=128)["n_mover_wg"] == \
        mk.MK_MOVERS_NONE
    assert mk.mk_select_tuning(16384, 7168, 256, 8, 0, 32, 2048, S=16, chunk_rows=128)["n_mover_wg"] == 256
    # compute workgroups keyed on the shape: the expected GEMM tasks plus a quarter, multiple of 8, >= 32;
    # 0 (all) once that reaches 256
    assert mk.mk_select_tuning(256, 512, 8, 2, 0, 8, 1024)["n_compute_wg"] == 40        # 32 tasks
    assert mk.mk_select_tuning(1024, 4096, 8, 2, 0, 8, 4096)["n_compute_wg"] == 160     # 128 tasks
    assert mk.mk_select_tuning(16, 512, 8, 2, 0, 8, 256)["n_compute_wg"] == 32          # 8 tasks: the floor
    assert mk.mk_select_tuning(128, 7168, 256, 8, 0, 32, 2048)["n_compute_wg"] == 0     # 256 tasks
    assert mk.mk_select_tuning(16384, 7168, 256, 8, 0, 32, 2048, S=16)["n_compute_wg"] == 0   # rows moved
    assert mk.mk_select_tuning(4096, 4096, 8, 2, 0, 8, 14336, S=16)["n_mover_wg"] > 0
    with pytest.raises(mk.MkError):
        mk.mk_select_tuning(4096, 4096, 8, 2, 0, 8, 14335)
    # task order: short tails last with at most three rounds of tasks on 256 workgroups
    assert mk.mk_select_tuning(16384, 7168, 256, 8, 0, 32, 2048, S=8, chunk_rows=128)["tile_order"] == \
        mk.MK_ORDER_TAILS_LAST                                                              # 512 tasks
    assert mk.mk_select_tuning(4096, 4096, 8, 2, 0, 8, 14336)["tile_order"] == mk.MK_ORDER_EXPERT   # 1792
    assert mk.mk_select_tuning(8192, 2048, 64, 6, 0, 64, 1408)["tile_order"] == mk.MK_ORDER_EXPERT  # 1152
    assert mk.mk_select_tuning(16384, 7168, 256, 8, 0, 32, 2048, S=16, chunk_rows=128)["tile_order"] == \
        mk.MK_ORDER_EXPERT                                                                  # rows moved


def test_next_steps_argument_errors_are_synchronous():
    """mk_combine, mk_swiglu, mk_grouped_gemm and mk_grouped_gemm_swiglu refuse bad arguments before touching the device, and
    their empty cases are no-ops."""
    lib = mk.load()
    fake = ctypes.c_void_p(0x1000)            # aligned, never dereferenced: every call below returns early
    odd = ctypes.c_void_p(0x1008)             # 8-byte aligned only
    # combine: k range, N % 8, T == 0 no-op, null and misaligned pointers
    assert lib.mk_combine(fake, 4, fake, fake, 4, 0, 64, fake, None) == mk.MK_EINVAL
    assert lib.mk_combine(fake, 4, fake, fake, 4, 33, 64, fake, None) == mk.MK_EINVAL
    assert lib.mk_combine(fake, 4, fake, fake, 4, 2, 60, fake, None) == mk.MK_EINVAL
    assert lib.mk_combine(None, 4, None, None, 0, 2, 64, None, None) == mk.MK_OK
    assert lib.mk_combine(fake, 4, None, fake, 4, 2, 64, fake, None) == mk.MK_EINVAL
    assert lib.mk_combine(fake, 4, fake, fake, 4, 2, 64, odd, None) == mk.MK_EINVAL
    # swiglu: F % 8, rows == 0 no-op, misaligned
    assert lib.mk_swiglu(fake, 4, 12, fake, None) == mk.MK_EINVAL
    assert lib.mk_swiglu(None, 0, 16, None, None) == mk.MK_OK
    assert lib.mk_swiglu(odd, 4, 16, fake, None) == mk.MK_EINVAL
    # grouped GEMM: E_local range, K % 128 unsupported, workspace size, N % 8
    assert lib.mk_grouped_gemm(fake, fake, 0, fake, 128, 64, fake, fake, 4096, None) == mk.MK_EINVAL
    assert lib.mk_grouped_gemm(fake, fake, 4, fake, 64, 64, fake, fake, 4096, None) == mk.MK_EUNSUPPORTED
    assert lib.mk_grouped_gemm(fake, fake, 4, fake, 128, 60, fake, fake, 4096, None) == mk.MK_EINVAL
    need = lib.mk_grouped_gemm_workspace_bytes(4)
    assert need > 0 and lib.mk_grouped_gemm_workspace_bytes(0) == 0
    assert lib.mk_grouped_gemm(fake, fake, 4, fake, 128, 64, fake, fake, need - 1, None) == mk.MK_EWORKSPACE
    # gate|up GEMM with the SwiGLU epilogue: the same checks, F % 8, and 32-bit W row offsets
    sw = lib.mk_grouped_gemm_swiglu
    assert sw(fake, fake, 0, fake, 128, 64, fake, fake, need, None) == mk.MK_EINVAL
    assert sw(fake, fake, 4, fake, 64, 64, fake, fake, need, None) == mk.MK_EUNSUPPORTED
    assert sw(fake, fake, 4, fake, 128, 60, fake, fake, need, None) == mk.MK_EINVAL
    assert sw(fake, fake, 4, fake, 128, 64, fake, fake, need - 1, None) == mk.MK_EWORKSPACE
    assert sw(fake, fake, 4, fake, 8192, 131072, fake, fake, need, None) == mk.MK_EUNSUPPORTED
    assert sw(fake, fake, 4, fake, 128, 64, odd, fake, need, None) == mk.MK_EINVAL


def test_dispatch_refusals_without_gpu():
    """mk_dispatch_gemm_swiglu refuses an odd feature count and a gate|up matrix past the 32-bit tile offsets, and
    the arrival simulator refuses more chunks than it holds, all before touching the device."""
    lib = mk.load()
    fake = ctypes.c_void_p(0x1000)
    xs = (ctypes.c_void_p * 8)(*([0x1000] * 8))

    def call(fn, shape, S=1, chunk_rows=0, sim=False):
        src = mk.MkSources(S, shape.T // S, ctypes.cast(xs, ctypes.POINTER(ctypes.c_void_p)), chunk_rows,
                           fake if chunk_rows else None, 1, fake if sim else None, None)
        return fn(ctypes.byref(shape), ctypes.byref(src), fake, None, None, fake, fake, fake, fake, None, None, None,
                  fake, 1 << 40, None, None)

    sw = lib.mk_dispatch_gemm_swiglu
    assert call(sw, mk.MkShape(256, 512, 8, 2, 0, 8, 1032)) == mk.MK_EINVAL           # F = 516, not a multiple of 8
    assert call(sw, mk.MkShape(256, 8192, 8, 2, 0, 8, 131072)) == mk.MK_EUNSUPPORTED  # (2F + 256) d 2 >= 2^31
    big = mk.MkShape(32768, 1024, 64, 4, 0, 16, 512)
    assert call(lib.mk_dispatch_gemm, big, S=8, chunk_rows=1, sim=True) == mk.MK_EUNSUPPORTED   # 32768 chunks
