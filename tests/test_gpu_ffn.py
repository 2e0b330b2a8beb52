"""Expert FFN after the gate|up GEMM (the next row): mk_swiglu and the
down-projection mk_grouped_gemm against the oracle on the same seeded bf16
inputs (made here, not by the HIP path).

Tolerances: SwiGLU is fp32 then one bf16 rounding, |h - ref| <= 2^-8 |ref| +
1e-6; the grouped GEMM is the expert-output bar, max(1e-2 |ref|, 1e-2)."""
import numpy as np
import pytest
import torch

import moe_dispatch_expert_amd as mk
import oracle
from gpu_cases import Y_FLOOR, Y_REL, sample_rows, say

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _name(request):
    say(f"\n[gpu case] {request.node.nodeid}")
    yield
    torch.cuda.synchronize()


def _bf16(shape, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(*shape, generator=g) * scale).to(torch.bfloat16)


@pytest.mark.parametrize("rows,F", [(300, 520), (1, 8), (64, 2048)])
def test_swiglu_matches_oracle(rows, F):
    gu = _bf16((rows, 2 * F), 21 + rows, scale=3.0)
    h = mk.mk_swiglu(gu.cuda())
    torch.cuda.synchronize()
    ref = oracle.swiglu(gu)
    got = h.float().cpu().numpy()
    bad = np.abs(got - ref) > 2.0 ** -8 * np.abs(ref) + 1e-6
    assert not bad.any(), f"{int(bad.sum())} of {bad.size}; first at {tuple(np.argwhere(bad)[0])}"


def _layout(counts):
    return np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)


@pytest.mark.parametrize("counts,K,N", [
    ([300, 0, 37, 256, 129], 256, 264),      # empty expert, ragged tails of every tile height
    ([1, 2, 513], 384, 520),                  # one-row experts, a tile and a half
    ([64] * 8, 128, 256),
])
def test_grouped_gemm_matches_oracle(counts, K, N):
    offsets = _layout(counts)
    R, E_local = int(offsets[-1]), len(counts)
    a = _bf16((R + 5, K), 31 + K)             # 5 rows past R that must not matter
    w = _bf16((E_local, N, K), 41 + N, scale=K ** -0.5)
    out = torch.full((R + 5, N), 7.0, dtype=torch.bfloat16, device="cuda")
    mk.mk_grouped_gemm(a.cuda(), torch.from_numpy(offsets).cuda(), w.cuda(), out=out)
    torch.cuda.synchronize()
    ref = oracle.grouped_rows(a[:R], w, offsets, np.arange(R))
    got = out[:R].float().cpu().numpy()
    bad = np.abs(got - ref) > np.maximum(Y_REL * np.abs(ref), Y_FLOOR)
    assert not bad.any(), f"{int(bad.sum())} of {bad.size}; first at {tuple(np.argwhere(bad)[0])}"
    assert (out[R:] == 7.0).all(), "rows past R were written"


def test_grouped_gemm_empty_layout_and_errors():
    """An empty layout (all offsets 0) launches no task: the outputs stay as they were; K % 128 != 0 is refused."""
    w = _bf16((3, 16, 128), 1)
    out = torch.full((4, 16), 7.0, dtype=torch.bfloat16, device="cuda")
    mk.mk_grouped_gemm(torch.zeros(4, 128, dtype=torch.bfloat16, device="cuda"),
                       torch.zeros(4, dtype=torch.int32, device="cuda"), w.cuda(), out=out)
    torch.cuda.synchronize()
    assert (out == 7.0).all()
    h = torch.full((4, 8), 7.0, dtype=torch.bfloat16, device="cuda")   # the SwiGLU variant: F = 8
    mk.mk_grouped_gemm_swiglu(torch.zeros(4, 128, dtype=torch.bfloat16, device="cuda"),
                              torch.zeros(4, dtype=torch.int32, device="cuda"), w.cuda(), out=h)
    torch.cuda.synchronize()
    assert (h == 7.0).all()
    with pytest.raises(mk.MkError):   # K % 128 != 0: unsupported, nothing launched
        mk.mk_grouped_gemm(torch.zeros(4, 64, dtype=torch.bfloat16, device="cuda"),
                           torch.zeros(4, dtype=torch.int32, device="cuda"),
                           torch.zeros(3, 16, 64, dtype=torch.bfloat16, device="cuda"))


def _silu(g):
    return g / (1.0 + np.exp(-g))


@pytest.mark.parametrize("counts,K,F", [
    ([300, 0, 37, 256, 129], 256, 264),      # empty expert, every tile height, a 8-feature last block
    ([1, 2, 513], 384, 136),                  # one-row experts; gate and up blocks overlap (F < 256)
    ([40, 3], 128, 8),                        # F < 128: the up rows sit before the tile's second half
    ([64] * 8, 128, 256),
])
def test_grouped_gemm_swiglu(counts, K, F):
    """The gate|up GEMM with the SwiGLU epilogue gives the bits of mk_grouped_gemm (N = 2F) followed by
    mk_swiglu, and matches the oracle chain (GEMM, bf16 rounding, SwiGLU) within the bar derived from
    one bf16 step of g or u: |dh| <= 2^-7 (|g silu'(g) u| + |silu(g) u|) + 2^-8 |h| + 1e-6."""
    offsets = _layout(counts)
    R, E_local = int(offsets[-1]), len(counts)
    a = _bf16((R + 3, K), 51 + K)
    w = _bf16((E_local, 2 * F, K), 61 + F, scale=2.0 * K ** -0.5)
    dev_off = torch.from_numpy(offsets).cuda()
    h = torch.full((R + 3, F), 7.0, dtype=torch.bfloat16, device="cuda")
    mk.mk_grouped_gemm_swiglu(a.cuda(), dev_off, w.cuda(), out=h)
    gu = mk.mk_grouped_gemm(a.cuda(), dev_off, w.cuda())
    h2 = mk.mk_swiglu(gu[:R].contiguous())
    torch.cuda.synchronize()
    assert (h[R:] == 7.0).all(), "rows past R were written"
    ne = (h[:R] != h2).cpu().numpy()
    assert not ne.any(), (f"fused epilogue differs from GEMM + SwiGLU at {int(ne.sum())} of {ne.size}; "
                          f"first at {tuple(np.argwhere(ne)[0])}")
    ref_gu = torch.from_numpy(oracle.grouped_rows(a[:R], w, offsets, np.arange(R))).to(torch.bfloat16)
    ref = oracle.swiglu(ref_gu)
    g = ref_gu[:, :F].double().numpy()
    u = ref_gu[:, F:].double().numpy()
    sig = 1.0 / (1.0 + np.exp(-g))
    dsilu = sig * (1.0 + g * (1.0 - sig))
    tol = 2.0 ** -7 * (np.abs(g * dsilu * u) + np.abs(_silu(g) * u)) + 2.0 ** -8 * np.abs(ref) + 1e-6
    got = h[:R].float().cpu().numpy()
    bad = np.abs(got - ref) > tol
    assert not bad.any(), f"{int(bad.sum())} of {bad.size}; first at {tuple(np.argwhere(bad)[0])}"


def test_grouped_gemm_swiglu_mixtral_size():
    """Mixtral's expert FFN shape (8 experts of 1024 rows plus a ragged 37-row tail on one, K = 4096, F = 7168):
    the SwiGLU-epilogue GEMM equals GEMM + SwiGLU bit for bit on every output, and sampled rows (every expert's
    first, middle and last row, plus 16 seeded random rows) match the oracle chain within the derived bar."""
    counts = [1024] * 7 + [1061]
    K, F = 4096, 7168
    offsets = _layout(counts)
    R, E_local = int(offsets[-1]), len(counts)
    a = _bf16((R, K), 71)
    w = _bf16((E_local, 2 * F, K), 81, scale=2.0 * K ** -0.5)
    dev_off = torch.from_numpy(offsets).cuda()
    a_d, w_d = a.cuda(), w.cuda()
    h = mk.mk_grouped_gemm_swiglu(a_d, dev_off, w_d)
    h2 = mk.mk_swiglu(mk.mk_grouped_gemm(a_d, dev_off, w_d))
    torch.cuda.synchronize()
    ne = int((h != h2).sum().item())
    assert ne == 0, f"fused epilogue differs from GEMM + SwiGLU at {ne} outputs"
    rows = sample_rows(offsets, 16, seed=5).astype(np.int64)   # first, middle, last of every expert + 16 seeded
    ref_gu = torch.from_numpy(oracle.grouped_rows(a, w, offsets, rows.astype(np.int32))).to(torch.bfloat16)
    ref = oracle.swiglu(ref_gu)
    g = ref_gu[:, :F].double().numpy()
    u = ref_gu[:, F:].double().numpy()
    sig = 1.0 / (1.0 + np.exp(-g))
    dsilu = sig * (1.0 + g * (1.0 - sig))
    tol = 2.0 ** -7 * (np.abs(g * dsilu * u) + np.abs(_silu(g) * u)) + 2.0 ** -8 * np.abs(ref) + 1e-6
    got = h[torch.from_numpy(rows).cuda()].float().cpu().numpy()
    bad = np.abs(got - ref) > tol
    assert not bad.any(), f"{int(bad.sum())} of {bad.size}; first at {tuple(np.argwhere(bad)[0])}"


def test_down_projection_mixtral_size():
    """The down-projection at Mixtral's expert FFN shape (K = F = 7168, N = d = 4096, 8 experts, a ragged tail):
    sampled rows (every expert's first, middle and last row, plus 16 seeded random rows) against the oracle
    within the expert-output bar; rows past R untouched."""
    counts = [1024] * 7 + [1061]
    K, N = 7168, 4096
    offsets = _layout(counts)
    R, E_local = int(offsets[-1]), len(counts)
    a = _bf16((R, K), 91)
    w = _bf16((E_local, N, K), 101, scale=K ** -0.5)
    out = torch.full((R + 4, N), 7.0, dtype=torch.bfloat16, device="cuda")
    mk.mk_grouped_gemm(a.cuda(), torch.from_numpy(offsets).cuda(), w.cuda(), out=out)
    torch.cuda.synchronize()
    assert (out[R:] == 7.0).all(), "rows past R were written"
    rows = sample_rows(offsets, 16, seed=5).astype(np.int64)   # first, middle, last of every expert + 16 seeded
    ref = oracle.grouped_rows(a, w, offsets, rows.astype(np.int32))
    got = out[torch.from_numpy(rows).cuda()].float().cpu().numpy()
    bad = np.abs(got - ref) > np.maximum(Y_REL * np.abs(ref), Y_FLOOR)
    assert not bad.any(), f"{int(bad.sum())} of {bad.size}; first at {tuple(np.argwhere(bad)[0])}"


# ---------------------------------------------------------------- the FFN over the dispatch's own layout

def _swiglu_tol(ref_gu: torch.Tensor, ref: np.ndarray, F: int) -> np.ndarray:
    """Per-element bar of h against the oracle chain: one bf16 ulp (2^-8 relative) in g or in u moves h by at
    most 2^-7 of its sensitivity to each, plus h's own bf16 rounding."""
    g = ref_gu[:, :F].double().numpy()
    u = ref_gu[:, F:].double().numpy()
    sig = 1.0 / (1.0 + np.exp(-g))
    dsilu = sig * (1.0 + g * (1.0 - sig))
    return 2.0 ** -7 * (np.abs(g * dsilu * u) + np.abs(_silu(g) * u)) + 2.0 ** -8 * np.abs(ref) + 1e-6


def _ffn_case(name, seed, **changes):
    import workloads as W
    wl = W.scaled(W.WORKLOADS[name], **changes) if changes else W.WORKLOADS[name]
    inp = W.make_inputs(wl, seed)
    dev = {"x": inp["x"].cuda(), "w_router": inp["w_router"].cuda(), "w": inp["w_experts"].cuda(),
           "bias": None if inp["bias"] is None else inp["bias"].cuda()}
    return wl, inp, dev


def _dispatch(wl, dev, swiglu, tune=None, out=None):
    o = mk.mk_dispatch_gemm(dev["x"], dev["w"], wl.k, w_router=dev["w_router"], bias=dev["bias"], E=wl.E,
                            e_begin=wl.e_begin, tune=tune, out=out, swiglu=swiglu)
    torch.cuda.synchronize()
    assert mk.mk_poll_error(o["workspace"])[0] == mk.MK_OK
    return o


@pytest.mark.parametrize("path", ["table", "movers", "staged"])
def test_dispatch_swiglu_equals_dispatch_then_swiglu(path):
    """mk_dispatch_gemm_swiglu (gate|up weights, SwiGLU in the epilogue, 2F = 1024, ragged expert tails) gives
    bit for bit mk_dispatch_gemm followed by mk_swiglu on every routed row, the same layout, and leaves rows
    >= R of its output alone, in each launch configuration.  2F = 1040: the last feature tile is ragged."""
    wl, inp, dev = _ffn_case("tiny", 11, T=700, N=1040)
    tune = {"table": {}, "movers": {"n_mover_wg": 64}, "staged": {"n_mover_wg": mk.MK_MOVERS_STAGED}}[path]
    F = wl.N // 2
    r_cap = wl.T * min(wl.k, wl.E_local)
    h = torch.full((r_cap + 3, F), 7.0, dtype=torch.bfloat16, device="cuda")
    o_h = _dispatch(wl, dev, True, tune, out={"y_perm": h})
    o_y = _dispatch(wl, dev, False, tune)
    R = int(o_y["expert_offsets"][-1].item())
    for key in ("expert_offsets", "slot_of", "topk_ids"):
        assert torch.equal(o_h[key], o_y[key]), key
    h2 = mk.mk_swiglu(o_y["y_perm"][:R].contiguous())
    torch.cuda.synchronize()
    ne = (h[:R] != h2).cpu().numpy()
    assert not ne.any(), f"{int(ne.sum())} of {ne.size} differ; first at {tuple(np.argwhere(ne)[0])}"
    assert (h[R:] == 7.0).all(), "rows past R were written"


def test_ffn_over_dispatch_layout_matches_oracle_chain():
    """The expert FFN on the Mixtral-shaped workload read as gate|up weights (2F = 14336): the fused
    dispatch + gate|up GEMM + SwiGLU, then the down-projection mk_grouped_gemm (W_down [8, 4096, 7168]) over the
    same layout.  Sampled rows (every expert's first, middle and last, plus 8 seeded) against the oracle chain
    (routing, layout, fp64 expert rows rounded to bf16, SwiGLU, fp64 down-projection); h within the SwiGLU bar,
    the down output within the expert-output bar widened by the h bar carried through W_down."""
    wl, inp, dev = _ffn_case("mixtral", 0)
    F = wl.N // 2
    o = _dispatch(wl, dev, True)
    lg, ids, _ = oracle.route(inp["x"], inp["w_router"].numpy(), wl.k)
    assert np.array_equal(o["topk_ids"].cpu().numpy(), ids)
    _, offsets, _, row_token = oracle.layout(ids, wl.e_begin, wl.E_local)
    assert np.array_equal(o["expert_offsets"].cpu().numpy(), offsets)
    R = int(offsets[-1])
    rows = sample_rows(offsets, 8, seed=3)
    ref_gu = torch.from_numpy(oracle.expert_rows(inp["x"], inp["w_experts"], offsets, row_token, rows)).to(
        torch.bfloat16)
    ref_h = oracle.swiglu(ref_gu)
    tol_h = _swiglu_tol(ref_gu, ref_h, F)
    idx = torch.from_numpy(rows.astype(np.int64)).cuda()
    got_h = o["y_perm"][idx].float().cpu().numpy()
    bad = np.abs(got_h - ref_h) > tol_h
    assert not bad.any(), f"h: {int(bad.sum())} of {bad.size}; first at {tuple(np.argwhere(bad)[0])}"
    wd = _bf16((wl.E_local, wl.d, F), 7, scale=F ** -0.5)
    z = mk.mk_grouped_gemm(o["y_perm"], o["expert_offsets"], wd.cuda())
    torch.cuda.synchronize()
    # the oracle's down-projection of its own h rows (rows not sampled are zero and not read)
    a = torch.zeros(R, F, dtype=torch.bfloat16)
    a[torch.from_numpy(rows.astype(np.int64))] = torch.from_numpy(ref_h.astype(np.float32)).to(torch.bfloat16)
    ref_z = oracle.grouped_rows(a, wd, offsets, rows)
    e_of = np.searchsorted(offsets, rows, side="right") - 1
    # |h_gpu - bf16(h_ref)| <= tol_h + 2^-8 |h_ref| per element, carried through |W_down| (one expert at a time)
    dh = tol_h + 2.0 ** -8 * np.abs(ref_h)
    carried = np.zeros((len(rows), wl.d))
    for e in np.unique(e_of):
        carried[e_of == e] = dh[e_of == e] @ np.abs(wd[e].double().numpy()).T
    got_z = z[idx].float().cpu().numpy()
    bad = np.abs(got_z - ref_z) > np.maximum(Y_REL * np.abs(ref_z), Y_FLOOR) + carried
    assert not bad.any(), f"down: {int(bad.sum())} of {bad.size}; first at {tuple(np.argwhere(bad)[0])}"
