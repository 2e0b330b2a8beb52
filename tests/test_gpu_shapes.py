"""Shape edges of the HIP path against the CPU oracle.

- Expert row counts on every tile-height boundary (the ragged last row tile of
  an expert runs as a 256-, 128-, 64- or 32-row tile): ids are given, so the
  counts are exact, and tagged-identity experts make every output row an
  exactly scaled copy of its token row (bit-exact), then random experts are
  checked to the tolerance.
- K depths with an odd number of slab pairs and the smallest legal d.
- Global expert counts above 64 that are not multiples of 64 (the
  token-per-wave selection with 2, 4, 8 and 16 keys per lane), k = 1 and the
  largest k.
- The layout's LDS capacities: the block-base table and the scan arrays full,
  and one block past each.
"""
import numpy as np
import pytest
import torch

import moe_dispatch_expert_amd as mk
import oracle
import workloads as W
from gpu_cases import assert_y_close, check_layout, full_check, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _name(request):
    say(f"\n[gpu case] {request.node.nodeid}")
    yield
    torch.cuda.synchronize()


def _run(inp, dev, **kw):
    wl = inp["wl"]
    out = mk.mk_dispatch_gemm(dev["x"], dev["w_experts"], wl.k, w_router=dev["w_router"], bias=dev["bias"],
                              E=wl.E, e_begin=wl.e_begin, **kw)
    torch.cuda.synchronize()
    st, detail = mk.mk_poll_error(out["workspace"])
    assert st == mk.MK_OK, (mk.mk_status_str(st), detail)
    return out


# Rows per expert: each side of the 32 / 64 / 128 / 256-row tile heights, and
# multi-tile experts whose last tile lands on each height.
BOUNDARY_COUNTS = [1, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257, 288, 320, 384, 511, 512, 513, 0]


def _ids_for_counts(counts, seed):
    """k = 1 ids giving exactly `counts` tokens per expert, in a seeded token order."""
    ids = np.concatenate([np.full(c, e, dtype=np.int32) for e, c in enumerate(counts)])
    rng = np.random.default_rng(seed)
    rng.shuffle(ids)
    return ids.reshape(-1, 1)


@pytest.mark.parametrize("fused", [True, False])
def test_tile_height_boundaries_bit_exact(fused):
    counts = BOUNDARY_COUNTS
    E = len(counts)
    T = int(sum(counts))
    wl = W.scaled(W.WORKLOADS["tiny"], T=T, d=256, E=E, k=1, E_local=E, N=256)
    inp = W.make_inputs(wl, 11, with_experts=False)
    inp["w_experts"] = torch.stack([torch.eye(256) * 2.0 ** -(e % 8) for e in range(E)]).to(torch.bfloat16)
    ids = _ids_for_counts(counts, 11)
    dev = to_dev(inp)
    tune = None if fused else {"n_mover_wg": -1}
    out = mk.mk_dispatch_gemm(dev["x"], dev["w_experts"], 1, topk_ids_in=torch.from_numpy(ids).cuda(), E=E,
                              tune=tune)
    torch.cuda.synchronize()
    assert mk.mk_poll_error(out["workspace"])[0] == mk.MK_OK
    count, offsets, _, row_token = check_layout(out, ids, wl, "boundaries")
    assert count.tolist() == counts
    y = out["y_perm"][:T].float().cpu()
    for e in range(E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        want = inp["x"][torch.from_numpy(row_token[a:b].astype(np.int64))].float() * 2.0 ** -(e % 8)
        assert torch.equal(y[a:b], want), f"expert {e} ({counts[e]} rows)"


def test_tile_height_boundaries_random_experts():
    counts = BOUNDARY_COUNTS
    E = len(counts)
    T = int(sum(counts))
    wl = W.scaled(W.WORKLOADS["tiny"], T=T, d=384, E=E, k=1, E_local=E, N=264)
    inp = W.make_inputs(wl, 12)
    ids = _ids_for_counts(counts, 12)
    dev = to_dev(inp)
    out = mk.mk_dispatch_gemm(dev["x"], dev["w_experts"], 1, topk_ids_in=torch.from_numpy(ids).cuda(), E=E)
    torch.cuda.synchronize()
    assert mk.mk_poll_error(out["workspace"])[0] == mk.MK_OK
    _, offsets, _, row_token = check_layout(out, ids, wl, "boundaries, random W")
    rows = np.arange(int(offsets[-1]), dtype=np.int32)
    y_ref = oracle.expert_rows(inp["x"], inp["w_experts"], offsets, row_token, rows)
    assert_y_close(out["y_perm"][:T].float().cpu().numpy(), y_ref, "boundaries, random W")


@pytest.mark.parametrize("d", [128, 384, 640])
def test_k_depths(d):
    wl = W.scaled(W.WORKLOADS["tiny"], T=300, d=d, N=520)
    inp = W.make_inputs(wl, 13)
    full_check(inp, _run(inp, to_dev(inp)), what=f"d={d}")


@pytest.mark.parametrize("E,E_local,e_begin,k,T", [(65, 65, 0, 1, 37), (100, 40, 30, 8, 130), (300, 16, 284, 5, 200),
                                                  (1000, 24, 500, 8, 70), (65, 65, 0, 2, 1500), (40, 40, 0, 3, 2100)])
def test_wide_expert_counts(E, E_local, e_begin, k, T):
    """Routing with E past one wave, groups of experts that end past E (router tasks of one, two or four
    groups of 8 experts, by the task count), local ranges inside E; against the oracle, fused and staged."""
    wl = W.scaled(W.WORKLOADS["decode"], T=T, d=512, E=E, k=k, E_local=E_local, e_begin=e_begin, N=256)
    inp = W.make_inputs(wl, 14)
    out = _run(inp, to_dev(inp))
    full_check(inp, out, what=f"E={E}")
    staged = _run(inp, to_dev(inp), tune={"n_mover_wg": -1})
    full_check(inp, staged, what=f"E={E} staged")


def test_largest_k():
    wl = W.scaled(W.WORKLOADS["tiny"], T=70, d=256, E=64, k=32, E_local=64, N=128)
    inp = W.make_inputs(wl, 15)
    r = full_check(inp, _run(inp, to_dev(inp)), what="k=32")
    assert r["R"] == 70 * 32


@pytest.mark.parametrize("T", [8192, 8256, 16384, 16448])
def test_layout_capacity_boundaries(T):
    """The fused kernel's layout at its LDS capacities (64 local experts, 64-token blocks): 8192 block bases,
    the most the GEMM keeps in LDS (no third barrier); 8256, one block more (row_token after a third barrier);
    16384, the most the scan holds; 16448, past it (the staged path takes over).  Every row against the oracle."""
    wl = W.scaled(W.WORKLOADS["tiny"], T=T, d=128, E=64, k=2, E_local=64, N=64)
    inp = W.make_inputs(wl, 16)
    r = full_check(inp, _run(inp, to_dev(inp)), what=f"T={T}")
    assert r["R"] == 2 * T
