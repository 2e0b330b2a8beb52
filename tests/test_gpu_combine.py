"""Combine (mk_combine, the step after the path) against the oracle's combine.

The GPU input is the GPU path's own output (y_perm, slot_of, topk_w of a
mk_dispatch_gemm call); the reference is computed by the oracle alone from
the same seeded inputs (its routing, layout, fp64 expert rows and fp64
gates).  Tolerance per element, derived from the arithmetic: each expert
output reaches the combine rounded to bf16 (relative error <= 2^-8), each
gate differs from the fp64 one by <= 1e-4 relative, fp32 accumulation adds
little, and the result is rounded to bf16 once (<= 2^-8 |out|):
    |out - ref| <= (2^-8 + 1e-4) * sum_j |w_j y_j| + 2^-8 |ref| + 1e-6.
Routing ids and slot_of are bit-exact (checked on the way).
"""
import numpy as np
import pytest
import torch

import moe_dispatch_expert_amd as mk
import oracle
import workloads as W
from gpu_cases import oracle_route, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _name(request):
    say(f"\n[gpu case] {request.node.nodeid}")
    yield
    torch.cuda.synchronize()


def _dispatch(wl, seed):
    inp = W.make_inputs(wl, seed)
    dev = to_dev(inp)
    out = mk.mk_dispatch_gemm(dev["x"], dev["w_experts"], wl.k, w_router=dev["w_router"], bias=dev["bias"],
                              E=wl.E, e_begin=wl.e_begin)
    torch.cuda.synchronize()
    return inp, out


def _reference(inp, tokens):
    """Oracle combine of the given tokens: (ref [n, N], bound [n, N] of sum_j |w_j y_j|, slot_of, ids)."""
    wl = inp["wl"]
    _, ids, w = oracle_route(inp)
    _, offsets, slot_of, row_token = oracle.layout(ids, wl.e_begin, wl.E_local)
    s = slot_of[tokens]
    need = np.unique(s[s >= 0]).astype(np.int32)
    y = oracle.expert_rows(inp["x"], inp["w_experts"], offsets, row_token, need)
    ref = oracle.combine(y, need, s, w[tokens])
    mag = oracle.combine(np.abs(y), need, s, np.abs(w[tokens]))
    return ref, mag, slot_of, ids


def _check(inp, out, comb, tokens, what):
    ref, mag, slot_of, ids = _reference(inp, tokens)
    assert np.array_equal(out["topk_ids"].cpu().numpy(), ids), what
    assert np.array_equal(out["slot_of"].cpu().numpy(), slot_of), what
    got = comb[torch.from_numpy(np.asarray(tokens, dtype=np.int64)).cuda()].float().cpu().numpy()
    tol = (2.0 ** -8 + 1e-4) * mag + 2.0 ** -8 * np.abs(ref) + 1e-6
    bad = np.abs(got - ref) > tol
    assert not bad.any(), (f"{what}: {int(bad.sum())} of {bad.size} out of tolerance; first at "
                           f"{tuple(np.argwhere(bad)[0])}")


@pytest.mark.parametrize("seed", [0, 1])
def test_combine_tiny_every_token(seed):
    wl = W.WORKLOADS["tiny"]
    inp, out = _dispatch(wl, seed)
    comb = mk.mk_combine(out["y_perm"], out["slot_of"], out["topk_w"], rows=int(out["expert_offsets"][-1]))
    _check(inp, out, comb, np.arange(wl.T), f"tiny seed {seed}")


def test_combine_mixtral_sampled_tokens():
    wl = W.WORKLOADS["mixtral"]
    inp, out = _dispatch(wl, 0)
    comb = mk.mk_combine(out["y_perm"], out["slot_of"], out["topk_w"], rows=int(out["expert_offsets"][-1]))
    tokens = np.array([0, 1, 777, 2048, 3000, wl.T - 1])
    _check(inp, out, comb, tokens, "mixtral")


def test_combine_local_choices_only():
    """A rank's share of a wide expert-parallel layer (experts 16..31 of 64, top-6): most choices are not
    local (slot -1); tokens without a local choice get an exact zero row."""
    wl = W.scaled(W.WORKLOADS["decode"], T=200, d=512, E=64, k=6, E_local=16, e_begin=16, N=520)
    inp, out = _dispatch(wl, 5)
    comb = mk.mk_combine(out["y_perm"], out["slot_of"], out["topk_w"], rows=int(out["expert_offsets"][-1]))
    _check(inp, out, comb, np.arange(wl.T), "local only")
    none_local = (out["slot_of"] < 0).all(dim=1)
    assert none_local.any()
    assert (comb[none_local] == 0).all()


def test_combine_shapes_and_empty():
    """k = 1 (the inverse permutation of the layout), a column count that is not a multiple of 512, and
    T = 0 (no-op)."""
    wl = W.scaled(W.WORKLOADS["tiny"], T=300, d=256, E=5, k=1, E_local=5, N=520)
    inp, out = _dispatch(wl, 2)
    comb = mk.mk_combine(out["y_perm"], out["slot_of"], out["topk_w"], rows=int(out["expert_offsets"][-1]))
    _check(inp, out, comb, np.arange(wl.T), "k=1")
    empty = torch.empty(0, 520, dtype=torch.bfloat16, device="cuda")
    mk.mk_combine(out["y_perm"], torch.empty(0, 1, dtype=torch.int32, device="cuda"),
                  torch.empty(0, 1, dtype=torch.float32, device="cuda"), out=empty)
