"""HIP path (through the C ABI) against the CPU oracle on the same seeded inputs.

Bit-exact: top-k ids, expert offsets, slot_of, row_token.  Tolerance:
y_perm within max(1e-2 |ref|, 1e-2) per element, gate weights within
max(1e-4 w, 1e-6).  Sizes: every row at small sizes (several tiles plus a
ragged tail), sampled rows at the full workload sizes in the launch
configuration the benchmark times.
"""
import json
import os

import numpy as np
import pytest
import torch

import moe_dispatch_expert_amd as mk
import oracle
import workloads as W
from gpu_cases import (assert_w_close, assert_y_close, check_layout, full_check, oracle_route, sample_rows, say,
                       to_dev, Y_FLOOR, Y_REL)

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


# ---------------------------------------------------------------- worked example

def test_worked_example(golden_dir):
    """The hand-worked fixture, zero-padded to d=128 and N=8 (the library needs d % 128 == 0, N % 8 == 0)."""
    with open(os.path.join(golden_dir, "worked_example.json")) as f:
        g = json.load(f)
    d, N = 128, 8
    x = torch.zeros(g["T"], d)
    x[:, :g["d"]] = torch.tensor(g["x"], dtype=torch.float32)
    wr = torch.zeros(d, g["E"])
    wr[:g["d"]] = torch.tensor(g["w_router"], dtype=torch.float32)
    we = torch.zeros(g["E_local"], N, d)
    we[:, :g["N"], :g["d"]] = torch.tensor(g["w_experts"], dtype=torch.float32)
    out = mk.mk_dispatch_gemm(x.to(torch.bfloat16).cuda(), we.to(torch.bfloat16).cuda(), g["k"],
                              w_router=wr.cuda(), E=g["E"])
    torch.cuda.synchronize()
    ex = g["expect"]
    assert out["topk_ids"].cpu().tolist() == ex["ids"]
    assert out["expert_offsets"].cpu().tolist() == ex["offsets"]
    assert out["slot_of"].cpu().tolist() == ex["slot_of"]
    assert out["row_token"][:8].cpu().tolist() == ex["row_token"]
    assert out["y_perm"][:8, :g["N"]].float().cpu().tolist() == ex["y"]
    assert (out["y_perm"][:8, g["N"]:].float() == 0).all()


# ---------------------------------------------------------------- router alone

@pytest.mark.parametrize("name", ["tiny", "skewed", "decode"])
def test_route_topk_matches_oracle(name):
    wl = W.WORKLOADS[name]
    inp = W.make_inputs(wl, 0, with_experts=False)
    ids, w = mk.mk_route_topk(inp["x"].cuda(), inp["w_router"].cuda(), wl.k,
                              bias=None if inp["bias"] is None else inp["bias"].cuda())
    torch.cuda.synchronize()
    _, ref_ids, ref_w = oracle_route(inp)
    assert np.array_equal(ids.cpu().numpy(), ref_ids)
    assert_w_close(w.cpu().numpy(), ref_w, name)


@pytest.mark.parametrize("name,changes", [
    ("tiny", {}), ("mixtral", {}), ("skewed", {}), ("decode", {}),
    ("tiny", dict(T=96, d=384, E=6, k=3, E_local=6)),      # 48-step segments, E % 4 != 0
    ("tiny", dict(T=700, d=256, E=10, k=3, E_local=10)),   # 32-step segments, a partial expert group
    ("tiny", dict(T=33, d=128, E=1, k=1, E_local=1)),       # one expert, 16-step segments, a 1-token block
])
def test_router_logits_bit_exact(name, changes):
    """The router's per-segment partial sums (left in the mk_route_topk workspace, [8, T, E] fp32),
    added in the fixed order, equal the oracle's fp32 logits bit for bit: every chain is the same
    sequence of fused multiply-adds."""
    wl = W.scaled(W.WORKLOADS[name], **changes) if changes else W.WORKLOADS[name]
    inp = W.make_inputs(wl, 3, with_experts=False)
    ws = torch.zeros(mk.mk_route_topk_workspace_bytes(wl.T, wl.E), dtype=torch.uint8, device="cuda")
    mk.mk_route_topk(inp["x"].cuda(), inp["w_router"].cuda(), wl.k, workspace=ws)
    torch.cuda.synchronize()
    part = ws[:8 * wl.T * wl.E * 4].view(torch.float32).reshape(8, wl.T, wl.E).cpu().numpy()
    lg = part[0].copy()
    for s in range(1, 8):
        lg = (lg + part[s]).astype(np.float32)
    ref = oracle.logits(inp["x"], inp["w_router"])
    bad = lg.view(np.uint32) != ref.view(np.uint32)
    assert not bad.any(), f"{int(bad.sum())} of {bad.size} logits differ; first at {tuple(np.argwhere(bad)[0])}"


@pytest.mark.parametrize("name,changes", [
    ("tiny", {}), ("skewed", {}), ("decode", {}),
    ("tiny", dict(T=96, d=384, E=6, k=3, E_local=6)),
    ("tiny", dict(T=33, d=128, E=1, k=1, E_local=1)),
])
def test_router_final_logits_bit_exact(name, changes):
    """The logits the selection ranks (mk_route_topk's optional logits output: the eight partial sums added
    left to right, then the bias) equal the oracle's fp32 logits bit for bit, bias included (the skewed
    workload carries the Zipf bias)."""
    wl = W.scaled(W.WORKLOADS[name], **changes) if changes else W.WORKLOADS[name]
    inp = W.make_inputs(wl, 5, with_experts=False)
    bias = None if inp["bias"] is None else inp["bias"]
    lg = torch.full((wl.T, wl.E), float("nan"), dtype=torch.float32, device="cuda")
    ids, _ = mk.mk_route_topk(inp["x"].cuda(), inp["w_router"].cuda(), wl.k,
                              bias=None if bias is None else bias.cuda(), logits=lg)
    torch.cuda.synchronize()
    ref_lg, ref_ids, _ = oracle_route(inp)
    got = lg.cpu().numpy()
    bad = got.view(np.uint32) != ref_lg.astype(np.float32).view(np.uint32)
    assert not bad.any(), f"{int(bad.sum())} of {bad.size} logits differ; first at {tuple(np.argwhere(bad)[0])}"
    assert np.array_equal(ids.cpu().numpy(), ref_ids)


# ---------------------------------------------------------------- the five workloads

@pytest.mark.parametrize("seed", [0, 1, 2])
def test_tiny_every_row(seed):
    inp = W.make_inputs(W.WORKLOADS["tiny"], seed)
    out = _run(inp, to_dev(inp))
    r = full_check(inp, out, what=f"tiny seed {seed}")
    assert r["R"] == 512


@pytest.mark.parametrize("name,n_random", [("mixtral", 24), ("skewed", 48), ("decode", 0)])
def test_workload_sampled_rows(name, n_random):
    """Full-size workloads: routing and layout bit-exact and sampled rows (decode: every row) against the oracle;
    then every row against an fp32 GEMM of the same bf16 operands on the GPU (the rows' tokens are the ones whose
    layout just matched the oracle), to the same bound."""
    wl = W.WORKLOADS[name]
    inp = W.make_inputs(wl, 0)
    dev = to_dev(inp)
    out = _run(inp, dev)
    _, ids, _ = oracle_route(inp)
    _, offsets, _, _ = oracle.layout(ids, wl.e_begin, wl.E_local)
    rows = None if name == "decode" else sample_rows(offsets, n_random)
    r = full_check(inp, out, rows=rows, what=name)
    if name == "skewed":
        assert (r["count"] == 0).sum() >= 4
    if name != "decode":
        _every_row_vs_fp32_gemm(out, dev["x"], dev["w_experts"], offsets, wl, name)


def _every_row_vs_fp32_gemm(out, x, w_experts, offsets, wl, what):
    """Every routed row against an fp32 GEMM of the same bf16 operands on the GPU, to the oracle's bound (the
    rows' tokens are row_token's, whose layout the caller has matched with the oracle)."""
    torch.backends.cuda.matmul.allow_tf32 = False
    rt = out["row_token"].long()
    n_bad = 0
    for e in range(wl.E_local):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if b == a:
            continue
        ref = torch.matmul(x[rt[a:b]].float(), w_experts[e].float().t().contiguous())
        got = out["y_perm"][a:b].float()
        tol = torch.clamp(Y_REL * ref.abs(), min=Y_FLOOR)
        n_bad += int(((got - ref).abs() > tol).sum())
    say(f"{what}: every one of {int(offsets[-1])} rows x {wl.N} columns against the fp32 GEMM, {n_bad} out of bound")
    assert n_bad == 0


def test_wide_ep_share_with_source_routing():
    """One GPU's share: 8 source shards, routing done per shard by the sources (mk_route_topk),
    ids handed to the dispatch call; local experts 0..31 of 256.  Sampled rows against the oracle, every row
    against an fp32 GEMM."""
    wl = W.WORKLOADS["wide_ep"]
    inp = W.make_inputs(wl, 0)
    dev = to_dev(inp)
    ids_parts = []
    for s in range(wl.S):
        ids_s, _ = mk.mk_route_topk(dev["x"][s], dev["w_router"], wl.k)
        ids_parts.append(ids_s)
    ids_in = torch.cat(ids_parts).contiguous()
    out = mk.mk_dispatch_gemm(dev["x"], dev["w_experts"], wl.k, topk_ids_in=ids_in, E=wl.E, e_begin=wl.e_begin)
    torch.cuda.synchronize()
    assert mk.mk_poll_error(out["workspace"])[0] == mk.MK_OK
    _, ref_ids, _ = oracle_route(inp)
    assert np.array_equal(ids_in.cpu().numpy(), ref_ids)
    assert np.array_equal(out["topk_ids"].cpu().numpy(), ref_ids)
    _, offsets, _, row_token = check_layout(out, ref_ids, wl, "wide_ep")
    rows = sample_rows(offsets, 32)
    y_ref = oracle.expert_rows(inp["x"], inp["w_experts"], offsets, row_token, rows)
    y_gpu = out["y_perm"][torch.from_numpy(rows.astype(np.int64)).cuda()].float().cpu().numpy()
    assert_y_close(y_gpu, y_ref, "wide_ep")
    _every_row_vs_fp32_gemm(out, torch.cat(dev["x"]), dev["w_experts"], offsets, wl, "wide_ep")


@pytest.mark.parametrize("seed", [1, 2])
def test_decode_every_row_other_seeds(seed):
    """The decode-shaped share at seeds 1 and 2, every routed row against the oracle."""
    inp = W.make_inputs(W.WORKLOADS["decode"], seed)
    out = _run(inp, to_dev(inp))
    full_check(inp, out, what=f"decode seed {seed}")


_CANARY_BF16 = 0x7FC1      # a quiet-NaN bf16 pattern no GEMM row produces from finite inputs
_CANARY_I32 = -7


def _canary_outputs(wl, dev):
    r_cap = wl.T * min(wl.k, wl.E_local)
    y = torch.empty(r_cap, wl.N, dtype=torch.bfloat16, device=dev)
    y.view(torch.int16).fill_(_CANARY_BF16)
    rt = torch.full((r_cap,), _CANARY_I32, dtype=torch.int32, device=dev)
    return {"y_perm": y, "row_token": rt}


def _assert_canaries(out, R, what):
    tail = out["y_perm"][R:].view(torch.int16)
    assert bool((tail == _CANARY_BF16).all()), f"{what}: y_perm rows >= R = {R} were written"
    assert bool((out["row_token"][R:] == _CANARY_I32).all()), f"{what}: row_token entries >= R = {R} were written"


@pytest.mark.parametrize("path", ["table", "movers", "staged"])
def test_decode_rows_beyond_R_untouched(path):
    """y_perm rows >= R (and row_token entries >= R) keep what the caller left there, on the decode share
    (R = 127 of R_cap = 1024 at seed 0) in each launch configuration: the table's (rows read in place), a mover role,
    and the staged launches; the routed rows still match the oracle."""
    wl = W.WORKLOADS["decode"]
    inp = W.make_inputs(wl, 0)
    dev = to_dev(inp)
    tune = {"table": {}, "movers": {"n_mover_wg": 64}, "staged": {"n_mover_wg": mk.MK_MOVERS_STAGED}}[path]
    out = _run(inp, dev, out=_canary_outputs(wl, "cuda"), tune=tune)
    r = full_check(inp, out, what=f"decode {path}")
    assert r["R"] < wl.T * wl.k
    _assert_canaries(out, r["R"], f"decode {path}")


@pytest.mark.parametrize("path", ["table", "staged"])
def test_wide_ep_reduced_rows_beyond_R_untouched(path):
    """The same on a reduced wide-EP share (8 sources x 256 rows, local experts 16..31 of 64, top-4, ids routed
    by the sources): rows >= R of y_perm and row_token untouched, routed rows against the oracle."""
    wl = W.scaled(W.WORKLOADS["wide_ep"], T=2048, d=1024, E=64, k=4, N=512, E_local=16, e_begin=16,
                  chunk_rows=32)
    inp = W.make_inputs(wl, 7)
    dev = to_dev(inp)
    _, ref_ids, _ = oracle_route(inp)
    tune = {"table": {}, "staged": {"n_mover_wg": mk.MK_MOVERS_STAGED}}[path]
    out = mk.mk_dispatch_gemm(dev["x"], dev["w_experts"], wl.k, topk_ids_in=torch.from_numpy(ref_ids).cuda(),
                              E=wl.E, e_begin=wl.e_begin, out=_canary_outputs(wl, "cuda"), tune=tune)
    torch.cuda.synchronize()
    assert mk.mk_poll_error(out["workspace"])[0] == mk.MK_OK
    _, offsets, _, row_token = check_layout(out, ref_ids, wl, f"wide_ep reduced {path}")
    R = int(offsets[-1])
    assert R < wl.T * min(wl.k, wl.E_local)
    rows = sample_rows(offsets, 64)
    y_ref = oracle.expert_rows(inp["x"], inp["w_experts"], offsets, row_token, rows)
    assert_y_close(out["y_perm"][torch.from_numpy(rows.astype(np.int64)).cuda()].float().cpu().numpy(), y_ref,
                   f"wide_ep reduced {path}")
    _assert_canaries(out, R, f"wide_ep reduced {path}")


# ---------------------------------------------------------------- edge cases

@pytest.mark.parametrize("T", [1, 63, 65, 100, 300])
def test_ragged_token_counts(T):
    wl = W.scaled(W.WORKLOADS["tiny"], T=T)
    inp = W.make_inputs(wl, 3)
    full_check(inp, _run(inp, to_dev(inp)), what=f"T={T}")


def test_empty_input():
    wl = W.scaled(W.WORKLOADS["tiny"], T=0)
    dev = dict(x=torch.empty(0, wl.d, dtype=torch.bfloat16).cuda(), w_router=W.make_w_router(wl).cuda(),
               w_experts=W.make_w_experts(wl).cuda())
    out = mk.mk_dispatch_gemm(dev["x"], dev["w_experts"], wl.k, w_router=dev["w_router"], E=wl.E)
    torch.cuda.synchronize()
    assert out["expert_offsets"].cpu().tolist() == [0] * (wl.E_local + 1)


def test_local_range_at_the_end():
    """256 global experts, local 224..255 (the last EP rank)."""
    wl = W.scaled(W.WORKLOADS["decode"], T=200, e_begin=224, N=256)
    inp = W.make_inputs(wl, 4)
    r = full_check(inp, _run(inp, to_dev(inp)), what="e_begin=224")
    assert 0 < r["R"] < wl.T * wl.k


def test_every_expert_chosen():
    wl = W.scaled(W.WORKLOADS["tiny"], T=96, E=6, k=6, E_local=6, N=256)
    inp = W.make_inputs(wl, 5)
    r = full_check(inp, _run(inp, to_dev(inp)), what="k=E")
    assert r["count"].tolist() == [96] * 6


def test_single_expert_is_a_plain_gemm():
    wl = W.scaled(W.WORKLOADS["tiny"], T=300, d=256, E=1, k=1, E_local=1, N=520)
    inp = W.make_inputs(wl, 6)
    out = _run(inp, to_dev(inp))
    ref = torch.matmul(inp["x"].double(), inp["w_experts"][0].double().t()).numpy()
    assert out["row_token"][:300].cpu().tolist() == list(range(300))
    assert_y_close(out["y_perm"][:300].float().cpu().numpy(), ref, "E=1")


def test_zero_input_closed_form():
    wl = W.scaled(W.WORKLOADS["tiny"], T=130, E=8, k=3, N=64)
    inp = W.make_inputs(wl, 7)
    inp["x"] = torch.zeros_like(inp["x"])
    out = _run(inp, to_dev(inp))
    T = wl.T
    assert (out["topk_ids"].cpu() == torch.arange(3, dtype=torch.int32)).all()
    assert out["slot_of"].cpu().tolist() == [[j * T + t for j in range(3)] for t in range(T)]
    assert torch.allclose(out["topk_w"].cpu(), torch.full((T, 3), 1 / 8), rtol=0, atol=1e-7)
    assert (out["y_perm"][:3 * T].float() == 0).all()


def test_tagged_identity_experts_are_bit_exact():
    """N = d and W_e = 2^-(e mod 8) I: every output row is an exactly scaled copy of its token row,
    which pins the gather, the tile edges and the epilogue independently of GEMM rounding."""
    wl = W.scaled(W.WORKLOADS["tiny"], T=700, d=256, E=10, k=3, E_local=10, N=256)
    inp = W.make_inputs(wl, 8)
    inp["w_experts"] = torch.stack([torch.eye(256) * 2.0 ** -(e % 8) for e in range(10)]).to(torch.bfloat16)
    out = _run(inp, to_dev(inp))
    _, ids, _ = oracle_route(inp)
    _, offsets, _, row_token = check_layout(out, ids, wl, "tagged")
    y = out["y_perm"][:int(offsets[-1])].float().cpu()
    for e in range(10):
        a, b = int(offsets[e]), int(offsets[e + 1])
        want = inp["x"][torch.from_numpy(row_token[a:b].astype(np.int64))].float() * 2.0 ** -(e % 8)
        assert torch.equal(y[a:b], want), f"expert {e}"


def test_duplicated_router_columns():
    wl = W.scaled(W.WORKLOADS["tiny"], T=256, N=128)
    inp = W.make_inputs(wl, 9)
    inp["w_router"][:, 5] = inp["w_router"][:, 2]
    full_check(inp, _run(inp, to_dev(inp)), what="duplicated columns")


def test_repeated_calls_identical():
    wl = W.scaled(W.WORKLOADS["skewed"], T=512, N=256)
    inp = W.make_inputs(wl, 10)
    dev = to_dev(inp)
    ws = torch.zeros(mk.mk_dispatch_gemm_workspace_bytes(wl.T, wl.d, wl.E, wl.k, 0, wl.E_local, wl.N),
                     dtype=torch.uint8, device="cuda")
    outs = [_run(inp, dev, workspace=ws) for _ in range(3)]
    for o in outs[1:]:
        for key in ("y_perm", "slot_of", "expert_offsets", "topk_ids", "topk_w"):
            R = int(outs[0]["expert_offsets"][-1])
            a = outs[0][key][:R] if key == "y_perm" else outs[0][key]
            b = o[key][:R] if key == "y_perm" else o[key]
            assert torch.equal(a, b), key
    full_check(inp, outs[-1], what="repeat")


def test_bad_source_ids_reported():
    wl = W.scaled(W.WORKLOADS["tiny"], T=64, N=64)
    inp = W.make_inputs(wl, 11)
    dev = to_dev(inp)
    ids = torch.tensor([[0, 1]] * 64, dtype=torch.int32)
    ids[17] = torch.tensor([3, 99])
    out = mk.mk_dispatch_gemm(dev["x"], dev["w_experts"], wl.k, topk_ids_in=ids.cuda(), E=wl.E)
    st, detail = mk.mk_poll_error(out["workspace"])
    assert st == mk.MK_EINVAL and detail == 17


def test_workspace_reusable_after_device_error():
    """A call that fails on the device leaves its grid barrier half passed: bad source ids raise MK_EINVAL
    while the workgroups arrive at the barrier after the histogram, and they give up there.  After
    mk_poll_error, a valid call through the same workspace must not pass that barrier early on the words
    the failed call left behind; its result is checked in full against the oracle."""
    wl = W.scaled(W.WORKLOADS["tiny"], T=64, N=64)
    inp = W.make_inputs(wl, 12)
    dev = to_dev(inp)
    ws = torch.zeros(mk.mk_dispatch_gemm_workspace_bytes(wl.T, wl.d, wl.E, wl.k, 0, wl.E_local, wl.N),
                     dtype=torch.uint8, device="cuda")
    ids = torch.tensor([[0, 1]] * 64, dtype=torch.int32)
    ids[5] = torch.tensor([2, 200])
    mk.mk_dispatch_gemm(dev["x"], dev["w_experts"], wl.k, topk_ids_in=ids.cuda(), E=wl.E, workspace=ws)
    st, detail = mk.mk_poll_error(ws)
    assert st == mk.MK_EINVAL and detail == 5
    for _ in range(2):
        out = _run(inp, dev, workspace=ws)
        full_check(inp, out, what="after a failed call")
