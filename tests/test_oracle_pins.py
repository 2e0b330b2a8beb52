"""Pins the CPU oracle to facts that do not come from the oracle itself.

Every oracle step is checked against something independent of its code:
hand-worked fixtures (tests/golden/), brute force over subsets or sorted
pairs, closed forms, exact sums (math.fsum) within a rounding-error bound, and
library fp64 matmul.  Each test names the oracle step it pins; the choices are
made so that a dropped term, a wrong sign or index, or a transposed operand in
the oracle fails at least one of them.
"""
import collections
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as W


def _bf16_bits(a) -> np.ndarray:
    t = torch.as_tensor(np.asarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _beats(la, a, lb, b):
    return la > lb or (la == lb and a < b)


# ---------------------------------------------------------------- step 1: logits

def test_router_order_golden(golden_dir):
    """Fixed fp32 order: hand-worked cases where other orders give other bits."""
    with open(os.path.join(golden_dir, "router_order.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        x = np.array([[float.fromhex(v) for v in c["x"]]], dtype=np.float32)
        wr = np.array([[float.fromhex(v)] for v in c["wr"]], dtype=np.float32)
        bias = None if c["bias"] is None else np.array([float.fromhex(c["bias"])], dtype=np.float32)
        xb = _bf16_bits(x)
        assert np.array_equal(torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).float().numpy(), x), \
            "fixture x must be bf16-exact"
        got = oracle.logits(xb, wr, bias)[0, 0]
        assert got == np.float32(float.fromhex(c["expect"])), (c["name"], float(got).hex())


@pytest.mark.parametrize("T,d,E", [(16, 64, 8), (8, 512, 16), (4, 7168, 5)])
def test_logits_within_error_bound_of_exact_sum(T, d, E):
    """|l - exact| <= gamma_(d/8+8) * sum|x_i w_i| (+ one rounding of the bias add)."""
    rng = np.random.default_rng(7)
    x = rng.standard_normal((T, d)).astype(np.float32)
    xb = _bf16_bits(x)
    xf = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).double().numpy()
    wr = (rng.standard_normal((d, E)) / math.sqrt(d)).astype(np.float32)
    bias = rng.standard_normal(E).astype(np.float32)
    got = oracle.logits(xb, wr, bias)
    u = 2.0 ** -24
    n = d // 8 + 8
    gamma = n * u / (1 - n * u)
    for t in range(T):
        for e in range(E):
            prods = [xf[t, i] * float(wr[i, e]) for i in range(d)]   # exact in fp64
            exact = math.fsum(prods + [float(bias[e])])
            bound = gamma * (math.fsum(abs(p) for p in prods) + abs(float(bias[e]))) + u * abs(exact)
            assert abs(float(got[t, e]) - exact) <= bound, (t, e, float(got[t, e]), exact, bound)


# ---------------------------------------------------------------- step 2: top-k

def _topk_bruteforce(l, k):
    E = len(l)
    winners = []
    for S in itertools.combinations(range(E), k):
        rest = [b for b in range(E) if b not in S]
        if all(_beats(l[a], a, l[b], b) for a in S for b in rest):
            winners.append(S)
    assert len(winners) == 1
    S = winners[0]
    # rank of a member = number of members that beat it
    return sorted(S, key=lambda a: sum(_beats(l[b], b, l[a], a) for b in S))


@pytest.mark.parametrize("E,k", [(7, 3), (6, 1), (5, 5), (8, 4)])
def test_topk_matches_subset_bruteforce(E, k):
    rng = np.random.default_rng(E * 10 + k)
    T = 60
    # small integer logits -> many exact ties; a few signed zeros mixed in
    lg = rng.integers(-2, 3, size=(T, E)).astype(np.float32)
    lg[rng.random((T, E)) < 0.1] = -0.0
    ids, _ = oracle.topk(lg, k)
    for t in range(T):
        assert list(ids[t]) == _topk_bruteforce([float(v) for v in lg[t]], k), (t, lg[t])


def test_topk_signed_zero_is_a_tie():
    lg = np.array([[-0.0, 0.0, -1.0], [0.0, -0.0, -1.0]], dtype=np.float32)
    ids, _ = oracle.topk(lg, 1)
    assert ids[:, 0].tolist() == [0, 0]


def test_duplicated_router_columns_pick_lower_id_first():
    wl = W.scaled(W.WORKLOADS["tiny"], T=128)
    x = W.make_x(wl, 3)
    wr = W.make_w_router(wl, 3).numpy().copy()
    wr[:, 5] = wr[:, 2]
    _, ids, w = oracle.route(x, wr, wl.k)
    seen = 0
    for t in range(wl.T):
        row = list(ids[t])
        if 5 in row:
            assert 2 in row and row.index(2) < row.index(5)
            seen += 1
        if row[0] == 2:   # the twin of the best expert ties with it and is ranked right after it
            assert row[1] == 5
    assert seen > 0, "no token chose the duplicated column: the case does not exercise the tie"


def test_huge_bias_expert_is_rank_zero():
    wl = W.scaled(W.WORKLOADS["tiny"], T=64)
    x = W.make_x(wl, 1)
    wr = W.make_w_router(wl, 1).numpy()
    bias = np.zeros(wl.E, dtype=np.float32)
    bias[6] = 1e4
    _, ids, w = oracle.route(x, wr, wl.k, bias)
    assert (ids[:, 0] == 6).all()
    assert np.allclose(w[:, 0], 1.0)


# ---------------------------------------------------------------- step 3: gate

def test_gate_uniform_when_x_is_zero():
    T, d, E, k = 9, 64, 6, 3
    x = np.zeros((T, d), dtype=np.uint16)
    wr = np.random.default_rng(0).standard_normal((d, E)).astype(np.float32)
    lg, ids, w = oracle.route(x, wr, k)
    assert (lg == 0).all()
    assert (ids == np.arange(k)).all()
    assert np.allclose(w, 1.0 / E, rtol=0, atol=1e-15)


def test_gate_two_experts_is_a_sigmoid():
    a = np.array([[0.5, -1.25], [3.0, 3.0], [-2.0, 1.0]], dtype=np.float32)
    ids, w = oracle.topk(a, 2)
    for t in range(3):
        hi, lo = (0, 1) if _beats(a[t, 0], 0, a[t, 1], 1) else (1, 0)
        delta = float(a[t, hi]) - float(a[t, lo])
        assert ids[t].tolist() == [hi, lo]
        assert abs(w[t, 0] - 1.0 / (1.0 + math.exp(-delta))) < 1e-15
        assert abs(w[t, 1] - 1.0 / (1.0 + math.exp(delta))) < 1e-15


def test_gate_rational_bias():
    """x = 0, bias[e] = fp32(ln(e+1)): gate of expert e is (e+1)/sum(1..E) up to the fp32 rounding of ln."""
    T, d, E, k = 3, 16, 5, 5
    x = np.zeros((T, d), dtype=np.uint16)
    wr = np.ones((d, E), dtype=np.float32)
    bias = np.log(np.arange(1, E + 1, dtype=np.float64)).astype(np.float32)
    _, ids, w = oracle.route(x, wr, k, bias)
    assert ids[0].tolist() == [4, 3, 2, 1, 0]
    for j, e in enumerate(ids[0]):
        assert abs(w[0, j] - (e + 1) / (E * (E + 1) / 2)) < 1e-6


def test_gate_invariants_random():
    wl = W.scaled(W.WORKLOADS["tiny"], T=200, E=12, k=12)
    x = W.make_x(wl, 2)
    wr = W.make_w_router(wl, 2).numpy()
    _, ids, w = oracle.route(x, wr, wl.k)
    assert np.allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-12)   # k == E: full softmax
    assert (np.diff(w, axis=1) <= 0).all()                       # rank order


# ---------------------------------------------------------------- steps 4-6: layout

def _layout_bruteforce(ids, e_begin, E_local):
    T, k = ids.shape
    pairs = sorted((int(ids[t, j]) - e_begin, t, j) for t in range(T) for j in range(k)
                   if 0 <= ids[t, j] - e_begin < E_local)
    cnt = collections.Counter(p[0] for p in pairs)
    count = np.array([cnt.get(e, 0) for e in range(E_local)], dtype=np.int32)
    offsets = np.concatenate([[0], np.cumsum(count)]).astype(np.int32)
    slot_of = -np.ones((T, k), dtype=np.int32)
    row_token = np.zeros(len(pairs), dtype=np.int32)
    for s, (e, t, j) in enumerate(pairs):
        slot_of[t, j] = s
        row_token[s] = t
    return count, offsets, slot_of, row_token


def _distinct_ids(rng, T, E, k):
    return np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)


@pytest.mark.parametrize("T,E,k,e_begin,E_local", [
    (50, 8, 2, 0, 8), (77, 64, 6, 0, 64), (40, 256, 8, 0, 32), (40, 256, 8, 224, 32), (0, 8, 2, 0, 8),
    (33, 5, 5, 0, 5)])
def test_layout_matches_sort_bruteforce(T, E, k, e_begin, E_local):
    rng = np.random.default_rng(T + E + k + e_begin)
    ids = _distinct_ids(rng, T, E, k) if T else np.zeros((0, k), dtype=np.int32)
    count, offsets, slot_of, row_token = oracle.layout(ids, e_begin, E_local)
    bc, bo, bs, br = _layout_bruteforce(ids, e_begin, E_local)
    assert np.array_equal(count, bc)
    assert np.array_equal(offsets, bo)
    assert np.array_equal(slot_of, bs)
    assert np.array_equal(row_token, br)
    R = int(offsets[-1])
    local = slot_of[slot_of >= 0]
    assert sorted(local.tolist()) == list(range(R))            # bijection onto [0, R)
    for e in range(E_local):                                    # ascending tokens per expert
        seg = row_token[offsets[e]:offsets[e + 1]]
        assert (np.diff(seg) > 0).all()
    if e_begin == 0 and E_local == E:
        assert R == T * k


def test_layout_x_zero_closed_form():
    T, d, E, k = 37, 32, 6, 4
    x = np.zeros((T, d), dtype=np.uint16)
    wr = np.random.default_rng(1).standard_normal((d, E)).astype(np.float32)
    _, ids, _ = oracle.route(x, wr, k)
    count, offsets, slot_of, row_token = oracle.layout(ids, 0, E)
    assert slot_of.tolist() == [[j * T + t for j in range(k)] for t in range(T)]
    assert count.tolist() == [T] * k + [0] * (E - k)


# ---------------------------------------------------------------- step 7: GEMM

def test_gemm_single_expert_equals_library_matmul():
    wl = W.scaled(W.WORKLOADS["tiny"], T=48, d=256, E=1, k=1, E_local=1, N=96)
    inp = W.make_inputs(wl, 4)
    res = oracle.run(inp["x"], inp["w_router"].numpy(), inp["w_experts"], 1)
    assert res["row_token"].tolist() == list(range(wl.T))
    ref = torch.matmul(inp["x"].double(), inp["w_experts"][0].double().t()).numpy()
    assert np.allclose(res["y"], ref, rtol=1e-12, atol=1e-12)


def test_gemm_tagged_identity_is_exact():
    wl = W.scaled(W.WORKLOADS["tiny"], T=40, d=64, E=10, k=3, E_local=10, N=64)
    x = W.make_x(wl, 5)
    wr = W.make_w_router(wl, 5).numpy()
    we = torch.stack([torch.eye(64) * 2.0 ** -(e % 8) for e in range(wl.E_local)]).to(torch.bfloat16)
    res = oracle.run(x, wr, we, wl.k)
    xf = x.double().numpy()
    for r in range(int(res["offsets"][-1])):
        e = int(np.searchsorted(res["offsets"], r, side="right") - 1)
        assert np.array_equal(res["y"][r], xf[res["row_token"][r]] * 2.0 ** -(e % 8))


def test_worked_example(golden_dir):
    with open(os.path.join(golden_dir, "worked_example.json")) as f:
        g = json.load(f)
    ex = g["expect"]
    xb = _bf16_bits(g["x"])
    wr = np.array(g["w_router"], dtype=np.float32)
    we = torch.tensor(g["w_experts"], dtype=torch.float32).to(torch.bfloat16)
    res = oracle.run(xb, wr, we, g["k"], g["e_begin"])
    assert res["logits"].tolist() == ex["logits"]
    assert res["ids"].tolist() == ex["ids"]
    for t, row in enumerate(ex["gate_exponents"]["w"]):
        for j, c in enumerate(row):
            want = math.exp(c["num"]) / math.fsum(math.exp(v) for v in c["den"])
            assert abs(res["w"][t, j] - want) < 1e-15
    assert res["count"].tolist() == ex["count"]
    assert res["offsets"].tolist() == ex["offsets"]
    assert res["slot_of"].tolist() == ex["slot_of"]
    assert res["row_token"].tolist() == ex["row_token"]
    assert res["y"].tolist() == ex["y"]


# ---------------------------------------------------------------- workload statistics

def test_skewed_workload_leaves_experts_idle():
    """The skewed workload must be heavily imbalanced with at least 4 experts receiving no token."""
    wl = W.WORKLOADS["skewed"]
    for seed in (0, 1):
        inp = W.make_inputs(wl, seed, with_experts=False)
        _, ids, _ = oracle.route(inp["x"], inp["w_router"].numpy(), wl.k, inp["bias"].numpy())
        count, *_ = oracle.layout(ids, 0, wl.E_local)
        assert (count == 0).sum() >= 4
        assert count.max() > 50 * np.median(count[count > 0])


def test_mixtral_workload_is_near_uniform():
    wl = W.WORKLOADS["mixtral"]
    inp = W.make_inputs(wl, 0, with_experts=False)
    _, ids, _ = oracle.route(inp["x"], inp["w_router"].numpy(), wl.k)
    count, *_ = oracle.layout(ids, 0, wl.E_local)
    mean = wl.T * wl.k / wl.E
    assert (np.abs(count - mean) < 0.1 * mean).all()


# ---------------------------------------------------------------- step 8 (next): combine

def test_combine_golden(golden_dir):
    """Hand-worked dyadic example (exact): weighted sum over the local choices only."""
    with open(os.path.join(golden_dir, "combine_example.json")) as f:
        g = json.load(f)
    y = np.array(g["y_rows"], dtype=np.float64)
    out = oracle.combine(y, np.arange(len(y)), np.array(g["slot_of"]), np.array(g["w"]))
    assert out.tolist() == g["expect"]


def test_combine_gate_normalisation():
    """k = E, every expert local, unit expert outputs: each token's output is the sum of its softmax gate
    over all experts, which is 1 (ties combine to the gate of step 3, computed independently)."""
    wl = W.scaled(W.WORKLOADS["tiny"], T=40, d=128, E=6, k=6, E_local=6)
    inp = W.make_inputs(wl, 7, with_experts=False)
    _, ids, w = oracle.route(inp["x"], inp["w_router"].numpy(), wl.k)
    _, offsets, slot_of, _ = oracle.layout(ids, 0, wl.E_local)
    R = int(offsets[-1])
    out = oracle.combine(np.ones((R, 3)), np.arange(R), slot_of, w)
    assert np.abs(out - 1.0).max() < 1e-12


def test_combine_choice_order_and_locality():
    """Permuting a token's choices (slots with their weights) leaves the output unchanged, and a
    non-local choice (slot -1) equals the same choice with weight 0 (dyadic data: every sum exact)."""
    rng = np.random.default_rng(11)
    T, k, N, R = 30, 5, 7, 60
    y = rng.integers(-64, 64, size=(R, N)) / 8.0
    slot_of = np.stack([rng.permutation(R)[:k] for _ in range(T)]).astype(np.int32)
    w = rng.integers(0, 32, size=(T, k)) / 64.0
    base = oracle.combine(y, np.arange(R), slot_of, w)
    perm = np.stack([rng.permutation(k) for _ in range(T)])
    rows = np.arange(T)[:, None]
    assert np.array_equal(oracle.combine(y, np.arange(R), slot_of[rows, perm], w[rows, perm]), base)
    drop = rng.random((T, k)) < 0.3
    s2 = np.where(drop, -1, slot_of).astype(np.int32)
    assert np.array_equal(oracle.combine(y, np.arange(R), s2, w), oracle.combine(y, np.arange(R), slot_of,
                                                                                  np.where(drop, 0.0, w)))
    # k = 1, weight 1: the combine is the inverse permutation of the layout (the token's own row)
    one = oracle.combine(y, np.arange(R), slot_of[:, :1], np.ones((T, 1)))
    assert np.array_equal(one, y[slot_of[:, 0]])


# ---------------------------------------------------------------- next row: expert FFN (SwiGLU, down-projection)

def test_swiglu_closed_forms():
    """silu(g) = g * sigmoid(g): with u = 1, h(g) - h(-g) = g and h(g) + h(-g) = g * tanh(g / 2) (library
    tanh), h(0) = 0; a row [g | u] pairs column f of g with column f of u."""
    g = np.array([0.0, 0.5, 1.0, 2.0, 3.0, -1.5, 8.0], dtype=np.float32)
    gb = torch.tensor(g).bfloat16().float().numpy().astype(np.float64)   # exact in bf16
    F = g.size
    rows = torch.tensor(np.stack([np.concatenate([g, np.ones(F)]), np.concatenate([-g, np.ones(F)])]),
                        dtype=torch.float32).bfloat16()
    h = oracle.swiglu(rows)
    assert np.allclose(h[0] - h[1], gb, rtol=0, atol=1e-13)
    assert np.allclose(h[0] + h[1], gb * np.tanh(gb / 2), rtol=1e-13, atol=1e-14)
    assert h[0][0] == 0.0
    # split: u_f scales only column f
    u = np.array([2.0, -1.0, 0.25, 4.0, 1.0, 0.5, -3.0], dtype=np.float32)
    h2 = oracle.swiglu(torch.tensor(np.concatenate([g, u])[None, :]).bfloat16())
    assert np.allclose(h2[0], h[0] * u.astype(np.float64), rtol=1e-14, atol=0)


def test_grouped_rows_matches_library_matmul():
    """Each row of the layout times its own expert's W^T: fp64 library matmul per expert range."""
    rng = np.random.default_rng(5)
    E_local, K, N = 4, 32, 12
    counts = np.array([3, 0, 5, 2])
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    R = int(offsets[-1])
    a = torch.tensor(rng.standard_normal((R, K)), dtype=torch.float32).bfloat16()
    w = torch.tensor(rng.standard_normal((E_local, N, K)), dtype=torch.float32).bfloat16()
    z = oracle.grouped_rows(a, w, offsets, np.arange(R))
    af, wf = a.double().numpy(), w.double().numpy()
    for e in range(E_local):
        lo, hi = offsets[e], offsets[e + 1]
        if hi > lo:
            assert np.allclose(z[lo:hi], af[lo:hi] @ wf[e].T, rtol=1e-12, atol=1e-12)
    sub = np.array([9, 0, 4])
    assert np.array_equal(oracle.grouped_rows(a, w, offsets, sub), z[sub])
