"""The persistent fused kernel: roles, tile counters, source-chunk arrival flags.

Bit-identity across schedules (role splits, arrival delays, arrival order,
staged vs fused launch), poison mode (source rows hold NaN until the arrival
simulator copies the real rows in and releases the chunk, so any read before
the release shows up), stale-data check (different inputs through one
workspace), and a withheld arrival flag that must end in MK_ETIMEOUT through
the kernel's own bounded wait.
"""
import os

import numpy as np
import pytest
import torch

import moe_dispatch_expert_amd as mk
import oracle
import workloads as W
from gpu_cases import assert_y_close, check_layout, full_check, oracle_route, sample_rows, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _name(request):
    say(f"\n[gpu case] {request.node.nodeid}")
    yield
    torch.cuda.synchronize()


KEYS = ("y_perm", "slot_of", "expert_offsets", "topk_ids", "row_token")


def _same(a, b, keys=KEYS):
    R = int(a["expert_offsets"][-1])
    for key in keys:
        x, y = a[key], b[key]
        if key in ("y_perm", "row_token"):
            x, y = x[:R], y[:R]
        assert torch.equal(x, y), key


def _call(inp, dev, **kw):
    wl = inp["wl"]
    out = mk.mk_dispatch_gemm(dev["x"], dev["w_experts"], wl.k, w_router=dev["w_router"], bias=dev["bias"],
                              E=wl.E, e_begin=wl.e_begin, **kw)
    st, detail = mk.mk_poll_error(out["workspace"])
    assert st == mk.MK_OK, (mk.mk_status_str(st), detail)
    return out


@pytest.mark.parametrize("name", ["tiny", "skewed", "decode"])
def test_fused_equals_staged(name):
    wl = W.WORKLOADS[name]
    if name != "tiny":
        wl = W.scaled(wl, T=min(wl.T, 1024), N=512)
    inp = W.make_inputs(wl, 20)
    dev = to_dev(inp)
    fused = _call(inp, dev)
    staged = _call(inp, dev, tune={"n_mover_wg": -1})
    _same(fused, staged, KEYS + ("topk_w",))
    full_check(inp, fused, what=f"{name} fused")


@pytest.mark.parametrize("n_mover", [1, 7, 64, 256])
def test_role_split_does_not_change_results(n_mover):
    wl = W.scaled(W.WORKLOADS["mixtral"], T=1024, N=1024)
    inp = W.make_inputs(wl, 21)
    dev = to_dev(inp)
    ref = _call(inp, dev, tune={"n_mover_wg": -1})
    out = _call(inp, dev, tune={"n_mover_wg": n_mover})
    _same(ref, out)


@pytest.mark.parametrize("n_compute", [8, 32, 100, 0])
def test_grid_size_does_not_change_results(n_compute):
    """The in-place path on 8, 32 or 100 workgroups, or the table's count (0), gives the staged launches'
    outputs bit for bit: the grid only changes which workgroup runs a phase's work or a GEMM tile."""
    wl = W.scaled(W.WORKLOADS["mixtral"], T=1024, N=1024)
    inp = W.make_inputs(wl, 22)
    dev = to_dev(inp)
    ref = _call(inp, dev, tune={"n_mover_wg": -1})
    out = _call(inp, dev, tune={"n_mover_wg": mk.MK_MOVERS_NONE, "n_compute_wg": n_compute})
    _same(ref, out, KEYS + ("topk_w",))


@pytest.mark.parametrize("name,changes,arrivals", [
    ("mixtral", dict(T=1024, N=1024), False),
    ("skewed", dict(T=2048, N=512), False),
    ("wide_ep", dict(T=2048, d=1024, E=64, k=4, N=512, E_local=16, e_begin=16, chunk_rows=32), True),
])
def test_tile_order_does_not_change_results(name, changes, arrivals):
    """The GEMM tasks in expert order or with the short last tiles after every full tile (rows read in place,
    with arrivals for the wide-EP share, and moved by 64 movers) give the same bits."""
    wl = W.scaled(W.WORKLOADS[name], **changes)
    inp = W.make_inputs(wl, 23)
    dev = to_dev(inp)
    for movers in (0, 64):
        outs = []
        for order in (mk.MK_ORDER_EXPERT, mk.MK_ORDER_TAILS_LAST):
            tune = {"tile_order": order, "n_mover_wg": movers}
            if arrivals:
                _, ref_ids, _ = oracle_route(inp)
                delays = torch.randint(0, 50, (wl.S * (wl.rows_per_src // wl.chunk_rows),),
                                       generator=torch.Generator().manual_seed(6)).to(torch.int32)
                out, st, detail, _ = _ep_run(wl, inp, dev, torch.from_numpy(ref_ids).cuda(), delays=delays, tune=tune)
                assert st == mk.MK_OK, (mk.mk_status_str(st), detail)
            else:
                out = _call(inp, dev, tune=tune)
            outs.append(out)
        _same(outs[0], outs[1], KEYS + ("topk_w",) if not arrivals else KEYS)


def test_new_inputs_through_one_workspace():
    """A second call with different inputs through the same workspace must not see the first call's rows."""
    wl = W.scaled(W.WORKLOADS["skewed"], T=2048, N=512)
    ws = torch.zeros(mk.mk_dispatch_gemm_workspace_bytes(wl.T, wl.d, wl.E, wl.k, 0, wl.E_local, wl.N),
                     dtype=torch.uint8, device="cuda")
    for seed in (30, 31, 32):
        inp = W.make_inputs(wl, seed)
        out = _call(inp, to_dev(inp), workspace=ws)
        _, ids, _ = oracle_route(inp)
        _, offsets, _, _ = oracle.layout(ids, 0, wl.E_local)
        full_check(inp, out, rows=sample_rows(offsets, 64, seed), what=f"seed {seed}")


# ---------------------------------------------------------------- arrivals

def _ep_small():
    """A reduced wide-EP share: 8 sources x 256 rows, 64 global experts, local 16..31, chunks of 32 rows."""
    return W.scaled(W.WORKLOADS["wide_ep"], T=2048, d=1024, E=64, k=4, N=512, E_local=16, e_begin=16,
                    chunk_rows=32)


def _ep_run(wl, inp, dev, ids_in, delays=None, payload=None, pre_release=False, epoch=1, **kw):
    n_chunks = wl.S * (-(-wl.rows_per_src // wl.chunk_rows))
    ready = torch.zeros(n_chunks, dtype=torch.int32, device="cuda")
    if pre_release:
        ready.fill_(epoch)
    out = mk.mk_dispatch_gemm(dev["x"], dev["w_experts"], wl.k, topk_ids_in=ids_in, E=wl.E, e_begin=wl.e_begin,
                              chunk_rows=wl.chunk_rows, chunk_ready=ready, epoch=epoch,
                              sim_delay_us=None if delays is None else delays.cuda(), sim_payload=payload, **kw)
    st, detail = mk.mk_poll_error(out["workspace"])
    return out, st, detail, ready


def _ep_inputs(wl, seed):
    inp = W.make_inputs(wl, seed)
    dev = to_dev(inp)
    _, ids, _ = oracle_route(inp)
    return inp, dev, torch.from_numpy(ids).cuda()


def test_arrival_flags_schedules_are_bit_identical():
    wl = _ep_small()
    inp, dev, ids_in = _ep_inputs(wl, 40)
    base, st, _, _ = _ep_run(wl, inp, dev, ids_in, pre_release=True)
    assert st == mk.MK_OK
    _, offsets, _, row_token = check_layout(base, ids_in.cpu().numpy(), wl, "ep pre-released")
    rows = sample_rows(offsets, 64)
    y_ref = oracle.expert_rows(inp["x"], inp["w_experts"], offsets, row_token, rows)
    assert_y_close(base["y_perm"][torch.from_numpy(rows.astype(np.int64)).cuda()].float().cpu().numpy(),
                   y_ref, "ep")
    n_chunks = wl.S * (wl.rows_per_src // wl.chunk_rows)
    g = torch.Generator().manual_seed(4)
    schedules = {
        "seeded U[0,100]": torch.randint(0, 101, (n_chunks,), generator=g, dtype=torch.int64).to(torch.int32),
        "all zero": torch.zeros(n_chunks, dtype=torch.int32),
        "reversed": torch.arange(n_chunks, 0, -1, dtype=torch.int32),
        "one source late": torch.tensor([300 if c // (n_chunks // wl.S) == 3 else 0 for c in range(n_chunks)],
                                        dtype=torch.int32),
    }
    for name, delays in schedules.items():
        for n_mover in (8, 64, mk.MK_MOVERS_NONE):   # movers, or tiles reading their rows in place
            out, st, detail, ready = _ep_run(wl, inp, dev, ids_in, delays=delays, tune={"n_mover_wg": n_mover})
            assert st == mk.MK_OK, (name, mk.mk_status_str(st), detail)
            assert (ready.cpu() == 1).all(), name
            _same(base, out)


def test_in_place_sources_equal_moved_rows():
    """Sources as regions of one receive buffer (in reverse order): the table reads their rows in place; the
    same inputs through separately allocated sources with every workgroup moving rows give the same bits."""
    wl = _ep_small()
    inp, dev, ids_in = _ep_inputs(wl, 44)
    t = mk.mk_select_tuning(wl.T, wl.d, wl.E, wl.k, wl.e_begin, wl.E_local, wl.N, chunk_rows=wl.chunk_rows,
                            xs=dev["x"])
    assert t["n_mover_wg"] == mk.MK_MOVERS_NONE
    in_place, st, _, _ = _ep_run(wl, inp, dev, ids_in, pre_release=True)
    assert st == mk.MK_OK
    moved, st, _, _ = _ep_run(wl, inp, to_dev(inp, separate=True), ids_in, pre_release=True,
                              tune={"n_mover_wg": 256})
    assert st == mk.MK_OK
    _same(in_place, moved)


def test_in_place_ragged_chunks_and_sources():
    """Sources of 250 rows (not a multiple of the 64-token blocks) in 32-row chunks (the last chunk of each
    source ragged), seeded arrivals: rows read in place give the bits of 64 movers and of all rows pre-released."""
    wl = W.scaled(_ep_small(), T=2000)
    inp, dev, ids_in = _ep_inputs(wl, 45)
    assert wl.rows_per_src == 250
    n_chunks = wl.S * (-(-wl.rows_per_src // wl.chunk_rows))
    delays = torch.randint(0, 40, (n_chunks,), generator=torch.Generator().manual_seed(7)).to(torch.int32)
    ref, st, _, _ = _ep_run(wl, inp, dev, ids_in, pre_release=True)
    assert st == mk.MK_OK
    for movers in (mk.MK_MOVERS_NONE, 64):
        out, st, detail, ready = _ep_run(wl, inp, dev, ids_in, delays=delays, tune={"n_mover_wg": movers})
        assert st == mk.MK_OK, (movers, mk.mk_status_str(st), detail)
        assert (ready.cpu() == 1).all()
        _same(ref, out)
    _, offsets, _, row_token = check_layout(ref, ids_in.cpu().numpy(), wl, "ragged ep")
    rows = sample_rows(offsets, 32)
    y_ref = oracle.expert_rows(inp["x"], inp["w_experts"], offsets, row_token, rows)
    assert_y_close(ref["y_perm"][torch.from_numpy(rows.astype(np.int64)).cuda()].float().cpu().numpy(), y_ref,
                   "ragged ep")


@pytest.mark.parametrize("n_mover", [16, mk.MK_MOVERS_NONE])
def test_poison_mode_reads_only_released_rows(n_mover):
    """Every source row holds NaN until the simulator copies its chunk in and releases the flag: movers, or
    GEMM tiles reading rows in place, must read only released rows."""
    wl = _ep_small()
    inp, dev, ids_in = _ep_inputs(wl, 41)
    base, st, _, _ = _ep_run(wl, inp, dev, ids_in, pre_release=True)
    assert st == mk.MK_OK
    payload = [t.clone() for t in dev["x"]]
    for t in dev["x"]:
        t.view(torch.int16).fill_(-1)             # 0xFFFF: bf16 NaN until the chunk arrives
    g = torch.Generator().manual_seed(5)
    delays = torch.randint(0, 60, (wl.S * (wl.rows_per_src // wl.chunk_rows),), generator=g,
                           dtype=torch.int64).to(torch.int32)
    out, st, detail, _ = _ep_run(wl, inp, dev, ids_in, delays=delays, payload=payload, tune={"n_mover_wg": n_mover})
    assert st == mk.MK_OK, (mk.mk_status_str(st), detail)
    R = int(out["expert_offsets"][-1])
    assert not torch.isnan(out["y_perm"][:R].float()).any()
    _same(base, out)
    for a, b in zip(dev["x"], payload):
        assert torch.equal(a, b)                  # every chunk was delivered


def test_full_size_wide_ep_with_arrivals():
    wl = W.WORKLOADS["wide_ep"]
    inp, dev, ids_in = _ep_inputs(wl, 0)
    delays = W.make_delays_us(wl, 0)
    out, st, detail, _ = _ep_run(wl, inp, dev, ids_in, delays=delays)
    assert st == mk.MK_OK, (mk.mk_status_str(st), detail)
    _, offsets, _, row_token = check_layout(out, ids_in.cpu().numpy(), wl, "wide_ep arrivals")
    rows = sample_rows(offsets, 32)
    y_ref = oracle.expert_rows(inp["x"], inp["w_experts"], offsets, row_token, rows)
    assert_y_close(out["y_perm"][torch.from_numpy(rows.astype(np.int64)).cuda()].float().cpu().numpy(), y_ref,
                   "wide_ep arrivals")


@pytest.mark.parametrize("n_mover", [64, 0])
def test_withheld_arrival_flag_times_out(n_mover):
    """One chunk is never released (no simulator, flag left at 0): the movers' bounded wait (64 movers), or
    the tiles' (the table: rows read in place), gives up, the call reports MK_ETIMEOUT and the kernel exits."""
    wl = _ep_small()
    inp, dev, ids_in = _ep_inputs(wl, 42)
    n_chunks = wl.S * (wl.rows_per_src // wl.chunk_rows)
    ready = torch.ones(n_chunks, dtype=torch.int32, device="cuda")
    ready[n_chunks // 2] = 0
    old = os.environ.get("MK_TIMEOUT_US")
    os.environ["MK_TIMEOUT_US"] = "20000"
    try:
        out = mk.mk_dispatch_gemm(dev["x"], dev["w_experts"], wl.k, topk_ids_in=ids_in, E=wl.E,
                                  e_begin=wl.e_begin, chunk_rows=wl.chunk_rows, chunk_ready=ready, epoch=1,
                                  tune={"n_mover_wg": n_mover})
        st, detail = mk.mk_poll_error(out["workspace"])
    finally:
        if old is None:
            del os.environ["MK_TIMEOUT_US"]
        else:
            os.environ["MK_TIMEOUT_US"] = old
    assert st == mk.MK_ETIMEOUT
    assert detail == (0x20000000 | (n_chunks // 2))


def test_workspace_reusable_after_timeout():
    """After a call that ended in MK_ETIMEOUT (a withheld arrival flag: movers, tile waits and grid state
    left mid-call), mk_poll_error and then a call with every chunk released through the same workspace
    give the same bits as a fresh workspace."""
    wl = _ep_small()
    inp, dev, ids_in = _ep_inputs(wl, 43)
    ref, st, _, _ = _ep_run(wl, inp, dev, ids_in, pre_release=True)
    assert st == mk.MK_OK
    n_chunks = wl.S * (wl.rows_per_src // wl.chunk_rows)
    ready = torch.ones(n_chunks, dtype=torch.int32, device="cuda")
    ready[3] = 0
    ws = torch.zeros_like(ref["workspace"])
    old = os.environ.get("MK_TIMEOUT_US")
    os.environ["MK_TIMEOUT_US"] = "20000"
    try:
        mk.mk_dispatch_gemm(dev["x"], dev["w_experts"], wl.k, topk_ids_in=ids_in, E=wl.E, e_begin=wl.e_begin,
                            chunk_rows=wl.chunk_rows, chunk_ready=ready, epoch=1, workspace=ws)
        st, _ = mk.mk_poll_error(ws)
    finally:
        if old is None:
            del os.environ["MK_TIMEOUT_US"]
        else:
            os.environ["MK_TIMEOUT_US"] = old
    assert st == mk.MK_ETIMEOUT
    ready.fill_(1)
    out = mk.mk_dispatch_gemm(dev["x"], dev["w_experts"], wl.k, topk_ids_in=ids_in, E=wl.E, e_begin=wl.e_begin,
                              chunk_rows=wl.chunk_rows, chunk_ready=ready, epoch=1, workspace=ws)
    st, detail = mk.mk_poll_error(ws)
    assert st == mk.MK_OK, (mk.mk_status_str(st), detail)
    _same(ref, out)
