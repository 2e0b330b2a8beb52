"""Benchmark of the fused MoE dispatch + expert GEMM on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload mixtral] [--seed 0]

One step = one mk_dispatch_gemm call over one batch of synthetic input
(routing, histogram, offsets, slots, row scatter, grouped GEMM), inputs
resident in HBM before the timed region.  Prints one JSON line for the named
workload (default the Mixtral-shaped one) with, on the default run, two
sub-records of the same form: "decode" (the weight-streaming bound share,
roofline in HBM GB/s) and "wide_ep" (rows arriving from eight simulated peers,
with the overlap efficiency against the serial sum).  Fields:
  value          whole-step TFLOP/s, 2*R*d*N flops per step (R = routed local rows)
  roofline       the dominant kernel's launch (the fused kernel, or with
                 --staged the grouped GEMM), timed with HIP events the library
                 records around it on its stream, against the dense bf16 MFMA
                 peak (or HBM when the flops per byte sit below the ridge);
                 traffic = counter-measured HBM bytes per launch when the
                 committed summary matches the kernel sources
  cpu_baseline   the CPU oracle timed on this host on a bounded sample
Only one GPU is used: --gpus above 1 exits with a message.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# MI355X dense bf16 matrix peak: 256 CUs x 4096 flop/clk x 2.4 GHz (vendor figure 2.5 PFLOP/s).
PEAK_BF16_TFLOPS = 256 * 4096 * 2.4e9 / 1e12
PEAK_HBM_GBS = 8000.0
METRIC = "fused MoE dispatch+GEMM TFLOP/s (% MFMA peak) + routed tokens/s, 1 GPU"


def _hip():
    lib = ctypes.CDLL("libamdhip64.so")
    lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    lib.hipEventSynchronize.argtypes = [ctypes.c_void_p]
    lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
    lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
    return lib


def _events(hip, n):
    evs = []
    for _ in range(n):
        e = ctypes.c_void_p()
        if hip.hipEventCreate(ctypes.byref(e)) != 0:
            raise RuntimeError("hipEventCreate failed")
        evs.append(e)
    return evs


def _elapsed_ms(hip, a, b) -> float:
    hip.hipEventSynchronize(b)
    ms = ctypes.c_float()
    if hip.hipEventElapsedTime(ctypes.byref(ms), a, b) != 0:
        raise RuntimeError("hipEventElapsedTime failed")
    return float(ms.value)


def _csrc_hash() -> str:
    h = hashlib.sha256()
    d = os.path.join(ROOT, "moe_dispatch_expert_amd", "csrc")
    for f in sorted(os.listdir(d)):
        with open(os.path.join(d, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def _traffic_path(kernel: str, workload: str) -> str:
    return os.path.join(ROOT, "profiles", f"{kernel}_{workload}_hbm_traffic.json")


def _traffic(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` (fused or gemm) from the committed rocprofv3 counter summary,
    if it was taken on the current kernel sources; else None."""
    p = _traffic_path(kernel, workload)
    if not os.path.exists(p):
        return None
    with open(p) as f:
        t = json.load(f)
    if t.get("csrc_sha256_16") != _csrc_hash():
        return None
    return t.get("bytes_per_launch")


def _pmc_per_dispatch(d: str, kernel_substr: str, counter: str) -> float:
    """Mean value of `counter` over the dispatches of kernels whose name contains kernel_substr, from a
    rocprofv3 --pmc -f csv output directory."""
    import csv
    import glob
    vals = []
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if kernel_substr in r["Kernel_Name"] and r["Counter_Name"] == counter:
                vals.append(float(r["Counter_Value"]))
    if not vals:
        raise SystemExit(f"no {counter} samples for '{kernel_substr}' under {d}")
    return sum(vals) / len(vals)


def write_traffic(out_dir: str, workload: str, kernel: str, copy_mib: int) -> dict:
    """HBM bytes per launch from four rocprofv3 --pmc runs (FETCH_SIZE and WRITE_SIZE, KiB per
    dispatch) of the kernel and of a plain copy of copy_mib MiB: each counter is scaled by
    (bytes the copy moves) / (what the counter reads for the copy)."""
    substr = {"fused": "k_fused", "gemm": "k_gemm"}[kernel]
    copy_bytes = copy_mib * 1024 * 1024
    f_k = _pmc_per_dispatch(os.path.join(out_dir, f"pmc_fetch_{kernel}_{workload}"), substr, "FETCH_SIZE")
    w_k = _pmc_per_dispatch(os.path.join(out_dir, f"pmc_write_{kernel}_{workload}"), substr, "WRITE_SIZE")
    f_c = _pmc_per_dispatch(os.path.join(out_dir, "pmc_fetch_copy"), "MulFunctor", "FETCH_SIZE")
    w_c = _pmc_per_dispatch(os.path.join(out_dir, "pmc_write_copy"), "MulFunctor", "WRITE_SIZE")
    fetch_scale, write_scale = copy_bytes / f_c, copy_bytes / w_c
    run = (f"python3 bench.py --workload {workload} --staged --no-sub --steps 3 --warmup 1 --no-cpu-baseline"
           if kernel == "gemm" else
           f"python3 bench.py --workload {workload} --no-sub --steps 3 --warmup 1 --no-cpu-baseline")
    commands = [f"export TMPDIR=/tmp; rocprofv3 --pmc {c} -f csv -d {out_dir}/pmc_{c.split('_')[0].lower()}_{kernel}_{workload} "
                f"-o run -- {run}" for c in ("FETCH_SIZE", "WRITE_SIZE")]
    commands += [f"export TMPDIR=/tmp; rocprofv3 --pmc {c} -f csv -d {out_dir}/pmc_{c.split('_')[0].lower()}_copy -o run "
                 f"-- python3 bench.py --copy-calibration {copy_mib}" for c in ("FETCH_SIZE", "WRITE_SIZE")]
    commands.append(f"python3 bench.py --write-traffic {out_dir} --workload {workload} --kernel {kernel}")
    rec = {"kernel": substr, "workload": workload, "commands": commands,
           "fetch_kib_per_dispatch": f_k, "write_kib_per_dispatch": w_k,
           "copy_bytes": copy_bytes, "copy_fetch_kib": f_c, "copy_write_kib": w_c,
           "fetch_scale": fetch_scale, "write_scale": write_scale,
           "bytes_per_launch": f_k * fetch_scale + w_k * write_scale, "csrc_sha256_16": _csrc_hash()}
    with open(_traffic_path(kernel, workload), "w") as f:
        json.dump(rec, f, indent=1)
    return rec


def _trace_command(out_dir: str, workload: str, kernel: str, extra: str = "") -> str:
    run = (f"python3 bench.py --workload {workload} --no-sub --no-cpu-baseline" + (" --staged" if kernel == "gemm" else "")
           + (f" {extra}" if extra else ""))
    return f"export TMPDIR=/tmp; rocprofv3 --kernel-trace --stats -f csv -d {out_dir} -o run -- {run}"


def summarize_trace(out_dir: str, workload: str, kernel: str, timed: int, extra: str = "", name: str = "",
                    path: str = "") -> str:
    """profiles/<kernel>_<workload>_kernel_trace.md from a rocprofv3 --kernel-trace --stats run of
    _trace_command: the per-kernel statistics over every dispatch, then the timed window alone (the last
    `timed` dispatches of the dominant kernel: the bench's timed steps, without its first call and warm-ups)."""
    import csv
    import glob
    substr = {"fused": "k_fused", "gemm": "k_gemm"}[kernel]
    stats = glob.glob(os.path.join(out_dir, "**", "*kernel_stats.csv"), recursive=True)
    trace = glob.glob(os.path.join(out_dir, "**", "*kernel_trace.csv"), recursive=True)
    if not stats or not trace:
        raise SystemExit(f"no kernel stats / trace csv under {out_dir}")
    tail = (f" --trace-extra '{extra}'" if extra else "") + (f" --trace-name {name}" if name else "")
    lines = [f"# Kernel trace: {substr}, {workload} workload" + (f" ({extra})" if extra else ""), "",
             "Commands (run from the repository root on one MI355X):", "", "```",
             _trace_command(out_dir, workload, kernel, extra), f"python3 bench.py --summarize-trace {out_dir} "
             f"--workload {workload} --kernel {kernel} --steps {timed}{tail}", "```", "",
             "All dispatches:", "",
             "| kernel | calls | total us | avg us | min us | max us | % |", "|---|---|---|---|---|---|---|"]
    for r in csv.DictReader(open(stats[0])):
        n = r["Name"] if len(r["Name"]) <= 90 else r["Name"][:87] + "..."
        f = lambda k: float(r[k]) / 1000.0
        lines.append(f"| `{n}` | {r['Calls']} | {f('TotalDurationNs'):.1f} | {f('AverageNs'):.1f} | "
                     f"{f('MinNs'):.1f} | {f('MaxNs'):.1f} | {float(r['Percentage']):.1f} |")
    d = sorted((int(r["Start_Timestamp"]), int(r["End_Timestamp"])) for r in csv.DictReader(open(trace[0]))
               if substr in r["Kernel_Name"])
    win = np.array([(e - b) / 1000.0 for b, e in d[-timed:]])
    lines += ["", f"Timed window (the last {len(win)} of {len(d)} `{substr}` dispatches, the bench's timed steps):", "",
              "| dispatches | avg us | p10 us | p50 us | p90 us |", "|---|---|---|---|---|",
              f"| {len(win)} | {win.mean():.1f} | {np.percentile(win, 10):.1f} | {np.percentile(win, 50):.1f} | "
              f"{np.percentile(win, 90):.1f} |"]
    path = path or os.path.join(ROOT, "profiles", f"{name or kernel + '_' + workload}_kernel_trace.md")
    with open(path, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    return path


def copy_calibration(mib: int, reps: int = 3):
    """A plain device copy of a known size, for counter calibration: an elementwise kernel that reads
    and writes every byte once (torch's multiply by one; a same-dtype copy_ may go to a DMA engine)."""
    import torch
    n = mib * 1024 * 1024
    src = torch.empty(n, dtype=torch.uint8, device="cuda").random_(0, 255)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        torch.mul(src, 1, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n, "reps": reps}), flush=True)


def library_gemm(wl, steps: int, warmup: int):
    """The library GEMM (torch linear, hipBLASLt) on the workload's expert shape, bf16 random data, R = T * k
    rows (what a uniform routing gives), two ways: one dense GEMM y[R, N] = x[R, d] . W[N, d]^T with a single
    W (reused by every row), and one GEMM per local expert on its R / E_local rows with its own W (the
    grouped problem: every expert's W is streamed once).  Each timed K times between two events."""
    import torch
    g = torch.Generator(device="cuda").manual_seed(0)
    R, N, K, E = wl.T * min(wl.k, wl.E_local), wl.N, wl.d, wl.E_local
    x = torch.randn(R, K, device="cuda", generator=g).to(torch.bfloat16)
    ws = [(torch.randn(N, K, device="cuda", generator=g) / K ** 0.5).to(torch.bfloat16) for _ in range(E)]
    xs = list(x.split(R // E))

    def timed(fn):
        for _ in range(warmup):
            fn()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for _ in range(steps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / steps

    flops = 2.0 * R * N * K
    res = {"library_gemm": "torch.nn.functional.linear (hipBLASLt), bf16", "M": R, "N": N, "K": K}
    for name, fn in (("dense_one_W", lambda: torch.nn.functional.linear(x, ws[0])),
                     ("per_expert", lambda: [torch.nn.functional.linear(xe, we) for xe, we in zip(xs, ws)])):
        ms = timed(fn)
        tf = flops / (ms * 1e-3) / 1e12
        res[name] = {"ms": round(ms, 4), "TFLOP/s": round(tf, 1), "frac": round(tf / PEAK_BF16_TFLOPS, 4)}
    print(json.dumps(res), flush=True)


def trace_summary(tr: dict) -> dict:
    """Phase boundaries of the fused kernel (max over workgroups, microseconds from the first start)."""
    live = tr["start"] > 0
    if not live.any():
        return {"note": "no trace records written"}
    t0 = tr["start"][live].min()
    us = lambda v: round(float(v - t0) / tr["ticks_per_us"], 2)
    out = {"start_spread_us": us(tr["start"][live].max())}
    for name in ("routed", "barrier_a", "selected", "counted", "barrier_b", "slots", "barrier_c", "moved", "done"):
        v = tr[name][live]
        v = v[v > 0]
        if v.size:
            out[name + "_max_us"] = us(v.max())
            out[name + "_p50_us"] = us(np.median(v))
    ft = tr["first_task"][live]
    ft = ft[ft > 0]
    if ft.size:
        out["first_task_min_us"] = us(ft.min())
        out["first_task_max_us"] = us(ft.max())
    out["tasks_min_max"] = [int(tr["tasks"][live].min()), int(tr["tasks"][live].max())]
    out["tile_wait_us_mean"] = round(float(tr["wait_ticks"][live].mean()) / tr["ticks_per_us"], 2)
    out["xcc_of_wg0_to_7"] = [int(v) for v in tr["xcc"][:8]]
    return out


def time_combine(bufs: dict, R: int, steps: int, warmup: int) -> dict:
    """mk_combine (weighted un-permute of y_perm back to token rows) on the outputs of a step: K launches
    between two events on the current stream.  Algorithmic bytes: every routed row of y_perm read once,
    the [T, N] output written once, slot_of and topk_w read once."""
    import torch
    import moe_dispatch_expert_amd as mk
    y, slot_of, gate = bufs["y_perm"], bufs["slot_of"], bufs["topk_w"]
    T, k = slot_of.shape
    N = y.shape[1]
    out = torch.empty(T, N, dtype=torch.bfloat16, device=y.device)
    for _ in range(warmup):
        mk.mk_combine(y, slot_of, gate, rows=R, out=out)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for _ in range(steps):
        mk.mk_combine(y, slot_of, gate, rows=R, out=out)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    alg = R * N * 2 + T * N * 2 + T * k * 8
    gbs = alg / (ms * 1e-3) / 1e9
    return {"kernel": "k_combine", "ms": round(ms, 4), "alg_bytes": alg, "achieved": round(gbs, 1),
            "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4)}


def time_ffn(case, R: int, steps: int, warmup: int, ms_step: float) -> dict:
    """The expert FFN over the dispatch's own layout, the workload's expert weights read as [gate | up]
    (F = N / 2), each part timed K times between two events on the current stream:
      dispatch_swiglu       mk_dispatch_gemm_swiglu: the whole step with SwiGLU in the GEMM epilogue, h [R, F]
      dispatch_then_swiglu  the step (mk_dispatch_gemm, timed above) plus mk_swiglu over its y_perm
      swiglu                mk_swiglu alone
      down                  the down-projection mk_grouped_gemm over h, seeded W_down [E_local, d, F] ~ N(0, 1/F)"""
    import torch
    import moe_dispatch_expert_amd as mk
    wl = case.wl
    y = case.bufs["y_perm"]
    F = wl.N // 2
    if wl.N % 16:
        return {"skipped": f"F = N / 2 = {wl.N / 2} is not a multiple of 8"}
    g = torch.Generator().manual_seed(case.seed * 1000 + 5)
    wd = torch.empty(wl.E_local, wl.d, F, dtype=torch.bfloat16)
    for e in range(wl.E_local):
        wd[e] = (torch.randn(wl.d, F, generator=g) / F ** 0.5).to(torch.bfloat16)
    wd = wd.to(y.device)
    h = torch.empty(y.shape[0], F, dtype=torch.bfloat16, device=y.device)
    h2 = torch.empty_like(h)
    z = torch.empty(y.shape[0], wl.d, dtype=torch.bfloat16, device=y.device)
    gws = torch.empty(mk.mk_grouped_gemm_workspace_bytes(wl.E_local), dtype=torch.uint8, device=y.device)
    off = case.bufs["expert_offsets"]
    out_h = dict(case.bufs, y_perm=h)

    def timed(fn):
        for _ in range(warmup):
            fn()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for _ in range(steps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / steps

    ms_dsw = timed(lambda: case.call(out=out_h, swiglu=True))
    st, detail = mk.mk_poll_error(case.ws)
    if st != mk.MK_OK:
        raise SystemExit(f"device error {mk.mk_status_str(st)} ({detail})")
    ms_act = timed(lambda: mk.mk_swiglu(y, rows=R, out=h2))
    ms_down = timed(lambda: mk.mk_grouped_gemm(h, off, wd, out=z, workspace=gws))
    gu_flops = 2.0 * R * wl.d * wl.N
    act_bytes = R * 3 * F * 2
    down_flops = 2.0 * R * F * wl.d
    tf = lambda fl, ms: round(fl / (ms * 1e-3) / 1e12, 2)
    return {"F": F,
            "dispatch_swiglu": {"kernel": "k_fused (SwiGLU epilogue)", "ms": round(ms_dsw, 4), "flops": gu_flops,
                                "TFLOP/s": tf(gu_flops, ms_dsw),
                                "frac": round(tf(gu_flops, ms_dsw) / PEAK_BF16_TFLOPS, 4)},
            "dispatch_then_swiglu": {"kernels": "k_fused + k_swiglu", "ms": round(ms_step + ms_act, 4),
                                     "TFLOP/s": tf(gu_flops, ms_step + ms_act)},
            "swiglu": {"kernel": "k_swiglu", "ms": round(ms_act, 4), "alg_bytes": act_bytes,
                       "achieved": round(act_bytes / (ms_act * 1e-3) / 1e9, 1), "unit": "GB/s",
                       "frac": round(act_bytes / (ms_act * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)},
            "down": {"kernel": "k_gemm", "ms": round(ms_down, 4), "flops": down_flops,
                     "TFLOP/s": tf(down_flops, ms_down), "frac": round(tf(down_flops, ms_down) / PEAK_BF16_TFLOPS, 4)}}


def cpu_baseline(inp, R_gpu: int, budget_s: float = 12.0) -> dict:
    import oracle
    wl = inp["wl"]
    t0 = time.perf_counter()
    b = None if inp["bias"] is None else inp["bias"].numpy()
    _, ids, _ = oracle.route(inp["x"], inp["w_router"].numpy(), wl.k, b)
    _, offsets, _, row_token = oracle.layout(ids, wl.e_begin, wl.E_local)
    t_route = time.perf_counter() - t0
    R = int(offsets[-1])
    rng = np.random.default_rng(0)
    # one probe row, then as many rows as fit the budget
    t1 = time.perf_counter()
    oracle.expert_rows(inp["x"], inp["w_experts"], offsets, row_token, np.array([0], dtype=np.int32))
    per_row = max(time.perf_counter() - t1, 1e-4)
    n = int(max(1, min(R, (budget_s - t_route) / per_row * oracle.num_threads())))
    rows = np.sort(rng.choice(R, size=n, replace=False)).astype(np.int32)
    t2 = time.perf_counter()
    oracle.expert_rows(inp["x"], inp["w_experts"], offsets, row_token, rows)
    t_gemm = time.perf_counter() - t2
    t_full = t_route + t_gemm * R / n          # extrapolated whole-job time
    flops = 2.0 * R * wl.d * wl.N
    return {"value": flops / t_full / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": (f"routing+layout of all {wl.T} tokens ({t_route:.2f} s) + fp64 GEMM of {n} of {R} "
                       f"expert rows ({t_gemm:.2f} s), GEMM time scaled to all rows"),
            "routed_rows_per_s": R / t_full, "matches_gpu_R": R == R_gpu}


def _roofline(flops: float, alg_bytes: float, launch_all, kernel: str, traffic) -> dict:
    """Roofline record of one launch kind: which roof bounds it (flops per algorithmic byte against the ridge
    point), what it achieved over the mean event-timed launch, and the spread of launch times."""
    ms = float(np.mean(launch_all))
    if flops / max(alg_bytes, 1) >= PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9):
        tf = flops / (ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(tf, 2), "peak": round(PEAK_BF16_TFLOPS, 1),
                "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4)}
    else:
        gbs = alg_bytes / (ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(gbs / PEAK_HBM_GBS, 4)}
    roof.update({"traffic": traffic, "kernel": kernel, "launch_ms": round(ms, 4),
                 "launch_ms_p10_p50_p90": [round(float(v), 4) for v in np.percentile(launch_all, [10, 50, 90])],
                 "flops_per_launch": flops, "alg_bytes_per_launch": alg_bytes})
    return roof


class Case:
    """One workload resident on the GPU: inputs, outputs, workspace, and a timed loop of mk_dispatch_gemm."""

    def __init__(self, wl, seed: int, base_tune: dict, inp=None):
        import torch
        import moe_dispatch_expert_amd as mk
        import workloads as W
        self.wl, self.mk, self.torch, self.seed = wl, mk, torch, seed
        self.inp = inp if inp is not None else W.make_inputs(wl, seed)
        dev = self.dev = torch.device("cuda:0")
        x = self.inp["x"]
        if wl.S > 1:   # the peers' rows land in per-peer regions of one receive buffer
            recv = torch.empty(wl.T, wl.d, dtype=x.dtype, device=dev)
            recv.copy_(x)
            self.xs = [recv[s * wl.rows_per_src:(s + 1) * wl.rows_per_src] for s in range(wl.S)]
        else:
            self.xs = x.to(dev)
        self.wr = self.inp["w_router"].to(dev)
        self.bias = None if self.inp["bias"] is None else self.inp["bias"].to(dev)
        self.we = self.inp["w_experts"].to(dev)
        self.ids_in = None
        if wl.route_outside:   # the sources route their own tokens before the payload arrives (untimed)
            parts = [mk.mk_route_topk(self.xs[s], self.wr, wl.k)[0] for s in range(wl.S)]
            self.ids_in = torch.cat(parts).contiguous()
        self.base_tune = dict(base_tune)
        self.arrivals = None
        xl = self.xs if isinstance(self.xs, list) else [self.xs]
        self.ws = torch.zeros(mk.mk_dispatch_gemm_workspace_bytes(
            wl.T, wl.d, wl.E, wl.k, wl.e_begin, wl.E_local, wl.N, wl.S, tune=self.base_tune, xs=xl),
            dtype=torch.uint8, device=dev)
        out = self._call(None, None)
        self.bufs = {k: out[k] for k in ("y_perm", "slot_of", "expert_offsets", "topk_ids", "topk_w", "row_token")}
        self.epoch = 1

    def with_arrivals(self, delays_us):
        """From now on every call models arriving rows: chunk flags released by the kernel's arrival simulator
        sim_delay_us[c] microseconds after the launch starts (flags only: the rows are already resident).
        Each call uses the next epoch, so no flag needs clearing between calls."""
        torch, wl = self.torch, self.wl
        n = wl.S * (-(-wl.rows_per_src // wl.chunk_rows))
        self.arrivals = {"ready": torch.zeros(n, dtype=torch.int32, device=self.dev),
                         "delays": delays_us.to(self.dev)}
        tu = dict(self.base_tune)
        xl = self.xs if isinstance(self.xs, list) else [self.xs]
        self.ws = torch.zeros(self.mk.mk_dispatch_gemm_workspace_bytes(
            wl.T, wl.d, wl.E, wl.k, wl.e_begin, wl.E_local, wl.N, wl.S, chunk_rows=wl.chunk_rows, tune=tu, xs=xl),
            dtype=torch.uint8, device=self.dev)
        return self

    def _call(self, ev_begin, ev_end, out=None, swiglu=False):
        wl, mk = self.wl, self.mk
        tune = dict(self.base_tune)
        if ev_begin is not None:
            tune.update({"ev_gemm_begin": ev_begin, "ev_gemm_end": ev_end})
        kw = {}
        if self.arrivals is not None:
            self.epoch += 1
            kw = dict(chunk_rows=wl.chunk_rows, chunk_ready=self.arrivals["ready"], epoch=self.epoch,
                      sim_delay_us=self.arrivals["delays"])
        return mk.mk_dispatch_gemm(self.xs, self.we, wl.k, w_router=self.wr, bias=self.bias, topk_ids_in=self.ids_in,
                                   E=wl.E, e_begin=wl.e_begin, workspace=self.ws,
                                   out=out if out is not None else getattr(self, "bufs", None), tune=tune,
                                   swiglu=swiglu, **kw)

    def call(self, out=None, swiglu=False):
        """One untimed call (out: other output buffers; swiglu: the gate|up reading of the weights)."""
        return self._call(None, None, out, swiglu)

    def run(self, steps: int, warmup: int, evict_mall: bool = False) -> dict:
        """W untimed calls, then K timed calls between two events (step time), each call's GEMM launch also
        between the library's own events on its stream (launch time)."""
        torch, mk = self.torch, self.mk
        hip = _hip()
        evs = _events(hip, 2 * steps)
        for _ in range(warmup):
            self._call(None, None)
        torch.cuda.synchronize()
        st, detail = mk.mk_poll_error(self.ws)
        if st != mk.MK_OK:
            raise SystemExit(f"device error {mk.mk_status_str(st)} ({detail})")
        t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        scratch = torch.ones(1 << 30, dtype=torch.uint8, device=self.dev) if evict_mall else None
        torch.cuda.synchronize()
        t_start.record()
        for i in range(steps):
            if scratch is not None:   # read, not write: evicted lines are clean, so no write-back lands in the step
                scratch.sum(dtype=torch.int64)
            self._call(evs[2 * i], evs[2 * i + 1])
        t_end.record()
        torch.cuda.synchronize()
        st, detail = mk.mk_poll_error(self.ws)
        if st != mk.MK_OK:
            raise SystemExit(f"device error {mk.mk_status_str(st)} ({detail})")
        launch_all = [_elapsed_ms(hip, evs[2 * i], evs[2 * i + 1]) for i in range(steps)]
        for e in evs:
            hip.hipEventDestroy(e)
        ms_step = t_start.elapsed_time(t_end) / steps
        if scratch is not None:   # the evicting reads sit between the steps: time the launches only
            ms_step = float(np.mean(launch_all))
        wl = self.wl
        R = int(self.bufs["expert_offsets"][-1].item())
        hit = int((torch.diff(self.bufs["expert_offsets"]) > 0).sum())
        alg_bytes = (hit * wl.N * wl.d * 2 + R * wl.N * 2      # weights of hit experts, y_perm
                     + wl.T * wl.d * 2 + (0 if self.ids_in is not None else wl.d * wl.E * 4))
        return {"ms_step": ms_step, "launch_all": launch_all, "R": R, "flops": 2.0 * R * wl.d * wl.N,
                "alg_bytes": alg_bytes}


def _device_record(torch) -> dict:
    """What the runtime reports about the GPU (the peaks above are the vendor's figures for MI355X)."""
    p = torch.cuda.get_device_properties(0)
    return {"name": p.name, "arch": getattr(p, "gcnArchName", ""), "compute_units": p.multi_processor_count,
            "hbm_GiB": round(p.total_memory / 2 ** 30, 1)}


def decode_record(seed: int, steps: int, warmup: int) -> dict:
    """Decode-shaped share (T=128, d=7168, 32 local of 256 experts, top-8, N=2048), routing inside the step:
    weight-streaming bound, so its roofline is HBM bytes (weights of the hit experts, x, router weights,
    y_perm) over the event-timed fused launch."""
    import workloads as W
    c = Case(W.WORKLOADS["decode"], seed, {})
    m = c.run(steps, warmup)
    roof = _roofline(m["flops"], m["alg_bytes"], m["launch_all"], "fused dispatch+GEMM (k_fused)",
                     _traffic("fused", "decode"))
    return {"workload": "decode", "R": m["R"], "ms_per_step": round(m["ms_step"], 4),
            "tokens_per_s": c.wl.T / (m["ms_step"] * 1e-3), "roofline": roof}


def wide_ep_record(seed: int, steps: int, warmup: int) -> dict:
    """One GPU's share of a wide EP layer (8 sources x 2048 rows, d=7168, 32 local of 256 experts, top-8,
    N=2048), ids routed by the sources (untimed), rows arriving in chunks of 128 whose ready flags the
    kernel's arrival simulator releases at seeded U[0, 100] us delays.  Also timed: the same arrivals with
    every workgroup first moving rows (the dispatch role), and all rows resident.  Overlap efficiency = (last arrival
    + the grouped GEMM alone on the same layout) / the fused launch: above 1 when the GEMM runs while rows
    are still arriving."""
    import torch
    import workloads as W
    wl = W.WORKLOADS["wide_ep"]
    inp = W.make_inputs(wl, seed)
    delays = inp["delays_us"]
    fused = Case(wl, seed, {}, inp=inp).with_arrivals(delays)
    mf = fused.run(steps, warmup)
    del fused
    movers = Case(wl, seed, {"n_mover_wg": 256}, inp=inp).with_arrivals(delays)
    mm = movers.run(steps, warmup)
    del movers
    at_zero = Case(wl, seed, {}, inp=inp).with_arrivals(torch.zeros_like(delays))
    mz = at_zero.run(steps, warmup)
    del at_zero
    resident = Case(wl, seed, {}, inp=inp)
    mr = resident.run(steps, warmup)
    del resident
    staged = Case(wl, seed, {"n_mover_wg": -1}, inp=inp)
    ms = staged.run(steps, warmup)
    del staged
    fused_ms = float(np.mean(mf["launch_all"]))
    gemm_ms = float(np.mean(ms["launch_all"]))
    arrival_ms = float(delays.max()) * 1e-3
    roof = _roofline(mf["flops"], mf["alg_bytes"], mf["launch_all"], "fused dispatch+GEMM (k_fused), arrivals",
                     _traffic("fused", "wide_ep"))
    return {"workload": "wide_ep", "R": mf["R"], "ms_per_step": round(mf["ms_step"], 4),
            "tflops_step": round(mf["flops"] / (mf["ms_step"] * 1e-3) / 1e12, 2),
            "arrivals": f"{delays.numel()} chunks of {wl.chunk_rows} rows, flags released at seeded U[0,100] us "
                        f"(last at {float(delays.max()):.0f} us), rows already resident",
            "roofline": roof,
            "path": "the per-shape table's (tiles read their rows in place, each waiting for its rows' chunks)",
            "fused_movers_arrivals_launch_ms": round(float(np.mean(mm["launch_all"])), 4),
            "fused_arrivals_all_at_0us_launch_ms": round(float(np.mean(mz["launch_all"])), 4),
            "fused_all_resident_launch_ms": round(float(np.mean(mr["launch_all"])), 4),
            "gemm_alone_launch_ms": round(gemm_ms, 4),
            "last_arrival_ms": round(arrival_ms, 4),
            "serial_sum_ms": round(arrival_ms + gemm_ms, 4),
            "overlap_efficiency": round((arrival_ms + gemm_ms) / fused_ms, 4)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="mixtral")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sub", action="store_true",
                    help="time the named workload only (no decode / wide_ep sub-records)")
    ap.add_argument("--trace", action="store_true", help="add the fused kernel's phase timeline of the last step")
    ap.add_argument("--staged", action="store_true", help="one launch per step instead of the fused kernel")
    ap.add_argument("--movers", type=int, default=0, help="override the per-shape mover count")
    ap.add_argument("--compute-wg", type=int, default=0, help="override the per-shape compute workgroup count")
    ap.add_argument("--tile-order", type=int, default=0, help="override the per-shape GEMM task order (1 or 2)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain MIB-MiB device copy (counter calibration) and exit")
    ap.add_argument("--write-traffic", default="", metavar="DIR",
                    help="only turn the rocprofv3 --pmc outputs under DIR into profiles/<kernel>_<workload>_hbm_traffic.json")
    ap.add_argument("--kernel", default="fused", choices=("fused", "gemm"),
                    help="kernel for --write-traffic / --summarize-trace")
    ap.add_argument("--trace-extra", default="", help="bench arguments the traced run added (--summarize-trace)")
    ap.add_argument("--trace-name", default="", help="profile name instead of <kernel>_<workload> (--summarize-trace)")
    ap.add_argument("--summarize-trace", default="", metavar="DIR",
                    help="only turn a rocprofv3 --kernel-trace --stats run under DIR into "
                         "profiles/<kernel>_<workload>_kernel_trace.md (timed window = the last --steps dispatches)")
    ap.add_argument("--evict-mall", action="store_true",
                    help="read 1 GiB before every step (outside the launch events) so no input is left in the "
                         "256 MiB Infinity Cache; value and roofline then come from the launch events")
    ap.add_argument("--ffn", action="store_true",
                    help="also time the expert FFN over the step's layout (the expert weights read as [gate | up], "
                         "F = N / 2): mk_dispatch_gemm_swiglu, mk_swiglu, and the down-projection mk_grouped_gemm "
                         "(reported apart, not in value)")
    ap.add_argument("--library-gemm", action="store_true",
                    help="only time the dense library GEMM (torch linear) of the workload's expert shape and exit")
    ap.add_argument("--combine", action="store_true",
                    help="also time the next step, mk_combine, on the step's outputs (reported apart, not in value)")
    args = ap.parse_args()
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.write_traffic:
        print(json.dumps(write_traffic(args.write_traffic, args.workload, args.kernel, 1024)), flush=True)
        return
    if args.summarize_trace:
        print(summarize_trace(args.summarize_trace, args.workload, args.kernel, args.steps, args.trace_extra,
                              args.trace_name), flush=True)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU's share only (asked for --gpus {args.gpus}); run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import moe_dispatch_expert_amd as mk
    import workloads as W

    wl = W.WORKLOADS[args.workload]
    if args.library_gemm:
        library_gemm(wl, args.steps, args.warmup)
        return
    base_tune = {}
    if args.staged:
        base_tune["n_mover_wg"] = mk.MK_MOVERS_STAGED
    elif args.movers:
        base_tune["n_mover_wg"] = args.movers
    if args.compute_wg:
        base_tune["n_compute_wg"] = args.compute_wg
    if args.tile_order:
        base_tune["tile_order"] = args.tile_order
    case = Case(wl, args.seed, base_tune)
    if wl.chunk_rows > 0 and not args.staged:   # rows arriving in chunks, flags released at seeded delays
        case.with_arrivals(case.inp["delays_us"])
    m = case.run(args.steps, args.warmup, args.evict_mall)
    ms_step, R, flops = m["ms_step"], m["R"], m["flops"]
    tflops = flops / (ms_step * 1e-3) / 1e12
    kernel = "gemm" if args.staged else "fused"
    traffic = _traffic(kernel, args.workload) if not (args.movers or args.compute_wg or args.tile_order) else None
    roof = _roofline(flops, m["alg_bytes"], m["launch_all"],
                     "grouped expert GEMM (k_gemm)" if args.staged else "fused dispatch+GEMM (k_fused)", traffic)
    rec = {
        "metric": METRIC, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": args.workload, "T": wl.T, "d": wl.d, "E": wl.E, "k": wl.k, "N": wl.N,
                   "E_local": wl.E_local, "e_begin": wl.e_begin, "sources": wl.S, "R": R, "seed": args.seed,
                   "routing": "by the sources (untimed)" if case.ids_in is not None else "inside the step",
                   "arrivals": ("chunk flags at seeded U[0,100] us delays" if case.arrivals is not None
                                else "all rows resident")},
        "mfma_frac_step": round(tflops / PEAK_BF16_TFLOPS, 4),
        "routed_rows_per_s": R / (ms_step * 1e-3), "tokens_per_s": wl.T / (ms_step * 1e-3),
        "hbm_GBs_step_alg": m["alg_bytes"] / (ms_step * 1e-3) / 1e9,
        "roofline": roof,
        "torch": torch.__version__,
        "device": _device_record(torch),
    }
    if args.staged or args.movers or args.compute_wg or args.tile_order:
        rec["config"]["path"] = ("staged" if args.staged else "fused") + (
            f", {args.movers} movers" if args.movers else "") + (
            f", {args.compute_wg} compute workgroups" if args.compute_wg else "") + (
            f", tile order {args.tile_order}" if args.tile_order else "")
    if args.evict_mall:
        rec["config"]["mall"] = "1 GiB read before every step; step time = launch time"
    if args.trace and not args.staged:
        rec["trace"] = trace_summary(mk.mk_dispatch_gemm_trace(case.ws, wl.T, wl.d, wl.E, wl.k, wl.e_begin,
                                                               wl.E_local, wl.N, wl.S))
    if args.combine:
        rec["combine"] = time_combine(case.bufs, R, args.steps, args.warmup)
    if args.ffn:
        rec["ffn"] = time_ffn(case, R, args.steps, args.warmup, ms_step)
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(case.inp, R)
        rec["cpu_baseline"]["value"] = round(rec["cpu_baseline"]["value"], 6)
    del case
    if not args.no_sub and not (args.staged or args.movers or args.compute_wg or args.tile_order) and \
            args.workload == "mixtral":
        torch.cuda.empty_cache()
        rec["decode"] = decode_record(args.seed, args.steps, args.warmup)
        torch.cuda.empty_cache()
        rec["wide_ep"] = wide_ep_record(args.seed, args.steps, args.warmup)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
