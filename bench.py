"""Benchmark of the MoE-FFN forward on one MI355X.

One step = one moe_ffn_forward call (router + top-k, dispatch, expert up and
down projections, combine, aux statistics) over one batch of seeded
synthetic input already resident in HBM.  Prints ONE JSON line.

  python bench.py [--steps K] [--warmup W] [--config NAME] [--no-cpu-baseline]

value = tokens per second of the whole step.  roofline = the up-projection
kernel (the dominant one), timed with HIP events on the launch stream in a
second pass of K steps made of the per-stage entry points.  cpu_baseline =
the float64 oracle on the host cores (never tuned), on a bounded sample.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16/fp16 MFMA
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E
METRIC = "MoE-FFN fwd tokens/s + TFLOP/s (% bf16 MFMA peak / % HBM BW), 1 MI355X"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--config", default=None, help="workload name (default: large_prefill)")
    ap.add_argument("--tokens", type=int, default=0,
                    help="run the workload's layer on this many tokens instead of its T "
                         "(the first T rows of its x draw; weights unchanged)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="also time the forward captured in a HIP graph (graph_ms_per_step)")
    ap.add_argument("--pass", dest="pass_", choices=("forward", "backward"), default="forward",
                    help="backward: time moe_ffn_backward (gradients of the task loss plus "
                         "alpha * L_aux) instead of the forward")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--gemm-policy", choices=("auto", "mf32", "mf16"), default="auto",
                    help="grouped GEMM main loop (moe_set_gemm_policy; results are identical)")
    ap.add_argument("--copy-calibration-mb", type=int, default=0,
                    help="only run a plain device copy of this many MiB (for counter scaling)")
    ap.add_argument("--record-traffic", nargs=6,
                    metavar=("KERNEL", "WORKLOAD", "NAME", "SOURCE", "FETCH_DIR", "WRITE_DIR"),
                    help="host only: write the traffic entry KERNEL:WORKLOAD of "
                         "profiles/traffic.json from two rocprofv3 --pmc output folders "
                         "(FETCH_SIZE, WRITE_SIZE), averaging the dispatches whose name "
                         "contains NAME; SOURCE = the kernel's file under csrc/")
    ap.add_argument("--calibration", nargs=3, metavar=("MIB", "FETCH_DIR", "WRITE_DIR"),
                    help="with --record-traffic: the --pmc folders of a "
                         "--copy-calibration-mb MIB run, giving the counter scales")
    return ap.parse_args()


def source_digest(path):
    """sha256 of a kernel source with its comments and whitespace removed:
    recorded counters stay valid across comment-only edits and become
    invalid when the code changes."""
    import re
    text = open(path, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return hashlib.sha256("".join(text.split()).encode()).hexdigest()


def _counter_rows(folder, counter):
    import csv
    import glob
    paths = glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True)
    if not paths:
        raise SystemExit(f"no counter_collection.csv under {folder}")
    rows = []
    for path in paths:
        with open(path) as fh:
            rows += [r for r in csv.DictReader(fh) if r["Counter_Name"] == counter]
    return rows


def record_traffic(a):
    """HBM bytes per launch of one kernel = FETCH_SIZE * fetch_scale + WRITE_SIZE *
    write_scale, where the scales make the counters of a plain device copy of
    known size read its true byte counts.  Writes profiles/traffic.json."""
    kernel, workload, name, source, fdir, wdir = a.record_traffic
    if not a.calibration:
        raise SystemExit("--record-traffic needs --calibration MIB FETCH_DIR WRITE_DIR")
    mib, cfdir, cwdir = int(a.calibration[0]), a.calibration[1], a.calibration[2]
    nbytes = mib * (1 << 20)

    def copy_kib(folder, counter):
        rows = [r for r in _counter_rows(folder, counter) if "copyBuffer" in r["Kernel_Name"]]
        return max(float(r["Counter_Value"]) for r in rows)   # the big copy

    def kernel_kib(folder, counter):
        vals = [float(r["Counter_Value"]) for r in _counter_rows(folder, counter)
                if name in r["Kernel_Name"]]
        if not vals:
            raise SystemExit(f"no dispatch of '{name}' in {folder}")
        return sum(vals) / len(vals), len(vals)

    cf, cw = copy_kib(cfdir, "FETCH_SIZE"), copy_kib(cwdir, "WRITE_SIZE")
    fs, ws = nbytes / (cf * 1024), nbytes / (cw * 1024)
    fk, nf = kernel_kib(fdir, "FETCH_SIZE")
    wk, nw = kernel_kib(wdir, "WRITE_SIZE")
    src = os.path.join(ROOT, "mixture_experts_sparse_gemv_amd", "csrc", source)
    path = os.path.join(ROOT, "profiles", "traffic.json")
    db = json.load(open(path)) if os.path.exists(path) else {}
    db["_about"] = ("HBM bytes per launch = FETCH_SIZE * fetch_scale + WRITE_SIZE * write_scale "
                    "(rocprofv3 --pmc, KiB per dispatch); the scales make a plain device copy's "
                    "counters read the bytes it moves. Valid while the kernel source file (comments and whitespace "
                    "removed) hashes to source_sha256.")
    db["calibration"] = {"copy_bytes_each_way": nbytes, "fetch_kib": cf, "write_kib": cw,
                         "fetch_scale": fs, "write_scale": ws}
    db[f"{kernel}:{workload}"] = {
        "source": source,
        "source_sha256": source_digest(src),
        "dispatch_name": name, "dispatches": [nf, nw],
        "fetch_kib": fk, "write_kib": wk,
        "bytes_per_launch": int(round(fk * 1024 * fs + wk * 1024 * ws)),
    }
    with open(path, "w") as fh:
        json.dump(db, fh, indent=1)
        fh.write("\n")
    print(json.dumps(db[f"{kernel}:{workload}"]))


def expert_flops(run, kept_rows):
    F1 = 2 * run.d_ff if run.activation == "swiglu" else run.d_ff
    up = 2.0 * kept_rows * run.d_model * F1
    down = 2.0 * kept_rows * run.d_ff * run.d_model
    return up, down


def main():
    a = parse()
    if a.record_traffic:
        record_traffic(a)
        return
    if a.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {a.gpus}); the layer runs on a "
              f"single MI355X with all experts resident, so there is no multi-GPU step.",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    from mixture_experts_sparse_gemv_amd import moe as M
    from synth import HEADLINE_RUN, RUNS, make_inputs

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    M.moe_set_gemm_policy({"auto": M.MOE_GEMM_AUTO, "mf32": M.MOE_GEMM_MF32,
                           "mf16": M.MOE_GEMM_MF16}[a.gemm_policy])

    if a.copy_calibration_mb:
        n = a.copy_calibration_mb * (1 << 20) // 4
        src = torch.ones(n, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_each_way": n * 4}))
        return

    name = a.config or HEADLINE_RUN
    run = RUNS[name]
    if a.tokens:
        from synth import scaled
        run = scaled(run, T=a.tokens, x_rows=max(run.rows_drawn, a.tokens))
        name = f"{name}_T{a.tokens}"
    inp = make_inputs(run)
    g = {k: (None if v is None else v.to(dev)) for k, v in inp.items()}
    if a.no_cpu_baseline:
        del inp
    if run.w_fp8:
        # one-time preparation (untimed): per-row FP8 E4M3 codes and scales
        for name_w, name_s in (("w_up", "s_up"), ("w_down", "s_down")):
            wt = g[name_w]
            q = torch.empty(wt.shape, dtype=torch.uint8, device=dev)
            sc = torch.empty(wt.numel() // wt.shape[-1], dtype=torch.float32, device=dev)
            M.moe_quantize_fp8(wt, q, sc)
            g[name_w], g[name_s] = q, sc
            del wt
        torch.cuda.synchronize()
    cap = M.moe_capacity(run.T, run.top_k, run.num_experts, run.capacity_factor or 0.0)
    p = M.make_problem(T=run.T, d_model=run.d_model, d_ff=run.d_ff, num_experts=run.num_experts,
                       top_k=run.top_k, num_shared=run.num_shared, capacity=cap,
                       dtype=run.dtype, gating=run.gating, activation=run.activation,
                       router_bias=run.router_bias != "none", expert_bias=run.expert_bias,
                       w_fp8=run.w_fp8, expert_choice=run.expert_choice)
    w = M.make_weights(g["w_router"], g["b_router"], g["w_up"], g["b_up"], g["w_down"],
                       g["b_down"], g.get("s_up"), g.get("s_down"))
    ws = M.workspace(p, dev)
    y = torch.empty(run.T * run.d_model, dtype=torch.float32, device=dev)
    E, k, T = run.num_experts, run.top_k, run.T
    i32 = dict(dtype=torch.int32, device=dev)
    if run.expert_choice:   # experts pick their tokens: E*cap rows, [T, E] rows and weights
        r = dict(probs=torch.empty(T * E, dtype=torch.float32, device=dev),
                 counts=torch.empty(E, **i32), kept=torch.empty(E, **i32),
                 offsets=torch.empty(E + 1, **i32), sorted_assign=torch.empty(E * cap, **i32),
                 assign_row=torch.empty(T * E, **i32), f=torch.empty(E, device=dev),
                 P=torch.empty(E, device=dev), l_aux=torch.empty(1, device=dev))
    else:
        r = dict(topk_idx=torch.empty(T * k, **i32),
                 topk_w=torch.empty(T * k, dtype=torch.float32, device=dev),
                 counts=torch.empty(E, **i32), kept=torch.empty(E, **i32),
                 offsets=torch.empty(E + 1, **i32), sorted_assign=torch.empty(T * k, **i32),
                 assign_row=torch.empty(T * k, **i32),
                 drop_mask=torch.empty(T * k, dtype=torch.uint8, device=dev),
                 f=torch.empty(E, device=dev), P=torch.empty(E, device=dev),
                 l_aux=torch.empty(1, device=dev))
    print(f"bench: {name} T={T} d={run.d_model} f={run.d_ff} E={E} k={k} S={run.num_shared} "
          f"cap={cap} warmup={a.warmup} steps={a.steps}", file=sys.stderr, flush=True)

    if a.pass_ == "backward":
        bench_backward(a, name, run, p, w, g, ws, y, r)
        return

    # ---- headline: K whole forward calls
    for _ in range(a.warmup):
        M.moe_ffn_forward(p, w, g["x"], y, ws, routing=r)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(a.steps):
        M.moe_ffn_forward(p, w, g["x"], y, ws, routing=r)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    step_s = (t1 - t0) / a.steps

    graph_ms = None
    if a.graph:   # the same step captured once and replayed
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph, stream=side):
                M.moe_ffn_forward(p, w, g["x"], y, ws, routing=r)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        for _ in range(a.warmup):
            graph.replay()
        torch.cuda.synchronize()
        g0 = time.perf_counter()
        for _ in range(a.steps):
            graph.replay()
        torch.cuda.synchronize()
        graph_ms = (time.perf_counter() - g0) / a.steps * 1e3

    kept = int(r["offsets"][E].item())
    rows = kept + run.num_shared * T
    counts = r["counts"].cpu().numpy()
    touched = int(np.count_nonzero(r["kept"].cpu().numpy())) + run.num_shared
    up_fl, down_fl = expert_flops(run, rows)
    router_fl = 2.0 * T * run.d_model * E
    step_flops = up_fl + down_fl + router_fl
    F1 = 2 * run.d_ff if run.activation == "swiglu" else run.d_ff
    esz = 4 if run.dtype == "f32" else 2
    wsz = 1 if run.w_fp8 else esz   # expert weight bytes per element (scales: 4 per row)
    w_bytes_touched = touched * ((F1 * run.d_model + run.d_model * run.d_ff) * wsz +
                                 ((F1 + run.d_model) * 4 if run.w_fp8 else 0))
    step_bytes = (T * run.d_model * esz + E * run.d_model * esz + w_bytes_touched +
                  T * run.d_model * 4)
    decode = run.dtype == "bf16" and T <= 128   # the library's weight-streaming path

    # ---- per-stage pass: the same steps through the stage entry points, with
    # events around each stage on the launch stream
    stream = torch.cuda.current_stream()
    names = ["router_topk", "dispatch", "expert_up", "expert_down", "combine"]
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
          for _ in range(a.steps)]
    h = torch.empty(M.max_rows(p) * run.d_ff, dtype=M.h_dtype(p), device=dev)
    y_exp = torch.empty(M.max_rows(p) * run.d_model, dtype=torch.float32, device=dev)
    part = torch.empty(E, dtype=torch.float32, device=dev)

    def staged(evs=None):
        rec = (lambda i: evs[i].record(stream)) if evs else (lambda i: None)
        rec(0)
        if run.expert_choice:
            M.moe_router_topk(p, g["x"], w, None, None, r["probs"], part, ws=ws)
            rec(1)
            M.moe_expert_choice(p, r["probs"], r["offsets"], r["sorted_assign"], r["assign_row"],
                                ws=ws)
        else:
            M.moe_router_topk(p, g["x"], w, r["topk_idx"], r["topk_w"], None, part, ws=ws)
            rec(1)
            M.moe_dispatch(p, r["topk_idx"], r["counts"], r["kept"], r["offsets"],
                           r["sorted_assign"], r["assign_row"], r["drop_mask"], ws=ws)
        rec(2)
        M.moe_expert_up(p, g["x"], w, r["offsets"], r["sorted_assign"], h)
        rec(3)
        M.moe_expert_down(p, w, r["offsets"], h, y_exp, ws)
        rec(4)
        M.moe_combine(p, r["probs"] if run.expert_choice else r["topk_w"], r["assign_row"],
                      r["offsets"], y_exp, y)
        rec(5)

    for _ in range(a.warmup):
        staged()
    torch.cuda.synchronize()
    for i in range(a.steps):
        staged(ev[i])
    torch.cuda.synchronize()
    stage_ms = {n: float(np.mean([ev[i][j].elapsed_time(ev[i][j + 1]) for i in range(a.steps)]))
                for j, n in enumerate(names)}
    up_ms = stage_ms["expert_up"]

    dn_ms = stage_ms["expert_down"]
    if decode:
        up_bytes = (touched * F1 * (run.d_model * wsz + (4 if run.w_fp8 else 0)) +
                    T * run.d_model * esz + rows * run.d_ff * 2)
        dn_bytes = touched * run.d_model * (run.d_ff * wsz + (4 if run.w_fp8 else 0))
        achieved = up_bytes / (up_ms * 1e-3) / 1e9
        roof = {"kernel": "decode_kernel (up)", "bound": "hbm", "achieved": round(achieved, 1),
                "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBPS, 4),
                "traffic": traffic_for("decode_kernel", name)}
        stage_frac = {"up": roof["frac"],
                      "down": round(dn_bytes / (dn_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4)}
    else:
        achieved = up_fl / (up_ms * 1e-3) / 1e12
        roof = {"kernel": "grouped_gemm_kernel (up)", "bound": "mfma",
                "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": traffic_for("grouped_gemm_kernel", name)}
        stage_frac = {"up": roof["frac"],
                      "down": round(down_fl / (dn_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}

    cpu = None
    if not a.no_cpu_baseline:
        cpu = cpu_baseline(run, cap, a.cpu_seconds, inp)

    step_tflops = step_flops / step_s / 1e12
    step_gbps = step_bytes / step_s / 1e9
    out = {
        "metric": METRIC,
        "value": round(T / step_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(step_s * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if run.dtype == "f32" else "bf16",
        "data": "synthetic (seeded; shapes and distributions of the workload, random weights)",
        "config": {"workload": run.description, "name": name, "T": T, "d_model": run.d_model,
                   "d_ff": run.d_ff, "num_experts": E, "top_k": k, "num_shared": run.num_shared,
                   "capacity": cap, "kept_rows": rows, "touched_experts": touched,
                   "parallelism": "single GPU"},
        "step_tflops": round(step_tflops, 2),
        "step_pct_bf16_peak": round(100 * step_tflops / PEAK_BF16_TFLOPS, 2),
        "step_gbps": round(step_gbps, 1),
        "step_pct_hbm": round(100 * step_gbps / PEAK_HBM_GBPS, 2),
        "stage_ms": {n: round(v, 5) for n, v in stage_ms.items()},
        "graph_ms_per_step": None if graph_ms is None else round(graph_ms, 5),
        "roofline": roof,
        "roofline_frac_by_projection": stage_frac,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out))


ALPHA = 0.01   # weight of L_aux in the training objective (the pages' usual value)


def bench_backward(a, name, run, p, w, g, ws, y, r):
    """One step = one moe_ffn_backward call over resident inputs: x, weights,
    the upstream gradient dy and the routing of one (untimed) forward call."""
    import numpy as np
    import torch

    from mixture_experts_sparse_gemv_amd import moe as M
    from synth import make_grad_output
    if run.dtype != "bf16" or run.w_fp8 or run.expert_choice:
        print(f"the backward pass supports bf16 token-choice problems; {name} is not one",
              file=sys.stderr)
        sys.exit(2)
    dev = g["x"].device
    T, E, k, S, d, f = run.T, run.num_experts, run.top_k, run.num_shared, run.d_model, run.d_ff
    F1 = 2 * f if run.activation == "swiglu" else f
    M.moe_ffn_forward(p, w, g["x"], y, ws, routing=r)
    dy = make_grad_output(run).to(dev)
    f32 = dict(dtype=torch.float32, device=dev)
    grads = dict(dx=torch.empty(T * d, **f32), dw_router=torch.empty(E * d, **f32),
                 dw_up=torch.empty((E + S) * F1 * d, **f32),
                 dw_down=torch.empty((E + S) * d * f, **f32))
    if run.router_bias != "none":
        grads["db_router"] = torch.empty(E, **f32)
    if run.expert_bias:
        grads["db_up"] = torch.empty((E + S) * f, **f32)
        grads["db_down"] = torch.empty((E + S) * d, **f32)
    bws = M.backward_workspace(p, dev)
    torch.cuda.synchronize()
    rows = int(r["offsets"][E].item()) + S * T
    for _ in range(a.warmup):
        M.moe_ffn_backward(p, w, g["x"], dy, ALPHA, r, grads, bws)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(a.steps + 1)]
    t0 = time.perf_counter()
    ev[0].record()
    for i in range(a.steps):
        M.moe_ffn_backward(p, w, g["x"], dy, ALPHA, r, grads, bws)
        ev[i + 1].record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    per = [ev[i].elapsed_time(ev[i + 1]) for i in range(a.steps)]
    step_s = float(np.median(per)) * 1e-3
    up_fl, dn_fl = expert_flops(run, rows)
    # dX and dW of both projections (twice the forward's expert flops), plus the
    # router's dlogits Wr and dlogits^T x; the recomputed pre-activations are not counted
    bwd_flops = 2.0 * (up_fl + dn_fl) + 4.0 * T * E * d
    achieved = bwd_flops / step_s / 1e12
    cpu = None if a.no_cpu_baseline else cpu_baseline_backward(run, a.cpu_seconds)
    out = {
        "metric": "MoE-FFN backward tokens/s + TFLOP/s (% bf16 MFMA peak), 1 MI355X",
        "value": round(T / step_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(step_s * 1e3, 5),
        "wall_ms_per_step": round((t1 - t0) * 1e3 / a.steps, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; shapes and distributions of the workload, random weights, "
                "dy ~ N(0, 1))",
        "config": {"workload": run.description + ", backward", "name": name, "T": T,
                   "d_model": d, "d_ff": f, "num_experts": E, "top_k": k, "num_shared": S,
                   "alpha": ALPHA, "rows": rows, "parallelism": "single GPU"},
        "step_tflops": round(achieved, 2),
        "step_pct_bf16_peak": round(100 * achieved / PEAK_BF16_TFLOPS, 2),
        "roofline": {"kernel": "moe_ffn_backward (whole pass)", "bound": "mfma",
                     "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": None},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out))


def cpu_baseline_backward(run, seconds):
    """The backward oracle on the first n <= 512 tokens of the workload (a
    batch of its own, same capacity factor), repeated for about `seconds`."""
    import oracle.moe_backward as OB
    from oracle import moe_oracle as O
    from synth import make_grad_output, make_inputs, scaled, to_f64
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count()
    n = min(run.T, 512)
    sub = scaled(run, T=n)
    inp, dy = make_inputs(sub), make_grad_output(sub).double().numpy()
    f64 = lambda t: None if t is None else _Lazy(t)
    cap = O.capacity(n, run.top_k, run.num_experts, run.capacity_factor)
    reps, t0 = 0, time.perf_counter()
    while True:
        OB.backward(to_f64(inp["x"]), to_f64(inp["w_router"]), to_f64(inp["b_router"]),
                    f64(inp["w_up"]), f64(inp["b_up"]), f64(inp["w_down"]), f64(inp["b_down"]),
                    dy, alpha=ALPHA, top_k=run.top_k, num_shared=run.num_shared,
                    gating=run.gating, activation=run.activation, cap=cap)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds or reps >= 50:
            break
    sample = f"oracle backward of a {n}-token batch of the workload, x{reps} repetitions in {el:.1f} s"
    return {"value": round(n * reps / el, 1), "unit": "tokens/s", "cores": threads,
            "kind": "oracle", "sample": sample}


def traffic_for(kernel, workload):
    """HBM bytes per launch measured by rocprofv3 counters (profiles/traffic.json),
    used only while the kernel's source is unchanged since the measurement."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        with open(path) as fh:
            db = json.load(fh)
        ent = db.get(f"{kernel}:{workload}")
        if not ent:
            return None
        src = os.path.join(ROOT, "mixture_experts_sparse_gemv_amd", "csrc", ent["source"])
        if source_digest(src) != ent["source_sha256"]:
            return None
        return ent["bytes_per_launch"]
    except Exception:
        return None


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(run, cap, seconds, inp):
    """The oracle's whole forward on the same workload (the same CPU input
    tensors), repeated until about `seconds` of host time have passed;
    tokens/s over the repetitions."""
    import numpy as np

    import oracle as O
    from synth import to_f64
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count()
    f64 = lambda t: None if t is None else _Lazy(t)
    # FP8 expert weights: the oracle's own quantization (codes computed once,
    # untimed, as the GPU path quantizes once), dequantized exactly per use
    if run.w_fp8:
        qup, qdown = _LazyFP8(inp["w_up"], O), _LazyFP8(inp["w_down"], O)
        f64w = lambda t: qup if t is inp["w_up"] else qdown
    else:
        f64w = f64
    x, wr = to_f64(inp["x"]), to_f64(inp["w_router"])
    br = None if inp["b_router"] is None else to_f64(inp["b_router"])
    ocap = O.capacity(run.T, run.top_k, run.num_experts, run.capacity_factor)
    # Bounded sample: at most 1024 tokens' expert FFNs per repetition (routing,
    # dispatch and aux statistics always cover the whole batch).
    sub = None if run.T <= 1024 else np.arange(1024)
    n_tok = run.T if sub is None else len(sub)
    reps, t0 = 0, time.perf_counter()
    while True:
        if run.expert_choice:
            O.forward_expert_choice(x, wr, br, f64w(inp["w_up"]), f64(inp["b_up"]),
                                    f64w(inp["w_down"]), f64(inp["b_down"]), capacity=ocap,
                                    num_shared=run.num_shared, gating=run.gating,
                                    activation=run.activation, token_subset=sub)
        else:
            O.forward(x, wr, br, f64w(inp["w_up"]), f64(inp["b_up"]), f64w(inp["w_down"]),
                      f64(inp["b_down"]), top_k=run.top_k, num_shared=run.num_shared,
                      gating=run.gating, activation=run.activation, cap=ocap, token_subset=sub)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds or reps >= 50:
            break
    sample = (f"float64 numpy oracle forward over the whole {run.T}-token batch (routing, "
              f"dispatch, aux) with expert FFNs for {n_tok} tokens, x{reps} repetitions in "
              f"{el:.1f} s, {threads} BLAS threads on {cpu_model()}")
    return {"value": round(n_tok * reps / el, 1), "unit": "tokens/s", "cores": threads,
            "kind": "oracle", "sample": sample}


class _Lazy:
    def __init__(self, t):
        self.t = t
        self.shape = tuple(t.shape)

    def __getitem__(self, i):
        return self.t[i].to(__import__("torch").float64).numpy()


class _LazyFP8(_Lazy):
    """The oracle's FP8 codes of every expert, computed once (several experts
    at a time); each access dequantizes one expert."""

    def __init__(self, t, oracle, workers=8):
        from concurrent.futures import ThreadPoolExecutor
        super().__init__(t)
        self.O = oracle
        torch = __import__("torch")
        one = lambda i: oracle.quantize_fp8_rows(t[i].to(torch.float32).numpy())
        with ThreadPoolExecutor(max_workers=workers) as ex:
            self.codes = list(ex.map(one, range(t.shape[0])))

    def __getitem__(self, i):
        return self.O.dequantize_fp8_rows(*self.codes[i])


if __name__ == "__main__":
    main()
