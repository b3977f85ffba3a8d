"""GPU parity of every step of the MoE-FFN forward against the float64 oracle,
through the C ABI.  Each test prints its case before the GPU work."""
import functools

import numpy as np
import pytest
import torch

import oracle as O
from mixture_experts_sparse_gemv_amd import moe as M
from synth import RUNS, make_inputs, scaled, to_f64

from _parity import (GAP, assert_close, check_dispatch_bitexact, compare_forward, gpu_inputs,
                     oracle_capacity, oracle_forward, problem_of, run_forward, weights_of)

pytestmark = pytest.mark.gpu

# Parity cases the oracle finishes in seconds: several tiles and a ragged tail.
SMALL = {
    "tiny": RUNS["tiny"],
    "gpt2_T700": scaled(RUNS["gpt2"], T=700),
    "gpt2_T700_cf1": scaled(RUNS["gpt2"], T=700, capacity_factor=1.0),
    "swiglu_skew_T3000": scaled(RUNS["swiglu_skew"], T=3000),
    "large_decode": RUNS["large_decode"],
    "large_T300": scaled(RUNS["large_prefill"], T=300),
    # bf16 widths that are multiples of 8 but not of 64 (the untiled grouped
    # GEMM, and the router's partial K step of 8, 16 or 24 elements)
    "gelu_bias_d776_f1416_T300": scaled(RUNS["gpt2"], T=300, d_model=776, d_ff=1416),
    "swiglu_d520_f2056_T200": scaled(RUNS["large_prefill"], T=200, d_model=520, d_ff=2056),
    "shared_sigmoid_d400_f328_T150": scaled(RUNS["fine_shared"], T=150, d_model=400, d_ff=328),
    "small_T12_d1048_f776": scaled(RUNS["large_prefill"], T=12, d_model=1048, d_ff=776),
    "relu_d64_f200_T500": scaled(RUNS["gpt2"], T=500, d_model=64, d_ff=200, activation="relu",
                                 capacity_factor=None),
    # the weight-streaming path with 2 and 4 groups of 16 token rows
    "decode_T40_d1024": scaled(RUNS["large_prefill"], T=40, d_model=1024, d_ff=2048),
    "decode_T64_shared_sigmoid": scaled(RUNS["fine_shared"], T=64, d_model=512, d_ff=768),
    # segments of more than 64 rows on the weight-streaming path (T <= 128):
    # two row passes, each streaming the weights again -- the skewed expert
    # takes nearly every token; the shared experts take all 100
    "decode_T128_skew_two_passes": scaled(RUNS["swiglu_skew"], T=128, top_k=2),
    "decode_T100_shared_two_passes": scaled(RUNS["fine_shared"], T=100, d_model=512, d_ff=768),
    "fine_shared_T1000": scaled(RUNS["fine_shared"], T=1000),
    "fine_shared_T1000_literal": scaled(RUNS["fine_shared"], T=1000, capacity_factor=1.25 / 6),
    # more than 64 16-token router blocks (8 waves each, not 16) with 64
    # experts and 2 shared ones, at a width the oracle finishes quickly
    "fine_shared_T1100_d256": scaled(RUNS["fine_shared"], T=1100, d_model=256, d_ff=128),
    # 64 experts of 683..1278 rows: exactly 256 full m-tiles and 35 half-empty
    # ones, so both grouped GEMMs take the two-list tile schedule (checked on
    # the oracle's routing in test_split_lists_case_takes_two_lists)
    "relu_E64_T16384_split_lists": scaled(RUNS["gpt2"], T=16384, d_model=256, d_ff=128,
                                          num_experts=64, top_k=4, activation="relu",
                                          capacity_factor=None),
}


@functools.lru_cache(maxsize=None)
def _inputs(name):
    run = SMALL.get(name) or RUNS[name]
    return run, make_inputs(run)


@functools.lru_cache(maxsize=None)
def _oracle(name):
    run, inp = _inputs(name)
    return oracle_forward(run, inp)


def _say(*a):
    print(*a, flush=True)


@pytest.mark.parametrize("name", list(SMALL))
def test_forward_small(name):
    run, inp = _inputs(name)
    _say(f"[forward] {name}: T={run.T} d={run.d_model} f={run.d_ff} E={run.num_experts} "
         f"k={run.top_k} S={run.num_shared} seed={run.seed}")
    g = gpu_inputs(inp)
    gpu = run_forward(run, g)
    compare_forward(run, gpu, _oracle(name), inp)


@pytest.mark.parametrize("name", list(SMALL))
def test_router_topk(name):
    run, inp = _inputs(name)
    _say(f"[router_topk] {name}")
    g = gpu_inputs(inp)
    p = problem_of(run)
    T, k, E = run.T, run.top_k, run.num_experts
    idx = torch.empty(T * k, dtype=torch.int32, device="cuda")
    w = torch.empty(T * k, dtype=torch.float32, device="cuda")
    probs = torch.empty(T * E, dtype=torch.float32, device="cuda")
    colsum = torch.empty(E, dtype=torch.float32, device="cuda")
    M.moe_router_topk(p, g["x"], weights_of(g), idx, w, probs, colsum, ws=M.workspace(p))
    torch.cuda.synchronize()
    logits = O.router_logits(to_f64(inp["x"]), to_f64(inp["w_router"]), to_f64(inp["b_router"]))
    pr = O.gate(logits, run.gating)
    oi, ow = O.topk_renorm(pr, k)
    gi = idx.view(T, k).cpu().numpy()
    gap = O.selection_gap(pr, k)
    same = np.all(np.sort(gi, 1) == np.sort(oi, 1), axis=1)
    assert np.all(same | (gap <= GAP))
    ex = np.all(gi == oi, axis=1)
    assert_close(w.view(T, k).cpu().numpy()[ex], ow[ex], "topk_w")
    assert_close(probs.view(T, E).cpu().numpy(), pr, "probs")
    assert_close(colsum.cpu().numpy(), pr.sum(0), "colsum", rel=1e-4, mabs=1e-2)


# Exact ties between experts: router rows duplicated in groups, so the
# duplicated experts' logits are equal in any precision; the selection must
# then take the lower expert index first (top-k with ties to the lower
# index, renormalized weights), on both top-k paths of the router kernel
# (up to 16 experts: a rank count over all experts; more: k extractions of
# the largest remaining logit at its lowest index).
TIE_CASES = {
    "E8_top2_softmax": (scaled(RUNS["gpt2"], T=300, d_model=256, d_ff=256, router_bias="none"),
                        [(0, 1), (2, 5), (3, 4, 7)]),
    "E64_top6_sigmoid": (scaled(RUNS["fine_shared"], T=300, d_model=256, d_ff=128,
                                router_bias="none"),
                         [(2 * q, 2 * q + 1) for q in range(24)] + [(50, 51, 52, 60)]),
}


@pytest.mark.parametrize("name", list(TIE_CASES))
def test_router_ties_to_lower_index(name):
    run, groups = TIE_CASES[name]
    _say(f"[router ties] {name}")
    inp = dict(make_inputs(run))
    wr = inp["w_router"].clone()
    for grp in groups:
        for e in grp[1:]:
            wr[e] = wr[grp[0]]
    inp["w_router"] = wr
    g = gpu_inputs(inp)
    p = problem_of(run)
    T, k, E = run.T, run.top_k, run.num_experts
    idx = torch.empty(T * k, dtype=torch.int32, device="cuda")
    w = torch.empty(T * k, dtype=torch.float32, device="cuda")
    M.moe_router_topk(p, g["x"], weights_of(g), idx, w, ws=M.workspace(p))
    torch.cuda.synchronize()
    logits = O.router_logits(to_f64(inp["x"]), to_f64(wr), None)
    pr = O.gate(logits, run.gating)
    oi, ow = O.topk_renorm(pr, k)
    gi = idx.view(T, k).cpu().numpy()
    # tokens whose top k+1 scores are exactly tied or clearly apart
    top = -np.sort(-pr, axis=1)[:, :k + 1]
    d = top[:, :-1] - top[:, 1:]
    clear = np.all((d == 0) | (d > GAP), axis=1)
    tied = np.any(d[clear] == 0, axis=1)
    _say(f"  tokens compared {clear.sum()} of {T}, with an exact tie among them {tied.sum()}")
    assert clear.sum() >= T // 2 and tied.sum() >= 20
    assert np.array_equal(gi[clear], oi[clear])
    assert_close(w.view(T, k).cpu().numpy()[clear], ow[clear], "topk_w")


def _dispatch_cases():
    rng = np.random.default_rng(123)
    cases = []
    for name in ("gpt2_T700", "fine_shared_T1000"):
        run = SMALL[name]
        cases.append((name, run.T, run.top_k, run.num_experts, None))
    # synthetic routings: skewed, all to one expert, many experts, > 64K assignments
    def rand_idx(T, k, E, skew):
        p = np.arange(E, 0, -1, dtype=np.float64) ** skew
        p /= p.sum()
        out = np.empty((T, k), dtype=np.int32)
        for t in range(T):
            out[t] = rng.choice(E, size=k, replace=False, p=p)
        return out
    cases.append(("skew_E64_k6", 3000, 6, 64, rand_idx(3000, 6, 64, 2.0)))
    cases.append(("uniform_E8_k2", 4096, 2, 8, rand_idx(4096, 2, 8, 0.0)))
    cases.append(("one_expert", 777, 1, 5, np.full((777, 1), 3, dtype=np.int32)))
    big = rand_idx(20000, 4, 16, 1.0)
    cases.append(("segments_80000", 20000, 4, 16, big))
    return cases


@pytest.mark.parametrize("case", _dispatch_cases(), ids=lambda c: c[0])
@pytest.mark.parametrize("cap_mode", ["none", "cf1.25", "cf1.0", "tight"])
def test_dispatch_bitexact(case, cap_mode):
    name, T, k, E, idx = case
    if idx is None:
        run, inp = _inputs(name)
        pr = O.gate(O.router_logits(to_f64(inp["x"]), to_f64(inp["w_router"]),
                                    to_f64(inp["b_router"])), run.gating)
        idx, _ = O.topk_renorm(pr, k)
    cap = {"none": None, "cf1.25": O.capacity(T, k, E, 1.25), "cf1.0": O.capacity(T, k, E, 1.0),
           "tight": 1}[cap_mode]
    _say(f"[dispatch] {name} T={T} k={k} E={E} cap={cap}")
    orc = O.dispatch(idx, E, cap)
    p = M.make_problem(T=T, d_model=64, d_ff=64, num_experts=E, top_k=k, capacity=cap or 0)
    n = T * k
    i32 = dict(dtype=torch.int32, device="cuda")
    out = dict(counts=torch.empty(E, **i32), kept=torch.empty(E, **i32),
               offsets=torch.empty(E + 1, **i32), sorted_assign=torch.empty(n, **i32),
               assign_row=torch.empty(n, **i32),
               drop_mask=torch.empty(n, dtype=torch.uint8, device="cuda"))
    M.moe_dispatch(p, torch.from_numpy(idx.reshape(-1).astype(np.int32)).cuda(), **out,
                   ws=M.workspace(p))
    torch.cuda.synchronize()
    check_dispatch_bitexact({k_: v.cpu().numpy() for k_, v in out.items()}, orc, E)


@pytest.mark.parametrize("name", list(SMALL))
def test_expert_ffn_and_combine_given_oracle_routing(name):
    run, inp = _inputs(name)
    _say(f"[expert_ffn+combine] {name}")
    g = gpu_inputs(inp)
    p = problem_of(run)
    orc = _oracle(name)
    T, k, d = run.T, run.top_k, run.d_model
    dev = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a).astype(dt)).cuda()
    offsets = dev(orc["offsets"], np.int32)
    sorted_assign = dev(orc["sorted_assign"], np.int32)
    assign_row = dev(orc["assign_row"], np.int32)
    topk_w = dev(orc["w"].reshape(-1), np.float32)
    ws = M.workspace(p)
    y_exp = torch.empty(M.max_rows(p) * d, dtype=torch.float32, device="cuda")
    M.moe_expert_ffn(p, g["x"], weights_of(g), offsets, sorted_assign, y_exp, ws)
    y = torch.empty(T * d, dtype=torch.float32, device="cuda")
    M.moe_combine(p, topk_w, assign_row, offsets, y_exp, y)
    torch.cuda.synchronize()
    assert_close(y.view(T, d).cpu().numpy(), orc["y"], "y")


def test_aux_stats_given_oracle_sums():
    run, inp = _inputs("fine_shared_T1000")
    _say("[aux_stats] fine_shared_T1000")
    orc = _oracle("fine_shared_T1000")
    p = problem_of(run)
    E = run.num_experts
    colsum = torch.from_numpy(orc["probs"].sum(0).astype(np.float32)).cuda()
    counts = torch.from_numpy(orc["counts"].astype(np.int32)).cuda()
    f = torch.empty(E, device="cuda")
    P = torch.empty(E, device="cuda")
    l = torch.empty(1, device="cuda")
    M.moe_aux_stats(p, colsum, counts, f, P, l)
    torch.cuda.synchronize()
    np.testing.assert_allclose(f.cpu().numpy(), orc["f"], rtol=1e-6)
    np.testing.assert_allclose(P.cpu().numpy(), orc["P"], rtol=1e-5)
    assert abs(float(l.item()) - orc["l_aux"]) <= 1e-4 * orc["l_aux"]


@pytest.mark.parametrize("name", ["fine_shared_T1000", "shared_sigmoid_d400_f328_T150"])
def test_deterministic_and_no_out_of_bounds_writes(name):
    run, inp = _inputs(name)
    _say(f"[determinism+canary] {name}")
    g = gpu_inputs(inp)
    p = problem_of(run)
    T, d = run.T, run.d_model
    pad = 4096
    ys = []
    for rep in range(2):
        y = torch.full((T * d + 2 * pad,), float("nan"), device="cuda")
        ws = M.workspace(p)
        M.moe_ffn_forward(p, weights_of(g), g["x"], y[pad:pad + T * d], ws)
        torch.cuda.synchronize()
        yy = y.cpu().numpy()
        assert np.all(np.isnan(yy[:pad])) and np.all(np.isnan(yy[-pad:])), "write outside y"
        assert np.all(np.isfinite(yy[pad:-pad]))
        ys.append(yy[pad:-pad].copy())
    assert np.array_equal(ys[0].view(np.uint32), ys[1].view(np.uint32)), "not bit-identical"


@pytest.mark.parametrize("name", ["gpt2_T700", "swiglu_skew_T3000", "large_T300", "large_decode",
                                  "gelu_bias_d776_f1416_T300"])
def test_stage_entry_points_equal_fused_forward(name):
    """The per-stage entry points (router, dispatch, up, down with its K slices
    folded, combine) give bit-identical y to the fused forward, which adds the
    down projection's K slices inside the combine."""
    run, inp = _inputs(name)
    _say(f"[staged==forward] {name}")
    g = gpu_inputs(inp)
    p = problem_of(run)
    T, k, E, d = run.T, run.top_k, run.num_experts, run.d_model
    fwd = run_forward(run, g, p)
    ws = M.workspace(p)
    i32 = dict(dtype=torch.int32, device="cuda")
    idx, tw = torch.empty(T * k, **i32), torch.empty(T * k, device="cuda")
    cnt, kept, off = torch.empty(E, **i32), torch.empty(E, **i32), torch.empty(E + 1, **i32)
    sa, ar = torch.empty(T * k, **i32), torch.empty(T * k, **i32)
    dm = torch.empty(T * k, dtype=torch.uint8, device="cuda")
    w = weights_of(g)
    M.moe_router_topk(p, g["x"], w, idx, tw, ws=ws)
    M.moe_dispatch(p, idx, cnt, kept, off, sa, ar, dm, ws=ws)
    h = torch.empty(M.max_rows(p) * run.d_ff, dtype=M.h_dtype(p), device="cuda")
    y_exp = torch.empty(M.max_rows(p) * d, device="cuda")
    M.moe_expert_up(p, g["x"], w, off, sa, h)
    M.moe_expert_down(p, w, off, h, y_exp, ws)
    y = torch.empty(T * d, device="cuda")
    M.moe_combine(p, tw, ar, off, y_exp, y)
    torch.cuda.synchronize()
    ys = y.view(T, d).cpu().numpy()
    assert np.array_equal(ys.view(np.uint32), fwd["y"].view(np.uint32)), "staged != forward"


def test_routing_stats_entry_point_given_oracle_inputs():
    from _parity import check_route_stats
    _say("[routing_stats] synthetic counts, drops and idle experts")
    rng = np.random.default_rng(11)
    for E in (1, 4, 8, 64):
        counts = rng.integers(0, 400, size=E)
        if E > 2:
            counts[1] = 0
        kept = np.minimum(counts, 250)
        Pv = rng.random(E)
        Pv /= Pv.sum()
        ref = O.routing_stats(counts, kept, Pv)
        p = M.make_problem(T=int(counts.sum()) + 1, d_model=64, d_ff=64, num_experts=E, top_k=1)
        st = M.route_stats_tensor()
        M.moe_routing_stats(p, torch.tensor(counts, dtype=torch.int32, device="cuda"),
                            torch.tensor(kept, dtype=torch.int32, device="cuda"),
                            torch.tensor(Pv, dtype=torch.float32, device="cuda"), st)
        torch.cuda.synchronize()
        check_route_stats(M.route_stats_dict(st), ref)


# Activations far beyond fp16's range: x drawn with std 128 (256 for the
# 16-token case, which has fewer rows to reach the tail), so that the SwiGLU
# intermediate silu(x Wg) * (x Wu) reaches |h| above 65504 (checked on the
# oracle's side below); the grouped GEMM path (T = 300) and the decode path
# (T = 16).  y then reaches about 1e4, so the absolute bound is taken
# relative to max |y|: 2e-3 max |y_ref| (the runs at the workloads' scale
# have max |y| of about 10 against the 2e-2 bound).
LARGE_H = {
    "swiglu_T300_x128": scaled(RUNS["large_prefill"], T=300, d_model=1024, d_ff=1024,
                               x_std=128.0, seed=31),
    "swiglu_decode_T16_x256": scaled(RUNS["large_prefill"], T=16, d_model=1024, d_ff=1024,
                                     x_std=256.0, seed=32),
}


@pytest.mark.parametrize("name", list(LARGE_H))
def test_forward_h_beyond_fp16_range(name):
    run = LARGE_H[name]
    _say(f"[forward large h] {name}: T={run.T} d={run.d_model} f={run.d_ff} x_std={run.x_std}")
    inp = make_inputs(run)
    g = gpu_inputs(inp)
    gpu = run_forward(run, g)
    orc = oracle_forward(run, inp, idx=gpu["topk_idx"].reshape(run.T, run.top_k))
    # the case exercises what it is for: |h| beyond 65504 on the selected rows
    x = to_f64(inp["x"])
    hmax = 0.0
    for e in range(run.num_experts):
        rows = orc["sorted_assign"][orc["offsets"][e]:orc["offsets"][e + 1]] // run.top_k
        if rows.size:
            z = x[rows] @ inp["w_up"][e].to(torch.float64).numpy().T
            hmax = max(hmax, float(np.abs(O.silu(z[:, :run.d_ff]) * z[:, run.d_ff:]).max()))
    _say(f"  max |h| = {hmax:.3e}")
    assert hmax > 65504.0
    check_dispatch_bitexact(gpu, orc, run.num_experts)
    ymax = float(np.abs(orc["y"]).max())
    assert_close(gpu["y"], orc["y"], "y", mabs=2e-3 * ymax)
