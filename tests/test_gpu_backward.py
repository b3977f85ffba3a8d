"""GPU parity of the backward pass (moe_ffn_backward, through the C ABI)
against the float64 backward oracle, evaluated at the GPU forward's top-k
selection.  Each test prints its case before the GPU work.

Tolerance of every gradient G (float32 out, bf16 operands, fp32
accumulation; dy, h and dZ are rounded to bf16 as MFMA operands, a relative
error of at most 2^-9 each): relative Frobenius error <= 1e-2 and maximum
absolute error <= 2e-2 * max|G_ref| (gradients carry the scale of dy, so
the absolute bound is taken relative to the largest reference entry)."""
import functools

import numpy as np
import pytest
import torch

from oracle import moe_backward as OB
from mixture_experts_sparse_gemv_amd import moe as M
from synth import RUNS, make_grad_output, make_inputs, scaled, to_f64

from _parity import (REL_FROB, gpu_inputs, oracle_capacity, problem_of, routing_outputs,
                     weights_of)

pytestmark = pytest.mark.gpu

MAX_ABS_REL = 2e-2

# name: (run, alpha)
CASES = {
    "gpt2_T700": (scaled(RUNS["gpt2"], T=700), 0.01),
    "gpt2_T700_cf1_drops": (scaled(RUNS["gpt2"], T=700, capacity_factor=1.0), 0.3),
    "swiglu_skew_T3000": (scaled(RUNS["swiglu_skew"], T=3000), 0.01),
    "fine_shared_T1000_d512": (scaled(RUNS["fine_shared"], T=1000, d_model=512, d_ff=384), 0.1),
    "decode_T16_d1024": (scaled(RUNS["large_decode"], d_model=1024, d_ff=2048), 0.01),
    "relu_T333": (scaled(RUNS["gpt2"], T=333, d_model=256, d_ff=512, activation="relu",
                         capacity_factor=1.0), 0.05),
    # edge cases: one token; one expert; every expert selected; capacity 1
    "one_token": (scaled(RUNS["gpt2"], T=1, d_model=256, d_ff=512), 0.1),
    "single_expert": (scaled(RUNS["swiglu_skew"], T=100, d_model=256, d_ff=256, num_experts=1),
                      0.1),
    "all_experts": (scaled(RUNS["gpt2"], T=200, d_model=256, d_ff=256, top_k=8), 0.1),
    "capacity_one": (scaled(RUNS["gpt2"], T=300, d_model=256, d_ff=256, capacity_factor=0.01),
                     0.1),
    # long shared-expert reductions (4500 rows each) next to short routed ones
    "fine_shared_T4500": (scaled(RUNS["fine_shared"], T=4500, d_model=256, d_ff=128), 0.01),
}


class LazyF64:
    def __init__(self, t):
        self.t = t
        self.shape = tuple(t.shape)

    def __getitem__(self, i):
        return self.t[i].to(torch.float64).numpy()


def grad_outputs(p, run, device="cuda"):
    f32 = dict(dtype=torch.float32, device=device)
    E, S, d, f = run.num_experts, run.num_shared, run.d_model, run.d_ff
    F1 = 2 * f if run.activation == "swiglu" else f
    g = dict(dx=torch.empty(run.T * d, **f32), dw_router=torch.empty(E * d, **f32),
             db_router=torch.empty(E, **f32), dw_up=torch.empty((E + S) * F1 * d, **f32),
             dw_down=torch.empty((E + S) * d * f, **f32),
             d_topk_w=torch.empty(run.T * run.top_k, **f32),
             d_logits=torch.empty(run.T * E, **f32))
    if run.expert_bias:
        g["db_up"] = torch.empty((E + S) * f, **f32)
        g["db_down"] = torch.empty((E + S) * d, **f32)
    return g


def run_gpu(run, alpha, inp, dy):
    p = problem_of(run)
    g = gpu_inputs(inp)
    w = weights_of(g)
    r = routing_outputs(p)
    y = torch.empty(run.T * run.d_model, dtype=torch.float32, device="cuda")
    M.moe_ffn_forward(p, w, g["x"], y, M.workspace(p), routing=r)
    grads = grad_outputs(p, run)
    ws = M.backward_workspace(p)
    dyg = dy.cuda()
    M.moe_ffn_backward(p, w, g["x"], dyg, alpha, r, grads, ws)
    torch.cuda.synchronize()
    out = {k: v.cpu().numpy() for k, v in grads.items()}
    # a second call must give bit-identical gradients (fixed reduction orders)
    grads2 = grad_outputs(p, run)
    M.moe_ffn_backward(p, w, g["x"], dyg, alpha, r, grads2, ws)
    torch.cuda.synchronize()
    for k, v in grads2.items():
        assert np.array_equal(v.cpu().numpy(), out[k]), f"{k} not deterministic"
    out["topk_idx"] = r["topk_idx"].cpu().numpy()
    return out


def assert_grad_close(got, ref, name):
    got = np.asarray(got, dtype=np.float64).reshape(ref.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    diff = got - ref
    nref = np.linalg.norm(ref)
    rf = np.linalg.norm(diff) / (nref if nref > 0 else 1.0)
    scale = float(np.abs(ref).max()) if ref.size else 0.0
    ma = float(np.abs(diff).max()) if diff.size else 0.0
    print(f"  {name}: rel_frob={rf:.3e} max_abs={ma:.3e} (max|ref|={scale:.3e})", flush=True)
    if nref == 0:
        assert ma == 0.0, f"{name}: reference is zero, got max {ma}"
        return
    assert rf <= REL_FROB, f"{name}: relative Frobenius error {rf:.3e} > {REL_FROB}"
    assert ma <= MAX_ABS_REL * scale, f"{name}: max abs error {ma:.3e} > {MAX_ABS_REL} * {scale:.3e}"


@functools.lru_cache(maxsize=None)
def _case(name):
    run, alpha = CASES[name]
    return run, alpha, make_inputs(run), make_grad_output(run)


@pytest.mark.parametrize("name", list(CASES))
def test_backward_parity(name):
    run, alpha, inp, dy = _case(name)
    print(f"case {name}: T={run.T} d={run.d_model} f={run.d_ff} E={run.num_experts} "
          f"k={run.top_k} S={run.num_shared} {run.gating} {run.activation} alpha={alpha}",
          flush=True)
    gpu = run_gpu(run, alpha, inp, dy)
    lazy = lambda t: None if t is None else LazyF64(t)
    ref = OB.backward(to_f64(inp["x"]), to_f64(inp["w_router"]), to_f64(inp["b_router"]),
                      lazy(inp["w_up"]), lazy(inp["b_up"]), lazy(inp["w_down"]),
                      lazy(inp["b_down"]), dy.double().numpy(), alpha=alpha, top_k=run.top_k,
                      num_shared=run.num_shared, gating=run.gating, activation=run.activation,
                      cap=oracle_capacity(run), idx=gpu["topk_idx"].reshape(run.T, run.top_k))
    assert_grad_close(gpu["d_topk_w"], ref["dw"], "d_topk_w")
    assert_grad_close(gpu["d_logits"], ref["dlogits"], "d_logits")
    assert_grad_close(gpu["dx"], ref["dx"], "dx")
    assert_grad_close(gpu["dw_router"], ref["dw_router"], "dw_router")
    if run.router_bias != "none":
        assert_grad_close(gpu["db_router"], ref["db_router"], "db_router")
    assert_grad_close(gpu["dw_up"], ref["dw_up"], "dw_up")
    assert_grad_close(gpu["dw_down"], ref["dw_down"], "dw_down")
    if run.expert_bias:
        assert_grad_close(gpu["db_up"], ref["db_up"], "db_up")
        assert_grad_close(gpu["db_down"], ref["db_down"], "db_down")
    # experts that received no rows have exactly zero weight gradients
    counts = np.bincount(gpu["topk_idx"], minlength=run.num_experts)
    F1 = 2 * run.d_ff if run.activation == "swiglu" else run.d_ff
    dwu = gpu["dw_up"].reshape(-1, F1, run.d_model)
    for e in np.nonzero(counts == 0)[0]:
        assert np.all(dwu[e] == 0.0)


def test_backward_validation():
    """Unsupported problems and missing arguments are rejected before any launch."""
    print("case backward validation", flush=True)
    run = scaled(RUNS["gpt2"], T=64)
    p = problem_of(run)
    with pytest.raises(M.MoeError, match="UNSUPPORTED"):
        M.moe_backward_workspace_size(problem_of(RUNS["tiny"]))   # float32 problem
    with pytest.raises(M.MoeError, match="UNSUPPORTED"):
        M.moe_backward_workspace_size(problem_of(RUNS["gpt2_ec"]))
    g = gpu_inputs(make_inputs(run))
    r = routing_outputs(p)
    grads = grad_outputs(p, run)
    dy = make_grad_output(run).cuda()
    ws = M.backward_workspace(p)
    for missing in ("dx", "dw_up", "db_up"):
        bad = {k: v for k, v in grads.items() if k != missing}
        with pytest.raises(M.MoeError, match="INVALID_ARG"):
            M.moe_ffn_backward(p, weights_of(g), g["x"], dy, 0.01, r, bad, ws)
    with pytest.raises(M.MoeError, match="WORKSPACE"):
        M.moe_ffn_backward(p, weights_of(g), g["x"], dy, 0.01, r, grads, ws[:1024])
    r2 = {k: v for k, v in r.items() if k != "assign_row"}
    with pytest.raises(M.MoeError, match="INVALID_ARG"):
        M.moe_ffn_backward(p, weights_of(g), g["x"], dy, 0.01, r2, grads, ws)
