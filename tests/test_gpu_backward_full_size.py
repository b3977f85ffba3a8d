"""GPU parity of the backward pass at the full workload sizes, in the launch
configuration `bench.py --pass backward` times (alpha 0.01, the workload's
capacity), against the float64 backward oracle at the GPU forward's top-k
selection.

gpt2: every gradient against the whole oracle backward.  The large
workloads: sampled entries the oracle computes one by one (a token's dx,
slot-weight and logit gradients; a row of dW1 with its bias gradient and a
column of dW2 of chosen experts), with the tolerances of the small-size
backward tests applied to each sampled vector, except for two quantities
whose single entries carry a cancellation:

* the slot weight's gradient dw = <dy, out> sums d_model terms of both
  signs; the GPU forms it from dy rounded to bf16 (relative error at most
  2^-9 per element), so its error bound is 2^-9 * sum_j |dy_j out_j| (the
  test allows twice that, plus 1e-4 |dw| for the fp32 sums);
* the logits' gradient takes differences of the slots' dw (renormalized
  top-k), so it is checked against the oracle's router backward evaluated
  at the GPU's own dw (relative 1e-3): that isolates the router arithmetic,
  while the whole-tensor checks at gpt2 size cover the combination."""
import numpy as np
import pytest
import torch

from oracle import moe_backward as OB
from oracle import moe_oracle as O
from mixture_experts_sparse_gemv_amd import moe as M
from synth import RUNS, make_grad_output, make_inputs, to_f64

from _parity import gpu_inputs, oracle_capacity, problem_of, routing_outputs, weights_of
from test_gpu_backward import assert_grad_close, grad_outputs

pytestmark = pytest.mark.gpu

ALPHA = 0.01


class CachedF64:
    """Per-expert float64 views of a [n, rows, K] tensor, the last two kept."""

    def __init__(self, t):
        self.t = t
        self.shape = tuple(t.shape)
        self.cache = {}

    def __getitem__(self, i):
        if i not in self.cache:
            if len(self.cache) >= 2:
                self.cache.pop(next(iter(self.cache)))
            self.cache[i] = self.t[i].to(torch.float64).numpy()
        return self.cache[i]


def run_gpu(run, inp, dy):
    p = problem_of(run)
    g = gpu_inputs(inp)
    w = weights_of(g)
    r = routing_outputs(p)
    y = torch.empty(run.T * run.d_model, dtype=torch.float32, device="cuda")
    M.moe_ffn_forward(p, w, g["x"], y, M.workspace(p), routing=r)
    grads = grad_outputs(p, run)
    M.moe_ffn_backward(p, w, g["x"], dy.cuda(), ALPHA, r, grads, M.backward_workspace(p))
    torch.cuda.synchronize()
    del g, w
    return r, grads


def test_backward_full_gpt2():
    run = RUNS["gpt2"]
    print(f"case backward full size gpt2: T={run.T} d={run.d_model} f={run.d_ff}", flush=True)
    inp, dy = make_inputs(run), make_grad_output(run)
    r, grads = run_gpu(run, inp, dy)
    f64 = lambda t: None if t is None else to_f64(t)
    ref = OB.backward(f64(inp["x"]), f64(inp["w_router"]), f64(inp["b_router"]), f64(inp["w_up"]),
                      f64(inp["b_up"]), f64(inp["w_down"]), f64(inp["b_down"]),
                      dy.double().numpy(), alpha=ALPHA, top_k=run.top_k,
                      num_shared=run.num_shared, gating=run.gating, activation=run.activation,
                      cap=oracle_capacity(run),
                      idx=r["topk_idx"].cpu().numpy().reshape(run.T, run.top_k))
    for name, rname in (("d_topk_w", "dw"), ("d_logits", "dlogits"), ("dx", "dx"),
                        ("dw_router", "dw_router"), ("db_router", "db_router"),
                        ("dw_up", "dw_up"), ("db_up", "db_up"), ("dw_down", "dw_down"),
                        ("db_down", "db_down")):
        assert_grad_close(grads[name].cpu().numpy(), ref[rname], name)


SAMPLED = {
    "large_prefill": dict(tokens=(0, 4095, 8191), segs=(0, 5)),
    "fine_shared": dict(tokens=(0, 3000, 8191), segs=(0, 63, 64)),
    "large_decode": dict(tokens=(0, 7, 15), segs=None),
}


@pytest.mark.parametrize("name", list(SAMPLED))
def test_backward_full_size_sampled(name):
    run = RUNS[name]
    spec = SAMPLED[name]
    print(f"case backward full size {name}: T={run.T} d={run.d_model} f={run.d_ff} "
          f"E={run.num_experts} k={run.top_k} S={run.num_shared}", flush=True)
    inp, dy = make_inputs(run), make_grad_output(run)
    r, grads = run_gpu(run, inp, dy)
    T, k, E, S, f = run.T, run.top_k, run.num_experts, run.num_shared, run.d_ff
    F1 = 2 * f if run.activation == "swiglu" else f
    idx = r["topk_idx"].cpu().numpy().reshape(T, k).astype(np.int64)
    disp = O.dispatch(idx, E, oracle_capacity(run))
    assert np.array_equal(disp["offsets"], r["offsets"].cpu().numpy())
    kept = disp["assign_row"].reshape(T, k) >= 0
    x, dyd = to_f64(inp["x"]), dy.double().numpy()
    wr, br = to_f64(inp["w_router"]), to_f64(inp["b_router"])
    w_up, w_down = CachedF64(inp["w_up"]), CachedF64(inp["w_down"])
    b_up = None if inp["b_up"] is None else CachedF64(inp["b_up"])
    b_down = None if inp["b_down"] is None else CachedF64(inp["b_down"])
    probs, keys = OB.gate_keys(O.router_logits(x, wr, br), run.gating)
    sel = np.take_along_axis(keys, idx, axis=1)
    topw = sel / sel.sum(axis=1, keepdims=True)

    gx = grads["dx"].view(T, -1)
    gw = grads["d_topk_w"].view(T, k)
    gl = grads["d_logits"].view(T, E)
    for t in spec["tokens"]:
        ref = OB.backward_token(t, x, wr, br, w_up, b_up, w_down, b_down, dyd, alpha=ALPHA,
                                top_k=k, num_shared=S, gating=run.gating,
                                activation=run.activation, idx=idx, kept_slots=kept[t],
                                counts=disp["counts"])
        assert_grad_close(gx[t].cpu().numpy(), ref["dx"], f"dx[{t}]")
        dw_gpu = gw[t].cpu().numpy().astype(np.float64)
        bound = 2.0 * 2.0 ** -9 * ref["dw_scale"] + 1e-4 * np.abs(ref["dw"]) + 1e-6
        err = np.abs(dw_gpu - ref["dw"])
        print(f"  d_topk_w[{t}]: err={err} bound={bound}", flush=True)
        assert np.all(err <= bound), f"d_topk_w[{t}] outside the bf16-dy bound"
        rr = OB.router_backward_token(t, x, wr, br, alpha=ALPHA, top_k=k, gating=run.gating,
                                      idx=idx, counts=disp["counts"], dw=dw_gpu)
        assert_grad_close(gl[t].cpu().numpy(), rr["dlogits"], f"d_logits[{t}] at the GPU's dw")
        rf = (np.linalg.norm(gl[t].cpu().numpy() - rr["dlogits"]) /
              max(np.linalg.norm(rr["dlogits"]), 1e-30))
        assert rf <= 1e-3, f"router backward of token {t}: {rf:.2e}"

    segs = spec["segs"]
    if segs is None:   # the experts the selection touches most
        segs = tuple(int(e) for e in np.argsort(-disp["kept"], kind="stable")[:2])
    dwu = grads["dw_up"].view(E + S, F1, run.d_model)
    dwd = grads["dw_down"].view(E + S, run.d_model, f)
    for seg in segs:
        for n in (0, F1 - 1):
            ref = OB.backward_weight_entries(seg, n, x, w_up, b_up, w_down, b_down, dyd,
                                             activation=run.activation, top_k=k, disp=disp,
                                             topk_weights=topw)
            assert_grad_close(dwu[seg, n].cpu().numpy(), ref["dw_up_row"], f"dw_up[{seg}][{n}]")
            assert_grad_close(dwd[seg, :, ref["col"]].cpu().numpy(), ref["dw_down_col"],
                              f"dw_down[{seg}][:, {ref['col']}]")
