"""GPU parity of the forward (and, for bf16 token choice, the backward) on a
seeded sweep of small, irregular layer shapes: token counts around the
decode bounds and the 256-row tile (1, 5, 16, 17, 65, 128, 129, 255, 257,
...), widths
that leave partial 256- and 128-column tiles, one to 64 experts with odd
counts, top-k up to 8, shared experts, both gates, every activation with and
without biases, and capacities from unlimited to tight.  Each case is drawn
from its own seed, prints its shape first, and is compared with the float64
oracle under the same rules as the fixed parity cases."""
import functools
import random

import numpy as np
import pytest
import torch

from oracle import moe_backward as OB
from mixture_experts_sparse_gemv_amd import moe as M
from synth import RUNS, make_grad_output, make_inputs, scaled, to_f64

from _parity import (compare_forward, gpu_inputs, oracle_capacity, oracle_forward, problem_of,
                     run_forward, weights_of, routing_outputs)
from test_gpu_backward import LazyF64, assert_grad_close, grad_outputs

N_CASES = 36


def _draw(i):
    rng = random.Random(1000 + i)
    dtype = "f32" if i % 8 == 7 else "bf16"
    T = rng.choice([1, 5, 16, 17, 33, 63, 64, 65, 200, 255, 257, 513, 777])
    if i >= 24:   # around the streaming path's bound (row passes of 64 above T = 64)
        T = rng.choice([65, 96, 127, 128, 129, 160])
    if dtype == "bf16":
        d = rng.choice([64, 128, 192, 320, 512])
        f = rng.choice([64, 128, 192, 448, 640])
    else:
        d = rng.choice([8, 24, 40])
        f = rng.choice([8, 16, 56])
    E = rng.choice([1, 2, 3, 5, 8, 13, 16, 33, 64])
    k = rng.randint(1, min(E, 8))
    S = rng.choice([0, 0, 1, 2])
    gating = rng.choice(["softmax", "sigmoid_norm"])
    act = rng.choice(["relu", "gelu", "swiglu"])
    ebias = act != "swiglu" and rng.random() < 0.5
    rbias = rng.choice(["none", "learned"])
    cf = rng.choice([None, None, 1.25, 1.0, 0.5])
    return scaled(RUNS["gpt2"], name=f"random{i}", T=T, d_model=d, d_ff=f, num_experts=E,
                  top_k=k, num_shared=S, gating=gating, activation=act, router_bias=rbias,
                  expert_bias=ebias, dtype=dtype, capacity_factor=cf, seed=500 + i)


CASES = [_draw(i) for i in range(N_CASES)]


def _describe(run):
    return (f"{run.name}: T={run.T} d={run.d_model} f={run.d_ff} E={run.num_experts} "
            f"k={run.top_k} S={run.num_shared} {run.gating} {run.activation} "
            f"ebias={run.expert_bias} rbias={run.router_bias} {run.dtype} cf={run.capacity_factor}")


@functools.lru_cache(maxsize=None)
def _inputs(i):
    return make_inputs(CASES[i])


def test_sweep_is_varied():
    """The drawn shapes cover the paths the sweep is for (CPU-side check)."""
    runs = CASES
    assert any(r.T <= 16 and r.dtype == "bf16" for r in runs)        # decode kernels
    assert any(16 < r.T <= 64 and r.dtype == "bf16" for r in runs)  # several token groups
    assert any(64 < r.T <= 128 and r.dtype == "bf16" for r in runs)  # row passes
    assert any(r.T > 256 and r.dtype == "bf16" for r in runs)        # several m-tiles
    assert any(r.num_shared > 0 for r in runs)
    assert any(r.capacity_factor is not None for r in runs)
    assert len({r.activation for r in runs}) == 3
    assert len({r.gating for r in runs}) == 2
    assert any(r.dtype == "f32" for r in runs)


@pytest.mark.gpu
@pytest.mark.parametrize("i", range(N_CASES), ids=[r.name for r in CASES])
def test_forward_random_shape(i):
    run = CASES[i]
    print(f"[random forward] {_describe(run)}", flush=True)
    inp = _inputs(i)
    g = gpu_inputs(inp)
    gpu = run_forward(run, g)
    compare_forward(run, gpu, oracle_forward(run, inp), inp)


BWD = [i for i, r in enumerate(CASES) if r.dtype == "bf16"][:10]


@pytest.mark.gpu
@pytest.mark.parametrize("i", BWD, ids=[CASES[i].name for i in BWD])
def test_backward_random_shape(i):
    run = CASES[i]
    alpha = 0.05
    print(f"[random backward] {_describe(run)} alpha={alpha}", flush=True)
    inp = _inputs(i)
    dy = make_grad_output(run)
    p = problem_of(run)
    g = gpu_inputs(inp)
    w = weights_of(g)
    r = routing_outputs(p)
    y = torch.empty(run.T * run.d_model, dtype=torch.float32, device="cuda")
    M.moe_ffn_forward(p, w, g["x"], y, M.workspace(p), routing=r)
    grads = grad_outputs(p, run)
    M.moe_ffn_backward(p, w, g["x"], dy.cuda(), alpha, r, grads, M.backward_workspace(p))
    torch.cuda.synchronize()
    idx = r["topk_idx"].cpu().numpy().reshape(run.T, run.top_k)
    lazy = lambda t: None if t is None else LazyF64(t)
    ref = OB.backward(to_f64(inp["x"]), to_f64(inp["w_router"]), to_f64(inp["b_router"]),
                      lazy(inp["w_up"]), lazy(inp["b_up"]), lazy(inp["w_down"]),
                      lazy(inp["b_down"]), dy.double().numpy(), alpha=alpha, top_k=run.top_k,
                      num_shared=run.num_shared, gating=run.gating, activation=run.activation,
                      cap=oracle_capacity(run), idx=idx)
    got = {k: v.cpu().numpy() for k, v in grads.items()}
    for name, rname in (("dx", "dx"), ("dw_router", "dw_router"), ("dw_up", "dw_up"),
                        ("dw_down", "dw_down"), ("d_topk_w", "dw"), ("d_logits", "dlogits")):
        assert_grad_close(got[name], ref[rname], name)
    if run.router_bias != "none":
        assert_grad_close(got["db_router"], ref["db_router"], "db_router")
    if run.expert_bias:
        assert_grad_close(got["db_up"], ref["db_up"], "db_up")
        assert_grad_close(got["db_down"], ref["db_down"], "db_down")
