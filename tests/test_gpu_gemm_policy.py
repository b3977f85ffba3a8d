"""The grouped GEMM's two main loops (16x16x32 MFMAs with 64-deep k-tiles, and
32x32x16 MFMAs with 32-deep k-tiles) on the same problems.  By default the up
projection takes the 16x16x32 loop and the down-style projections take it
only when long, so only full-size layers would reach it there; here
moe_set_gemm_policy forces each loop everywhere, on shapes the oracle
finishes in seconds: ragged and half-empty m-tiles, waves without rows,
shared experts, biases, every activation, one-k-tile and odd k-tile
reductions, K-sliced down projections, and the two-list tile schedule.  Both
loops accumulate every output in the same order, so their outputs are
compared bit for bit, and the forced 16x16x32 forward is compared with the
float64 oracle."""
import contextlib
import functools

import numpy as np
import pytest
import torch

from mixture_experts_sparse_gemv_amd import moe as M
from synth import RUNS, make_grad_output, make_inputs, scaled

from _parity import (compare_forward, gpu_inputs, oracle_forward, problem_of, routing_outputs,
                     run_forward, weights_of)
from test_gpu_backward import grad_outputs

pytestmark = pytest.mark.gpu

CASES = {
    "gpt2_T700": scaled(RUNS["gpt2"], T=700),
    "gpt2_T700_cf1": scaled(RUNS["gpt2"], T=700, capacity_factor=1.0),
    "swiglu_skew_T3000": scaled(RUNS["swiglu_skew"], T=3000),
    "large_T300": scaled(RUNS["large_prefill"], T=300),
    "fine_shared_T1000": scaled(RUNS["fine_shared"], T=1000),
    "fine_shared_T1100_d256": scaled(RUNS["fine_shared"], T=1100, d_model=256, d_ff=128),
    # one 64-deep k-tile in the up projection, three (odd) in the down one
    "relu_bias_d64_f192_T900": scaled(RUNS["gpt2"], T=900, d_model=64, d_ff=192,
                                      activation="relu", capacity_factor=None),
    # five 64-deep k-tiles up, K-sliced down projection (f = 1280)
    "gelu_d320_f1280_T1500": scaled(RUNS["gpt2"], T=1500, d_model=320, d_ff=1280),
    # SwiGLU with 3 shared experts and a tight capacity
    "swiglu_shared3_T777": scaled(RUNS["fine_shared"], T=777, d_model=384, d_ff=448,
                                  num_experts=13, top_k=3, num_shared=3, capacity_factor=0.5),
    "relu_E64_T16384_split_lists": scaled(RUNS["gpt2"], T=16384, d_model=256, d_ff=128,
                                          num_experts=64, top_k=4, activation="relu",
                                          capacity_factor=None),
}


@contextlib.contextmanager
def gemm_policy(policy):
    M.moe_set_gemm_policy(policy)
    try:
        yield
    finally:
        M.moe_set_gemm_policy(M.MOE_GEMM_AUTO)


@functools.lru_cache(maxsize=None)
def _inputs(name):
    return make_inputs(CASES[name])


def _describe(name):
    r = CASES[name]
    return (f"{name}: T={r.T} d={r.d_model} f={r.d_ff} E={r.num_experts} k={r.top_k} "
            f"S={r.num_shared} {r.activation} ebias={r.expert_bias} cf={r.capacity_factor}")


@pytest.mark.parametrize("name", list(CASES))
def test_forward_mf16_matches_oracle_and_mf32(name):
    run = CASES[name]
    print(f"[gemm policy forward] {_describe(name)}", flush=True)
    inp = _inputs(name)
    g = gpu_inputs(inp)
    with gemm_policy(M.MOE_GEMM_MF16):
        a = run_forward(run, g)
    with gemm_policy(M.MOE_GEMM_MF32):
        b = run_forward(run, g)
    assert np.array_equal(a["y"].view(np.uint32), b["y"].view(np.uint32)), \
        "16x16x32 and 32x32x16 loops differ"
    compare_forward(run, a, oracle_forward(run, inp), inp)


@pytest.mark.parametrize("name", ["gpt2_T700", "large_T300", "fine_shared_T1000",
                                  "swiglu_shared3_T777", "relu_bias_d64_f192_T900"])
def test_backward_mf16_equals_mf32(name):
    run = CASES[name]
    alpha = 0.05
    print(f"[gemm policy backward] {_describe(name)}", flush=True)
    inp = _inputs(name)
    dy = make_grad_output(run).cuda()
    g = gpu_inputs(inp)
    p = problem_of(run)
    w = weights_of(g)
    r = routing_outputs(p)
    y = torch.empty(run.T * run.d_model, dtype=torch.float32, device="cuda")
    M.moe_ffn_forward(p, w, g["x"], y, M.workspace(p), routing=r)
    out = []
    for policy in (M.MOE_GEMM_MF16, M.MOE_GEMM_MF32):
        grads = grad_outputs(p, run)
        with gemm_policy(policy):
            M.moe_ffn_backward(p, w, g["x"], dy, alpha, r, grads, M.backward_workspace(p))
            torch.cuda.synchronize()
        out.append({k: v.cpu().numpy() for k, v in grads.items()})
    for k in out[0]:
        assert np.array_equal(out[0][k].view(np.uint32), out[1][k].view(np.uint32)), \
            f"{k}: 16x16x32 and 32x32x16 loops differ"
