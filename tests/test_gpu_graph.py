"""The forward and backward entry points under HIP graph capture: every
kernel they launch is a plain launch on the caller's stream (no memset, no
allocation, no synchronization), so a captured call replays the same work.
Each replay, with unrelated eager work and synchronizations between the
replays, must reproduce the eager results bit for bit (the kernels are
deterministic)."""
import numpy as np
import pytest
import torch

from mixture_experts_sparse_gemv_amd import moe as M
from synth import RUNS, make_grad_output, make_inputs, scaled

from _parity import gpu_inputs, problem_of, routing_outputs, weights_of
from test_gpu_backward import grad_outputs

pytestmark = pytest.mark.gpu

CASES = {
    "gpt2_T700": scaled(RUNS["gpt2"], T=700),
    "fine_shared_T1000_d512": scaled(RUNS["fine_shared"], T=1000, d_model=512, d_ff=384),
    "decode_T16_d1024": scaled(RUNS["large_decode"], d_model=1024, d_ff=2048),
}


def _snap(tensors):
    return {k: v.detach().cpu().numpy().copy() for k, v in tensors.items() if k != "stats"}


@pytest.mark.parametrize("name", list(CASES))
def test_forward_and_backward_replay(name):
    run = CASES[name]
    print(f"case graph {name}: T={run.T} d={run.d_model} f={run.d_ff} E={run.num_experts}",
          flush=True)
    p = problem_of(run)
    g = gpu_inputs(make_inputs(run))
    w = weights_of(g)
    ws, bws = M.workspace(p), M.backward_workspace(p)
    y = torch.empty(run.T * run.d_model, dtype=torch.float32, device="cuda")
    r = routing_outputs(p)
    grads = grad_outputs(p, run)
    dy = make_grad_output(run).cuda()

    M.moe_ffn_forward(p, w, g["x"], y, ws, routing=r)
    M.moe_ffn_backward(p, w, g["x"], dy, 0.01, r, grads, bws)
    torch.cuda.synchronize()
    ref_fwd = _snap(dict(y=y, **r))
    ref_bwd = _snap(grads)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # capture needs a non-default stream
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=side):
            M.moe_ffn_forward(p, w, g["x"], y, ws, routing=r)
            M.moe_ffn_backward(p, w, g["x"], dy, 0.01, r, grads, bws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    for rep in range(3):
        # unrelated eager work between replays, and outputs overwritten
        y.fill_(float("nan"))
        for v in grads.values():
            v.fill_(float("nan"))
        junk = torch.randn(1 << 20, device="cuda")
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        del junk
        got_fwd, got_bwd = _snap(dict(y=y, **r)), _snap(grads)
        for k, v in ref_fwd.items():
            assert np.array_equal(got_fwd[k], v, equal_nan=True), f"replay {rep}: {k} differs"
        for k, v in ref_bwd.items():
            assert np.array_equal(got_bwd[k], v, equal_nan=True), f"replay {rep}: {k} differs"
