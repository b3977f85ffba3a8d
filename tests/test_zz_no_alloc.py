"""moe_ffn_forward_static (the forward with the library's own device scratch
array, for callers that cannot allocate) against moe_ffn_forward with a
caller workspace, through the C ABI: two calls in a row, the second on a
smaller problem, each bit-identical to the workspace entry point (the same
kernels on the same inputs); and a problem whose workspace exceeds the array
is refused before any launch."""
import numpy as np
import pytest
import torch

from mixture_experts_sparse_gemv_amd import moe as M
from synth import RUNS, make_inputs, scaled

from _parity import gpu_inputs, problem_of, routing_outputs, weights_of

pytestmark = pytest.mark.gpu


def _forward(run, g, static):
    p = problem_of(run)
    y = torch.empty(run.T * run.d_model, dtype=torch.float32, device="cuda")
    r = routing_outputs(p)
    if static:
        M.moe_ffn_forward_static(p, weights_of(g), g["x"], y, routing=r)
    else:
        M.moe_ffn_forward(p, weights_of(g), g["x"], y, M.workspace(p), routing=r)
    torch.cuda.synchronize()
    out = {k: v.cpu().numpy() for k, v in r.items()}
    out["y"] = y.cpu().numpy()
    return out


@pytest.mark.parametrize("first,second", [(("gpt2", 1500), ("gpt2", 300)),
                                          (("fine_shared", 1200), ("swiglu_skew", 700))])
def test_static_scratch_forward_matches_workspace_forward(first, second):
    for name, T in (first, second):    # the second call is smaller than the first
        run = scaled(RUNS[name], T=T)
        print(f"[static scratch] {name} T={T} workspace "
              f"{M.moe_workspace_size(problem_of(run))} bytes", flush=True)
        assert M.moe_workspace_size(problem_of(run)) <= M.STATIC_SCRATCH_BYTES
        g = gpu_inputs(make_inputs(run))
        ref = _forward(run, g, static=False)
        got = _forward(run, g, static=True)
        for key in ref:
            assert np.array_equal(got[key], ref[key]), key


def test_static_scratch_refuses_a_problem_beyond_its_size():
    run = RUNS["large_prefill"]
    p = problem_of(run)
    assert M.moe_workspace_size(p) > M.STATIC_SCRATCH_BYTES
    x = torch.empty(run.T * run.d_model, dtype=torch.bfloat16, device="cuda")
    y = torch.empty(run.T * run.d_model, dtype=torch.float32, device="cuda")
    with pytest.raises(M.MoeError, match="MOE_ERR_WORKSPACE"):
        M.moe_ffn_forward_static(p, M.moe_weights(), x, y)
