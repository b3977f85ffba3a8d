"""Parity at the workloads' full sizes, in the launch configuration the
benchmark times (one moe_ffn_forward call): the GPU's routing against the
oracle's own over every token, then the whole layer against the oracle
evaluated at the GPU's selection: dispatch bit-exact, and every element of
y, topk_w and probs within the tolerances."""
import time

import numpy as np
import pytest
import torch

from synth import RUNS, make_inputs

from _parity import compare_forward, gpu_inputs, oracle_routing, run_forward

pytestmark = pytest.mark.gpu


def _run_whole(run):
    print(f"[full-size forward] {run.name}: T={run.T} d={run.d_model} f={run.d_ff} "
          f"E={run.num_experts} k={run.top_k} S={run.num_shared} fp8={run.w_fp8}", flush=True)
    inp = make_inputs(run)
    g = gpu_inputs(inp, w_fp8=run.w_fp8)
    gpu = run_forward(run, g)
    del g
    torch.cuda.empty_cache()
    t0 = time.perf_counter()
    compare_forward(run, gpu, oracle_routing(run, inp), inp)
    print(f"  oracle and comparison over all {run.T} x {run.d_model} outputs: "
          f"{time.perf_counter() - t0:.1f} s", flush=True)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["gpt2", "swiglu_skew", "large_prefill", "fine_shared"])
def test_forward_full_size_every_output(name):
    _run_whole(RUNS[name])


@pytest.mark.timeout(900)
def test_forward_full_size_fp8_decode():
    # the FP8 decode workload at its full shape (d_model 4096, SwiGLU 14336,
    # 8 experts): the oracle quantizes the bf16 weights itself
    _run_whole(RUNS["large_decode_fp8"])
