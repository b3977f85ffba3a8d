"""Parity at the workloads' full sizes, in the launch configuration the
benchmark times (one moe_ffn_forward call): routing, dispatch and the aux
statistics are compared over every token; y over a seeded sample of tokens
that the oracle computes one by one (a token's y needs only its own expert
rows once the batch-wide dispatch is known)."""
import numpy as np
import pytest

from synth import RUNS, make_inputs

from _parity import compare_forward, gpu_inputs, oracle_forward, run_forward

pytestmark = pytest.mark.gpu

SAMPLE = 48


@pytest.mark.parametrize("name", ["gpt2", "swiglu_skew", "large_prefill", "fine_shared"])
def test_forward_full_size_sampled_tokens(name):
    run = RUNS[name]
    print(f"[full-size forward] {name}: T={run.T} d={run.d_model} f={run.d_ff} "
          f"E={run.num_experts} k={run.top_k} S={run.num_shared}", flush=True)
    inp = make_inputs(run)
    g = gpu_inputs(inp)
    gpu = run_forward(run, g)
    del g
    rng = np.random.default_rng(1000 + run.seed)
    sub = np.sort(rng.choice(run.T, size=SAMPLE, replace=False))
    orc = oracle_forward(run, inp, token_subset=sub)
    compare_forward(run, gpu, orc, token_subset=sub)
