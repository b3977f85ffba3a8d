"""Expert-choice routing through the C ABI: the selection against the
oracle's on the same float32 probabilities (exact, ties included), and whole
forwards against the oracle's expert-choice forward."""
import numpy as np
import pytest
import torch

import oracle as O
from mixture_experts_sparse_gemv_amd import moe as M
from synth import RUNS, make_inputs, scaled

from _parity import compare_forward_ec, gpu_inputs, oracle_forward, run_forward

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


@pytest.mark.parametrize("T,E,C,levels", [(64, 4, 16, 0), (1000, 8, 250, 7), (1000, 8, 1, 0),
                                          (4097, 64, 300, 0), (3000, 3, 3000, 5),
                                          (16384, 8, 4096, 11), (16, 8, 5, 3)])
def test_expert_choice_selection_exact(T, E, C, levels):
    _say(f"[expert_choice] T={T} E={E} C={C} levels={levels}")
    rng = np.random.default_rng(T + E + C)
    probs = rng.random((T, E)).astype(np.float32)
    if levels:                      # few distinct scores: many ties
        probs = (np.floor(probs * levels) / levels).astype(np.float32)
    p = M.make_problem(T=T, d_model=64, d_ff=64, num_experts=E, top_k=1, capacity=C,
                       expert_choice=True)
    i32 = dict(dtype=torch.int32, device="cuda")
    off, sa = torch.empty(E + 1, **i32), torch.empty(E * C, **i32)
    row_of, te = torch.empty(T * E, **i32), torch.empty(T, **i32)
    M.moe_expert_choice(p, torch.from_numpy(probs).cuda(), off, sa, row_of, te,
                        ws=M.workspace(p))
    torch.cuda.synchronize()
    sel, rows, tex = O.expert_choice_select(probs.astype(np.float64), C)
    assert np.array_equal(off.cpu().numpy(), np.arange(E + 1) * C)
    assert np.array_equal(sa.cpu().numpy().reshape(E, C), sel)
    assert np.array_equal(row_of.cpu().numpy().reshape(T, E), rows)
    assert np.array_equal(te.cpu().numpy(), tex)


EC_CASES = {
    "gpt2_ec_T700": scaled(RUNS["gpt2_ec"], T=700),
    "ec_swiglu_shared_sigmoid": scaled(RUNS["gpt2_ec"], T=1000, d_model=512, d_ff=1408,
                                       activation="swiglu", expert_bias=False, num_shared=2,
                                       gating="sigmoid_norm", num_experts=16, top_k=2,
                                       capacity_factor=0.75, router_bias="zipf", seed=12),
    "ec_decode_T16": scaled(RUNS["gpt2_ec"], T=16, d_model=1024, d_ff=2048,
                            activation="swiglu", expert_bias=False, router_bias="none",
                            capacity_factor=1.0, seed=13),
    "ec_d392_f584_T500": scaled(RUNS["gpt2_ec"], T=500, d_model=392, d_ff=584, seed=16),
    # the streaming path with 128 rows per expert: two row passes
    "ec_T128_two_passes": scaled(RUNS["gpt2_ec"], T=128, d_model=256, d_ff=512, num_experts=2,
                                 seed=17),
    "gpt2_ec": RUNS["gpt2_ec"],
}


@pytest.mark.parametrize("name", list(EC_CASES))
def test_forward_expert_choice(name):
    run = EC_CASES[name]
    _say(f"[forward ec] {name}: T={run.T} d={run.d_model} f={run.d_ff} E={run.num_experts} "
         f"S={run.num_shared} {run.gating} {run.activation}")
    inp = make_inputs(run)
    g = gpu_inputs(inp)
    gpu = run_forward(run, g)
    del g
    orc = oracle_forward(run, inp)
    compare_forward_ec(run, gpu, orc, inp)
    _say(f"  orphans={int((gpu['token_experts'] == 0).sum())} "
         f"max experts per token={int(gpu['token_experts'].max())}")
