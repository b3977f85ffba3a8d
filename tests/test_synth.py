"""The seeded generator: determinism, shapes, dtypes and the bias recipes
of the skewed and Zipf workloads (CPU only)."""
import math

import numpy as np
import torch

import oracle as O
from synth import RUNS, make_inputs, scaled, to_f64


def test_deterministic_and_shapes():
    for name in ("tiny", "gpt2"):
        r = RUNS[name]
        a, b = make_inputs(r), make_inputs(r)
        for key in a:
            if a[key] is None:
                assert b[key] is None
                continue
            assert torch.equal(a[key], b[key])
        E, S = r.num_experts, r.num_shared
        assert a["x"].shape == (r.T, r.d_model)
        assert a["w_up"].shape == (E + S, r.up_rows, r.d_model)
        assert a["w_down"].shape == (E + S, r.d_model, r.d_ff)
        assert a["x"].dtype == (torch.float32 if r.dtype == "f32" else torch.bfloat16)
        assert (a["b_up"] is not None) == r.expert_bias


def test_distribution_scales():
    r = RUNS["gpt2"]
    a = make_inputs(r)
    assert abs(a["x"].float().std().item() - 1.0) < 0.01
    assert abs(a["w_up"].float().std().item() - 0.02) < 0.001
    t = make_inputs(RUNS["tiny"])
    assert abs(t["w_router"].std().item() - 1 / math.sqrt(32)) < 0.03


def test_decode_inputs_are_prefix_of_prefill():
    small_p = scaled(RUNS["large_prefill"], d_model=64, d_ff=128, T=64)
    small_d = scaled(RUNS["large_decode"], d_model=64, d_ff=128, T=16, x_rows=64)
    p, d = make_inputs(small_p), make_inputs(small_d)
    assert torch.equal(d["x"], p["x"][:16])
    assert torch.equal(d["w_up"], p["w_up"]) and torch.equal(d["w_down"], p["w_down"])


def test_zipf_bias_recipe():
    r = scaled(RUNS["fine_shared"], d_model=64, d_ff=64, T=8)
    b = make_inputs(r)["b_router"].float()
    ref = torch.tensor([-1.1 * math.log(e + 1) for e in range(64)]).to(torch.bfloat16).float()
    assert torch.equal(b, ref)


def test_skew_gives_half_of_tokens_to_expert0():
    r = RUNS["swiglu_skew"]
    a = make_inputs(scaled(r, d_ff=64))       # same x / router draws, smaller experts
    p = O.softmax(O.router_logits(to_f64(a["x"]), to_f64(a["w_router"]), to_f64(a["b_router"])))
    idx, _ = O.topk_renorm(p, 1)
    share = float(np.mean(idx[:, 0] == 0))
    assert 0.49 <= share <= 0.51
