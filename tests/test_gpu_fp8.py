"""FP8 E4M3 expert weights (per-row scales) on the weight-streaming decode
path: the GPU quantizer against the oracle's (bit-exact codes and scales),
and decode-sized forwards against the oracle run on its own dequantized
weights.  The quantization error itself (against the bf16 weights) is
reported and bounded separately: it is the method's error budget, not a
parity criterion."""
import numpy as np
import pytest
import torch

import oracle as O
from mixture_experts_sparse_gemv_amd import moe as M
from synth import RUNS, make_inputs, scaled

from _parity import compare_forward, gpu_inputs, oracle_forward, run_forward

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


@pytest.mark.parametrize("rows,cols,std", [(7, 128, 0.02), (33, 4096, 1.0), (5, 14336, 0.02)])
def test_quantize_fp8_bitexact(rows, cols, std):
    _say(f"[quantize_fp8] rows={rows} cols={cols} std={std}")
    g = torch.Generator().manual_seed(rows * 1000 + cols)
    w = (torch.randn(rows, cols, generator=g) * std)
    w[0, :] = 0.0                                   # all-zero row: scale 1, codes 0
    w[1, :5] = torch.tensor([448.0, -1e-30, 2.0 ** -12, -3.0, 1e-5]) * std
    w[2, :3] = torch.tensor([1.0, 1.0625, 1.1875])  # ties after scaling by this row's max
    wb = w.to(torch.bfloat16)
    q = torch.empty(rows, cols, dtype=torch.uint8, device="cuda")
    s = torch.empty(rows, dtype=torch.float32, device="cuda")
    M.moe_quantize_fp8(wb.cuda(), q, s)
    torch.cuda.synchronize()
    codes, scales = O.quantize_fp8_rows(wb.to(torch.float32).numpy())
    assert np.array_equal(s.cpu().numpy().view(np.uint32), scales.view(np.uint32)), "scales"
    qq = q.cpu().numpy()
    bad = np.argwhere(qq != codes)
    assert bad.size == 0, f"{len(bad)} codes differ, first at {bad[:3]}: {qq[tuple(bad[0])]} vs {codes[tuple(bad[0])]}"


FP8_CASES = {
    "fp8_swiglu_T7": scaled(RUNS["large_decode_fp8"], T=7, d_model=256, d_ff=512, x_rows=0),
    "fp8_gelu_bias_T16": scaled(RUNS["large_decode_fp8"], T=16, d_model=384, d_ff=640,
                                activation="gelu", expert_bias=True, router_bias="learned",
                                num_experts=6, x_rows=0, seed=9),
    "fp8_shared_T5": scaled(RUNS["large_decode_fp8"], T=5, d_model=256, d_ff=384, num_shared=2,
                            gating="sigmoid_norm", num_experts=16, top_k=4, x_rows=0, seed=10),
    # K long enough for the steady state of the decode ring (at least 5 stages
    # of 128 in both projections: d = 1024, and d_ff = 8192 in 8 K slices)
    "fp8_swiglu_T16_d1024_f8192": scaled(RUNS["large_decode_fp8"], d_model=1024, d_ff=8192,
                                         x_rows=0, seed=11),
    # 2 and 4 groups of 16 token rows per weight stage
    "fp8_swiglu_T29": scaled(RUNS["large_decode_fp8"], T=29, d_model=512, d_ff=1024, x_rows=0,
                             seed=14),
    "fp8_gelu_bias_T64_shared": scaled(RUNS["large_decode_fp8"], T=64, d_model=256, d_ff=384,
                                       activation="gelu", expert_bias=True, num_shared=1,
                                       router_bias="learned", x_rows=0, seed=15),
    # two row passes for the shared expert's 100 rows
    "fp8_swiglu_T100_shared_two_passes": scaled(RUNS["large_decode_fp8"], T=100, d_model=256,
                                                d_ff=384, num_shared=1, x_rows=0, seed=16),
}


@pytest.mark.parametrize("name", list(FP8_CASES))
def test_forward_fp8_weights(name):
    run = FP8_CASES[name]
    _say(f"[forward fp8] {name}: T={run.T} d={run.d_model} f={run.d_ff} E={run.num_experts} "
         f"k={run.top_k} S={run.num_shared} {run.activation}")
    inp = make_inputs(run)
    g = gpu_inputs(inp, w_fp8=True)
    gpu = run_forward(run, g)
    del g
    orc = oracle_forward(run, inp)
    compare_forward(run, gpu, orc, inp)
    # error budget: FP8 weights against the bf16 weights (oracle both ways)
    ref = oracle_forward(run, inp, w_fp8=False)
    e = orc["y"] - ref["y"]
    rel = float(np.linalg.norm(e) / np.linalg.norm(ref["y"]))
    _say(f"  fp8 quantization error of y: rel_frob={rel:.3e} max_abs={np.abs(e).max():.3e}")
    assert rel < 0.06
