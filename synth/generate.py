"""Seeded input generator shared by the oracle-side tests and the HIP path.

Draw recipe (fixed order, one torch CPU generator seeded with run.seed):
  1. x          [rows_drawn, d_model]   ~ N(0, x_std^2)
  2. w_router   [E, d_model]            ~ N(0, router_w_std^2)
  3. b_router   [E]  "learned": N(0, w_std^2); "skew": (skew_b0, 0, ..., 0);
                     "zipf": -s*ln(e+1) for expert e (Zipf(s) log-prior,
                     expert 0 is the head); "none": absent
  4. for each expert q = 0..E+S-1 (routed first, then shared):
        w_up[q]   [F1, d_model] ~ N(0, w_std^2)   (F1 = d_ff, or 2*d_ff for
                                                   SwiGLU: gate rows then up rows)
        b_up[q]   [F1]          ~ N(0, w_std^2)   (only with expert biases)
        w_down[q] [d_model, d_ff] ~ N(0, w_std^2)
        b_down[q] [d_model]     ~ N(0, w_std^2)   (only with expert biases)
Every draw is fp32; bf16 runs round each tensor to bf16 (round to nearest
even) right after drawing it.  Both the oracle and the kernels read these
same bytes (the oracle upcasts bf16 exactly).

make_grad_output draws the upstream gradient of the backward pass.

This module performs no step of the method: no router product, no gate, no
routing, no FFN.  The weights follow the nn.Linear [out, in] layout.
"""
import math
from typing import Dict

import torch

from .configs import Run


def _dtype(run: Run):
    return torch.float32 if run.dtype == "f32" else torch.bfloat16


def make_inputs(run: Run) -> Dict[str, torch.Tensor]:
    """Return CPU tensors x, w_router, b_router (or None), w_up, b_up (or None),
    w_down, b_down (or None), all of the run's dtype.  x has run.T rows (the
    first run.T of the rows_drawn drawn)."""
    g = torch.Generator(device="cpu")
    g.manual_seed(run.seed)
    dt = _dtype(run)
    E, S, d, f = run.num_experts, run.num_shared, run.d_model, run.d_ff
    F1 = run.up_rows

    def draw(shape, std):
        t = torch.randn(shape, generator=g, dtype=torch.float32) * std
        return t.to(dt)

    x = draw((run.rows_drawn, d), run.x_std)[: run.T].contiguous()
    w_router = draw((E, d), run.router_w_std)
    if run.router_bias == "learned":
        b_router = draw((E,), run.w_std)
    elif run.router_bias == "skew":
        b = torch.zeros(E, dtype=torch.float32)
        b[0] = run.skew_b0
        b_router = b.to(dt)
    elif run.router_bias == "zipf":
        b = torch.tensor([-run.zipf_s * math.log(e + 1.0) for e in range(E)],
                         dtype=torch.float32)
        b_router = b.to(dt)
    elif run.router_bias == "none":
        b_router = None
    else:
        raise ValueError(run.router_bias)

    n_all = E + S
    w_up = torch.empty((n_all, F1, d), dtype=dt)
    w_down = torch.empty((n_all, d, f), dtype=dt)
    b_up = torch.empty((n_all, F1), dtype=dt) if run.expert_bias else None
    b_down = torch.empty((n_all, d), dtype=dt) if run.expert_bias else None
    for q in range(n_all):
        w_up[q] = draw((F1, d), run.w_std)
        if b_up is not None:
            b_up[q] = draw((F1,), run.w_std)
        w_down[q] = draw((d, f), run.w_std)
        if b_down is not None:
            b_down[q] = draw((d,), run.w_std)
    return dict(x=x, w_router=w_router, b_router=b_router, w_up=w_up, b_up=b_up,
                w_down=w_down, b_down=b_down)


def make_grad_output(run: Run) -> torch.Tensor:
    """Upstream gradient dy [T, d_model] for the backward pass: float32
    N(0, 1), from its own CPU generator seeded with run.seed + 1000 (so the
    forward inputs above are unchanged)."""
    g = torch.Generator(device="cpu")
    g.manual_seed(run.seed + 1000)
    return torch.randn((run.T, run.d_model), generator=g, dtype=torch.float32)


def to_f64(t):
    """Exact upcast of a generated tensor to a float64 numpy array (None stays None)."""
    if t is None:
        return None
    return t.to(torch.float64).numpy()
