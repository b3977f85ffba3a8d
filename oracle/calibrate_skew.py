"""Choose the router bias of expert 0 for the skewed SwiGLU run.

Test-infrastructure script: it calls only the oracle (router logits, softmax,
top-1) on the seeded x and router weight of that run and bisects the bias b0,
taken on the bf16 grid the run stores, until expert 0 receives about half of
the tokens.  Run it from the repository root:

    python -m oracle.calibrate_skew

and copy the printed value into synth/configs.py (C3_SKEW_B0)."""
import numpy as np
import torch

from synth import RUNS, make_inputs, to_f64
from synth.configs import scaled

from . import moe_oracle as O


def share_of_expert0(x, wr, b0):
    E = wr.shape[0]
    br = np.zeros(E)
    br[0] = float(torch.tensor(b0, dtype=torch.float32).to(torch.bfloat16).to(torch.float64))
    idx, _ = O.topk_renorm(O.softmax(O.router_logits(x, wr, br)), 1)
    return float(np.mean(idx[:, 0] == 0)), br[0]


def main():
    run = scaled(RUNS["swiglu_skew"], skew_b0=0.0)
    inp = make_inputs(run)
    x, wr = to_f64(inp["x"]), to_f64(inp["w_router"])
    lo, hi = 0.0, 2.0
    for _ in range(40):
        mid = 0.5 * (lo + hi)
        s, _ = share_of_expert0(x, wr, mid)
        if s < 0.5:
            lo = mid
        else:
            hi = mid
    s, b = share_of_expert0(x, wr, hi)
    print(f"b0 = {b!r}  share of expert 0 = {s:.4f}")


if __name__ == "__main__":
    main()
