"""Seeded synthetic inputs for the MoE-FFN forward: the run table and the
generator.  Shared by the oracle-side tests and the HIP path; holds no step
of the method."""
from .configs import RUNS, HEADLINE_RUN, Run, scaled
from .generate import make_grad_output, make_inputs, to_f64

__all__ = ["RUNS", "HEADLINE_RUN", "Run", "scaled", "make_inputs", "make_grad_output", "to_f64"]
