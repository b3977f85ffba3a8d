"""The six seeded synthetic workloads of the MoE-FFN forward.

Each run fixes the layer's shape (tokens T, d_model, d_ff, routed experts E,
top-k, shared experts S), its gate and expert activation, which biases exist,
the storage dtype, the capacity factor and the recipe of the random draws.
This module holds shapes and the input recipe only; it computes nothing of
the method itself (no routing, no capacity, no FFN).

Sources for the shapes (the pages have no measured workloads, so every input
is synthetic):
  * tiny ReLU expert with biases: "手撕一个极简 MoE-FFN" (kamacoder notes),
    section 四 (Expert = Linear -> ReLU -> Linear);
  * GPT-2 width 768 / 3072 with GELU experts and biases: "MoE混合专家模型：
    Transformer稀疏前馈网络原理与PyTorch实现" (0539edu), sections 1.1 and 4.1;
  * SwiGLU experts: learn-minimind MoE guide (gitcode), section 二;
  * shared experts, fine-grained experts and normalized sigmoid gating:
    "MoE架构解析" (bojinhu), section 四 (技术飞跃 ①②③);
  * capacity factor 1.25: "MoE架构解析" section 三 (关键技术①) and the 0539edu
    page section 3.2.
"""
from dataclasses import dataclass, field
from typing import Optional


@dataclass(frozen=True)
class Run:
    name: str
    T: int                    # tokens (B*L flattened)
    d_model: int
    d_ff: int                 # expert FFN width (SwiGLU intermediate for swiglu)
    num_experts: int          # routed experts E
    top_k: int
    num_shared: int           # always-on shared experts S (index E..E+S-1)
    gating: str               # "softmax" | "sigmoid_norm"
    activation: str           # "relu" | "gelu" | "swiglu"
    router_bias: str          # "none" | "learned" | "skew" | "zipf"
    expert_bias: bool
    dtype: str                # "f32" | "bf16" (x, all weights and biases)
    capacity_factor: Optional[float]   # None = no capacity limit
    seed: int
    x_rows: int = 0           # rows of x drawn (>= T); 0 means T
    x_std: float = 1.0
    w_std: float = 0.02       # expert weights and biases, learned router bias
    router_w_std: float = 0.02
    skew_b0: float = 0.0      # router bias of expert 0 for router_bias == "skew"
    zipf_s: float = 1.1       # exponent for router_bias == "zipf"
    w_fp8: bool = False       # expert weights prepared as per-row FP8 E4M3 (drawn as for bf16)
    expert_choice: bool = False   # experts pick their tokens; capacity from capacity_factor
    description: str = ""

    @property
    def rows_drawn(self) -> int:
        return self.x_rows or self.T

    @property
    def up_rows(self) -> int:
        """Rows of one expert's up-projection weight: d_ff, or 2*d_ff for
        SwiGLU (gate rows first, then up rows)."""
        return 2 * self.d_ff if self.activation == "swiglu" else self.d_ff


# Router bias of expert 0 in the skewed SwiGLU run.  It was chosen by
# oracle/calibrate_skew.py (bisection over bf16 values on the seeded x and
# router weight) so that expert 0 receives about half of all tokens; the
# script prints the value and the resulting share.
C3_SKEW_B0 = 0.388671875


RUNS = {
    "tiny": Run(
        name="tiny", T=64, d_model=32, d_ff=64, num_experts=4, top_k=1, num_shared=0,
        gating="softmax", activation="relu", router_bias="learned", expert_bias=True,
        dtype="f32", capacity_factor=None, seed=1,
        router_w_std=(1.0 / 32) ** 0.5,
        description="T=64 d=32 f=64 E=4 top-1 softmax+bias ReLU fp32, no capacity"),
    "gpt2": Run(
        name="gpt2", T=4096, d_model=768, d_ff=3072, num_experts=8, top_k=2, num_shared=0,
        gating="softmax", activation="gelu", router_bias="learned", expert_bias=True,
        dtype="bf16", capacity_factor=1.25, seed=2,
        description="T=4096 (8x512) d=768 f=3072 E=8 top-2 softmax GELU bf16, CF 1.25"),
    "swiglu_skew": Run(
        name="swiglu_skew", T=16384, d_model=512, d_ff=1408, num_experts=4, top_k=1,
        num_shared=0, gating="softmax", activation="swiglu", router_bias="skew",
        expert_bias=False, dtype="bf16", capacity_factor=None, seed=3,
        skew_b0=C3_SKEW_B0,
        description="T=16384 d=512 f=1408 E=4 top-1 softmax SwiGLU bf16, ~50% to expert 0"),
    "gpt2_ec": Run(
        name="gpt2_ec", T=4096, d_model=768, d_ff=3072, num_experts=8, top_k=2, num_shared=0,
        gating="softmax", activation="gelu", router_bias="learned", expert_bias=True,
        dtype="bf16", capacity_factor=1.0, seed=2, expert_choice=True,
        description="T=4096 (8x512) d=768 f=3072 E=8 softmax GELU bf16, expert choice: each "
                    "expert takes T*2/E = 1024 tokens"),
    "large_decode": Run(
        name="large_decode", T=16, d_model=4096, d_ff=14336, num_experts=8, top_k=2,
        num_shared=0, gating="softmax", activation="swiglu", router_bias="none",
        expert_bias=False, dtype="bf16", capacity_factor=None, seed=4, x_rows=8192,
        description="T=16 d=4096 f=14336 E=8 top-2 softmax SwiGLU bf16 (decode)"),
    "large_decode_fp8": Run(
        name="large_decode_fp8", T=16, d_model=4096, d_ff=14336, num_experts=8, top_k=2,
        num_shared=0, gating="softmax", activation="swiglu", router_bias="none",
        expert_bias=False, dtype="bf16", capacity_factor=None, seed=4, x_rows=8192, w_fp8=True,
        description="T=16 d=4096 f=14336 E=8 top-2 softmax SwiGLU, bf16 activations, "
                    "FP8 E4M3 expert weights with per-row scales (decode)"),
    "large_prefill": Run(
        name="large_prefill", T=8192, d_model=4096, d_ff=14336, num_experts=8, top_k=2,
        num_shared=0, gating="softmax", activation="swiglu", router_bias="none",
        expert_bias=False, dtype="bf16", capacity_factor=None, seed=4,
        description="T=8192 d=4096 f=14336 E=8 top-2 softmax SwiGLU bf16 (prefill)"),
    "fine_shared": Run(
        name="fine_shared", T=8192, d_model=2048, d_ff=1408, num_experts=64, top_k=6,
        num_shared=2, gating="sigmoid_norm", activation="swiglu", router_bias="zipf",
        expert_bias=False, dtype="bf16", capacity_factor=1.25, seed=5,
        description="T=8192 d=2048 f=1408 E=64 top-6 + 2 shared, normalized sigmoid, "
                    "Zipf(1.1) router bias, SwiGLU bf16, CF 1.25"),
}

# The run whose throughput is the headline figure: the largest one-GPU
# workload (Mixtral-sized experts, an 8192-token prefill batch).
HEADLINE_RUN = "large_prefill"


def scaled(run: Run, **changes) -> Run:
    """A copy of `run` with some fields replaced (smaller parity cases keep the
    structure of a workload: gate, activation, bias recipe, dtype, k, E)."""
    d = {f: getattr(run, f) for f in run.__dataclass_fields__}
    d.update(changes)
    if "T" in changes and "x_rows" not in changes:
        d["x_rows"] = 0
    return Run(**d)
