"""Shared helpers of the GPU parity tests: seeded inputs on the GPU, the
oracle on the same bytes, and the comparison rules.

Tolerances (from the statement of the layer's accuracy for bf16 inputs with
fp32 accumulation):
  * routing indices: identical sets on every token whose oracle score gap
    between the k-th and (k+1)-th expert exceeds GAP; slot order identical
    where adjacent selected scores differ by more than GAP; on the other
    tokens every selected expert must score within GAP of the k-th best;
  * dispatch outputs: bit-exact given the same routing;
  * floating-point outputs: relative Frobenius error <= 1e-2 and max abs
    error <= 2e-2 against the float64 oracle;
  * L_aux: relative error <= 1e-4.
"""
import math

import numpy as np
import torch

import oracle as O
from mixture_experts_sparse_gemv_amd import moe as M
from synth import make_inputs, to_f64

GAP = 1e-4
REL_FROB = 1e-2
MAX_ABS = 2e-2
LAUX_REL = 1e-4


class LazyF64:
    """Indexable view of a [n, ...] torch tensor that upcasts one slice at a
    time to float64 numpy (keeps the oracle's memory bounded at large sizes)."""

    def __init__(self, t):
        self.t = t
        self.shape = tuple(t.shape)

    def __getitem__(self, i):
        return self.t[i].to(torch.float64).numpy()


def problem_of(run, capacity=None):
    cap = capacity
    if cap is None:
        cap = M.moe_capacity(run.T, run.top_k, run.num_experts, run.capacity_factor or 0.0)
    return M.make_problem(
        T=run.T, d_model=run.d_model, d_ff=run.d_ff, num_experts=run.num_experts,
        top_k=run.top_k, num_shared=run.num_shared, capacity=cap, dtype=run.dtype,
        gating=run.gating, activation=run.activation,
        router_bias=run.router_bias != "none", expert_bias=run.expert_bias, w_fp8=run.w_fp8,
        expert_choice=run.expert_choice)


def oracle_capacity(run):
    return O.capacity(run.T, run.top_k, run.num_experts, run.capacity_factor)


def gpu_inputs(inp, w_fp8=False):
    """The inputs on the GPU; with w_fp8 the expert weights are replaced by
    their per-row FP8 codes (moe_quantize_fp8) and scales s_up, s_down."""
    g = {k: (None if v is None else v.cuda()) for k, v in inp.items()}
    if w_fp8:
        for name, sname in (("w_up", "s_up"), ("w_down", "s_down")):
            w = g[name]
            q = torch.empty(w.shape, dtype=torch.uint8, device="cuda")
            sc = torch.empty(w.numel() // w.shape[-1], dtype=torch.float32, device="cuda")
            M.moe_quantize_fp8(w, q, sc)
            g[name], g[sname] = q, sc
            del w
        torch.cuda.synchronize()
    return g


def weights_of(g):
    return M.make_weights(g["w_router"], g["b_router"], g["w_up"], g["b_up"], g["w_down"],
                          g["b_down"], g.get("s_up"), g.get("s_down"))


class LazyDeqFP8:
    """Per-expert float64 weights of a [n, rows, K] bf16 tensor as the oracle
    quantizes them (codes and scales from the oracle's own quantizer).  The
    codes of all experts are computed up front, several experts at a time
    (numpy releases the interpreter lock in its array operations), with a
    line per expert; each access dequantizes one expert."""

    def __init__(self, t, workers=8):
        from concurrent.futures import ThreadPoolExecutor
        self.t = t
        self.shape = tuple(t.shape)

        def one(i):
            q = O.quantize_fp8_rows(t[i].to(torch.float32).numpy())
            print(f"  oracle FP8 codes of expert {i} ({tuple(t.shape[1:])})", flush=True)
            return q
        with ThreadPoolExecutor(max_workers=workers) as ex:
            self.codes = list(ex.map(one, range(t.shape[0])))

    def __getitem__(self, i):
        return O.dequantize_fp8_rows(*self.codes[i])


def oracle_forward(run, inp, cap="run", token_subset=None, w_fp8=None, idx=None, sel=None):
    """w_fp8 (default: run.w_fp8): expert weights as the oracle's own FP8
    quantization of the bf16 weights, dequantized exactly.  idx (token
    choice) / sel (expert choice): evaluate the layer at that selection."""
    c = oracle_capacity(run) if cap == "run" else cap
    fp8 = run.w_fp8 if w_fp8 is None else w_fp8
    lazy = lambda t: None if t is None else LazyF64(t)
    lazyw = (lambda t: LazyDeqFP8(t)) if fp8 else lazy
    if run.expert_choice:
        return O.forward_expert_choice(
            to_f64(inp["x"]), to_f64(inp["w_router"]), to_f64(inp["b_router"]),
            lazyw(inp["w_up"]), lazy(inp["b_up"]), lazyw(inp["w_down"]), lazy(inp["b_down"]),
            capacity=c, num_shared=run.num_shared, gating=run.gating,
            activation=run.activation, token_subset=token_subset, sel=sel)
    return O.forward(to_f64(inp["x"]), to_f64(inp["w_router"]), to_f64(inp["b_router"]),
                     lazyw(inp["w_up"]), lazy(inp["b_up"]), lazyw(inp["w_down"]),
                     lazy(inp["b_down"]), top_k=run.top_k, num_shared=run.num_shared,
                     gating=run.gating, activation=run.activation, cap=c,
                     token_subset=token_subset, idx=idx)


def oracle_routing(run, inp):
    """The oracle's own routing over every token (logits, probs, idx, w, gap),
    without the expert FFNs (token choice)."""
    return O.routing(to_f64(inp["x"]), to_f64(inp["w_router"]), to_f64(inp["b_router"]),
                     top_k=run.top_k, gating=run.gating)


def assert_close(got, ref, name, rel=REL_FROB, mabs=MAX_ABS):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    diff = got - ref
    nref = np.linalg.norm(ref)
    rf = np.linalg.norm(diff) / (nref if nref > 0 else 1.0)
    ma = float(np.abs(diff).max()) if diff.size else 0.0
    print(f"  {name}: rel_frob={rf:.3e} max_abs={ma:.3e}", flush=True)
    assert rf <= rel, f"{name}: relative Frobenius error {rf:.3e} > {rel}"
    assert ma <= mabs, f"{name}: max abs error {ma:.3e} > {mabs}"
    return rf, ma


def check_routing(gpu_idx, orc, k):
    """Returns the mask of tokens whose selected set equals the oracle's."""
    oi = orc["idx"]
    gi = np.asarray(gpu_idx).reshape(oi.shape)
    same = np.all(np.sort(gi, axis=1) == np.sort(oi, axis=1), axis=1)
    gap = orc["gap"]
    bad = ~same & (gap > GAP)
    assert not bad.any(), f"routing differs on {int(bad.sum())} tokens with a clear gap"
    probs = orc["probs"]
    E = probs.shape[1]
    assert gi.min() >= 0 and gi.max() < E
    assert np.all(np.array([len(set(r)) for r in gi]) == k), "repeated expert in a token"
    # near-tie tokens: the GPU's choices must be valid within GAP
    kth = np.sort(probs, axis=1)[:, ::-1][:, k - 1]
    sel = np.take_along_axis(probs, gi.astype(np.int64), axis=1)
    assert np.all(sel >= kth[:, None] - GAP)
    # slot order where it is well defined
    osel = np.take_along_axis(probs, oi.astype(np.int64), axis=1)
    if k > 1:
        clear = np.all(np.abs(np.diff(osel, axis=1)) > GAP, axis=1) & same
        assert np.array_equal(gi[clear], oi[clear]), "slot order differs"
    return same


def check_dispatch_bitexact(gpu, orc, E):
    assert np.array_equal(gpu["counts"], orc["counts"]), "counts"
    assert np.array_equal(gpu["kept"], orc["kept"]), "kept"
    assert np.array_equal(gpu["offsets"], orc["offsets"]), "offsets"
    assert np.array_equal(gpu["sorted_assign"], orc["sorted_assign"]), "sorted_assign"
    assert np.array_equal(gpu["assign_row"], orc["assign_row"]), "assign_row"
    assert np.array_equal(gpu["drop_mask"], orc["drop_mask"]), "drop_mask"


def routing_outputs(p, device="cuda"):
    T, k, E = p.T, p.top_k, p.num_experts
    i32 = dict(dtype=torch.int32, device=device)
    f32 = dict(dtype=torch.float32, device=device)
    if p.flags & M.MOE_EXPERT_CHOICE:
        n = E * p.capacity
        return dict(probs=torch.empty(T * E, **f32), counts=torch.empty(E, **i32),
                    kept=torch.empty(E, **i32), offsets=torch.empty(E + 1, **i32),
                    sorted_assign=torch.empty(n, **i32), assign_row=torch.empty(T * E, **i32),
                    f=torch.empty(E, **f32), P=torch.empty(E, **f32),
                    l_aux=torch.empty(1, **f32), stats=M.route_stats_tensor(device),
                    token_experts=torch.empty(T, **i32))
    return dict(topk_idx=torch.empty(T * k, **i32), topk_w=torch.empty(T * k, **f32),
                probs=torch.empty(T * E, **f32), counts=torch.empty(E, **i32),
                kept=torch.empty(E, **i32), offsets=torch.empty(E + 1, **i32),
                sorted_assign=torch.empty(T * k, **i32), assign_row=torch.empty(T * k, **i32),
                drop_mask=torch.empty(T * k, dtype=torch.uint8, device=device),
                f=torch.empty(E, **f32), P=torch.empty(E, **f32), l_aux=torch.empty(1, **f32),
                stats=M.route_stats_tensor(device))


def run_forward(run, g, p=None, routing=True):
    p = p or problem_of(run)
    ws = M.workspace(p)
    y = torch.empty(run.T * run.d_model, dtype=torch.float32, device="cuda")
    r = routing_outputs(p) if routing else None
    M.moe_ffn_forward(p, weights_of(g), g["x"], y, ws, routing=r)
    torch.cuda.synchronize()
    out = {k: v.cpu().numpy() for k, v in (r or {}).items() if k != "stats"}
    if r:
        out["stats"] = M.route_stats_dict(r["stats"])
    out["y"] = y.view(run.T, run.d_model).cpu().numpy()
    return out


def compare_forward(run, gpu, orc, inp=None, token_subset=None, w_fp8=None):
    """Full comparison of a forward pass against the oracle.

    orc: the oracle's own forward (or only its routing, oracle_routing).  The
    GPU's selection is checked against the oracle's own (check_routing); then
    the layer is compared at the GPU's selection: when that differs from the
    oracle's (a near-tie flip, or slots in another order) or orc holds no y,
    the oracle is evaluated again at the GPU's topk_idx (needs inp), so the
    dispatch outputs are bit-exact and y is compared on every token."""
    k, E, T = run.top_k, run.num_experts, run.T
    gi = gpu["topk_idx"].reshape(T, k)
    same = check_routing(gi, orc, k)
    if not np.array_equal(gi, orc["idx"]) or "y" not in orc:
        assert inp is not None, "the oracle at the GPU's selection needs the inputs"
        n_flip = int((~np.all(gi == orc["idx"], axis=1)).sum())
        print(f"  oracle evaluated at the GPU's selection ({n_flip} tokens differ from its own)",
              flush=True)
        orc = oracle_forward(run, inp, token_subset=token_subset, w_fp8=w_fp8, idx=gi)
    check_dispatch_bitexact(gpu, orc, E)
    assert_close(gpu["topk_w"].reshape(T, k), orc["w"], "topk_w")
    assert_close(gpu["probs"].reshape(T, E), orc["probs"], "probs")
    toks = orc["tokens"]
    assert_close(gpu["y"][toks], orc["y"], "y")
    # aux statistics (f from the shared selection's counts, P from the gate)
    print(f"  l_aux gpu={float(gpu['l_aux'][0]):.6f} oracle={orc['l_aux']:.6f}", flush=True)
    assert abs(float(gpu["l_aux"][0]) - orc["l_aux"]) <= LAUX_REL * abs(orc["l_aux"])
    assert_close(gpu["P"], orc["P"], "P", rel=1e-4, mabs=1e-5)
    np.testing.assert_allclose(gpu["f"], orc["f"], rtol=1e-6)
    check_route_stats(gpu["stats"], orc["stats"])
    return same


def check_route_stats(got, ref):
    """Routing health indicators: integers exact; float32 sums over at most 64
    experts within 1e-5 relative (entropies and CV also 1e-6 absolute)."""
    print(f"  stats gpu={got}", flush=True)
    assert got["dropped"] == ref["dropped"] and got["idle"] == ref["idle"]
    for key in ("entropy", "entropy_p", "entropy_max", "util_mean", "util_var", "util_cv"):
        assert abs(got[key] - ref[key]) <= 1e-5 * abs(ref[key]) + 1e-6, (key, got[key], ref[key])


def inputs_for(run):
    return make_inputs(run)


def compare_forward_ec(run, gpu, orc, inp=None, token_subset=None):
    """Expert-choice forward against the oracle.  Selection: experts whose
    C-th and (C+1)-th best scores differ by more than GAP pick exactly the
    oracle's tokens; elsewhere every picked token scores within GAP of the
    oracle's C-th best.  When the selections differ the oracle is evaluated
    again at the GPU's selection (needs inp); y is compared on every token."""
    T, E = run.T, run.num_experts
    C = oracle_capacity(run)
    probs = orc["probs"]
    assert_close(gpu["probs"].reshape(T, E), probs, "probs")
    assert np.array_equal(gpu["offsets"], np.arange(E + 1) * C)
    assert np.all(gpu["counts"] == C) and np.all(gpu["kept"] == C)
    gsel = gpu["sorted_assign"].reshape(E, C)
    kth = -np.sort(-probs, axis=0)[C - 1]
    for e in range(E):
        assert np.all(np.diff(gsel[e]) > 0), "tokens of an expert not ascending"
        if orc["gap"][e] > GAP:
            assert np.array_equal(gsel[e], orc["sel"][e]), f"expert {e} picked other tokens"
        else:
            assert np.all(probs[gsel[e], e] >= kth[e] - GAP)
    if not np.array_equal(gsel, orc["sel"]):
        assert inp is not None, "the oracle at the GPU's selection needs the inputs"
        n = int((gsel != orc["sel"]).any(axis=1).sum())
        print(f"  oracle evaluated at the GPU's selection ({n} experts differ)", flush=True)
        orc = oracle_forward(run, inp, token_subset=token_subset, sel=gsel)
    row_of = gpu["assign_row"].reshape(T, E)
    assert np.array_equal(row_of, orc["row_of"]), "row_of"
    assert np.array_equal(gpu["token_experts"], orc["token_experts"])
    toks = orc["tokens"]
    assert_close(gpu["y"][toks], orc["y"], "y")
    np.testing.assert_allclose(gpu["f"], np.full(E, 1.0 / E), rtol=1e-6)
    assert_close(gpu["P"], probs.mean(0), "P", rel=1e-4, mabs=1e-5)
    check_route_stats(gpu["stats"], O.routing_stats(gpu["counts"], gpu["kept"], gpu["P"]))
