"""Pins of the float64 oracle against what the pages and the mathematics fix:
the pages' worked top-k example, closed forms, library routines and brute
force on tiny inputs.  CPU only."""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F
from scipy.special import ndtr

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as fh:
        return json.load(fh)


# ---------------------------------------------------------------- top-k + renorm

def test_worked_example_exact():
    g = _golden("worked_example_topk.json")
    idx, w = O.topk_renorm(np.array([g["scores"]]), g["k"])
    assert idx[0].tolist() == g["indices"]
    np.testing.assert_allclose(w[0], g["weights"], rtol=0, atol=1e-15)


def test_worked_example_via_router_softmax():
    # Logits ln(p) reproduce the example's scores through the softmax gate.
    g = _golden("worked_example_topk.json")
    logits = np.log(np.array([g["scores"]]))
    p = O.softmax(logits)
    np.testing.assert_allclose(p[0], g["scores"], rtol=1e-14)
    idx, w = O.topk_renorm(p, g["k"])
    assert idx[0].tolist() == g["indices"]
    np.testing.assert_allclose(w[0], g["weights"], rtol=1e-12)


def test_topk_ties_go_to_lower_index():
    idx, w = O.topk_renorm(np.array([[0.25, 0.25, 0.25, 0.25]]), 2)
    assert idx[0].tolist() == [0, 1]
    np.testing.assert_allclose(w[0], [0.5, 0.5])
    idx, _ = O.topk_renorm(np.array([[0.1, 0.3, 0.3, 0.3]]), 2)
    assert idx[0].tolist() == [1, 2]
    # the worked example's tie (0.1 at experts 0 and 3) decides the third slot
    idx, _ = O.topk_renorm(np.array([[0.1, 0.5, 0.3, 0.1]]), 3)
    assert idx[0].tolist() == [1, 2, 0]
    # many experts in few tie groups: within a group, ascending index
    s = np.repeat(np.array([0.2, 0.5, 0.1, 0.5, 0.2]), 13)[None, :]
    s = np.concatenate([s, s[:, ::-1]])
    idx, _ = O.topk_renorm(s, 30)
    n = s.shape[1]
    for row in range(2):
        order = sorted(range(n), key=lambda e: (-s[row, e], e))
        assert idx[row].tolist() == order[:30]


def test_topk_descending_slots_and_weights_sum_to_one():
    rng = np.random.default_rng(7)
    s = rng.random((200, 9))
    for k in (1, 2, 3, 9):
        idx, w = O.topk_renorm(s, k)
        sel = np.take_along_axis(s, idx.astype(np.int64), axis=1)
        assert np.all(np.diff(sel, axis=1) <= 0)
        # every unselected score is below the k-th selected one
        mask = np.ones_like(s, dtype=bool)
        np.put_along_axis(mask, idx.astype(np.int64), False, axis=1)
        other = np.where(mask, s, -np.inf).max(axis=1)
        assert np.all(other <= sel[:, -1])
        np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-15)
        if k == 1:
            assert np.all(w == 1.0)
    # agrees with torch.topk where no ties exist
    tv, ti = torch.topk(torch.from_numpy(s), 3, dim=1)
    idx, _ = O.topk_renorm(s, 3)
    assert np.array_equal(idx, ti.numpy())


def test_selection_gap():
    gap = O.selection_gap(np.array([[0.1, 0.5, 0.3, 0.1], [0.4, 0.4, 0.1, 0.1]]), 2)
    np.testing.assert_allclose(gap, [0.2, 0.3])
    assert O.selection_gap(np.array([[0.5, 0.5]]), 2)[0] == np.inf


# ---------------------------------------------------------------- gates

def test_softmax_closed_form():
    p = O.softmax(np.log(np.array([[1.0, 2.0, 3.0, 4.0]])))
    np.testing.assert_allclose(p[0], [0.1, 0.2, 0.3, 0.4], rtol=1e-14)
    # shift invariance and large logits (max subtraction keeps it finite)
    p2 = O.softmax(np.log(np.array([[1.0, 2.0, 3.0, 4.0]])) + 1000.0)
    np.testing.assert_allclose(p2, p, rtol=1e-12)
    rng = np.random.default_rng(1)
    z = rng.normal(size=(50, 7)) * 3
    np.testing.assert_allclose(O.softmax(z), torch.softmax(torch.from_numpy(z), 1).numpy(),
                               rtol=1e-13)


def test_sigmoid_normalized_closed_form():
    # sigma(0) = 1/2, sigma(ln 3) = 3/4 -> normalized (0.4, 0.6)
    p = O.sigmoid_normalized(np.array([[0.0, math.log(3.0)]]))
    np.testing.assert_allclose(p[0], [0.4, 0.6], rtol=1e-14)
    rng = np.random.default_rng(2)
    z = rng.normal(size=(40, 6)) * 2
    p = O.sigmoid_normalized(z)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=1e-14)
    sig = torch.sigmoid(torch.from_numpy(z)).numpy()
    np.testing.assert_allclose(p, sig / sig.sum(axis=1, keepdims=True), rtol=1e-13)


def test_sigmoid_renorm_equals_selected_sigmoid_share():
    # Renormalizing the globally normalized scores over the selected experts
    # gives sigma_i / sum of the selected sigmas: logits (2, 1, 0, -1), k = 2.
    z = np.array([[2.0, 1.0, 0.0, -1.0]])
    idx, w = O.topk_renorm(O.sigmoid_normalized(z), 2)
    s0, s1 = 1 / (1 + math.exp(-2.0)), 1 / (1 + math.exp(-1.0))
    assert idx[0].tolist() == [0, 1]
    np.testing.assert_allclose(w[0], [s0 / (s0 + s1), s1 / (s0 + s1)], rtol=1e-14)


def test_router_logits_is_nn_linear():
    rng = np.random.default_rng(3)
    x, W, b = rng.normal(size=(11, 6)), rng.normal(size=(4, 6)), rng.normal(size=4)
    ref = F.linear(torch.from_numpy(x), torch.from_numpy(W), torch.from_numpy(b)).numpy()
    np.testing.assert_allclose(O.router_logits(x, W, b), ref, rtol=1e-13)
    ref0 = F.linear(torch.from_numpy(x), torch.from_numpy(W)).numpy()
    np.testing.assert_allclose(O.router_logits(x, W), ref0, rtol=1e-13)


# ---------------------------------------------------------------- activations / FFN

def test_gelu_is_exact_erf_form():
    assert O.gelu(np.array([0.0]))[0] == 0.0
    # gelu(z) = z * Phi(z); Phi(1) from the normal CDF
    np.testing.assert_allclose(O.gelu(np.array([1.0, -1.0, 2.5])),
                               np.array([1.0, -1.0, 2.5]) * ndtr([1.0, -1.0, 2.5]), rtol=1e-14)
    z = np.linspace(-6, 6, 241)
    ref = F.gelu(torch.from_numpy(z), approximate="none").numpy()
    np.testing.assert_allclose(O.gelu(z), ref, rtol=1e-12, atol=1e-15)
    tanh_form = F.gelu(torch.from_numpy(z), approximate="tanh").numpy()
    assert np.abs(O.gelu(z) - tanh_form).max() > 1e-4


def test_silu_values():
    np.testing.assert_allclose(O.silu(np.array([0.0, 1.0])), [0.0, 1.0 / (1.0 + math.exp(-1.0))],
                               rtol=1e-15)
    z = np.linspace(-8, 8, 161)
    np.testing.assert_allclose(O.silu(z), F.silu(torch.from_numpy(z)).numpy(), rtol=1e-13,
                               atol=1e-16)


def _torch_ffn(x, w_up, b_up, w_down, b_down, act):
    t = lambda a: None if a is None else torch.from_numpy(a)
    z = F.linear(t(x), t(w_up), t(b_up))
    if act == "relu":
        h = F.relu(z)
    elif act == "gelu":
        h = F.gelu(z)
    else:
        f = w_up.shape[0] // 2
        h = F.silu(z[:, :f]) * z[:, f:]
    return F.linear(h, t(w_down), t(b_down)).numpy()


@pytest.mark.parametrize("act", ["relu", "gelu", "swiglu"])
def test_expert_ffn_matches_linear_layers(act):
    rng = np.random.default_rng(4)
    d, f, m = 12, 20, 9
    F1 = 2 * f if act == "swiglu" else f
    x = rng.normal(size=(m, d))
    wu, wd = rng.normal(size=(F1, d)) * 0.3, rng.normal(size=(d, f)) * 0.3
    bu, bd = (None, None) if act == "swiglu" else (rng.normal(size=F1), rng.normal(size=d))
    np.testing.assert_allclose(O.expert_ffn(x, wu, bu, wd, bd, act),
                               _torch_ffn(x, wu, bu, wd, bd, act), rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------- dispatch

def _random_routing(rng, T, k, E, p=None):
    idx = np.empty((T, k), dtype=np.int32)
    for t in range(T):
        idx[t] = rng.choice(E, size=k, replace=False, p=p)
    return idx


def _bruteforce_dispatch(idx, E, cap):
    T, k = idx.shape
    flat = idx.reshape(-1)
    counts = np.array([np.count_nonzero(flat == e) for e in range(E)])
    kept = counts if cap is None else np.array([min(c, cap) for c in counts])
    rows, dropped = [], []
    for e in range(E):
        lst = np.nonzero(flat == e)[0]
        rows += list(lst[: kept[e]])
        dropped += list(lst[kept[e]:])
    return counts, kept, np.array(rows + dropped)


@pytest.mark.parametrize("T,k,E,cap", [(1, 1, 1, None), (37, 2, 5, None), (37, 2, 5, 9),
                                       (64, 3, 8, 1), (50, 4, 4, 0), (200, 6, 64, 20)])
def test_dispatch_bruteforce_and_invariants(T, k, E, cap):
    rng = np.random.default_rng(T * 131 + E)
    skew = np.arange(E, 0, -1, dtype=np.float64)
    idx = _random_routing(rng, T, k, E, skew / skew.sum())
    dsp = O.dispatch(idx, E, cap)
    counts, kept, perm = _bruteforce_dispatch(idx, E, cap)
    assert np.array_equal(dsp["counts"], counts)
    assert np.array_equal(dsp["kept"], kept)
    assert dsp["counts"].sum() == T * k
    assert np.array_equal(dsp["offsets"], np.concatenate([[0], np.cumsum(kept)]))
    assert np.array_equal(dsp["sorted_assign"], perm)
    assert sorted(dsp["sorted_assign"].tolist()) == list(range(T * k))
    nk = dsp["offsets"][-1]
    assert np.array_equal(dsp["assign_row"][dsp["sorted_assign"][:nk]], np.arange(nk))
    assert np.all(dsp["assign_row"][dsp["sorted_assign"][nk:]] == -1)
    assert np.array_equal(dsp["drop_mask"], (dsp["assign_row"] < 0).astype(np.uint8))
    # rows within each expert segment are in ascending token order
    for e in range(E):
        seg = dsp["sorted_assign"][dsp["offsets"][e]:dsp["offsets"][e + 1]]
        assert np.all(np.diff(seg // k) > 0)
        assert np.all(idx.reshape(-1)[seg] == e)


def test_capacity_values():
    assert O.capacity(4096, 2, 8, 1.25) == 1280
    assert O.capacity(8192, 6, 64, 1.25) == 960
    # the page's literal (tokens / experts) x CF for top-1
    assert O.capacity(4096, 1, 8, 1.25) == 640
    assert O.capacity(8192, 1, 64, 1.25) == 160
    assert O.capacity(10, 1, 3, 1.0) == 4          # rounds up
    assert O.capacity(10, 1, 3, None) is None


# ---------------------------------------------------------------- aux statistics

def test_aux_uniform_probs_gives_exactly_one():
    rng = np.random.default_rng(5)
    x = rng.normal(size=(64, 8))
    for E, k in ((4, 1), (8, 2), (6, 3)):
        p = O.softmax(O.router_logits(x, np.zeros((E, 8)), np.zeros(E)))
        idx, _ = O.topk_renorm(p, k)
        # ties send every token to experts 0..k-1, yet P is uniform
        assert np.all(idx == np.arange(k))
        f, P, L = O.aux_stats(idx, p, E)
        assert abs(L - 1.0) < 1e-14
        g = _golden("page_numbers.json")["uniform_aux"]["value"]
        assert abs(L - g) < 1e-14


def test_aux_uniform_assignment_gives_one_and_collapse_gives_E_P():
    rng = np.random.default_rng(6)
    E, k, T = 8, 2, 64
    p = rng.dirichlet(np.ones(E), size=T)
    idx = np.array([[(2 * t) % E, (2 * t + 1) % E] for t in range(T)], dtype=np.int32)
    f, P, L = O.aux_stats(idx, p, E)
    np.testing.assert_allclose(f, 1.0 / E)
    assert abs(L - 1.0) < 1e-14
    assert abs(f.sum() - 1.0) < 1e-15 and abs(P.sum() - 1.0) < 1e-14
    # collapse onto expert 3 with top-1: L = E * P_3
    idx1 = np.full((T, 1), 3, dtype=np.int32)
    f, P, L = O.aux_stats(idx1, p, E)
    assert abs(L - E * P[3]) < 1e-14
    # a single expert
    f, P, L = O.aux_stats(np.zeros((T, 1), dtype=np.int32), np.ones((T, 1)), 1)
    assert L == 1.0


# ---------------------------------------------------------------- whole forward

def _tiny_problem(rng, T, d, f, E, S, act, bias, router_bias=True):
    F1 = 2 * f if act == "swiglu" else f
    return dict(
        x=rng.normal(size=(T, d)),
        w_router=rng.normal(size=(E, d)) * 0.7,
        b_router=rng.normal(size=E) * 0.1 if router_bias else None,
        w_up=rng.normal(size=(E + S, F1, d)) * 0.3,
        b_up=rng.normal(size=(E + S, F1)) * 0.1 if bias else None,
        w_down=rng.normal(size=(E + S, d, f)) * 0.3,
        b_down=rng.normal(size=(E + S, d)) * 0.1 if bias else None)


def _dense_masked(P, T, E, S, k, gating, act, cap):
    """Every expert on every token, multiplied by a dense (token, expert)
    weight that is w for kept selections and 0 otherwise, plus the shared
    experts unmasked (the dense-masked MoE layer of the yunthe page).
    Routing uses torch.topk on tie-free scores; drops use a direct recount."""
    logits = F.linear(torch.from_numpy(P["x"]), torch.from_numpy(P["w_router"]),
                      None if P["b_router"] is None else torch.from_numpy(P["b_router"]))
    if gating == "softmax":
        scores = torch.softmax(logits, dim=1)
    else:
        sg = torch.sigmoid(logits)
        scores = sg / sg.sum(dim=1, keepdim=True)
    top, ti = torch.topk(scores, k, dim=1)
    tw = top / top.sum(dim=1, keepdim=True)
    mask = torch.zeros(T, E, dtype=torch.float64)
    seen = [0] * E
    for t in range(T):
        for s in range(k):
            e = int(ti[t, s])
            if cap is None or seen[e] < cap:
                mask[t, e] = tw[t, s]
            seen[e] += 1
    y = torch.zeros(T, P["x"].shape[1], dtype=torch.float64)
    bu = lambda q: None if P["b_up"] is None else P["b_up"][q]
    bd = lambda q: None if P["b_down"] is None else P["b_down"][q]
    for e in range(E):
        out = _torch_ffn(P["x"], P["w_up"][e], bu(e), P["w_down"][e], bd(e), act)
        y += mask[:, e:e + 1] * torch.from_numpy(out)
    for q in range(E, E + S):
        y += torch.from_numpy(_torch_ffn(P["x"], P["w_up"][q], bu(q), P["w_down"][q], bd(q), act))
    return y.numpy(), scores.numpy(), ti.numpy()


@pytest.mark.parametrize("T,d,f,E,S,k,gating,act,bias,cap", [
    (23, 8, 12, 5, 0, 2, "softmax", "gelu", True, None),
    (23, 8, 12, 5, 0, 2, "softmax", "relu", True, 7),
    (30, 8, 6, 6, 2, 3, "sigmoid_norm", "swiglu", False, 12),
    (17, 4, 8, 4, 1, 1, "softmax", "swiglu", False, 3),
])
def test_forward_equals_dense_masked_bruteforce(T, d, f, E, S, k, gating, act, bias, cap):
    rng = np.random.default_rng(T + 100 * E + k)
    P = _tiny_problem(rng, T, d, f, E, S, act, bias)
    out = O.forward(**P, top_k=k, num_shared=S, gating=gating, activation=act, cap=cap)
    y_ref, scores, ti = _dense_masked(P, T, E, S, k, gating, act, cap)
    assert np.all(out["gap"] > 1e-6)          # tie-free, so torch.topk is unique
    np.testing.assert_allclose(out["probs"], scores, rtol=1e-13)
    assert np.array_equal(out["idx"], ti)
    np.testing.assert_allclose(out["y"], y_ref, rtol=1e-11, atol=1e-12)
    if cap is not None:
        assert out["drop_mask"].sum() > 0 or k * T <= cap * E


def test_single_expert_top1_is_the_dense_ffn():
    # E = 1, k = 1: the layer reduces to one FFN (kamacoder section 一 FeedForward)
    rng = np.random.default_rng(8)
    P = _tiny_problem(rng, 19, 8, 16, 1, 0, "relu", True)
    out = O.forward(**P, top_k=1, num_shared=0, gating="softmax", activation="relu")
    ref = _torch_ffn(P["x"], P["w_up"][0], P["b_up"][0], P["w_down"][0], P["b_down"][0], "relu")
    np.testing.assert_allclose(out["y"], ref, rtol=1e-12, atol=1e-14)
    assert out["l_aux"] == 1.0


def test_all_experts_selected_is_probability_mixture():
    # k = E with softmax and no capacity: y = sum_e p_e FFN_e(x)
    rng = np.random.default_rng(9)
    E = 4
    P = _tiny_problem(rng, 15, 6, 10, E, 0, "gelu", True)
    out = O.forward(**P, top_k=E, num_shared=0, gating="softmax", activation="gelu")
    p = out["probs"]
    ref = sum(p[:, e:e + 1] * _torch_ffn(P["x"], P["w_up"][e], P["b_up"][e], P["w_down"][e],
                                         P["b_down"][e], "gelu") for e in range(E))
    np.testing.assert_allclose(out["y"], ref, rtol=1e-11, atol=1e-13)


def test_token_subset_and_combine_rows_agree_with_full_forward():
    rng = np.random.default_rng(10)
    T, E, S, k = 40, 6, 2, 2
    P = _tiny_problem(rng, T, 8, 12, E, S, "swiglu", False)
    full = O.forward(**P, top_k=k, num_shared=S, gating="softmax", activation="swiglu", cap=12)
    sub = [3, 17, 39]
    part = O.forward(**P, top_k=k, num_shared=S, gating="softmax", activation="swiglu", cap=12,
                     token_subset=sub)
    np.testing.assert_allclose(part["y"], full["y"][sub], rtol=1e-13, atol=1e-15)
    # combine_rows from per-row expert outputs
    nk = int(full["offsets"][-1])
    y_rows = np.zeros((nk + S * T, 8))
    for r in range(nk):
        a = int(full["sorted_assign"][r])
        e = int(full["idx"].reshape(-1)[a])
        y_rows[r] = O.expert_ffn(P["x"][a // k][None], P["w_up"][e], None, P["w_down"][e], None,
                                 "swiglu")[0]
    for q in range(S):
        y_rows[nk + q * T: nk + (q + 1) * T] = O.expert_ffn(P["x"], P["w_up"][E + q], None,
                                                             P["w_down"][E + q], None, "swiglu")
    y = O.combine_rows(y_rows, full["w"], full["assign_row"], nk, S)
    np.testing.assert_allclose(y, full["y"], rtol=1e-12, atol=1e-14)


def test_page_parameter_counts():
    g = _golden("page_numbers.json")
    d, f = g["dense_ffn_params"]["d_model"], g["dense_ffn_params"]["ffn_dim"]
    from synth import RUNS
    r = RUNS["gpt2"]
    assert (r.d_model, r.d_ff) == (d, f)
    per_expert = r.up_rows * r.d_model + r.d_model * r.d_ff      # weight matrices
    assert abs(per_expert / g["dense_ffn_params"]["approx_params"] - 1) < g["dense_ffn_params"]["rel_tol"]
    four = g["four_expert_params"]
    assert abs(four["num_experts"] * per_expert / four["approx_params"] - 1) < four["rel_tol"]
    # k of E experts: the rows the experts evaluate are k/E of the dense all-expert work
    sf = g["sparse_fraction"]
    rng = np.random.default_rng(11)
    idx = _random_routing(rng, 32, sf["top_k"], sf["num_experts"])
    dsp = O.dispatch(idx, sf["num_experts"], None)
    assert dsp["offsets"][-1] / (32 * sf["num_experts"]) == sf["fraction"]


# ---------------------------------------------------------------- routing health statistics

def test_routing_stats_uniform_is_maximal_and_balanced():
    E = 8
    st = O.routing_stats(np.full(E, 100), np.full(E, 100), np.full(E, 1.0 / E))
    assert st["entropy"] == pytest.approx(math.log(E), rel=1e-15)
    assert st["entropy_p"] == pytest.approx(math.log(E), rel=1e-15)
    assert st["entropy_max"] == pytest.approx(math.log(E), rel=1e-15)
    assert st["util_var"] == 0.0 and st["util_cv"] == 0.0
    assert st["dropped"] == 0 and st["idle"] == 0


def test_routing_stats_collapse_to_one_expert():
    # all n assignments to one expert: entropy 0; kept values (n, 0, ..., 0)
    # have mean n/E, population std n sqrt(E-1)/E, so CV = sqrt(E-1)
    E, n = 6, 600
    counts = np.zeros(E, dtype=np.int64)
    counts[2] = n
    st = O.routing_stats(counts, counts, np.eye(E)[2])
    assert st["entropy"] == 0.0 and st["entropy_p"] == 0.0
    assert st["util_mean"] == pytest.approx(n / E)
    assert st["util_var"] == pytest.approx(n * n * (E - 1) / E ** 2)
    assert st["util_cv"] == pytest.approx(math.sqrt(E - 1), rel=1e-14)
    assert st["idle"] == E - 1 and st["dropped"] == 0


def test_routing_stats_hand_example_and_drops():
    # shares (1/2, 1/4, 1/4): H = ln2/2 + 2 * ln4/4 = 1.5 ln 2
    counts = np.array([4, 2, 2])
    kept = np.array([3, 2, 0])   # capacity 3 drops one; an expert whose kept rows were all dropped is idle
    st = O.routing_stats(counts, kept, np.array([0.5, 0.3, 0.2]))
    assert st["entropy"] == pytest.approx(1.5 * math.log(2.0), rel=1e-15)
    assert st["entropy_p"] == pytest.approx(-(0.5 * math.log(0.5) + 0.3 * math.log(0.3) +
                                             0.2 * math.log(0.2)), rel=1e-15)
    assert st["dropped"] == 3 and st["idle"] == 1
    m = 5.0 / 3.0
    var = ((3 - m) ** 2 + (2 - m) ** 2 + (0 - m) ** 2) / 3.0
    assert st["util_var"] == pytest.approx(var, rel=1e-14)
    assert st["util_cv"] == pytest.approx(math.sqrt(var) / m, rel=1e-14)


def test_routing_stats_invariant_under_expert_relabeling():
    rng = np.random.default_rng(7)
    counts = rng.integers(0, 50, size=16)
    kept = np.minimum(counts, 30)
    P = rng.random(16)
    P /= P.sum()
    perm = rng.permutation(16)
    a = O.routing_stats(counts, kept, P)
    b = O.routing_stats(counts[perm], kept[perm], P[perm])
    for key in a:
        assert a[key] == pytest.approx(b[key], rel=1e-13, abs=1e-15)


def test_routing_stats_of_forward_match_its_dispatch():
    rng = np.random.default_rng(3)
    T, d, f, E, k = 40, 8, 16, 5, 2
    x = rng.standard_normal((T, d))
    wr = rng.standard_normal((E, d))
    w_up = rng.standard_normal((E, f, d)) * 0.1
    w_dn = rng.standard_normal((E, d, f)) * 0.1
    out = O.forward(x, wr, None, w_up, None, w_dn, None, top_k=k, num_shared=0,
                    gating="softmax", activation="relu", cap=10)
    st = out["stats"]
    assert st["dropped"] == int(np.sum(out["drop_mask"]))
    assert st["dropped"] == T * k - int(out["offsets"][-1])
    share = np.bincount(out["idx"].reshape(-1), minlength=E) / (T * k)
    assert np.allclose(share, out["f"])


# ---------------------------------------------------------------- FP8 E4M3 expert weights

def _q1(v):
    """Code of one value with scale 1 (a row [448, v] keeps scale 448/448 = 1)."""
    c, s = O.quantize_fp8_rows(np.array([[448.0, v]], dtype=np.float32))
    assert s[0] == 1.0
    return int(c[0, 1])


def test_e4m3_table_matches_the_format_definition():
    vals = O.e4m3_values()
    assert vals.size == 127 and vals[0] == 0.0 and vals[-1] == 448.0
    assert vals[1] == 2.0 ** -9 and vals[8] == 2.0 ** -6 and vals[0x38] == 1.0
    assert np.all(np.diff(vals) > 0)          # codes are ordered by value
    assert len(set(vals.tolist())) == 127
    # the spacing within a binade is an eighth of its lower bound
    assert vals[0x39] - vals[0x38] == 0.125 and vals[0x79] - vals[0x78] == 32.0


def test_e4m3_known_codes_ties_and_saturation():
    assert _q1(0.0) == 0x00 and _q1(1.0) == 0x38 and _q1(-1.0) == 0xB8
    assert _q1(0.5) == 0x30 and _q1(1.125) == 0x39 and _q1(2.0 ** -9) == 0x01
    assert _q1(2.0 ** -6) == 0x08 and _q1(-448.0) == 0xFE
    assert _q1(1.0625) == 0x38           # tie between 1.0 (even) and 1.125
    assert _q1(1.1875) == 0x3A           # tie between 1.125 and 1.25 (even)
    assert _q1(1.5 * 2.0 ** -9) == 0x02  # subnormal tie goes to the even code
    assert _q1(0.5 * 2.0 ** -9) == 0x00  # half the smallest subnormal rounds to zero
    assert _q1(1.01 * 2.0 ** -10) == 0x01
    assert _q1(447.0) == 0x7E and _q1(431.0) == 0x7D   # 416 and 448 are neighbours
    # the row maximum maps to +-448 whatever its size (so magnitudes never exceed it)
    c, s = O.quantize_fp8_rows(np.array([[1000.0, -1000.0, 500.0]], dtype=np.float32))
    assert c[0, 0] == 0x7E and c[0, 1] == 0xFE and s[0] == np.float32(1000.0) / np.float32(448.0)


def test_e4m3_every_finite_value_round_trips():
    vals = O.e4m3_values()
    row = np.concatenate([[448.0], vals, -vals[1:]]).astype(np.float32)[None, :]
    codes, scales = O.quantize_fp8_rows(row)
    assert scales[0] == 1.0
    back = O.dequantize_fp8_rows(codes, scales)
    assert np.array_equal(back, row.astype(np.float64))


def test_fp8_rows_scale_error_bound_and_zero_row():
    rng = np.random.default_rng(5)
    w = (rng.standard_normal((6, 300)) * 0.02).astype(np.float32)
    w[3] = 0.0
    codes, scales = O.quantize_fp8_rows(w)
    assert scales[3] == 1.0 and not codes[3].any()
    amax = np.abs(w).max(axis=1)
    nz = amax > 0
    assert np.array_equal(scales[nz], (amax[nz] / np.float32(448.0)).astype(np.float32))
    # each row's largest magnitude maps to +-448
    for r in np.flatnonzero(nz):
        assert (int(codes[r, np.argmax(np.abs(w[r]))]) & 0x7F) == 0x7E
    back = O.dequantize_fp8_rows(codes, scales)
    # nearest-value rounding: error <= half a step, i.e. 2^-4 relative in the
    # normal range, half the subnormal step 2^-10 * s below it
    err = np.abs(back - w.astype(np.float64))
    bound = np.maximum(np.abs(w) * 2.0 ** -4, scales[:, None].astype(np.float64) * 2.0 ** -10)
    assert np.all(err <= bound * (1 + 1e-6))
    # and the rounding is to the nearest representable value
    vals = np.concatenate([-O.e4m3_values()[::-1], O.e4m3_values()[1:]])
    v = (w[0] / scales[0]).astype(np.float64)
    nearest = np.abs(vals[None, :] - v[:, None]).min(axis=1)
    assert np.allclose(np.abs(back[0] / scales[0] - v), nearest, rtol=0, atol=1e-12)


# ---------------------------------------------------------------- expert-choice routing

def test_expert_choice_hand_example():
    # 4 tokens, 2 experts, C = 2.  Expert 0 scores (.5, .2, .5, .1): tie at .5
    # -> tokens 0 and 2; expert 1 scores (.5, .8, .5, .9) -> tokens 3 and 1.
    probs = np.array([[0.5, 0.5], [0.2, 0.8], [0.5, 0.5], [0.1, 0.9]])
    sel, row_of, te = O.expert_choice_select(probs, 2)
    assert sel.tolist() == [[0, 2], [1, 3]]
    assert row_of.tolist() == [[0, -1], [-1, 2], [1, -1], [-1, 3]]
    assert te.tolist() == [1, 1, 1, 1]
    # ties go to the lower token index
    sel, _, te = O.expert_choice_select(np.array([[0.3, 0.7]] * 5), 3)
    assert sel.tolist() == [[0, 1, 2], [0, 1, 2]] and te.tolist() == [2, 2, 2, 0, 0]


def test_expert_choice_bruteforce_and_balance():
    rng = np.random.default_rng(4)
    for T, E, C in [(9, 3, 4), (20, 5, 7), (6, 4, 6)]:
        probs = np.round(rng.random((T, E)), 1)   # many ties
        sel, row_of, te = O.expert_choice_select(probs, C)
        for e in range(E):
            ranked = sorted(range(T), key=lambda t: (-probs[t, e], t))[:C]
            assert sel[e].tolist() == sorted(ranked)
            assert np.array_equal(np.flatnonzero(row_of[:, e] >= 0), sel[e])
            assert np.array_equal(row_of[sel[e], e], e * C + np.arange(C))
        assert te.sum() == E * C                   # exactly C tokens per expert
        assert np.array_equal(te, (row_of >= 0).sum(1))


def test_expert_choice_capacity_T_is_the_probability_mixture():
    # every expert takes every token: y = sum_e p[t,e] FFN_e(x_t), the dense
    # soft mixture, which equals token choice with k = E
    rng = np.random.default_rng(8)
    T, d, f, E = 6, 5, 7, 3
    x = rng.standard_normal((T, d))
    wr = rng.standard_normal((E, d))
    w_up = rng.standard_normal((E, f, d)) * 0.3
    w_dn = rng.standard_normal((E, d, f)) * 0.3
    ec = O.forward_expert_choice(x, wr, None, w_up, None, w_dn, None, capacity=T, num_shared=0,
                                 gating="softmax", activation="relu")
    tc = O.forward(x, wr, None, w_up, None, w_dn, None, top_k=E, num_shared=0,
                   gating="softmax", activation="relu")
    assert np.allclose(ec["y"], tc["y"], rtol=1e-12, atol=1e-13)
    assert np.all(ec["token_experts"] == E)


def test_expert_choice_orphans_get_only_shared_experts():
    rng = np.random.default_rng(9)
    T, d, f, E, S = 10, 4, 6, 2, 1
    x = rng.standard_normal((T, d))
    wr = rng.standard_normal((E, d))
    w_up = rng.standard_normal((E + S, f, d)) * 0.3
    w_dn = rng.standard_normal((E + S, d, f)) * 0.3
    out = O.forward_expert_choice(x, wr, None, w_up, None, w_dn, None, capacity=2, num_shared=S,
                                  gating="softmax", activation="gelu")
    orphans = np.flatnonzero(out["token_experts"] == 0)
    assert orphans.size >= T - 2 * E
    shared = O.expert_ffn(x[orphans], w_up[E], None, w_dn[E], None, "gelu")
    assert np.allclose(out["y"][orphans], shared, rtol=1e-13, atol=1e-14)
    # a picked token: its experts' weighted outputs plus the shared expert
    t = int(np.flatnonzero(out["token_experts"] > 0)[0])
    ref = O.expert_ffn(x[[t]], w_up[E], None, w_dn[E], None, "gelu")[0]
    for e in range(E):
        if out["row_of"][t, e] >= 0:
            ref = ref + out["probs"][t, e] * O.expert_ffn(x[[t]], w_up[e], None, w_dn[e], None,
                                                          "gelu")[0]
    assert np.allclose(out["y"][t], ref, rtol=1e-12, atol=1e-14)


def test_expert_choice_gap_hand_values():
    # expert 0 column (.9, .5, .3, .2): C = 2 -> .5 - .3; C = 3 -> .3 - .2
    # expert 1 column (.4, .4, .1, 0): C = 1 -> an exact tie, gap 0
    probs = np.array([[0.9, 0.4], [0.5, 0.4], [0.3, 0.1], [0.2, 0.0]])
    g2 = O.expert_choice_gap(probs, 2)
    assert g2[0] == pytest.approx(0.2, abs=1e-15) and g2[1] == pytest.approx(0.3, abs=1e-15)
    g1 = O.expert_choice_gap(probs, 1)
    assert g1[0] == pytest.approx(0.4, abs=1e-15) and g1[1] == 0.0
    g3 = O.expert_choice_gap(probs, 3)
    assert g3[0] == pytest.approx(0.1, abs=1e-15) and g3[1] == pytest.approx(0.1, abs=1e-15)
    # every token taken: nothing is left out, the gap is infinite
    assert np.all(O.expert_choice_gap(probs, 4) == np.inf)
    assert np.all(O.expert_choice_gap(probs, 9) == np.inf)
    # the gap is the C-th best minus the (C+1)-th best, whatever the token order
    rng = np.random.default_rng(12)
    p = rng.random((11, 3))
    for C in range(1, 11):
        for e in range(3):
            col = sorted(p[:, e], reverse=True)
            assert O.expert_choice_gap(p, C)[e] == col[C - 1] - col[C]


def _selection_bruteforce(P, idx, probs, E, S, act, cap):
    """y at a given selection, written out per token: w = the selected
    probabilities renormalized, a slot is dropped once its expert already holds
    cap earlier assignments (token order, then slot), shared experts unmasked."""
    T, k = idx.shape
    bu = lambda q: None if P["b_up"] is None else P["b_up"][q]
    bd = lambda q: None if P["b_down"] is None else P["b_down"][q]
    outs = [_torch_ffn(P["x"], P["w_up"][q], bu(q), P["w_down"][q], bd(q), act)
            for q in range(E + S)]
    seen = [0] * E
    y = np.zeros((T, P["x"].shape[1]))
    for t in range(T):
        tot = sum(probs[t, int(e)] for e in idx[t])
        for s in range(k):
            e = int(idx[t, s])
            if cap is None or seen[e] < cap:
                y[t] += probs[t, e] / tot * outs[e][t]
            seen[e] += 1
        for q in range(E, E + S):
            y[t] += outs[q][t]
    return y


@pytest.mark.parametrize("gating,act,cap", [("softmax", "gelu", None), ("softmax", "relu", 5),
                                            ("sigmoid_norm", "swiglu", 4)])
def test_forward_at_a_given_selection(gating, act, cap):
    rng = np.random.default_rng(21)
    T, d, f, E, S, k = 16, 6, 8, 5, 1, 2
    P = _tiny_problem(rng, T, d, f, E, S, act, act != "swiglu")
    own = O.forward(**P, top_k=k, num_shared=S, gating=gating, activation=act, cap=cap)
    # the oracle's own selection given back reproduces the forward exactly
    same = O.forward(**P, top_k=k, num_shared=S, gating=gating, activation=act, cap=cap,
                     idx=own["idx"])
    for key in ("y", "w", "l_aux", "f", "counts", "offsets", "sorted_assign", "assign_row",
                "drop_mask"):
        assert np.array_equal(np.asarray(same[key]), np.asarray(own[key])), key
    # another selection: second-best and third-best experts on every other
    # token, slot order reversed on token 1
    order = np.argsort(-own["probs"], axis=1, kind="stable")
    idx = own["idx"].copy()
    idx[::2] = order[::2, 1:3]
    idx[1] = idx[1, ::-1]
    out = O.forward(**P, top_k=k, num_shared=S, gating=gating, activation=act, cap=cap, idx=idx)
    assert np.array_equal(out["idx"], idx)
    np.testing.assert_allclose(out["w"].sum(1), 1.0, rtol=1e-15)
    sel = np.take_along_axis(own["probs"], idx.astype(np.int64), axis=1)
    np.testing.assert_allclose(out["w"], sel / sel.sum(1, keepdims=True), rtol=1e-15)
    ref = _selection_bruteforce(P, idx, own["probs"], E, S, act, cap)
    np.testing.assert_allclose(out["y"], ref, rtol=1e-11, atol=1e-12)
    # f follows the given selection, P the gate (unchanged), gap the own scores
    np.testing.assert_array_equal(out["f"], np.bincount(idx.reshape(-1), minlength=E) / (T * k))
    np.testing.assert_array_equal(out["P"], own["P"])
    np.testing.assert_array_equal(out["gap"], own["gap"])
    assert out["l_aux"] == pytest.approx(E * np.sum(out["f"] * own["P"]), rel=1e-15)


def test_routing_matches_the_forward():
    rng = np.random.default_rng(22)
    P = _tiny_problem(rng, 12, 6, 8, 4, 0, "relu", True)
    r = O.routing(P["x"], P["w_router"], P["b_router"], top_k=2, gating="softmax")
    fw = O.forward(**P, top_k=2, num_shared=0, gating="softmax", activation="relu")
    for key in ("logits", "probs", "idx", "w", "gap"):
        assert np.array_equal(r[key], fw[key]), key


def test_expert_choice_at_a_given_selection():
    rng = np.random.default_rng(23)
    T, d, f, E, S, C = 12, 5, 6, 3, 1, 4
    x = rng.standard_normal((T, d))
    wr = rng.standard_normal((E, d))
    w_up = rng.standard_normal((E + S, f, d)) * 0.3
    w_dn = rng.standard_normal((E + S, d, f)) * 0.3
    kw = dict(capacity=C, num_shared=S, gating="softmax", activation="relu")
    own = O.forward_expert_choice(x, wr, None, w_up, None, w_dn, None, **kw)
    same = O.forward_expert_choice(x, wr, None, w_up, None, w_dn, None, sel=own["sel"], **kw)
    for key in ("y", "sel", "row_of", "token_experts"):
        assert np.array_equal(same[key], own[key]), key
    # expert 0 takes its C worst tokens instead
    sel = own["sel"].copy()
    sel[0] = np.sort(np.argsort(own["probs"][:, 0], kind="stable")[:C])
    out = O.forward_expert_choice(x, wr, None, w_up, None, w_dn, None, sel=sel, **kw)
    ref = O.expert_ffn(x, w_up[E], None, w_dn[E], None, "relu")
    for e in range(E):
        fe = O.expert_ffn(x, w_up[e], None, w_dn[e], None, "relu")
        for t in sel[e]:
            ref[t] += own["probs"][t, e] * fe[t]
    np.testing.assert_allclose(out["y"], ref, rtol=1e-12, atol=1e-13)
    row_of = out["row_of"]
    for e in range(E):
        assert np.array_equal(np.flatnonzero(row_of[:, e] >= 0), sel[e])
        assert np.array_equal(row_of[sel[e], e], e * C + np.arange(C))
    assert np.array_equal(out["token_experts"], (row_of >= 0).sum(1))
