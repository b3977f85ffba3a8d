"""Pins of the backward oracle (CPU only).

1. Central finite differences of the forward oracle: the objective
   L = <dy, y> + alpha * L_aux is evaluated by oracle.forward at theta +- h
   for every entry of x and of every parameter; tie-free random inputs keep
   the top-k selection and the capacity drops fixed within +- h (checked).
2. float64 torch autograd of the same layer written as a torch expression
   with the oracle's selection held fixed.
3. Invariants: dropped slots get zero gate gradient; an expert with no kept
   rows gets zero weight gradients; alpha enters linearly.
4. The single-entry functions (a token's gradients, a row of dW1, a column
   of dW2) reproduce the full backward entry by entry.
"""
import numpy as np
import pytest
import torch

from oracle import moe_backward as B
from oracle import moe_oracle as O

CASES = {
    # name: activation, gating, shared, router bias, expert bias, capacity
    "gelu_softmax_drops": ("gelu", "softmax", 0, True, True, 4),
    "relu_softmax_shared": ("relu", "softmax", 1, True, True, None),
    "swiglu_sigmoid_shared_drops": ("swiglu", "sigmoid_norm", 2, True, False, 4),
    "gelu_sigmoid": ("gelu", "sigmoid_norm", 0, False, True, 3),
}
T, D, F, E, K = 9, 5, 4, 4, 2
ALPHA = 0.37


def make(case, seed=11):
    act, gating, S, rb, eb, cap = CASES[case]
    rng = np.random.default_rng(seed)
    F1 = 2 * F if act == "swiglu" else F
    p = dict(
        x=rng.normal(size=(T, D)),
        w_router=rng.normal(size=(E, D)) * 0.8,
        b_router=rng.normal(size=E) * 0.3 if rb else None,
        w_up=rng.normal(size=(E + S, F1, D)) * 0.5,
        b_up=rng.normal(size=(E + S, F1)) * 0.2 if eb else None,
        w_down=rng.normal(size=(E + S, D, F)) * 0.5,
        b_down=rng.normal(size=(E + S, D)) * 0.2 if eb else None,
    )
    dy = rng.normal(size=(T, D))
    kw = dict(top_k=K, num_shared=S, gating=gating, activation=act, cap=cap)
    return p, dy, kw


def objective(p, dy, kw, alpha):
    fw = O.forward(p["x"], p["w_router"], p["b_router"], p["w_up"], p["b_up"], p["w_down"],
                   p["b_down"], **kw)
    return float(np.sum(dy * fw["y"]) + alpha * fw["l_aux"]), fw


GRAD_OF = {"x": "dx", "w_router": "dw_router", "b_router": "db_router", "w_up": "dw_up",
           "b_up": "db_up", "w_down": "dw_down", "b_down": "db_down"}


@pytest.mark.parametrize("case", list(CASES))
def test_backward_matches_finite_differences(case):
    p, dy, kw = make(case)
    _, base = objective(p, dy, kw, ALPHA)
    # the inputs are tie-free: the k-th and (k+1)-th keys are well apart
    assert np.min(base["gap"]) > 1e-3
    g = B.backward(p["x"], p["w_router"], p["b_router"], p["w_up"], p["b_up"], p["w_down"],
                   p["b_down"], dy, alpha=ALPHA, **kw)
    assert np.array_equal(g["idx"], base["idx"])
    h = 1e-6
    for name, gname in GRAD_OF.items():
        if p[name] is None:
            assert g[gname] is None or gname == "db_router"
            continue
        arr = p[name]
        num = np.zeros_like(arr)
        for i in np.ndindex(arr.shape):
            old = arr[i]
            arr[i] = old + h
            lp, fp = objective(p, dy, kw, ALPHA)
            arr[i] = old - h
            lm, fm = objective(p, dy, kw, ALPHA)
            arr[i] = old
            assert np.array_equal(fp["idx"], base["idx"]) and np.array_equal(fm["idx"], base["idx"])
            num[i] = (lp - lm) / (2 * h)
        np.testing.assert_allclose(g[gname], num, rtol=1e-6, atol=1e-7, err_msg=f"{case}: {name}")


def test_backward_matches_torch_autograd():
    """The layer as a torch float64 expression (selection and drops fixed at
    the oracle's), differentiated by autograd."""
    for case in CASES:
        p, dy, kw = make(case, seed=5)
        act, gating, S = kw["activation"], kw["gating"], kw["num_shared"]
        g = B.backward(p["x"], p["w_router"], p["b_router"], p["w_up"], p["b_up"], p["w_down"],
                       p["b_down"], dy, alpha=ALPHA, **kw)
        idx = torch.tensor(g["idx"])
        keep = torch.tensor(g["assign_row"].reshape(T, K) >= 0)
        tp = {n: (None if v is None else torch.tensor(v, requires_grad=True)) for n, v in p.items()}
        x = tp["x"]
        logits = x @ tp["w_router"].T + (tp["b_router"] if tp["b_router"] is not None else 0)
        if gating == "softmax":
            probs = torch.softmax(logits, dim=1)
            keys = probs
        else:
            keys = torch.sigmoid(logits)
            probs = keys / keys.sum(dim=1, keepdim=True)
        sel = torch.gather(keys, 1, idx)
        w = sel / sel.sum(dim=1, keepdim=True)

        def ffn(q, xr):
            z = xr @ tp["w_up"][q].T
            if tp["b_up"] is not None:
                z = z + tp["b_up"][q]
            if act == "relu":
                hh = torch.relu(z)
            elif act == "gelu":
                hh = torch.nn.functional.gelu(z)
            else:
                hh = torch.nn.functional.silu(z[:, :F]) * z[:, F:]
            o = hh @ tp["w_down"][q].T
            if tp["b_down"] is not None:
                o = o + tp["b_down"][q]
            return o

        y = torch.zeros(T, D, dtype=torch.float64)
        for t in range(T):
            for s in range(K):
                if keep[t, s]:
                    y[t] = y[t] + w[t, s] * ffn(int(idx[t, s]), x[t:t + 1])[0]
        for q in range(S):
            y = y + ffn(E + q, x)
        f = torch.bincount(idx.reshape(-1), minlength=E).double() / (T * K)
        l_aux = E * torch.sum(f * probs.mean(dim=0))
        loss = torch.sum(torch.tensor(dy) * y) + ALPHA * l_aux
        loss.backward()
        for name, gname in GRAD_OF.items():
            if tp[name] is None:
                continue
            np.testing.assert_allclose(g[gname], tp[name].grad.numpy(), rtol=1e-9, atol=1e-12,
                                       err_msg=f"{case}: {name}")


def test_backward_invariants():
    p, dy, kw = make("gelu_softmax_drops")
    g = B.backward(p["x"], p["w_router"], p["b_router"], p["w_up"], p["b_up"], p["w_down"],
                   p["b_down"], dy, alpha=ALPHA, **kw)
    dropped = g["drop_mask"].reshape(T, K) == 1
    assert dropped.any()                       # the case exercises drops
    assert np.all(g["dw"][dropped] == 0.0)
    # alpha enters linearly, and only through the router
    g0 = B.backward(p["x"], p["w_router"], p["b_router"], p["w_up"], p["b_up"], p["w_down"],
                    p["b_down"], dy, alpha=0.0, **kw)
    g2 = B.backward(p["x"], p["w_router"], p["b_router"], p["w_up"], p["b_up"], p["w_down"],
                    p["b_down"], dy, alpha=2 * ALPHA, **kw)
    np.testing.assert_allclose(g2["dlogits"] - g0["dlogits"], 2 * (g["dlogits"] - g0["dlogits"]),
                               rtol=1e-12, atol=1e-14)
    np.testing.assert_array_equal(g2["dw_up"], g0["dw_up"])
    # an expert that receives no rows gets zero weight gradients
    p2 = dict(p)
    p2["b_router"] = np.array([0.0, 0.0, 0.0, -50.0])   # expert 3 never selected
    g3 = B.backward(p2["x"], p2["w_router"], p2["b_router"], p2["w_up"], p2["b_up"],
                    p2["w_down"], p2["b_down"], dy, alpha=ALPHA, **kw)
    assert g3["counts"][3] == 0
    assert np.all(g3["dw_up"][3] == 0) and np.all(g3["dw_down"][3] == 0)
    assert np.all(g3["db_up"][3] == 0) and np.all(g3["db_down"][3] == 0)


def test_activation_derivatives_closed_forms():
    z = np.linspace(-4, 4, 41)
    h = 1e-6
    np.testing.assert_allclose(B.gelu_grad(z), (O.gelu(z + h) - O.gelu(z - h)) / (2 * h),
                               rtol=1e-7, atol=1e-9)
    np.testing.assert_allclose(B.silu_grad(z), (O.silu(z + h) - O.silu(z - h)) / (2 * h),
                               rtol=1e-7, atol=1e-9)
    # GELU'(0) = 1/2, silu'(0) = 1/2; both tend to 1 for large z and 0 for very negative z
    assert B.gelu_grad(np.array([0.0]))[0] == 0.5 and B.silu_grad(np.array([0.0]))[0] == 0.5
    assert abs(B.gelu_grad(np.array([8.0]))[0] - 1) < 1e-12
    assert abs(B.silu_grad(np.array([-40.0]))[0]) < 1e-15


@pytest.mark.parametrize("case", list(CASES))
def test_single_entries_match_full_backward(case):
    """The per-token and per-weight-row entry functions (used for checks at
    full sizes) reproduce the full backward oracle entry by entry."""
    p, dy, kw = make(case)
    args = (p["x"], p["w_router"], p["b_router"], p["w_up"], p["b_up"], p["w_down"], p["b_down"], dy)
    g = B.backward(*args, alpha=ALPHA, **kw)
    kept = g["assign_row"].reshape(T, K) >= 0
    for t in range(T):
        tok = B.backward_token(t, *args, alpha=ALPHA, top_k=K, num_shared=kw["num_shared"],
                               gating=kw["gating"], activation=kw["activation"], idx=g["idx"],
                               kept_slots=kept[t], counts=g["counts"])
        np.testing.assert_allclose(tok["dx"], g["dx"][t], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(tok["dw"], g["dw"][t], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(tok["dlogits"], g["dlogits"][t], rtol=1e-12, atol=1e-13)
    F1 = p["w_up"].shape[1]
    for seg in range(E + kw["num_shared"]):
        for n in range(F1):
            ent = B.backward_weight_entries(seg, n, p["x"], p["w_up"], p["b_up"], p["w_down"],
                                            p["b_down"], dy, activation=kw["activation"],
                                            top_k=K, disp=g, topk_weights=g["w"])
            np.testing.assert_allclose(ent["dw_up_row"], g["dw_up"][seg][n], rtol=1e-12, atol=1e-13)
            if p["b_up"] is not None:
                np.testing.assert_allclose(ent["db_up"], g["db_up"][seg][n], rtol=1e-12, atol=1e-13)
            np.testing.assert_allclose(ent["dw_down_col"], g["dw_down"][seg][:, ent["col"]],
                                       rtol=1e-12, atol=1e-13)


def test_router_backward_token_is_linear_in_dw():
    """router_backward_token at the oracle's own dw gives the full backward's
    logit gradients; it is affine in dw (the aux term is the constant)."""
    p, dy, kw = make("swiglu_sigmoid_shared_drops")
    g = B.backward(p["x"], p["w_router"], p["b_router"], p["w_up"], p["b_up"], p["w_down"],
                   p["b_down"], dy, alpha=ALPHA, **kw)
    for t in range(T):
        r = B.router_backward_token(t, p["x"], p["w_router"], p["b_router"], alpha=ALPHA, top_k=K,
                                    gating=kw["gating"], idx=g["idx"], counts=g["counts"],
                                    dw=g["dw"][t])
        np.testing.assert_allclose(r["dlogits"], g["dlogits"][t], rtol=1e-12, atol=1e-13)
        r0 = B.router_backward_token(t, p["x"], p["w_router"], p["b_router"], alpha=ALPHA, top_k=K,
                                     gating=kw["gating"], idx=g["idx"], counts=g["counts"],
                                     dw=np.zeros(K))
        r2 = B.router_backward_token(t, p["x"], p["w_router"], p["b_router"], alpha=ALPHA, top_k=K,
                                     gating=kw["gating"], idx=g["idx"], counts=g["counts"],
                                     dw=2 * g["dw"][t])
        np.testing.assert_allclose(r2["dlogits"] - r0["dlogits"], 2 * (r["dlogits"] - r0["dlogits"]),
                                   rtol=1e-10, atol=1e-13)
