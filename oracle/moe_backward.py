"""Plain CPU oracle of the MoE-FFN backward pass, in float64 numpy.

TEST INFRASTRUCTURE ONLY (like the forward oracle beside it): only the tests,
the smoke check of the package entry file and the cpu_baseline leg of the
benchmark may import or run this module; it shares no code with the HIP
library.

What is differentiated.  The training use of the layer ([0539edu] 4.3, aux
loss merged into the task loss before one backward; [kamacoder] 七 total loss
= task loss + load-balancing loss) makes the objective

    L = <dy, y> + alpha * L_aux,

where dy is the upstream gradient of the task loss with respect to the layer
output y, and L_aux = E * sum_e f_e * P_e ([kamacoder] 七).  The gradient is
the one automatic differentiation of the pages' forward code gives:

  * the top-k selection, the capacity drops and the counts f_e are piecewise
    constant: no gradient flows through them (f_e is a count in the pages'
    load_balancing_loss; top-k passes gradient only to the selected values);
  * gradient reaches the router through the renormalized top-k weights and
    through P_e (the mean gate probability);
  * a dropped slot contributes nothing to y, so it sends no gradient to its
    expert nor to its gate weight;
  * shared experts have weight 1 and no gate.

Readings carried over from the forward: normalized sigmoid gating ranks and
weights by sigma (w = sigma_sel / sum_sel sigma) and P uses p = sigma / sum_all
sigma; the GELU is the exact erf form; SwiGLU has no biases.

Every step cites the forward passage it differentiates.  The derivatives
used are the textbook ones, written out below; nothing is blocked or fused.

Parity pins: central finite differences of the forward oracle on tie-free
inputs (every gradient, every activation and gating, drops and shared
experts), and float64 torch autograd on expressions of the same layer.
"""
import math

import numpy as np
from scipy.special import erf

from .moe_oracle import dispatch, gate, router_logits, silu


def gelu_grad(z):
    """d/dz of 0.5 z (1 + erf(z / sqrt 2)) = Phi(z) + z phi(z), with Phi and
    phi the standard normal distribution and density."""
    cdf = 0.5 * (1.0 + erf(z / math.sqrt(2.0)))
    pdf = np.exp(-0.5 * z * z) / math.sqrt(2.0 * math.pi)
    return cdf + z * pdf


def silu_grad(z):
    """d/dz of z * sigma(z) = sigma(z) * (1 + z * (1 - sigma(z)))."""
    s = 1.0 / (1.0 + np.exp(-z))
    return s * (1.0 + z * (1.0 - s))


def expert_ffn_backward(xr, w_up, b_up, w_down, b_down, activation, d_out):
    """Backward of one expert on rows xr [m, d] (the Linear -> activation ->
    Linear expert of [kamacoder] 四 / [0539edu] 4.1, SwiGLU form for
    activation == "swiglu") given d_out [m, d], the gradient of the objective
    with respect to the expert's output rows.

    Returns dict(dx [m, d], dw_up, db_up, dw_down, db_down, out [m, d]),
    where out is the expert's forward output (needed for the gate weights'
    gradient).  Linear layer y = W u + b: du = W^T dy, dW = dy^T u, db =
    sum of dy over rows."""
    z = xr @ w_up.T
    if b_up is not None:
        z = z + b_up[None, :]
    if activation == "relu":
        h = np.maximum(z, 0.0)
    elif activation == "gelu":
        erf_part = 0.5 * (1.0 + erf(z / math.sqrt(2.0)))
        h = z * erf_part
    elif activation == "swiglu":
        f = w_up.shape[0] // 2
        g, u = z[:, :f], z[:, f:]
        h = silu(g) * u
    else:
        raise ValueError(activation)
    out = h @ w_down.T
    if b_down is not None:
        out = out + b_down[None, :]

    dh = d_out @ w_down                    # [m, f]
    dw_down = d_out.T @ h                  # [d, f]
    db_down = d_out.sum(axis=0)
    if activation == "relu":
        dz = dh * (z > 0.0)
    elif activation == "gelu":
        dz = dh * gelu_grad(z)
    else:
        dz = np.concatenate([dh * u * silu_grad(g), dh * silu(g)], axis=1)
    dx = dz @ w_up                         # [m, d]
    dw_up = dz.T @ xr                      # [F1, d]
    db_up = dz.sum(axis=0)
    return dict(dx=dx, dw_up=dw_up, db_up=db_up, dw_down=dw_down, db_down=db_down, out=out)


def topk_renorm_backward(keys, idx, dw):
    """w[t, s] = key[t, idx_s] / S_t with S_t = sum over the k selected keys
    ([0539edu] 2.1 renormalization; [kamacoder] 三 top_k_routing).
    d key[t, idx_s] = (dw[t, s] - sum_s' w[t, s'] dw[t, s']) / S_t; keys that
    were not selected get zero."""
    T, k = idx.shape
    dkey = np.zeros_like(keys)
    for t in range(T):
        sel = keys[t, idx[t]]
        S = sel.sum()
        w = sel / S
        inner = float(np.dot(w, dw[t]))
        for s in range(k):
            dkey[t, idx[t, s]] += (dw[t, s] - inner) / S
    return dkey


def softmax_backward(p, dp):
    """p = softmax(l) per row ([0539edu] 2.1): dl = p * (dp - sum_e p_e dp_e)."""
    return p * (dp - np.sum(p * dp, axis=1, keepdims=True))


def sigmoid_normalized_backward(logits, dsig, dp):
    """Normalized sigmoid gating ([bojinhu] 四 技术飞跃③): sigma = 1/(1+e^-l)
    per expert, p = sigma / sum_all sigma.  dsig is the gradient that reaches
    sigma directly (through the top-k weights), dp the gradient on p
    (through P).  d sigma_j += (dp_j - sum_e p_e dp_e) / sum sigma;
    dl = d sigma * sigma (1 - sigma)."""
    sig = 1.0 / (1.0 + np.exp(-logits))
    tot = sig.sum(axis=1, keepdims=True)
    p = sig / tot
    dsig = dsig + (dp - np.sum(p * dp, axis=1, keepdims=True)) / tot
    return dsig * sig * (1.0 - sig)


def backward(x, w_router, b_router, w_up, b_up, w_down, b_down, dy, *, alpha, top_k,
             num_shared, gating, activation, cap=None, idx=None):
    """Gradients of L = <dy, y> + alpha * L_aux with respect to x and every
    parameter of the layer, for token-choice routing.

    idx: the top-k selection to differentiate at (default: the oracle's own;
    a GPU's selection can be passed so that both sides use the same
    piecewise-constant routing).  Returns dict(dx, dw_router, db_router,
    dw_up, db_up, dw_down, db_down, dw [T, k] gradient of the slot weights
    (0 for dropped slots), dlogits [T, E], idx, w, probs)."""
    T, d = x.shape
    E = w_router.shape[0]
    k = top_k
    logits = router_logits(x, w_router, b_router)
    probs = gate(logits, gating)
    if gating == "softmax":
        keys = probs
    else:
        keys = 1.0 / (1.0 + np.exp(-logits))
    if idx is None:
        order = np.argsort(-keys, axis=1, kind="stable")
        idx = order[:, :k]
    idx = np.asarray(idx, dtype=np.int64)
    sel = np.take_along_axis(keys, idx, axis=1)
    w = sel / sel.sum(axis=1, keepdims=True)
    disp = dispatch(idx, E, cap)

    dx = np.zeros_like(x)
    dw_up = np.zeros(w_up.shape)        # weights may be per-expert lazy views
    dw_down = np.zeros(w_down.shape)
    db_up = np.zeros((w_up.shape[0], w_up.shape[1]))
    db_down = np.zeros((w_down.shape[0], w_down.shape[1]))
    dw = np.zeros((T, k))
    # routed experts: only kept rows ([kamacoder] 五/六 dispatch and combine)
    for e in range(E):
        lo, hi = int(disp["offsets"][e]), int(disp["offsets"][e + 1])
        if hi == lo:
            continue
        a = disp["sorted_assign"][lo:hi]
        tt, ss = a // k, a % k
        d_out = w[tt, ss][:, None] * dy[tt]       # y_t += w_ts * out_ts
        g = expert_ffn_backward(x[tt], w_up[e], None if b_up is None else b_up[e], w_down[e],
                                None if b_down is None else b_down[e], activation, d_out)
        dx[tt] += g["dx"]                          # a token meets expert e at most once
        dw_up[e] += g["dw_up"]
        dw_down[e] += g["dw_down"]
        db_up[e] += g["db_up"]
        db_down[e] += g["db_down"]
        dw[tt, ss] = np.sum(dy[tt] * g["out"], axis=1)
    # shared experts: weight 1 on every token ([bojinhu] 四 技术飞跃②)
    for q in range(num_shared):
        qq = E + q
        g = expert_ffn_backward(x, w_up[qq], None if b_up is None else b_up[qq], w_down[qq],
                                None if b_down is None else b_down[qq], activation, dy)
        dx += g["dx"]
        dw_up[qq] += g["dw_up"]
        dw_down[qq] += g["dw_down"]
        db_up[qq] += g["db_up"]
        db_down[qq] += g["db_down"]

    # router: top-k weights, then the aux term through P_e = mean_t p[t, e]
    dkey = topk_renorm_backward(keys, idx, dw)
    counts = np.bincount(idx.reshape(-1), minlength=E).astype(np.float64)
    f = counts / (T * k)
    dp = np.broadcast_to(alpha * E * f / T, (T, E)).copy()
    if gating == "softmax":
        dlogits = softmax_backward(probs, dkey + dp)
    else:
        dlogits = sigmoid_normalized_backward(logits, dkey, dp)
    dx += dlogits @ w_router
    dw_router = dlogits.T @ x
    db_router = dlogits.sum(axis=0)
    return dict(dx=dx, dw_router=dw_router, db_router=db_router, dw_up=dw_up,
                db_up=db_up if b_up is not None else None, dw_down=dw_down,
                db_down=db_down if b_down is not None else None, dw=dw, dlogits=dlogits,
                idx=idx, w=w, probs=probs, **disp)


# ----------------------------------------------------------------------------
# Single gradient entries, for checks at sizes where the whole backward is
# too large for the host: each follows the same chain rule as `backward`,
# restricted to what one entry depends on.
# ----------------------------------------------------------------------------


def gate_keys(logits, gating):
    """(p, keys): the gate probabilities and the values the top-k ranks and
    renormalizes (p for softmax, sigma for the normalized sigmoid)."""
    probs = gate(logits, gating)
    keys = probs if gating == "softmax" else 1.0 / (1.0 + np.exp(-logits))
    return probs, keys


def router_backward_token(t, x, w_router, b_router, *, alpha, top_k, gating, idx, counts, dw):
    """Router part of token t's gradients for given slot-weight gradients
    dw [k]: the renormalized top-k, the gate and the aux term
    ([0539edu] 2.1, 2.3).  Returns dlogits [E] and dx_router = dlogits Wr."""
    T = x.shape[0]
    E = w_router.shape[0]
    logits = router_logits(x[t:t + 1], w_router, b_router)
    probs, keys = gate_keys(logits, gating)
    dkey = topk_renorm_backward(keys, idx[t:t + 1], np.asarray(dw, dtype=np.float64)[None, :])
    f = np.asarray(counts, dtype=np.float64) / (T * top_k)
    dp = (alpha * E * f / T)[None, :]
    if gating == "softmax":
        dl = softmax_backward(probs, dkey + dp)
    else:
        dl = sigmoid_normalized_backward(logits, dkey, dp)
    return dict(dlogits=dl[0], dx_router=(dl @ w_router)[0])


def backward_token(t, x, w_router, b_router, w_up, b_up, w_down, b_down, dy, *, alpha, top_k,
                   num_shared, gating, activation, idx, kept_slots, counts):
    """Gradients belonging to token t: dx[t], the slot weights' gradient
    dw[t, :] and dlogits[t, :].  idx [T, k] is the selection, kept_slots[s]
    whether slot s of token t survived the capacity, counts [E] the routed
    counts over the whole batch (they fix f_e).  Also returns dw_scale[s] =
    sum_j |dy[t, j] out_s[j]|, the magnitude behind the sum dw[s] =
    <dy[t], out_s> (what a rounding of dy scales with)."""
    E = w_router.shape[0]
    k = top_k
    xt = x[t:t + 1]
    _, keys = gate_keys(router_logits(xt, w_router, b_router), gating)
    sel = keys[0, idx[t]]
    w = sel / sel.sum()
    dx = np.zeros(x.shape[1])
    dw = np.zeros(k)
    dw_scale = np.zeros(k)
    for s in range(k):
        if not kept_slots[s]:
            continue
        e = int(idx[t, s])
        g = expert_ffn_backward(xt, w_up[e], None if b_up is None else b_up[e], w_down[e],
                                None if b_down is None else b_down[e], activation,
                                w[s] * dy[t:t + 1])
        dx += g["dx"][0]
        dw[s] = float(np.dot(dy[t], g["out"][0]))
        dw_scale[s] = float(np.sum(np.abs(dy[t] * g["out"][0])))
    for q in range(num_shared):
        qq = E + q
        g = expert_ffn_backward(xt, w_up[qq], None if b_up is None else b_up[qq], w_down[qq],
                                None if b_down is None else b_down[qq], activation, dy[t:t + 1])
        dx += g["dx"][0]
    r = router_backward_token(t, x, w_router, b_router, alpha=alpha, top_k=k, gating=gating,
                              idx=idx, counts=counts, dw=dw)
    return dict(dx=dx + r["dx_router"], dw=dw, dw_scale=dw_scale, dlogits=r["dlogits"])


def _segment_rows(seg, E, T, k, disp, topk_weights):
    """(tokens, gate weights) of the rows of segment seg: an expert's kept
    assignments in dispatch order, or every token with weight 1 (shared)."""
    if seg < E:
        lo, hi = int(disp["offsets"][seg]), int(disp["offsets"][seg + 1])
        a = np.asarray(disp["sorted_assign"][lo:hi], dtype=np.int64)
        return a // k, topk_weights[a // k, a % k]
    return np.arange(T), np.ones(T)


def _preact_column(x_rows, w_up_e, b_up_e, n):
    z = x_rows @ w_up_e[n]
    return z + b_up_e[n] if b_up_e is not None else z


def backward_weight_entries(seg, n, x, w_up, b_up, w_down, b_down, dy, *, activation, top_k,
                            disp, topk_weights):
    """Row n of dW1[seg] (with db1[seg][n]) and column n of dW2[seg] (with
    nothing else), for segment seg (expert, or E + q for shared expert q).
    For SwiGLU, row n < f of W1 is a gate row and row f + n the matching up
    row; column n of W2 multiplies h[:, n].  disp: the dispatch of the
    selection; topk_weights [T, k] the renormalized gate weights."""
    T, d = x.shape
    E = len(disp["offsets"]) - 1
    toks, wts = _segment_rows(seg, E, T, top_k, disp, topk_weights)
    xr, dyr = x[toks], dy[toks]
    w_up_e, w_down_e = w_up[seg], w_down[seg]
    b_up_e = None if b_up is None else b_up[seg]
    f = w_down_e.shape[1]
    col = n if n < f else n - f                  # h column this W1 row feeds
    # G[r] = (W2_e^T dy_r)[col]: the unweighted gradient reaching h[r, col]
    G = dyr @ w_down_e[:, col]
    dh = wts * G
    if activation == "swiglu":
        g = _preact_column(xr, w_up_e, b_up_e, col)
        u = _preact_column(xr, w_up_e, b_up_e, f + col)
        h = silu(g) * u
        dz = dh * u * silu_grad(g) if n < f else dh * silu(g)
    else:
        z = _preact_column(xr, w_up_e, b_up_e, col)
        if activation == "relu":
            h = np.maximum(z, 0.0)
            dz = dh * (z > 0.0)
        else:
            h = 0.5 * z * (1.0 + erf(z / math.sqrt(2.0)))
            dz = dh * gelu_grad(z)
    dw_up_row = dz @ xr                          # dW1[seg][n, :] = sum_r dz_r x_r
    db_up = float(dz.sum())
    dw_down_col = (wts[:, None] * dyr).T @ h     # dW2[seg][:, col] = sum_r (w_r dy_r) h_r[col]
    return dict(dw_up_row=dw_up_row, db_up=db_up, dw_down_col=dw_down_col, col=col)
