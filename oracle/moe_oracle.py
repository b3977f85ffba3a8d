"""Plain CPU oracle of the MoE-FFN forward, in float64 numpy.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check of the package
entry file and the cpu_baseline leg of the benchmark may import or run this
module.  It shares no code with the HIP library and imports nothing from it.

Every function follows one step as the pages state it; library primitives
(numpy matmul, exp, a stable argsort, scipy's erf) serve as single steps, and
nothing is blocked, fused or reordered beyond what the step's definition says.
Inputs are float64 arrays (bf16 data upcast exactly by the caller).

Pages (cited by title and section):
  [0539edu] "MoE混合专家模型：Transformer稀疏前馈网络原理与PyTorch实现"
  [bojinhu] "MoE架构解析"
  [kamacoder] "手撕一个极简 MoE-FFN"
  [yunthe] "Mixture of Experts混合专家模型架构原理与路由策略实现"
  [minimind] "术业有专攻：learn-minimind MoE混合专家模型架构入门指南"

Readings taken where the pages are silent, ambiguous or inconsistent (the
design notes list them with reasons):
  * f_e counts routing decisions before capacity drops and divides by T*k;
  * L_aux is returned without the weight alpha;
  * capacity C = ceil(CF * T * k / E); each expert keeps its C lowest-token
    assignments; a dropped slot contributes zero and the surviving weights
    are not renormalized; shared experts still apply;
  * normalized sigmoid: p_e = sigma_e / sum over all experts of sigma; the
    top-k weights renormalize p over the selected experts;
  * ties in the top-k go to the lower expert index; slots are in descending
    score order;
  * GELU is the exact erf form; SwiGLU is W2 (silu(Wg x) * (Wu x));
  * shared experts have weight 1.

Parity pins: every function here is pinned by a `-m "not gpu"` test against
the pages' worked example, closed forms, library routines or brute force.
"""
import math

import numpy as np
from scipy.special import erf

# ----------------------------------------------------------------------------
# Router and gate
# ----------------------------------------------------------------------------


def router_logits(x, w_router, b_router=None):
    """logits[t, e] = sum_j x[t, j] * Wr[e, j] + br[e].

    The router is one linear layer over the token vector with one output per
    expert ([0539edu] 2.1; [kamacoder] 三 Router; [yunthe] gate formula).
    Wr has the nn.Linear [E, d_model] layout."""
    logits = x @ w_router.T
    if b_router is not None:
        logits = logits + b_router[None, :]
    return logits


def softmax(logits):
    """p[t, e] = exp(l[t, e] - m_t) / sum_e' exp(l[t, e'] - m_t), m_t = max_e l[t, e]
    ([0539edu] 2.1; [kamacoder] 三; [bojinhu] 2.1 step 2)."""
    m = logits.max(axis=1, keepdims=True)
    ex = np.exp(logits - m)
    return ex / ex.sum(axis=1, keepdims=True)


def sigmoid_normalized(logits):
    """sigma_e = 1 / (1 + exp(-l_e)) for each expert independently, then
    normalized over all experts: p_e = sigma_e / sum_e' sigma_e'
    ([bojinhu] 四, 技术飞跃③ normalized sigmoid gating)."""
    sig = 1.0 / (1.0 + np.exp(-logits))
    return sig / sig.sum(axis=1, keepdims=True)


def gate(logits, gating):
    if gating == "softmax":
        return softmax(logits)
    if gating == "sigmoid_norm":
        return sigmoid_normalized(logits)
    raise ValueError(gating)


def topk_renorm(scores, k):
    """Top-k experts per token by descending score, ties to the lower expert
    index; weights are the selected scores divided by their sum
    ([0539edu] 2.1: topk, then renormalize the K probabilities to sum 1;
    [kamacoder] 三 top_k_routing and its worked example).

    Returns idx [T, k] int32 (slot 0 = highest score) and w [T, k] float64."""
    scores = np.asarray(scores, dtype=np.float64)
    # A stable sort of the negated scores keeps equal scores in ascending
    # expert order, so a tie goes to the lower index.
    order = np.argsort(-scores, axis=1, kind="stable")
    idx = order[:, :k].astype(np.int32)
    return idx, renorm(scores, idx)


def renorm(scores, idx):
    """w[t, s] = scores[t, idx[t, s]] / sum over the token's selected experts
    of their scores: the selected probabilities renormalized to sum to 1
    ([0539edu] 2.1; [kamacoder] 三 top_k_routing), for a given selection."""
    sel = np.take_along_axis(np.asarray(scores, dtype=np.float64),
                             np.asarray(idx, dtype=np.int64), axis=1)
    return sel / sel.sum(axis=1, keepdims=True)


def routing(x, w_router, b_router, *, top_k, gating):
    """Router -> gate -> top-k + renorm over all tokens: logits, probs, the
    oracle's own selection idx [T, k] with weights w, and the selection gap."""
    logits = router_logits(x, w_router, b_router)
    probs = gate(logits, gating)
    idx, w = topk_renorm(probs, top_k)
    return dict(logits=logits, probs=probs, idx=idx, w=w, gap=selection_gap(probs, top_k))


def selection_gap(scores, k):
    """Score of the k-th selected expert minus the score of the best
    unselected one (inf when k == E); the parity rule compares routing indices
    only where this gap exceeds a threshold."""
    s = np.sort(np.asarray(scores, dtype=np.float64), axis=1)[:, ::-1]
    if k >= s.shape[1]:
        return np.full(s.shape[0], np.inf)
    return s[:, k - 1] - s[:, k]


# ----------------------------------------------------------------------------
# Capacity and dispatch
# ----------------------------------------------------------------------------


def capacity(T, k, E, capacity_factor):
    """Per-expert capacity C = ceil(CF * T * k / E); None (no limit) when CF is
    None.  [bojinhu] 三 关键技术① gives (tokens per batch / experts) x CF, and
    [0539edu] 3.2 calls C a multiple of the ideal even share; with top-k the
    even share of the T*k assignments is T*k/E (equal to the page's formula
    for k = 1)."""
    if capacity_factor is None:
        return None
    return int(math.ceil(capacity_factor * T * k / E))


def dispatch(idx, E, cap=None):
    """Group the T*k assignments a = t*k + s by expert, stable in token order,
    and apply the capacity limit.

    counts[e]        assignments routed to e (before drops)
    kept[e]          min(counts[e], C) (counts[e] without a limit)
    offsets[e]       row where expert e's kept rows start; offsets[E] = total kept
    sorted_assign[r] assignment held by row r for r < offsets[E]; after that,
                     the dropped assignments, grouped by expert, token order
    assign_row[a]    row of assignment a, or -1 if dropped
    drop_mask[a]     1 if dropped
    Capacity and dropping: [bojinhu] 三 关键技术① (tokens beyond capacity skip
    the layer); which tokens are dropped is not stated, the later tokens of
    an expert are dropped first (stable by token index)."""
    T, k = idx.shape
    flat = idx.reshape(-1)
    n = T * k
    counts = np.zeros(E, dtype=np.int64)
    members = [[] for _ in range(E)]
    for a in range(n):          # ascending a == ascending token, then slot
        e = int(flat[a])
        members[e].append(a)
        counts[e] += 1
    kept = counts.copy() if cap is None else np.minimum(counts, cap)
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(kept)
    assign_row = np.full(n, -1, dtype=np.int64)
    drop_mask = np.zeros(n, dtype=np.uint8)
    sorted_assign = np.empty(n, dtype=np.int64)
    pos_drop = int(offsets[E])
    for e in range(E):
        for rank, a in enumerate(members[e]):
            if rank < kept[e]:
                r = int(offsets[e]) + rank
                assign_row[a] = r
                sorted_assign[r] = a
            else:
                drop_mask[a] = 1
                sorted_assign[pos_drop] = a
                pos_drop += 1
    return dict(counts=counts, kept=kept, offsets=offsets, sorted_assign=sorted_assign,
                assign_row=assign_row, drop_mask=drop_mask)


# ----------------------------------------------------------------------------
# Expert FFN
# ----------------------------------------------------------------------------


def gelu(z):
    """Exact GELU, 0.5 z (1 + erf(z / sqrt 2)) (F.gelu without the tanh
    approximation, as the GELU experts of [0539edu] 4.1 and [yunthe] call it)."""
    return 0.5 * z * (1.0 + erf(z / math.sqrt(2.0)))


def silu(z):
    """silu(z) = z / (1 + exp(-z))."""
    return z / (1.0 + np.exp(-z))


def expert_ffn(xr, w_up, b_up, w_down, b_down, activation):
    """One expert on the rows xr [m, d]: Linear -> activation -> Linear.

    relu / gelu: out = W2 act(W1 x + b1) + b2 ([kamacoder] 四 Expert with
    ReLU; [0539edu] 4.1 ExpertFFN with GELU; dropout is the identity in a
    forward pass).  swiglu: w_up holds [Wg; Wu] (2f rows), out =
    W2 (silu(Wg x) * (Wu x)) — the experts the minimind page names SwiGLU
    ([minimind] 二), taken in the standard GLU-variant form without biases."""
    z = xr @ w_up.T
    if b_up is not None:
        z = z + b_up[None, :]
    if activation == "relu":
        h = np.maximum(z, 0.0)
    elif activation == "gelu":
        h = gelu(z)
    elif activation == "swiglu":
        f = w_up.shape[0] // 2
        h = silu(z[:, :f]) * z[:, f:]
    else:
        raise ValueError(activation)
    out = h @ w_down.T
    if b_down is not None:
        out = out + b_down[None, :]
    return out


# ----------------------------------------------------------------------------
# Combine and auxiliary statistics
# ----------------------------------------------------------------------------


def combine_rows(y_rows, w, assign_row, shared_base=0, num_shared=0):
    """y[t] = sum over kept slots s of w[t, s] * y_rows[assign_row[t*k + s]]
             + sum over shared experts q of y_rows[shared_base + q*T + t].

    y_rows holds one expert output per row (routed rows by assign_row,
    shared expert q's output for token t at shared_base + q*T + t).
    Gate-weighted sum: [0539edu] 1.3 and 2.1; [kamacoder] 五 (output +=
    weight * expert_out); shared experts are always active with weight 1
    ([bojinhu] 四 技术飞跃②); a dropped slot (row -1) adds nothing."""
    T, k = w.shape
    d = y_rows.shape[1]
    y = np.zeros((T, d), dtype=np.float64)
    for t in range(T):
        for s in range(k):
            r = int(assign_row[t * k + s])
            if r >= 0:
                y[t] += w[t, s] * y_rows[r]
        for q in range(num_shared):
            y[t] += y_rows[shared_base + q * T + t]
    return y


def aux_stats(idx, probs, E):
    """f_e = (assignments routed to e) / (T * k); P_e = mean over tokens of
    p[t, e]; L_aux = E * sum_e f_e * P_e, without the weight alpha
    ([0539edu] 2.3; [kamacoder] 七 load_balancing_loss)."""
    T, k = idx.shape
    counts = np.bincount(idx.reshape(-1), minlength=E).astype(np.float64)
    f = counts / (T * k)
    P = probs.mean(axis=0)
    l_aux = E * float(np.sum(f * P))
    return f, P, l_aux


def routing_stats(counts, kept, P):
    """Routing health indicators ([0539edu] 3.3, observability: log per step the
    tokens each expert actually processes, the entropy of the routing
    distribution against the uniform entropy ln N, and the variance of expert
    utilization; its troubleshooting list judges balance by the coefficient of
    variation of utilization; experts at zero usage are the failure to watch).

    Readings: the routing distribution is the share of routing decisions per
    expert before capacity drops, counts_e / (T*k) (the same basis as f);
    entropy H = -sum_e s_e ln s_e with 0 ln 0 = 0, beside it the entropy of the
    mean gate probabilities P; utilization is the tokens actually processed,
    kept_e, with the population variance over experts and CV = std / mean
    (0 when nothing is kept); dropped = sum_e (counts_e - kept_e); idle =
    number of experts with kept_e = 0."""
    counts = np.asarray(counts, dtype=np.float64)
    kept = np.asarray(kept, dtype=np.float64)
    P = np.asarray(P, dtype=np.float64)
    E = counts.size

    def entropy(v):
        nz = v[v > 0]
        return float(-np.sum(nz * np.log(nz)))

    share = counts / counts.sum()
    mean = float(kept.mean())
    var = float(np.mean((kept - mean) ** 2))
    cv = float(np.sqrt(var) / mean) if mean > 0 else 0.0
    return dict(entropy=entropy(share), entropy_p=entropy(P), entropy_max=float(np.log(E)),
                util_mean=mean, util_var=var, util_cv=cv,
                dropped=int(np.sum(counts - kept)), idle=int(np.sum(kept == 0)))


# ----------------------------------------------------------------------------
# Expert-choice routing ([bojinhu] 二 2.2: each expert picks the Top-K tokens it
# is best at; every expert's load is then exactly equal, a token can be picked
# by several experts or by none)
# ----------------------------------------------------------------------------


def expert_choice_select(probs, C):
    """Each expert e keeps the C tokens with the largest probs[t, e]; equal
    scores go to the lower token index.  Readings: the affinity is the gate
    probability of token-choice routing, C is the per-expert capacity.
    Returns sel [E, C] (each expert's tokens in ascending order), row_of [T, E]
    (row e*C + position of (t, e), -1 if e did not pick t) and token_experts
    [T] (how many experts picked each token; 0 = an orphan token)."""
    T, E = probs.shape
    sel = np.empty((E, C), dtype=np.int64)
    for e in range(E):
        order = np.lexsort((np.arange(T), -probs[:, e]))   # by score desc, then token asc
        sel[e] = np.sort(order[:C])
    row_of, token_experts = expert_choice_rows(sel, T)
    return sel, row_of, token_experts


def expert_choice_gap(probs, C):
    """Per expert, the score gap between its C-th and (C+1)-th best tokens
    (inf when C >= T): selections agree wherever this gap is clear."""
    T, E = probs.shape
    if C >= T:
        return np.full(E, np.inf)
    srt = -np.sort(-probs, axis=0)
    return srt[C - 1] - srt[C]


def expert_choice_rows(sel, T):
    """row_of [T, E] (row e*C + position of (t, e) in expert e's ascending
    token list, -1 if e did not pick t) and token_experts [T] for a given
    selection sel [E, C] of ascending token lists."""
    sel = np.asarray(sel, dtype=np.int64)
    E, C = sel.shape
    row_of = np.full((T, E), -1, dtype=np.int64)
    for e in range(E):
        row_of[sel[e], e] = e * C + np.arange(C)
    return row_of, (row_of >= 0).sum(axis=1)


def forward_expert_choice(x, w_router, b_router, w_up, b_up, w_down, b_down, *, capacity,
                          num_shared, gating, activation, token_subset=None, sel=None):
    """MoE-FFN forward with expert-choice routing: router -> gate -> each
    expert takes its top-C tokens -> expert FFNs -> y[t] = sum over the
    experts e that picked t of p[t, e] * FFN_e(x_t) (no renormalization; an
    orphan token gets only the shared experts) + shared experts.

    sel [E, C]: evaluate the layer at this selection (each expert's tokens in
    ascending order) instead of the oracle's own; gap stays that of the
    oracle's own scores."""
    T, d = x.shape
    E = w_router.shape[0]
    logits = router_logits(x, w_router, b_router)
    probs = gate(logits, gating)
    if sel is None:
        sel, row_of, token_experts = expert_choice_select(probs, capacity)
    else:
        sel = np.asarray(sel, dtype=np.int64).reshape(E, capacity)
        row_of, token_experts = expert_choice_rows(sel, T)
    toks = np.arange(T) if token_subset is None else np.asarray(token_subset)
    pos = {int(t): i for i, t in enumerate(toks)}
    y = np.zeros((len(toks), d), dtype=np.float64)
    for e in range(E):
        tt = np.array([t for t in sel[e] if int(t) in pos], dtype=np.int64)
        if tt.size == 0:
            continue
        out = expert_ffn(x[tt], w_up[e], None if b_up is None else b_up[e],
                         w_down[e], None if b_down is None else b_down[e], activation)
        for i, t in enumerate(tt):
            y[pos[int(t)]] += probs[t, e] * out[i]
    for q in range(num_shared):
        qq = E + q
        y += expert_ffn(x[toks], w_up[qq], None if b_up is None else b_up[qq],
                        w_down[qq], None if b_down is None else b_down[qq], activation)
    return dict(logits=logits, probs=probs, sel=sel, row_of=row_of, token_experts=token_experts,
                gap=expert_choice_gap(probs, capacity), y=y, tokens=toks)


# ----------------------------------------------------------------------------
# FP8 expert weights ([0539edu] 5.2: quantize expert parameters from 16 bits
# to INT8 or FP8 to halve their memory)
# ----------------------------------------------------------------------------

FP8_MAX = 448.0


def e4m3_values():
    """Non-negative finite values of OCP FP8 E4M3 indexed by code 0..126 (code
    127 is NaN; there are no infinities).  Code bits eeee mmm: exponent
    field e with bias 7, mantissa m; e = 0 is subnormal, m/8 * 2^-6; otherwise
    (1 + m/8) * 2^(e - 7).  The largest value, code 126, is 448."""
    vals = []
    for code in range(127):
        e, m = code >> 3, code & 7
        vals.append(m / 8.0 * 2.0 ** -6 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7))
    return np.array(vals, dtype=np.float64)


def quantize_fp8_rows(w):
    """Per-row (output channel) FP8 E4M3 quantization of a [rows, K] matrix.

    Reading (the page names the format only): scale s = max_j |w[r, j]| / 448
    in float32 (1 where the row is all zero); each value v = w / s in float32
    is rounded to the nearest E4M3 value, ties to the even code, magnitudes
    above 448 saturating to 448.  Both divisions are taken in float32, the
    precision the kernels use, so that the codes are reproducible.
    Returns (codes uint8 [rows, K], scales float32 [rows])."""
    w32 = np.asarray(w, dtype=np.float32)
    absmax = np.abs(w32).max(axis=1)
    scales = np.where(absmax > 0, absmax / np.float32(FP8_MAX), np.float32(1.0)).astype(np.float32)
    v = (w32 / scales[:, None]).astype(np.float32)
    a = np.minimum(np.abs(v).astype(np.float64), FP8_MAX)
    vals = e4m3_values()
    hi = np.searchsorted(vals, a, side="left")          # vals[hi] >= a
    lo = np.maximum(hi - 1, 0)
    d_lo = a - vals[lo]
    d_hi = vals[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(vals[hi] == a, hi, np.where(pick_hi, hi, lo)).astype(np.uint8)
    code = code | np.where(v < 0, 0x80, 0).astype(np.uint8)
    return code, scales


def dequantize_fp8_rows(codes, scales):
    """w~[r, j] = value(codes[r, j]) * scales[r], exactly, in float64."""
    vals = e4m3_values()
    c = np.asarray(codes, dtype=np.uint8)
    mag = vals[(c & 0x7F).astype(np.int64)]
    return np.where(c & 0x80, -mag, mag) * np.asarray(scales, dtype=np.float64)[:, None]


# ----------------------------------------------------------------------------
# Whole forward
# ----------------------------------------------------------------------------


def forward(x, w_router, b_router, w_up, b_up, w_down, b_down, *, top_k, num_shared,
            gating, activation, cap=None, token_subset=None, idx=None):
    """The whole MoE-FFN forward: router -> gate -> top-k + renorm -> dispatch
    with capacity -> expert FFNs -> gate-weighted combine (+ shared experts)
    -> f, P, L_aux.  ([0539edu] 1.3 flow and 4.1 MoEFFN; [kamacoder] 二 data
    flow.)

    Routing, dispatch and the aux statistics always cover all T tokens (the
    capacity couples tokens).  If token_subset is given, y is evaluated only
    for those tokens (rows of y in subset order); otherwise for all.

    idx [T, k]: evaluate the layer at this selection (slot order as given)
    instead of the oracle's own top-k; the weights, dispatch, drops, FFNs,
    combine and f then follow from it, and gap stays that of the oracle's
    own scores."""
    T, d = x.shape
    E = w_router.shape[0]
    logits = router_logits(x, w_router, b_router)
    probs = gate(logits, gating)
    if idx is None:
        idx, w = topk_renorm(probs, top_k)
    else:
        idx = np.asarray(idx, dtype=np.int32).reshape(T, top_k)
        w = renorm(probs, idx)
    disp = dispatch(idx, E, cap)
    f, P, l_aux = aux_stats(idx, probs, E)

    toks = np.arange(T) if token_subset is None else np.asarray(token_subset)
    pos = {int(t): i for i, t in enumerate(toks)}
    y = np.zeros((len(toks), d), dtype=np.float64)
    k = top_k
    for e in range(E):
        lo, hi = int(disp["offsets"][e]), int(disp["offsets"][e + 1])
        rows = [(int(disp["sorted_assign"][r]) // k, int(disp["sorted_assign"][r]) % k)
                for r in range(lo, hi)]
        rows = [(t, s) for (t, s) in rows if t in pos]
        if not rows:
            continue
        tt = np.array([t for t, _ in rows])
        out = expert_ffn(x[tt], w_up[e], None if b_up is None else b_up[e],
                         w_down[e], None if b_down is None else b_down[e], activation)
        for i, (t, s) in enumerate(rows):
            y[pos[t]] += w[t, s] * out[i]
    for q in range(num_shared):
        qq = E + q
        y += expert_ffn(x[toks], w_up[qq], None if b_up is None else b_up[qq],
                        w_down[qq], None if b_down is None else b_down[qq], activation)
    stats = routing_stats(disp["counts"], disp["kept"], P)
    return dict(logits=logits, probs=probs, idx=idx, w=w, gap=selection_gap(probs, top_k),
                f=f, P=P, l_aux=l_aux, y=y, tokens=toks, stats=stats, **disp)
