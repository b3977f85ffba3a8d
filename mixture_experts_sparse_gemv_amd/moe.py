"""Python binding of libmoe_mi355x (ctypes).

Argument marshalling only: every function takes torch tensors, checks their
device, dtype and size on the host, and passes data pointers plus torch's
current HIP stream to the C entry point of the same name.  Every step of the
computation runs in the library's HIP kernels.  If the library is missing
the import fails (run __graft_entry__.build() or
python mixture_experts_sparse_gemv_amd/build.py first).
"""
import ctypes
import os

import torch  # noqa: F401  (loads the HIP runtime the library links against)

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_mi355x.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(5)
MOE_F32, MOE_BF16 = 0, 1
MOE_SOFTMAX, MOE_SIGMOID_NORM = 0, 1
MOE_RELU, MOE_GELU, MOE_SWIGLU = 0, 1, 2
MOE_ROUTER_BIAS, MOE_EXPERT_BIAS, MOE_W_FP8, MOE_EXPERT_CHOICE = 1, 2, 8, 16
MOE_GEMM_AUTO, MOE_GEMM_MF32, MOE_GEMM_MF16 = 0, 1, 2

# Every symbol include/moe.h declares.
EXPORTS = ("moe_capacity", "moe_workspace_size", "moe_router_topk", "moe_dispatch",
           "moe_expert_ffn", "moe_expert_up", "moe_expert_down", "moe_combine", "moe_aux_stats",
           "moe_routing_stats", "moe_quantize_fp8", "moe_expert_choice", "moe_ffn_forward",
           "moe_ffn_forward_static",
           "moe_backward_workspace_size", "moe_ffn_backward", "moe_set_gemm_policy",
           "moe_status_string", "moe_last_hip_error")


class moe_problem(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("T", "d_model", "d_ff", "num_experts", "top_k", "num_shared", "capacity",
                 "dtype", "gating", "activation", "flags")]


class moe_weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("w_router", "b_router", "w_up", "b_up", "w_down", "b_down", "s_up", "s_down")]


class moe_routing(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("topk_idx", "topk_w", "probs", "counts", "kept", "offsets", "sorted_assign",
                 "assign_row", "drop_mask", "f", "P", "l_aux", "stats", "token_experts")]


class moe_grads(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("dx", "dw_router", "db_router", "dw_up", "db_up", "dw_down", "db_down",
                 "d_topk_w", "d_logits")]


# moe_route_stats: six float32 then two int32 (32 bytes, device memory)
ROUTE_STATS_FLOATS = ("entropy", "entropy_p", "entropy_max", "util_mean", "util_var", "util_cv")
ROUTE_STATS_INTS = ("dropped", "idle")


class MoeError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        msg = _lib.moe_status_string(status).decode()
        if status == MOE_ERR_HIP:
            msg += f" (hipError {_lib.moe_last_hip_error()})"
        super().__init__(f"{fn}: {msg}")


def _load(path=LIB_PATH):
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run __graft_entry__.build()")
    lib = ctypes.CDLL(path)
    P, V, I32, SZ = ctypes.POINTER, ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    pp, pw, pr, pg = P(moe_problem), P(moe_weights), P(moe_routing), P(moe_grads)
    sig = {
        "moe_capacity": (I32, [I32, I32, I32, ctypes.c_float]),
        "moe_workspace_size": (I32, [pp, P(SZ)]),
        "moe_router_topk": (I32, [pp, V, pw, V, V, V, V, V, SZ, V]),
        "moe_dispatch": (I32, [pp, V, V, V, V, V, V, V, V, SZ, V]),
        "moe_expert_ffn": (I32, [pp, V, pw, V, V, V, V, SZ, V]),
        "moe_expert_up": (I32, [pp, V, pw, V, V, V, V, SZ, V]),
        "moe_expert_down": (I32, [pp, pw, V, V, V, V, SZ, V]),
        "moe_combine": (I32, [pp, V, V, V, V, V, V]),
        "moe_aux_stats": (I32, [pp, V, V, V, V, V, V]),
        "moe_routing_stats": (I32, [pp, V, V, V, V, V]),
        "moe_quantize_fp8": (I32, [V, ctypes.c_int64, I32, V, V, V]),
        "moe_expert_choice": (I32, [pp, V, V, V, V, V, V, SZ, V]),
        "moe_ffn_forward": (I32, [pp, pw, V, V, pr, V, SZ, V]),
        "moe_ffn_forward_static": (I32, [pp, pw, V, V, pr, V]),
        "moe_backward_workspace_size": (I32, [pp, P(SZ)]),
        "moe_ffn_backward": (I32, [pp, pw, V, V, ctypes.c_float, pr, pg, V, SZ, V]),
        "moe_set_gemm_policy": (I32, [I32]),
        "moe_status_string": (ctypes.c_char_p, [I32]),
        "moe_last_hip_error": (I32, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype, fn.argtypes = res, args
    return lib


_lib = _load()


# ---------------------------------------------------------------- helpers

def make_problem(T, d_model, d_ff, num_experts, top_k, num_shared=0, capacity=0,
                 dtype="bf16", gating="softmax", activation="swiglu", router_bias=False,
                 expert_bias=False, w_fp8=False, expert_choice=False):
    return moe_problem(
        T=T, d_model=d_model, d_ff=d_ff, num_experts=num_experts, top_k=top_k,
        num_shared=num_shared, capacity=capacity or 0,
        dtype={"f32": MOE_F32, "bf16": MOE_BF16}[dtype],
        gating={"softmax": MOE_SOFTMAX, "sigmoid_norm": MOE_SIGMOID_NORM}[gating],
        activation={"relu": MOE_RELU, "gelu": MOE_GELU, "swiglu": MOE_SWIGLU}[activation],
        flags=(MOE_ROUTER_BIAS if router_bias else 0) | (MOE_EXPERT_BIAS if expert_bias else 0) |
        (MOE_W_FP8 if w_fp8 else 0) | (MOE_EXPERT_CHOICE if expert_choice else 0))


def make_weights(w_router, b_router, w_up, b_up, w_down, b_down, s_up=None, s_down=None):
    """s_up / s_down: the FP8 row scales when w_up / w_down hold E4M3 codes.
    The tensors stay attached to the returned struct, so that every entry
    point checks their dtypes and sizes against its problem."""
    t = (w_router, b_router, w_up, b_up, w_down, b_down, s_up, s_down)
    w = moe_weights(*[_ptr(v) for v in t])
    w._tensors = dict(zip(("w_router", "b_router", "w_up", "b_up", "w_down", "b_down", "s_up",
                           "s_down"), t))
    return w


def _act_dtype(p):
    return torch.bfloat16 if p.dtype == MOE_BF16 else torch.float32


def _check_x(p, x):
    if x is None:
        raise ValueError("x is required")
    _need(x, p.T * p.d_model, _act_dtype(p), "x")


def _check_weights(p, w):
    """dtype and size of each weight tensor the problem reads (FP8 codes are
    uint8 with float32 row scales)."""
    t = getattr(w, "_tensors", None)
    if t is None:
        return
    E, S, d, f = p.num_experts, p.num_shared, p.d_model, p.d_ff
    F1 = 2 * f if p.activation == MOE_SWIGLU else f
    act = _act_dtype(p)
    wdt = torch.uint8 if p.flags & MOE_W_FP8 else act
    _need(t["w_router"], E * d, act, "w_router")
    _need(t["b_router"], E, act, "b_router")
    _need(t["w_up"], (E + S) * F1 * d, wdt, "w_up")
    _need(t["w_down"], (E + S) * d * f, wdt, "w_down")
    _need(t["b_up"], (E + S) * F1, act, "b_up")
    _need(t["b_down"], (E + S) * d, act, "b_down")
    if p.flags & MOE_W_FP8:
        _need(t["s_up"], (E + S) * F1, torch.float32, "s_up")
        _need(t["s_down"], (E + S) * d, torch.float32, "s_down")


def routing_sizes(p):
    """(element count, dtype) of every moe_routing field for problem p."""
    T, k, E = p.T, p.top_k, p.num_experts
    i32, f32 = torch.int32, torch.float32
    if p.flags & MOE_EXPERT_CHOICE:
        n = E * p.capacity
        return dict(topk_idx=(0, i32), topk_w=(0, f32), probs=(T * E, f32), counts=(E, i32),
                    kept=(E, i32), offsets=(E + 1, i32), sorted_assign=(n, i32),
                    assign_row=(T * E, i32), drop_mask=(0, torch.uint8), f=(E, f32), P=(E, f32),
                    l_aux=(1, f32), stats=(8, i32), token_experts=(T, i32))
    return dict(topk_idx=(T * k, i32), topk_w=(T * k, f32), probs=(T * E, f32), counts=(E, i32),
                kept=(E, i32), offsets=(E + 1, i32), sorted_assign=(T * k, i32),
                assign_row=(T * k, i32), drop_mask=(T * k, torch.uint8), f=(E, f32), P=(E, f32),
                l_aux=(1, f32), stats=(8, i32), token_experts=(0, i32))


def _routing_struct(p, routing):
    sizes = routing_sizes(p)
    for name, t in routing.items():
        if name not in sizes:
            raise ValueError(f"unknown routing field {name}")
        n, dt = sizes[name]
        if name == "stats" and t is not None and t.numel() * t.element_size() < 32:
            raise ValueError("stats: need 32 bytes")
        elif name != "stats":
            _need(t, n, dt, name)
    return moe_routing(**{k: _ptr(v) for k, v in routing.items()})


def _ptr(t):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch tensor")
    if t.device.type != "cuda":
        raise ValueError("tensors must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _check(fn, status):
    if status != MOE_OK:
        raise MoeError(fn, status)


def _need(t, numel, dtype, name):
    if t is None:
        return
    if t.dtype != dtype or t.numel() < numel:
        raise ValueError(f"{name}: need >= {numel} elements of {dtype}, got {t.numel()} of {t.dtype}")


def _ws(ws):
    return (ws.data_ptr(), ws.numel() * ws.element_size()) if ws is not None else (None, 0)


def h_dtype(p):
    """Storage dtype of the intermediate h: fp16 for bf16 problems, fp32 for fp32."""
    return torch.float16 if p.dtype == MOE_BF16 else torch.float32


def routed_rows(p):
    """Rows of the routed experts: T*k assignments, or E*capacity (expert choice)."""
    if p.flags & MOE_EXPERT_CHOICE:
        return p.num_experts * p.capacity
    return p.T * p.top_k


def max_rows(p):
    return routed_rows(p) + p.num_shared * p.T


# ---------------------------------------------------------------- entry points

def moe_capacity(T, k, E, capacity_factor):
    return _lib.moe_capacity(T, k, E, float(capacity_factor))


def moe_workspace_size(p):
    n = ctypes.c_size_t(0)
    _check("moe_workspace_size", _lib.moe_workspace_size(ctypes.byref(p), ctypes.byref(n)))
    return n.value


def workspace(p, device="cuda"):
    """A workspace tensor of moe_workspace_size(p) bytes (torch allocations are
    256-byte aligned)."""
    return torch.empty(moe_workspace_size(p), dtype=torch.uint8, device=device)


def moe_router_topk(p, x, w, topk_idx, topk_w, probs=None, prob_colsum=None, ws=None,
                    stream=None):
    _check_x(p, x)
    _check_weights(p, w)
    _need(topk_idx, p.T * p.top_k, torch.int32, "topk_idx")
    _need(topk_w, p.T * p.top_k, torch.float32, "topk_w")
    _need(probs, p.T * p.num_experts, torch.float32, "probs")
    _need(prob_colsum, p.num_experts, torch.float32, "prob_colsum")
    wp, wb = _ws(ws)
    _check("moe_router_topk", _lib.moe_router_topk(
        ctypes.byref(p), _ptr(x), ctypes.byref(w), _ptr(topk_idx), _ptr(topk_w), _ptr(probs),
        _ptr(prob_colsum), wp, wb, _stream(stream)))


def moe_dispatch(p, topk_idx, counts, kept, offsets, sorted_assign, assign_row, drop_mask,
                 ws=None, stream=None):
    E, n = p.num_experts, p.T * p.top_k
    _need(topk_idx, n, torch.int32, "topk_idx")
    for t, m, nm in ((counts, E, "counts"), (kept, E, "kept"), (offsets, E + 1, "offsets"),
                     (sorted_assign, n, "sorted_assign"), (assign_row, n, "assign_row")):
        _need(t, m, torch.int32, nm)
    _need(drop_mask, n, torch.uint8, "drop_mask")
    wp, wb = _ws(ws)
    _check("moe_dispatch", _lib.moe_dispatch(
        ctypes.byref(p), _ptr(topk_idx), _ptr(counts), _ptr(kept), _ptr(offsets),
        _ptr(sorted_assign), _ptr(assign_row), _ptr(drop_mask), wp, wb, _stream(stream)))


def moe_expert_ffn(p, x, w, offsets, sorted_assign, y_exp, ws, stream=None):
    _check_x(p, x)
    _check_weights(p, w)
    _need(y_exp, max_rows(p) * p.d_model, torch.float32, "y_exp")
    wp, wb = _ws(ws)
    _check("moe_expert_ffn", _lib.moe_expert_ffn(
        ctypes.byref(p), _ptr(x), ctypes.byref(w), _ptr(offsets), _ptr(sorted_assign),
        _ptr(y_exp), wp, wb, _stream(stream)))


def moe_expert_up(p, x, w, offsets, sorted_assign, h, ws=None, stream=None):
    _check_x(p, x)
    _check_weights(p, w)
    _need(h, max_rows(p) * p.d_ff, h_dtype(p), "h")
    wp, wb = _ws(ws)
    _check("moe_expert_up", _lib.moe_expert_up(
        ctypes.byref(p), _ptr(x), ctypes.byref(w), _ptr(offsets), _ptr(sorted_assign), _ptr(h),
        wp, wb, _stream(stream)))


def moe_expert_down(p, w, offsets, h, y_exp, ws, stream=None):
    _check_weights(p, w)
    _need(h, max_rows(p) * p.d_ff, h_dtype(p), "h")
    _need(y_exp, max_rows(p) * p.d_model, torch.float32, "y_exp")
    wp, wb = _ws(ws)
    _check("moe_expert_down", _lib.moe_expert_down(
        ctypes.byref(p), ctypes.byref(w), _ptr(offsets), _ptr(h), _ptr(y_exp), wp, wb,
        _stream(stream)))


def moe_combine(p, topk_w, assign_row, offsets, y_exp, y, stream=None):
    """Expert choice: topk_w = probs [T, E], assign_row = row_of [T, E]."""
    _need(y, p.T * p.d_model, torch.float32, "y")
    _check("moe_combine", _lib.moe_combine(
        ctypes.byref(p), _ptr(topk_w), _ptr(assign_row), _ptr(offsets), _ptr(y_exp), _ptr(y),
        _stream(stream)))


def moe_aux_stats(p, prob_colsum, counts, f, P, l_aux, stream=None):
    _check("moe_aux_stats", _lib.moe_aux_stats(
        ctypes.byref(p), _ptr(prob_colsum), _ptr(counts), _ptr(f), _ptr(P), _ptr(l_aux),
        _stream(stream)))


def route_stats_tensor(device="cuda"):
    """Device buffer for one moe_route_stats (8 x 4 bytes)."""
    return torch.empty(8, dtype=torch.int32, device=device)


def route_stats_dict(t):
    """Decodes a moe_route_stats buffer (copied to the host)."""
    raw = t.detach().to("cpu").contiguous()
    fl = raw.view(torch.float32)
    out = {n: float(fl[i]) for i, n in enumerate(ROUTE_STATS_FLOATS)}
    out.update({n: int(raw[6 + i]) for i, n in enumerate(ROUTE_STATS_INTS)})
    return out


def moe_expert_choice(p, probs, offsets, sorted_assign, row_of, token_experts=None, ws=None,
                      stream=None):
    T, E = p.T, p.num_experts
    _need(probs, T * E, torch.float32, "probs")
    _need(offsets, E + 1, torch.int32, "offsets")
    _need(sorted_assign, E * p.capacity, torch.int32, "sorted_assign")
    _need(row_of, T * E, torch.int32, "row_of")
    _need(token_experts, T, torch.int32, "token_experts")
    wp, wb = _ws(ws)
    _check("moe_expert_choice", _lib.moe_expert_choice(
        ctypes.byref(p), _ptr(probs), _ptr(offsets), _ptr(sorted_assign), _ptr(row_of),
        _ptr(token_experts), wp, wb, _stream(stream)))


def moe_routing_stats(p, counts, kept, P, stats, stream=None):
    _need(counts, p.num_experts, torch.int32, "counts")
    _need(kept, p.num_experts, torch.int32, "kept")
    _need(P, p.num_experts, torch.float32, "P")
    _need(stats, 8, torch.int32, "stats")
    _check("moe_routing_stats", _lib.moe_routing_stats(
        ctypes.byref(p), _ptr(counts), _ptr(kept), _ptr(P), _ptr(stats), _stream(stream)))


def moe_quantize_fp8(w, q, scale, stream=None):
    """Per-row FP8 E4M3 codes of a bf16 tensor whose last dimension is the
    row length: q (uint8, same shape), scale (float32, one per row)."""
    cols = w.shape[-1]
    rows = w.numel() // cols
    if w.dtype != torch.bfloat16:
        raise ValueError("w must be bfloat16")
    _need(q, w.numel(), torch.uint8, "q")
    _need(scale, rows, torch.float32, "scale")
    _check("moe_quantize_fp8", _lib.moe_quantize_fp8(_ptr(w), rows, cols, _ptr(q), _ptr(scale),
                                                     _stream(stream)))


def moe_ffn_forward(p, w, x, y, ws, routing=None, stream=None):
    """routing: optional dict of output tensors named as moe_routing's fields."""
    _need(y, p.T * p.d_model, torch.float32, "y")
    _check_x(p, x)
    _check_weights(p, w)
    r = None
    if routing:
        r = _routing_struct(p, routing)
    wp, wb = _ws(ws)
    _check("moe_ffn_forward", _lib.moe_ffn_forward(
        ctypes.byref(p), ctypes.byref(w), _ptr(x), _ptr(y),
        ctypes.byref(r) if r is not None else None, wp, wb, _stream(stream)))


# bytes of the library's own scratch array (moe_ffn_forward_static)
STATIC_SCRATCH_BYTES = 128 << 20


def moe_ffn_forward_static(p, w, x, y, routing=None, stream=None):
    """moe_ffn_forward with the library's own device scratch array instead
    of a workspace (allocates nothing; calls that overlap on one GPU race)."""
    _need(y, p.T * p.d_model, torch.float32, "y")
    _check_x(p, x)
    _check_weights(p, w)
    r = _routing_struct(p, routing) if routing else None
    _check("moe_ffn_forward_static", _lib.moe_ffn_forward_static(
        ctypes.byref(p), ctypes.byref(w), _ptr(x), _ptr(y),
        ctypes.byref(r) if r is not None else None, _stream(stream)))


def moe_set_gemm_policy(policy):
    """Process-wide grouped GEMM main loop: MOE_GEMM_AUTO (by launch size),
    MOE_GEMM_MF32 or MOE_GEMM_MF16; outputs are the same bit for bit."""
    _check("moe_set_gemm_policy", _lib.moe_set_gemm_policy(int(policy)))


def moe_backward_workspace_size(p):
    n = ctypes.c_size_t(0)
    _check("moe_backward_workspace_size",
           _lib.moe_backward_workspace_size(ctypes.byref(p), ctypes.byref(n)))
    return n.value


def backward_workspace(p, device="cuda"):
    return torch.empty(moe_backward_workspace_size(p), dtype=torch.uint8, device=device)


GRAD_FIELDS = ("dx", "dw_router", "db_router", "dw_up", "db_up", "dw_down", "db_down",
               "d_topk_w", "d_logits")


def moe_ffn_backward(p, w, x, dy, alpha, routing, grads, ws, stream=None):
    """routing: dict of the forward's routing tensors (moe_routing field
    names; topk_idx, topk_w, counts, offsets, sorted_assign, assign_row
    required).  grads: dict of float32 output tensors named as moe_grads'
    fields (dx, dw_router, dw_up, dw_down required)."""
    _need(dy, p.T * p.d_model, torch.float32, "dy")
    F1 = 2 * p.d_ff if p.activation == MOE_SWIGLU else p.d_ff
    nseg = p.num_experts + p.num_shared
    sizes = dict(dx=p.T * p.d_model, dw_router=p.num_experts * p.d_model,
                 db_router=p.num_experts, dw_up=nseg * F1 * p.d_model, db_up=nseg * p.d_ff,
                 dw_down=nseg * p.d_model * p.d_ff, db_down=nseg * p.d_model,
                 d_topk_w=p.T * p.top_k, d_logits=p.T * p.num_experts)
    for k, v in grads.items():
        if k not in sizes:
            raise ValueError(f"unknown gradient {k}")
        _need(v, sizes[k], torch.float32, k)
    _check_x(p, x)
    _check_weights(p, w)
    r = _routing_struct(p, routing)
    g = moe_grads(**{k: _ptr(v) for k, v in grads.items()})
    wp, wb = _ws(ws)
    _check("moe_ffn_backward", _lib.moe_ffn_backward(
        ctypes.byref(p), ctypes.byref(w), _ptr(x), _ptr(dy), float(alpha), ctypes.byref(r),
        ctypes.byref(g), wp, wb, _stream(stream)))
