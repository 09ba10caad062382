"""fp64 CPU oracle for the routed-expert MoE layer -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It never imports the HIP product
package and shares no code with it; both sides take their inputs from
``synthdata``.

The arithmetic lives in ``k3oracle.c`` (plain loops, fp64, sequential
reductions).  This module loads it through ctypes and composes the layer in
the order the pages give for one MoE layer and one token: router scores ->
choose the experts -> run each chosen expert on its packed MXFP4 weights ->
weighted sum (fiv.co.kr "kimi-k3-in-c deep dive": invariant #5 row and the
MoE/routing study-plan row; the expert FFN is SwiGLU,
down(silu(gate x) * up x)).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "k3oracle.c")
_SO = os.path.join(_HERE, "libk3oracle.so")
_lib = None

BIAS_NONE, BIAS_LOGITS, BIAS_SELECT_ONLY = 0, 1, 2
SCORE_SOFTMAX, SCORE_SIGMOID = 0, 1


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc (no fast-math, OpenMP)."""
    if force or not os.path.exists(_SO):
        tmp = _SO + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp",
                               "-Wall", "-Wextra", "-Werror", "-fno-fast-math",
                               _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _SO)
    return _SO


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build(force=True)
        L = ctypes.CDLL(_SO)
        P = ctypes.c_void_p
        I, LG, D = ctypes.c_int, ctypes.c_long, ctypes.c_double
        L.k3o_e2m1.argtypes, L.k3o_e2m1.restype = [I], D
        L.k3o_e8m0.argtypes, L.k3o_e8m0.restype = [I], D
        L.k3o_silu.argtypes, L.k3o_silu.restype = [D], D
        L.k3o_mx_dequant.argtypes = [LG, LG, P, P, P]
        L.k3o_router_logits.argtypes = [I, I, I, P, P, P]
        L.k3o_select_topk.argtypes = [I, I, I, P, P]
        L.k3o_topk_weights.argtypes = [I, I, I, P, P, P]
        L.k3o_sigmoid.argtypes = [LG, P, P]
        L.k3o_sigmoid_weights.argtypes = [I, I, I, P, P, P]
        L.k3o_permute.argtypes, L.k3o_permute.restype = [I, I, I, P, P, P, P, P], I
        L.k3o_mx_quantize.argtypes = [LG, P, P, P]
        L.k3o_gateup.argtypes = [I, I, P, P, P, P, P, P, P, P]
        L.k3o_down.argtypes = [I, I, P, P, P, P]
        L.k3o_num_threads.restype = I
        L.k3o_set_num_threads.argtypes = [I]
        _lib = L
    return _lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# ---------------------------------------------------------------- format ---
def e2m1(code: int) -> float:
    return lib().k3o_e2m1(int(code))


def e8m0(s: int) -> float:
    return lib().k3o_e8m0(int(s))


def silu(z: float) -> float:
    return lib().k3o_silu(float(z))


def num_threads() -> int:
    return lib().k3o_num_threads()


def set_num_threads(n: int) -> None:
    lib().k3o_set_num_threads(int(n))


def mx_dequant(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """[rows, cols/2] codes + [rows, cols/32] scales -> fp64 [rows, cols]."""
    codes, scales = _c(codes, np.uint8), _c(scales, np.uint8)
    rows, cols = codes.shape[0], codes.shape[1] * 2
    assert scales.shape == (rows, cols // 32)
    out = np.empty((rows, cols), np.float64)
    lib().k3o_mx_dequant(rows, cols, _p(codes), _p(scales), _p(out))
    return out


def mx_quantize(v: np.ndarray):
    """Quantise rows of v (length a multiple of 32) to MX: returns codes u8
    [..., n/2] and scales u8 [..., n/32].  fp32 inputs are widened exactly."""
    v = np.asarray(v)
    shp = v.shape
    flat = _c(v.reshape(-1), np.float64)
    assert flat.size % 32 == 0
    nb = flat.size // 32
    codes = np.empty(nb * 16, np.uint8)
    scales = np.empty(nb, np.uint8)
    lib().k3o_mx_quantize(nb, _p(flat), _p(codes), _p(scales))
    return codes.reshape(shp[:-1] + (shp[-1] // 2,)), scales.reshape(shp[:-1] + (shp[-1] // 32,))


# ---------------------------------------------------------------- router ---
def router_logits(x: np.ndarray, wr: np.ndarray) -> np.ndarray:
    x, wr = _c(x, np.float32), _c(wr, np.float32)
    T, d = x.shape
    E = wr.shape[0]
    out = np.empty((T, E), np.float64)
    lib().k3o_router_logits(T, E, d, _p(x), _p(wr), _p(out))
    return out


def select_topk(key: np.ndarray, k: int) -> np.ndarray:
    key = _c(key, np.float64)
    T, E = key.shape
    idx = np.empty((T, k), np.int32)
    lib().k3o_select_topk(T, E, k, _p(key), _p(idx))
    return idx


def topk_weights(logits: np.ndarray, idx: np.ndarray) -> np.ndarray:
    logits, idx = _c(logits, np.float64), _c(idx, np.int32)
    T, E = logits.shape
    k = idx.shape[1]
    w = np.empty((T, k), np.float64)
    lib().k3o_topk_weights(T, E, k, _p(logits), _p(idx), _p(w))
    return w


def sigmoid(logits: np.ndarray) -> np.ndarray:
    logits = _c(logits, np.float64)
    s = np.empty_like(logits)
    lib().k3o_sigmoid(logits.size, _p(logits), _p(s))
    return s


def sigmoid_weights(scores: np.ndarray, idx: np.ndarray) -> np.ndarray:
    scores, idx = _c(scores, np.float64), _c(idx, np.int32)
    T, E = scores.shape
    k = idx.shape[1]
    w = np.empty((T, k), np.float64)
    lib().k3o_sigmoid_weights(T, E, k, _p(scores), _p(idx), _p(w))
    return w


def permute(idx: np.ndarray, E: int) -> dict:
    idx = _c(idx, np.int32)
    T, k = idx.shape
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    perm_pair = np.empty(T * k, np.int32)
    row_of_pair = np.empty(T * k, np.int32)
    rc = lib().k3o_permute(T, E, k, _p(idx), _p(counts), _p(offsets), _p(perm_pair), _p(row_of_pair))
    if rc != 0:
        raise ValueError("expert index out of range or repeated within a token")
    return dict(counts=counts, offsets=offsets, perm_pair=perm_pair, row_of_pair=row_of_pair)


def route(x: np.ndarray, wr: np.ndarray, k: int, bias=None, bias_mode: int = BIAS_NONE,
          score_fn: int = SCORE_SOFTMAX) -> dict:
    """Router (O2-O5): fp64 logits, optional per-expert bias, top-k selection
    with lower-index ties, renormalised weights, expert grouping.

    bias_mode BIAS_LOGITS adds the bias to the logits (it changes both the
    choice and the weights); BIAS_SELECT_ONLY adds it to the selection key only
    and weights come from the unbiased scores (fiv.co.kr deep dive, invariant
    #5: the routing bias steers selection only).

    score_fn SCORE_SOFTMAX selects on the logits and weights by the softmax
    restricted to the selection; SCORE_SIGMOID (the pages' router) scores
    s = sigmoid(l), selects on s (+ bias under BIAS_SELECT_ONLY) and weights
    by the chosen s renormalised to sum to one."""
    logits = router_logits(x, wr)
    b = None
    if bias is not None and bias_mode != BIAS_NONE:
        b = np.asarray(bias, np.float32).astype(np.float64)
        if bias_mode == BIAS_LOGITS:
            logits = logits + b[None, :]
        elif bias_mode != BIAS_SELECT_ONLY:
            raise ValueError("unknown bias mode")
    if score_fn == SCORE_SOFTMAX:
        score = logits
    elif score_fn == SCORE_SIGMOID:
        score = sigmoid(logits)
    else:
        raise ValueError("unknown score function")
    key = score + b[None, :] if (b is not None and bias_mode == BIAS_SELECT_ONLY) else score
    idx = select_topk(key, k)
    w = topk_weights(logits, idx) if score_fn == SCORE_SOFTMAX else sigmoid_weights(score, idx)
    out = dict(logits=logits, key=key, topk_idx=idx, topk_w=w)
    out.update(permute(idx, wr.shape[0]))
    return out


# ----------------------------------------------------------------- expert ---
def gateup(x: np.ndarray, gate, up, return_gu: bool = False):
    """h = silu(Wg x) * (Wu x) for one expert; gate/up are (codes, scales) of
    [f, d] MX matrices; x is fp64 [d]."""
    gc, gs = (_c(a, np.uint8) for a in gate)
    uc, us = (_c(a, np.uint8) for a in up)
    f, d = gc.shape[0], gc.shape[1] * 2
    x = _c(x, np.float64)
    assert x.shape == (d,)
    h = np.empty(f, np.float64)
    g = np.empty(f, np.float64) if return_gu else None
    u = np.empty(f, np.float64) if return_gu else None
    lib().k3o_gateup(d, f, _p(x), _p(gc), _p(gs), _p(uc), _p(us), _p(h),
                     _p(g) if return_gu else None, _p(u) if return_gu else None)
    return (h, g, u) if return_gu else h


def down(h: np.ndarray, dn) -> np.ndarray:
    """o = Wd h for one expert; dn = (codes, scales) of a [d, f] MX matrix."""
    dc, ds = (_c(a, np.uint8) for a in dn)
    d, f = dc.shape[0], dc.shape[1] * 2
    h = _c(h, np.float64)
    assert h.shape == (f,)
    o = np.empty(d, np.float64)
    lib().k3o_down(d, f, _p(h), _p(dc), _p(ds), _p(o))
    return o


def expert_ffn(x: np.ndarray, ex: dict) -> np.ndarray:
    return down(gateup(x, ex["gate"], ex["up"]), ex["down"])


def mx_roundtrip(v: np.ndarray) -> np.ndarray:
    """deq(Q(v)) for a vector whose length is a multiple of 32."""
    c, s = mx_quantize(v)
    return mx_dequant(c.reshape(1, -1), s.reshape(1, -1)).reshape(-1)


def token_forward(x_t: np.ndarray, experts_t, w_t, get_expert, act_mode: str = "fp32",
                  h_override=None, keep: dict | None = None) -> np.ndarray:
    """y_t = sum_j w_j * FFN_{e_j}(x_t), j ascending, fp64 (O6 / O7).

    act_mode "mxfp4": x_t is replaced by deq(Q(x_t)) once for all experts and
    each expert's h by deq(Q(h)) before the down projection.  ``h_override``
    (optional, one fp32/fp64 h vector per j) replaces the oracle's own h before
    that quantisation; it is how the split-step checks feed the device's h in.
    ``keep`` (optional dict) receives the intermediates."""
    x = np.asarray(x_t, np.float64)
    if act_mode == "mxfp4":
        x = mx_roundtrip(np.asarray(x_t, np.float32))
    elif act_mode != "fp32":
        raise ValueError("unknown activation mode")
    y = np.zeros(x.shape[0], np.float64)
    hs, hq = [], []
    for j, e in enumerate(experts_t):
        ex = get_expert(int(e))
        h = gateup(x, ex["gate"], ex["up"])
        hs.append(h)
        if h_override is not None:
            h = np.asarray(h_override[j])
        if act_mode == "mxfp4":
            c, s = mx_quantize(h.reshape(1, -1))
            hq.append((c, s))
            h = mx_dequant(c, s).reshape(-1)
        y += float(w_t[j]) * down(h, ex["down"])
    if keep is not None:
        keep.update(x_used=x, h=hs, h_q=hq)
    return y


def layer_forward(x: np.ndarray, route: dict, tokens, get_expert, act_mode: str = "fp32",
                  h_override=None, keep: dict | None = None) -> np.ndarray:
    """y rows (fp64) of the given tokens: for each, exactly the sum
    token_forward forms (y_t = sum_j w_j * FFN_{e_j}(x_t), j ascending, from
    y = 0), but the experts are visited once each, in ascending id, for all of
    their pairs among these tokens, so that each expert's weights are fetched
    once.  ``get_expert`` is called with the needed ids in ascending order.
    ``h_override(t)`` (optional) returns the k h vectors of token t that
    replace the oracle's own h, as in token_forward.  ``keep`` (optional
    dict) receives keep["h"][(t, j)], the oracle's own h of each pair (from
    the quantised x in "mxfp4" mode), computed even where h_override
    replaces it."""
    if act_mode not in ("fp32", "mxfp4"):
        raise ValueError("unknown activation mode")
    tokens = [int(t) for t in tokens]
    idx, w = route["topk_idx"], route["topk_w"]
    k = idx.shape[1]
    xin = {}
    for t in tokens:
        xin[t] = (mx_roundtrip(np.asarray(x[t], np.float32)) if act_mode == "mxfp4"
                  else np.asarray(x[t], np.float64))
    by_expert = {}
    for t in tokens:
        for j in range(k):
            by_expert.setdefault(int(idx[t, j]), []).append((t, j))
    hov = {t: h_override(t) for t in tokens} if h_override is not None else None
    o = {}
    for e in sorted(by_expert):
        ex = get_expert(e)
        for t, j in by_expert[e]:
            h = None
            if hov is None or keep is not None:
                h = gateup(xin[t], ex["gate"], ex["up"])
                if keep is not None:
                    keep.setdefault("h", {})[(t, j)] = h
            if hov is not None:
                h = np.asarray(hov[t][j])
            if act_mode == "mxfp4":
                c, s = mx_quantize(h.reshape(1, -1))
                h = mx_dequant(c, s).reshape(-1)
            o[(t, j)] = down(h, ex["down"])
    out = np.empty((len(tokens), x.shape[1]), np.float64)
    for i, t in enumerate(tokens):
        y = np.zeros(x.shape[1], np.float64)
        for j in range(k):
            y += float(w[t][j]) * o[(t, j)]
        out[i] = y
    return out
