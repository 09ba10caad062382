"""Python binding of the k3moe C ABI (include/k3moe.h) -- argument marshalling only.

Every step of the routed-expert MoE layer runs in the gfx950 HIP library
``libk3moe.so``; this module only turns torch tensors into device pointers,
sizes and the current HIP stream.  PyTorch provides device memory and streams.

The library must be built first (``python -m mxfp4_routed_expert_softmax_amd.build``);
importing this package without it raises ImportError: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  -- loads torch's HIP runtime first, so the library binds to the same one

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libk3moe.so")

K3MOE_OK, K3MOE_EINVAL, K3MOE_EWORKSPACE, K3MOE_ENOTSUP, K3MOE_EHIP = 0, -1, -2, -3, -4
K3MOE_BIAS_NONE, K3MOE_BIAS_LOGITS, K3MOE_BIAS_SELECT_ONLY = 0, 1, 2
K3MOE_ACT_FP32, K3MOE_ACT_MXFP4 = 0, 1
K3MOE_SCORE_SOFTMAX, K3MOE_SCORE_SIGMOID = 0, 1

EXPORTS = ("k3moe_workspace_size", "k3moe_route", "k3moe_ffn", "k3moe_forward", "k3moe_forward_noalloc",
           "k3moe_cache_state_bytes", "k3moe_cache_reset", "k3moe_forward_cached", "k3moe_cache_read",
           "k3moe_set_stage_marks", "k3moe_status_string", "k3moe_last_hip_error")
NOALLOC_SCRATCH_BYTES = 64 << 20  # K3MOE_NOALLOC_SCRATCH_BYTES
MAX_MARKS = 8  # K3MOE_MAX_MARKS
KERNEL_KINDS = {1: "active_list", 2: "quantize", 3: "gateup", 4: "down", 5: "down_combine", 6: "combine"}

_BIAS = {"none": K3MOE_BIAS_NONE, "logits": K3MOE_BIAS_LOGITS, "select_only": K3MOE_BIAS_SELECT_ONLY}
_ACT = {"fp32": K3MOE_ACT_FP32, "mxfp4": K3MOE_ACT_MXFP4}
_SCORE = {"softmax": K3MOE_SCORE_SOFTMAX, "sigmoid": K3MOE_SCORE_SIGMOID}


class Dims(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("E", ctypes.c_int32), ("k", ctypes.c_int32),
                ("d_model", ctypes.c_int32), ("d_ff", ctypes.c_int32)]


class MX(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p)]


class Experts(ctypes.Structure):
    _fields_ = [("gate", MX), ("up", MX), ("down", MX)]


class Debug(ctypes.Structure):
    _fields_ = [("x_codes", ctypes.c_void_p), ("x_scales", ctypes.c_void_p), ("h", ctypes.c_void_p),
                ("h_codes", ctypes.c_void_p), ("h_scales", ctypes.c_void_p)]


class K3MoEError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = _lib().k3moe_status_string(status).decode()
        if status == K3MOE_EHIP:
            msg += f" (hipError_t {_lib().k3moe_last_hip_error()})"
        super().__init__(f"{where}: {msg} [{status}]")


_L = None


def _lib():
    global _L
    if _L is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run python -m mxfp4_routed_expert_softmax_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        P, I, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        DP = ctypes.POINTER(Dims)
        L.k3moe_workspace_size.argtypes = [DP, I, ctypes.POINTER(SZ)]
        L.k3moe_route.argtypes = [DP, P, P, P, I, I, P, P, P, P, P, P, P, SZ, P]
        L.k3moe_ffn.argtypes = [DP, P, ctypes.POINTER(Experts), P, P, P, P, P, P, I, P,
                                ctypes.POINTER(Debug), P, SZ, P]
        L.k3moe_forward.argtypes = [DP, P, P, P, I, I, ctypes.POINTER(Experts), I, P, P, P, P, P, P, P,
                                    ctypes.POINTER(Debug), P, SZ, P]
        L.k3moe_forward_noalloc.argtypes = [DP, P, P, P, I, I, ctypes.POINTER(Experts), I, P, P, P, P, P, P, P,
                                            ctypes.POINTER(Debug), P]
        L.k3moe_cache_state_bytes.argtypes = [I, I, ctypes.POINTER(SZ)]
        L.k3moe_cache_reset.argtypes = [P, I, I, P]
        L.k3moe_forward_cached.argtypes = [DP, P, P, P, I, I, ctypes.POINTER(Experts), ctypes.POINTER(Experts), I, P,
                                           I, P, P, P, P, P, P, P, P, SZ, P]
        L.k3moe_cache_read.argtypes = [P, I, I, P, P, P, P]
        L.k3moe_set_stage_marks.argtypes = [ctypes.POINTER(P), I, P, P]
        L.k3moe_status_string.argtypes = [I]
        L.k3moe_status_string.restype = ctypes.c_char_p
        L.k3moe_last_hip_error.argtypes = []
        for name in ("k3moe_workspace_size", "k3moe_route", "k3moe_ffn", "k3moe_forward", "k3moe_forward_noalloc",
                     "k3moe_cache_state_bytes", "k3moe_cache_reset", "k3moe_forward_cached", "k3moe_cache_read",
                     "k3moe_set_stage_marks", "k3moe_last_hip_error"):
            getattr(L, name).restype = I
        _L = L
    return _L


def lib():
    """The loaded ctypes library (raises ImportError if it is not built)."""
    return _lib()


def _ptr(t):
    if t is None:
        return None
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _check(rc, where):
    if rc != K3MOE_OK:
        raise K3MoEError(rc, where)


def _need(t, dtype, shape, name):
    if t.dtype != dtype or tuple(t.shape) != tuple(shape) or not t.is_contiguous() or not t.is_cuda:
        raise ValueError(f"{name}: expected contiguous {dtype} cuda tensor of shape {tuple(shape)}, "
                         f"got {t.dtype} {tuple(t.shape)} on {t.device}")


def make_experts(experts: dict, E: int, d: int, f: int, host: bool = False) -> Experts:
    """{'gate': (codes, scales), 'up': ..., 'down': ...} of uint8 cuda tensors
    ([E, f, d/2] + [E, f, d/32] for gate/up, [E, d, f/2] + [E, d, f/32] for
    down) -> the C struct.  host=True: pinned CPU tensors instead (the host
    store of the expert cache; pinned memory is readable by the device at its
    host address)."""
    shp = {"gate": (f, d), "up": (f, d), "down": (d, f)}
    mats = []
    for w in ("gate", "up", "down"):
        c, s = experts[w]
        rows, cols = shp[w]
        if host:
            for t, n, sh in ((c, "codes", (E, rows, cols // 2)), (s, "scales", (E, rows, cols // 32))):
                if t.dtype != torch.uint8 or tuple(t.shape) != sh or not t.is_contiguous() or t.is_cuda \
                        or not t.is_pinned():
                    raise ValueError(f"{w}.{n}: expected a contiguous pinned uint8 CPU tensor of shape {sh}")
        else:
            _need(c, torch.uint8, (E, rows, cols // 2), f"{w}.codes")
            _need(s, torch.uint8, (E, rows, cols // 32), f"{w}.scales")
        mats.append(MX(c.data_ptr(), s.data_ptr()))
    return Experts(*mats)


def k3moe_workspace_size(T: int, E: int, k: int, d_model: int, d_ff: int, act_mode="fp32") -> int:
    dims = Dims(T, E, k, d_model, d_ff)
    n = ctypes.c_size_t(0)
    _check(_lib().k3moe_workspace_size(ctypes.byref(dims), _ACT[act_mode], ctypes.byref(n)),
           "k3moe_workspace_size")
    return n.value


def alloc_workspace(T, E, k, d_model, d_ff, act_mode="fp32", device="cuda"):
    n = k3moe_workspace_size(T, E, k, d_model, d_ff, act_mode)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def alloc_route(T: int, E: int, k: int, device="cuda") -> dict:
    i32 = dict(dtype=torch.int32, device=device)
    return dict(topk_idx=torch.empty((T, k), **i32), topk_w=torch.empty((T, k), dtype=torch.float32, device=device),
                counts=torch.empty(E, **i32), offsets=torch.empty(E + 1, **i32),
                perm_pair=torch.empty(T * k, **i32), row_of_pair=torch.empty(T * k, **i32))


def k3moe_route(x, w_router, k, bias=None, bias_mode="none", out=None, ws=None, stream=None,
                score_fn="softmax") -> dict:
    T, d = x.shape
    E = w_router.shape[0]
    _need(x, torch.float32, (T, d), "x")
    _need(w_router, torch.float32, (E, d), "w_router")
    if bias is not None:
        _need(bias, torch.float32, (E,), "bias")
    out = out if out is not None else alloc_route(T, E, k, x.device)
    ws = ws if ws is not None else alloc_workspace(T, E, k, d, 32, "mxfp4", x.device)
    dims = Dims(T, E, k, d, 32)  # d_ff does not enter routing; any valid value
    rc = _lib().k3moe_route(ctypes.byref(dims), _ptr(x), _ptr(w_router), _ptr(bias), _BIAS[bias_mode],
                            _SCORE[score_fn], _ptr(out["topk_idx"]), _ptr(out["topk_w"]), _ptr(out["counts"]),
                            _ptr(out["offsets"]), _ptr(out["perm_pair"]), _ptr(out["row_of_pair"]),
                            _ptr(ws), ws.numel(), _stream(stream))
    _check(rc, "k3moe_route")
    return out


def _debug_struct(dbg):
    if dbg is None:
        return None
    return Debug(*(dbg[k].data_ptr() if dbg.get(k) is not None else None
                   for k in ("x_codes", "x_scales", "h", "h_codes", "h_scales")))


def k3moe_ffn(x, experts, route, act_mode="fp32", y=None, dbg=None, ws=None, stream=None):
    T, d = x.shape
    E = route["counts"].shape[0]
    k = route["topk_idx"].shape[1] if T else 1
    f = experts["gate"][0].shape[1]
    _need(x, torch.float32, (T, d), "x")
    ex = make_experts(experts, E, d, f)
    y = y if y is not None else torch.empty((T, d), dtype=torch.float32, device=x.device)
    ws = ws if ws is not None else alloc_workspace(T, E, k, d, f, act_mode, x.device)
    dims = Dims(T, E, k, d, f)
    dstruct = _debug_struct(dbg)
    rc = _lib().k3moe_ffn(ctypes.byref(dims), _ptr(x), ctypes.byref(ex), _ptr(route["topk_idx"]),
                          _ptr(route["topk_w"]), _ptr(route["counts"]), _ptr(route["offsets"]),
                          _ptr(route["perm_pair"]), _ptr(route["row_of_pair"]), _ACT[act_mode], _ptr(y),
                          ctypes.byref(dstruct) if dstruct is not None else None,
                          _ptr(ws), ws.numel(), _stream(stream))
    _check(rc, "k3moe_ffn")
    return y


class Forward:
    """The layer bound once to fixed buffers, so repeated calls (a decode loop,
    a benchmark) cost one ctypes call each.  ``run_route`` / ``run_ffn`` issue
    k3moe_route / k3moe_ffn, ``__call__`` issues k3moe_forward; all on the
    current torch stream unless ``stream`` is given.  ``set_x`` rebinds the
    activations to another tensor of the same shape."""

    def __init__(self, x, w_router, experts, k, bias=None, bias_mode="none", act_mode="fp32",
                 dbg=None, stream=None, score_fn="softmax"):
        T, d = x.shape
        E = w_router.shape[0]
        f = experts["gate"][0].shape[1]
        _need(x, torch.float32, (T, d), "x")
        _need(w_router, torch.float32, (E, d), "w_router")
        if bias is not None:
            _need(bias, torch.float32, (E,), "bias")
        self.dims = Dims(T, E, k, d, f)
        self.experts = make_experts(experts, E, d, f)
        self.route = alloc_route(T, E, k, x.device)
        self.y = torch.empty((T, d), dtype=torch.float32, device=x.device)
        self.ws = alloc_workspace(T, E, k, d, f, act_mode, x.device)
        self._keep = [x, w_router, bias, experts, dbg]
        self._dbg = _debug_struct(dbg)
        self._dbgp = ctypes.byref(self._dbg) if self._dbg is not None else None
        self._x = _ptr(x)
        self._bias_mode = _BIAS[bias_mode]
        self._score = _SCORE[score_fn]
        self._act = _ACT[act_mode]
        self._wr, self._bias = _ptr(w_router), _ptr(bias)
        r = self.route
        self._r = [_ptr(r[n]) for n in ("topk_idx", "topk_w", "counts", "offsets", "perm_pair",
                                        "row_of_pair")]
        self._y, self._ws, self._wsn = _ptr(self.y), _ptr(self.ws), self.ws.numel()
        self.stream = stream

    def set_x(self, x):
        _need(x, torch.float32, (self.dims.T, self.dims.d_model), "x")
        self._x = _ptr(x)
        self._keep[0] = x

    def run_route(self):
        rc = _lib().k3moe_route(ctypes.byref(self.dims), self._x, self._wr, self._bias, self._bias_mode,
                                self._score, *self._r, self._ws, self._wsn, _stream(self.stream))
        _check(rc, "k3moe_route")

    def run_ffn(self):
        rc = _lib().k3moe_ffn(ctypes.byref(self.dims), self._x, ctypes.byref(self.experts), *self._r,
                              self._act, self._y, self._dbgp, self._ws, self._wsn, _stream(self.stream))
        _check(rc, "k3moe_ffn")
        return self.y

    def __call__(self):
        rc = _lib().k3moe_forward(ctypes.byref(self.dims), self._x, self._wr, self._bias, self._bias_mode,
                                  self._score, ctypes.byref(self.experts), self._act, *self._r, self._y, self._dbgp,
                                  self._ws, self._wsn, _stream(self.stream))
        _check(rc, "k3moe_forward")
        return self.y


class StageMarks:
    """Kernel timing marks of the expert-FFN stage (k3moe_set_stage_marks).
    ``set()`` makes this object's n event pairs the marks of this host
    thread, ``clear()`` switches marking off.  After a marked call,
    ``kernel_ms(i)`` is kernel i's own duration (its dispatch's start and end
    events), ``kinds()`` names the kernels and ``launched`` is the number the
    stage launched."""

    def __init__(self, n=MAX_MARKS, stream=None):
        if not 1 <= n <= MAX_MARKS:
            raise ValueError(f"1 <= n <= {MAX_MARKS}")
        st = stream if stream is not None else torch.cuda.current_stream()
        self.n = n
        self.events = [torch.cuda.Event(enable_timing=True) for _ in range(2 * n)]
        for e in self.events:
            e.record(st)  # the HIP event is created on the first record
        self._handles = (ctypes.c_void_p * (2 * n))(*[e.cuda_event for e in self.events])
        self._kinds = (ctypes.c_int * n)()
        self._launched = ctypes.c_int(0)

    def set(self):
        rc = _lib().k3moe_set_stage_marks(self._handles, self.n, ctypes.cast(self._kinds, ctypes.c_void_p),
                                          ctypes.c_void_p(ctypes.addressof(self._launched)))
        _check(rc, "k3moe_set_stage_marks")

    @staticmethod
    def clear():
        _check(_lib().k3moe_set_stage_marks(None, 0, None, None), "k3moe_set_stage_marks")

    @property
    def launched(self):
        return self._launched.value

    def kinds(self):
        return [KERNEL_KINDS.get(self._kinds[i], "?") for i in range(min(self.launched, self.n))]

    def kernel_ms(self, i):
        return self.events[2 * i].elapsed_time(self.events[2 * i + 1])


def k3moe_forward(x, w_router, experts, k, bias=None, bias_mode="none", act_mode="fp32", dbg=None,
                  stream=None, score_fn="softmax"):
    """Route + expert FFN + combine in one C call; returns (y, routing dict)."""
    fw = Forward(x, w_router, experts, k, bias, bias_mode, act_mode, dbg, stream, score_fn)
    y = fw()
    return y, fw.route


def k3moe_forward_noalloc(x, w_router, experts, k, bias=None, bias_mode="none", act_mode="fp32", dbg=None,
                          stream=None, score_fn="softmax", out=None):
    """Route + expert FFN + combine through k3moe_forward_noalloc: no
    workspace; the library's fixed per-device scratch is used instead.
    ``out`` optionally gives (y, routing dict) to write into.  Returns (y,
    routing dict)."""
    T, d = x.shape
    E = w_router.shape[0]
    f = experts["gate"][0].shape[1]
    _need(x, torch.float32, (T, d), "x")
    _need(w_router, torch.float32, (E, d), "w_router")
    if bias is not None:
        _need(bias, torch.float32, (E,), "bias")
    if out is None:
        y = torch.empty((T, d), dtype=torch.float32, device=x.device)
        route = alloc_route(T, E, k, x.device)
    else:
        y, route = out
        _need(y, torch.float32, (T, d), "y")
    ex = make_experts(experts, E, d, f)
    dims = Dims(T, E, k, d, f)
    dstruct = _debug_struct(dbg)
    r = [_ptr(route[n]) for n in ("topk_idx", "topk_w", "counts", "offsets", "perm_pair", "row_of_pair")]
    rc = _lib().k3moe_forward_noalloc(ctypes.byref(dims), _ptr(x), _ptr(w_router), _ptr(bias), _BIAS[bias_mode],
                                      _SCORE[score_fn], ctypes.byref(ex), _ACT[act_mode], *r, _ptr(y),
                                      ctypes.byref(dstruct) if dstruct is not None else None, _stream(stream))
    _check(rc, "k3moe_forward_noalloc")
    return y, route


# ---- HBM expert cache ---------------------------------------------------------
def k3moe_cache_state_bytes(E: int, n_slots: int) -> int:
    n = ctypes.c_size_t(0)
    _check(_lib().k3moe_cache_state_bytes(E, n_slots, ctypes.byref(n)), "k3moe_cache_state_bytes")
    return n.value


class CachedForward:
    """k3moe_forward_cached bound to fixed buffers: the experts of a layer in
    pinned host memory (``host_experts``, same dict layout as the device
    experts but pinned CPU tensors), ``n_slots`` experts' worth of HBM slots
    and the cache state, all allocated here; ``reset`` empties the cache,
    ``__call__`` runs one step (routing, policy update, copy of the missed
    experts, expert FFN) and returns y; ``read`` returns the cache state."""

    def __init__(self, x, w_router, host_experts, n_slots, k, bias=None, bias_mode="none", act_mode="fp32",
                 stream=None, score_fn="softmax"):
        T, d = x.shape
        E = w_router.shape[0]
        f = host_experts["gate"][0].shape[1]
        _need(x, torch.float32, (T, d), "x")
        _need(w_router, torch.float32, (E, d), "w_router")
        if bias is not None:
            _need(bias, torch.float32, (E,), "bias")
        dev = x.device
        self.E, self.n_slots = E, n_slots
        self.dims = Dims(T, E, k, d, f)
        self.host = make_experts(host_experts, E, d, f, host=True)
        shp = {"gate": (f, d), "up": (f, d), "down": (d, f)}
        self.slots = {w: (torch.empty((n_slots, r, c // 2), dtype=torch.uint8, device=dev),
                          torch.empty((n_slots, r, c // 32), dtype=torch.uint8, device=dev))
                      for w, (r, c) in shp.items()}
        self.slot_struct = make_experts(self.slots, n_slots, d, f)
        self.state = torch.empty(max(k3moe_cache_state_bytes(E, n_slots), 256), dtype=torch.uint8, device=dev)
        self.route = alloc_route(T, E, k, dev)
        self.y = torch.empty((T, d), dtype=torch.float32, device=dev)
        self.ws = alloc_workspace(T, E, k, d, f, act_mode, dev)
        self._keep = [x, w_router, bias, host_experts]
        self._x, self._wr, self._bias = _ptr(x), _ptr(w_router), _ptr(bias)
        self._bias_mode, self._score, self._act = _BIAS[bias_mode], _SCORE[score_fn], _ACT[act_mode]
        self._r = [_ptr(self.route[n]) for n in ("topk_idx", "topk_w", "counts", "offsets", "perm_pair",
                                                 "row_of_pair")]
        self.stream = stream
        self.reset()

    def set_x(self, x):
        _need(x, torch.float32, (self.dims.T, self.dims.d_model), "x")
        self._x = _ptr(x)
        self._keep[0] = x

    def reset(self):
        _check(_lib().k3moe_cache_reset(_ptr(self.state), self.E, self.n_slots, _stream(self.stream)),
               "k3moe_cache_reset")

    def __call__(self):
        rc = _lib().k3moe_forward_cached(ctypes.byref(self.dims), self._x, self._wr, self._bias, self._bias_mode,
                                         self._score, ctypes.byref(self.host), ctypes.byref(self.slot_struct),
                                         self.n_slots, _ptr(self.state), self._act, *self._r, _ptr(self.y),
                                         _ptr(self.ws), self.ws.numel(), _stream(self.stream))
        _check(rc, "k3moe_forward_cached")
        return self.y

    def read(self) -> dict:
        stats = (ctypes.c_int64 * 4)()
        slot_of = (ctypes.c_int32 * self.E)()
        expert_in = (ctypes.c_int32 * self.n_slots)()
        _check(_lib().k3moe_cache_read(_ptr(self.state), self.E, self.n_slots, stats, slot_of, expert_in,
                                       _stream(self.stream)), "k3moe_cache_read")
        return {"steps": stats[0], "hits": stats[1], "misses": stats[2], "last_misses": stats[3],
                "slot_of": list(slot_of), "expert_in": list(expert_in)}
