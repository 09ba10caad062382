"""CPU checks of the C ABI: the library loads, exports every declared entry
point, and refuses bad arguments before any HIP call (no GPU needed)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "k3moe.h")

k3 = pytest.importorskip("mxfp4_routed_expert_softmax_amd")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(k3moe_[a-z_]+)\s*\(", src)))


def test_every_declared_symbol_is_exported():
    names = _declared()
    assert set(names) == set(k3.EXPORTS)
    lib = k3.lib()
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    lib = k3.lib()
    for rc in (0, -1, -2, -3, -4):
        assert lib.k3moe_status_string(rc)
    assert lib.k3moe_status_string(7) == b"unknown status"


def _ws(T, E, k, d, f, mode=0):
    lib = k3.lib()
    dims = k3.Dims(T, E, k, d, f)
    n = ctypes.c_size_t(0)
    rc = lib.k3moe_workspace_size(ctypes.byref(dims), mode, ctypes.byref(n))
    return rc, n.value


@pytest.mark.parametrize("dims,rc", [
    ((1, 16, 2, 256, 128), 0),
    ((0, 16, 2, 256, 128), 0),
    ((-1, 16, 2, 256, 128), -1),
    ((1, 0, 1, 256, 128), -1),
    ((1, 16, 0, 256, 128), -1),
    ((1, 16, 17, 256, 128), -1),     # k > E
    ((1, 16, 2, 250, 128), -1),      # d % 32
    ((1, 16, 2, 256, 100), -1),      # f % 32
    ((1, 2048, 2, 256, 128), -3),    # E > 1024
    ((1, 64, 33, 256, 128), -3),     # k > 32
    ((1, 16, 2, 16384, 16384), 0),   # the widest rows the GEMVs cover
    ((1, 16, 2, 16416, 128), -3),    # d_model > 16384: refused, never truncated
    ((1, 16, 2, 256, 16416), -3),    # d_ff > 16384
    ((4096, 896, 16, 16416, 2048), -3),
])
def test_dims_validation(dims, rc):
    assert _ws(*dims)[0] == rc


def test_unknown_act_mode_refused():
    assert _ws(1, 16, 2, 256, 128, mode=7)[0] == k3.K3MOE_ENOTSUP


def test_workspace_grows_with_tokens():
    sizes = [_ws(T, 896, 16, 7168, 2048)[1] for T in (1, 2, 64, 65, 4096)]
    assert all(a < b for a, b in zip(sizes, sizes[1:]))
    mx = [_ws(T, 896, 16, 7168, 2048, 1)[1] for T in (1, 64, 4096)]
    assert all(a < b for a, b in zip(mx, mx[1:]))


def test_route_rejects_bad_arguments_without_touching_the_gpu():
    lib = k3.lib()
    dims = k3.Dims(4, 16, 2, 256, 128)
    fake = ctypes.c_void_p(0x10000)  # never dereferenced: checks fail first
    # x, w_router, bias, bias_mode, score_fn, 6 outputs, ws, ws_bytes, stream
    args = [fake] * 2 + [None, 0, 0] + [fake] * 6 + [fake, 1 << 30, None]
    # null x
    a = list(args)
    a[0] = None
    assert lib.k3moe_route(ctypes.byref(dims), *a) == k3.K3MOE_EINVAL
    # bias required for a bias mode
    a = list(args)
    a[3] = k3.K3MOE_BIAS_LOGITS
    assert lib.k3moe_route(ctypes.byref(dims), *a) == k3.K3MOE_EINVAL
    # unknown bias mode
    a = list(args)
    a[3] = 9
    assert lib.k3moe_route(ctypes.byref(dims), *a) == k3.K3MOE_ENOTSUP
    # unknown score function (refused, never defaulted)
    a = list(args)
    a[4] = 2
    assert lib.k3moe_route(ctypes.byref(dims), *a) == k3.K3MOE_ENOTSUP
    a[4] = -1
    assert lib.k3moe_route(ctypes.byref(dims), *a) == k3.K3MOE_ENOTSUP
    # workspace too small / missing
    a = list(args)
    a[12] = 16
    assert lib.k3moe_route(ctypes.byref(dims), *a) == k3.K3MOE_EWORKSPACE
    a = list(args)
    a[11] = None
    assert lib.k3moe_route(ctypes.byref(dims), *a) == k3.K3MOE_EWORKSPACE
    # misaligned activations
    a = list(args)
    a[0] = ctypes.c_void_p(0x10004)
    assert lib.k3moe_route(ctypes.byref(dims), *a) == k3.K3MOE_EINVAL
    # T == 0 is a no-op that succeeds without any pointer
    z = k3.Dims(0, 16, 2, 256, 128)
    assert lib.k3moe_route(ctypes.byref(z), *([None] * 3 + [0, 0] + [None] * 6 + [None, 0, None])) == 0


def test_ffn_rejects_bad_arguments_without_touching_the_gpu():
    lib = k3.lib()
    dims = k3.Dims(4, 16, 2, 256, 128)
    fake = ctypes.c_void_p(0x10000)
    mx = k3.MX(0x10000, 0x10000)
    ex = k3.Experts(mx, mx, mx)
    base = [fake, ctypes.byref(ex)] + [fake] * 6 + [0, fake, None, fake, 1 << 34, None]
    a = list(base)
    a[8] = 5  # unknown activation mode
    assert lib.k3moe_ffn(ctypes.byref(dims), *a) == k3.K3MOE_ENOTSUP
    bad = k3.Experts(k3.MX(0x10008, 0x10000), mx, mx)  # codes not 16-byte aligned
    a = list(base)
    a[1] = ctypes.byref(bad)
    assert lib.k3moe_ffn(ctypes.byref(dims), *a) == k3.K3MOE_EINVAL
    nul = k3.Experts(k3.MX(0x10000, None), mx, mx)
    a = list(base)
    a[1] = ctypes.byref(nul)
    assert lib.k3moe_ffn(ctypes.byref(dims), *a) == k3.K3MOE_EINVAL
    a = list(base)
    a[9] = None  # y
    assert lib.k3moe_ffn(ctypes.byref(dims), *a) == k3.K3MOE_EINVAL


def test_binding_refuses_wrong_tensors():
    import torch
    x = torch.zeros((2, 256), dtype=torch.float64)
    with pytest.raises(ValueError):
        k3._need(x, torch.float32, (2, 256), "x")


def test_noalloc_scratch_limit_matches_header():
    src = open(HEADER).read()
    m = re.search(r"#define K3MOE_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", src)
    assert m and int(m.group(1)) << int(m.group(2)) == k3.NOALLOC_SCRATCH_BYTES


def test_noalloc_refuses_dimensions_beyond_its_scratch_without_touching_the_gpu():
    lib = k3.lib()
    fake = ctypes.c_void_p(0x10000)
    mx = k3.MX(0x10000, 0x10000)
    ex = k3.Experts(mx, mx, mx)
    # x, w_router, bias, bias_mode, score_fn, experts, act, 6 routing outputs, y, dbg, stream
    args = [fake, fake, None, 0, 0, ctypes.byref(ex), 0] + [fake] * 6 + [fake, None, None]
    for T, act in ((4096, 0), (4096, 1), (200, 0)):
        dims = k3.Dims(T, 896, 16, 7168, 2048)
        a = list(args)
        a[6] = act
        assert _ws(T, 896, 16, 7168, 2048, act)[1] > k3.NOALLOC_SCRATCH_BYTES
        assert lib.k3moe_forward_noalloc(ctypes.byref(dims), *a) == k3.K3MOE_EWORKSPACE
    # the usual argument checks come first, as in k3moe_forward
    dims = k3.Dims(1, 896, 16, 7168, 2048)
    a = list(args)
    a[0] = None
    assert lib.k3moe_forward_noalloc(ctypes.byref(dims), *a) == k3.K3MOE_EINVAL
    a = list(args)
    a[6] = 9
    assert lib.k3moe_forward_noalloc(ctypes.byref(dims), *a) == k3.K3MOE_ENOTSUP
    z = k3.Dims(0, 896, 16, 7168, 2048)
    assert lib.k3moe_forward_noalloc(ctypes.byref(z), *([None] * 3 + [0, 0, None, 0] + [None] * 9)) == 0
    # single-token decode fits
    assert _ws(1, 896, 16, 7168, 2048, 0)[1] <= k3.NOALLOC_SCRATCH_BYTES


def test_cache_state_size_and_dimension_checks():
    lib = k3.lib()
    n = ctypes.c_size_t(0)
    assert lib.k3moe_cache_state_bytes(896, 256, ctypes.byref(n)) == k3.K3MOE_OK
    # header + slot_of[E] + five int32 arrays of n_slots, each 256-aligned
    up = lambda b: (b + 255) // 256 * 256
    assert n.value == up(32) + up(896 * 4) + 5 * up(256 * 4)
    assert k3.k3moe_cache_state_bytes(16, 4) == up(32) + up(64) + 5 * up(16)
    for E, S, rc in ((896, 0, k3.K3MOE_EINVAL), (16, 17, k3.K3MOE_EINVAL), (2048, 64, k3.K3MOE_ENOTSUP),
                     (0, 1, k3.K3MOE_EINVAL)):
        assert lib.k3moe_cache_state_bytes(E, S, ctypes.byref(n)) == rc
    assert lib.k3moe_cache_state_bytes(16, 4, None) == k3.K3MOE_EINVAL
    assert lib.k3moe_cache_reset(None, 16, 4, None) == k3.K3MOE_EINVAL
    assert lib.k3moe_cache_reset(ctypes.c_void_p(0x10010), 16, 4, None) == k3.K3MOE_EINVAL  # not 256-aligned


def test_forward_cached_rejects_bad_arguments_without_touching_the_gpu():
    lib = k3.lib()
    fake = ctypes.c_void_p(0x10000)
    mx = k3.MX(0x10000, 0x10000)
    ex = k3.Experts(mx, mx, mx)
    state = ctypes.c_void_p(0x20000)
    # x, w_router, bias, bias_mode, score_fn, host, slots, n_slots, state, act, 6 routing outputs, y, ws, ws_bytes, stream
    T, E, k = 1, 896, 16
    ws = _ws(T, E, k, 7168, 2048, 0)[1]

    def call(dims, **kw):
        a = dict(x=fake, wr=fake, bias=None, bm=0, sf=0, host=ctypes.byref(ex), slots=ctypes.byref(ex), ns=32,
                 state=state, act=0, ws=ctypes.c_void_p(0x40000), wsn=ws)
        a.update(kw)
        return lib.k3moe_forward_cached(ctypes.byref(dims), a["x"], a["wr"], a["bias"], a["bm"], a["sf"], a["host"],
                                        a["slots"], a["ns"], a["state"], a["act"], *([fake] * 6), fake, a["ws"],
                                        a["wsn"], None)

    d1 = k3.Dims(T, E, k, 7168, 2048)
    assert call(d1, ns=15) == k3.K3MOE_EINVAL          # a step's 16 experts do not fit 15 slots
    assert call(d1, ns=E + 1) == k3.K3MOE_EINVAL
    assert call(d1, state=None) == k3.K3MOE_EINVAL
    assert call(d1, state=ctypes.c_void_p(0x20010)) == k3.K3MOE_EINVAL
    assert call(d1, host=None) == k3.K3MOE_EINVAL
    bad = k3.Experts(k3.MX(0x10000, 0x10004), mx, mx)  # scales not 16-byte aligned
    assert call(d1, slots=ctypes.byref(bad)) == k3.K3MOE_EINVAL
    assert call(d1, act=9) == k3.K3MOE_ENOTSUP
    assert call(d1, wsn=ws - 1) == k3.K3MOE_EWORKSPACE
    assert call(k3.Dims(3, E, k, 7168, 2048)) == k3.K3MOE_EINVAL  # 48 pairs > 32 slots
    assert call(k3.Dims(2, E, k, 7168, 2048)) == k3.K3MOE_EWORKSPACE  # 32 pairs fit; the workspace is for T = 1
    z = k3.Dims(0, E, k, 7168, 2048)
    assert call(z) == k3.K3MOE_OK


def test_stage_marks_constants_match_header():
    src = open(HEADER).read()
    m = re.search(r"#define K3MOE_MAX_MARKS (\d+)", src)
    assert m and int(m.group(1)) == k3.MAX_MARKS
    kinds = {int(v): n.lower() for n, v in re.findall(r"#define K3MOE_KERNEL_([A-Z_]+)\s+(\d+)", src)}
    assert kinds == k3.KERNEL_KINDS


def test_stage_marks_validation_without_touching_the_gpu():
    lib = k3.lib()
    P = ctypes.c_void_p
    ev = (P * 4)(P(0x1000), P(0x2000), P(0x3000), P(0x4000))  # never used: only checked for NULL here
    assert lib.k3moe_set_stage_marks(ev, -1, None, None) == k3.K3MOE_EINVAL
    assert lib.k3moe_set_stage_marks(ev, k3.MAX_MARKS + 1, None, None) == k3.K3MOE_EINVAL
    assert lib.k3moe_set_stage_marks(None, 1, None, None) == k3.K3MOE_EINVAL
    # two events per kernel: the end event of kernel 1 missing
    assert lib.k3moe_set_stage_marks((P * 4)(P(0x1000), P(0x2000), P(0x3000), None), 2, None, None) == k3.K3MOE_EINVAL
    # switching marks off always succeeds (and leaves none set for later calls)
    assert lib.k3moe_set_stage_marks(None, 0, None, None) == k3.K3MOE_OK
