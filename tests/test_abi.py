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
