"""k3moe_forward_noalloc (the library's fixed per-device scratch instead of a
workspace) against k3moe_forward on the same inputs: two calls in a row, the
second with fewer tokens, so the second runs on scratch the first left behind.
Routing bit-exact, y within the parity tolerance, every output poisoned
before each call."""
import numpy as np
import pytest
import torch

import synthdata
from helpers import assert_y_close

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import mxfp4_routed_expert_softmax_amd as k3  # noqa: E402

DEV = torch.device("cuda:0")


def _poisoned(T, E, k, d):
    y = torch.full((T, d), float("nan"), dtype=torch.float32, device=DEV)
    route = k3.alloc_route(T, E, k, DEV)
    for t in route.values():
        t.fill_(-7)
    return y, route


def _compare(x, wr, experts, k, act, bias=None, bias_mode="none"):
    T, d = x.shape
    E = wr.shape[0]
    print(f"noalloc vs forward: T={T} E={E} k={k} d={d} act={act}", flush=True)
    y_ref, r_ref = k3.k3moe_forward(x, wr, experts, k, bias, bias_mode, act)
    out = _poisoned(T, E, k, d)
    y, r = k3.k3moe_forward_noalloc(x, wr, experts, k, bias, bias_mode, act, out=out)
    torch.cuda.synchronize()
    for name in r_ref:
        assert torch.equal(r[name], r_ref[name]), f"{name} differs"
    yn = y.cpu().numpy()
    assert np.isfinite(yn).all()
    assert_y_close(yn, y_ref.cpu().numpy())


def _dev_experts(sh):
    host = synthdata.all_experts_host(sh)
    return {w: (torch.from_numpy(host[w][0]).to(DEV), torch.from_numpy(host[w][1]).to(DEV)) for w in host}


@pytest.mark.parametrize("act", ["fp32", "mxfp4"])
def test_noalloc_small_layers(act):
    for sh, Ts in ((synthdata.TINY, (70, 5)), (synthdata.SMALL_F1536, (90, 2))):
        ex = _dev_experts(sh)
        wr = torch.from_numpy(synthdata.router_weight(sh)).to(DEV)
        for T in Ts:
            x = torch.from_numpy(synthdata.tokens(sh, T, first=300 + T)).to(DEV)
            _compare(x, wr, ex, sh.k, act)


def test_noalloc_full_layer():
    sh = synthdata.K3
    ex = synthdata.upload_experts(sh, DEV)
    wr = torch.from_numpy(synthdata.router_weight(sh)).to(DEV)
    bias = torch.from_numpy(synthdata.zipf_bias(sh)).to(DEV)
    for T, act, bm in ((64, "fp32", "none"), (1, "fp32", "none"), (80, "mxfp4", "logits"), (3, "mxfp4", "logits")):
        x = torch.from_numpy(synthdata.tokens(sh, T, first=900 + T)).to(DEV)
        _compare(x, wr, ex, sh.k, act, bias if bm != "none" else None, bm)
    # beyond the scratch: refused, outputs untouched
    T = 4096
    x = torch.zeros((T, sh.d), dtype=torch.float32, device=DEV)
    with pytest.raises(k3.K3MoEError) as ei:
        k3.k3moe_forward_noalloc(x, wr, ex, sh.k, act_mode="mxfp4")
    assert ei.value.status == k3.K3MOE_EWORKSPACE
