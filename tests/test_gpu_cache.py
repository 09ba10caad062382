"""GPU tests of the HBM expert cache (k3moe_forward_cached), through the C ABI.

Per step: y and every routing output equal k3moe_forward's bit for bit (the
same kernels read the same bytes, from a slot instead of the expert's own
place), and the cache state after the step -- which expert sits in which
slot, hits and misses -- equals the oracle's step-batched LRU
(oracle/cache.py) replayed on the step's selection.  Routing is biased
toward a few experts so that the trace has both hits and evictions.  The
tiny layer runs both activation modes and two tokens per step; a layer of
64 full-size experts (d_model 7168, d_ff 2048, top-16) streams 23.4 MB per
missed expert over the host link."""
import numpy as np
import pytest
import torch

import synthdata
from oracle import cache as oc

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import mxfp4_routed_expert_softmax_amd as k3  # noqa: E402

DEV = torch.device("cuda:0")


def _log(msg):
    print(msg, flush=True)


def _pinned_copy(dev_experts):
    out = {}
    for w, (c, s) in dev_experts.items():
        hc = torch.empty(c.shape, dtype=torch.uint8, pin_memory=True)
        hs = torch.empty(s.shape, dtype=torch.uint8, pin_memory=True)
        hc.copy_(c)
        hs.copy_(s)
        out[w] = (hc, hs)
    return out


def _run_trace(sh, dev_experts, host_experts, wr_dev, n_slots, T, steps, act, bias):
    bias_dev = torch.from_numpy(bias).to(DEV)
    xs = [torch.from_numpy(synthdata.tokens(sh, T, first=7000 + T * i)).to(DEV) for i in range(steps)]
    ref = k3.Forward(xs[0], wr_dev, dev_experts, sh.k, bias_dev, "logits", act)
    cf = k3.CachedForward(xs[0], wr_dev, host_experts, n_slots, sh.k, bias_dev, "logits", act)
    trace = []
    for i in range(steps):
        ref.set_x(xs[i])
        cf.set_x(xs[i])
        ref.y.fill_(float("nan"))
        cf.y.fill_(float("nan"))
        for t in cf.route.values():
            t.fill_(-7)
        ref()
        cf()
        torch.cuda.synchronize()
        for name in ref.route:
            assert torch.equal(ref.route[name], cf.route[name]), f"step {i}: {name} differs"
        assert torch.equal(ref.y, cf.y), f"step {i}: y differs from k3moe_forward"
        assert torch.isfinite(cf.y).all()
        trace.append(cf.route["topk_idx"].cpu().numpy().ravel().tolist())
        want = oc.lru_replay(trace, n_slots)
        st = cf.read()
        slot_of = {e: s for e, s in enumerate(st["slot_of"]) if s >= 0}
        assert slot_of == want[-1]["slot_of"], f"step {i}: slot map differs from the oracle's LRU"
        assert st["expert_in"] == want[-1]["expert_in"], f"step {i}: slot contents differ"
        assert st["steps"] == i + 1
        assert st["hits"] == sum(w["hits"] for w in want) and st["misses"] == sum(w["misses"] for w in want)
        assert st["last_misses"] == want[-1]["misses"]
    return st


@pytest.mark.parametrize("act,T", [("fp32", 1), ("fp32", 2), ("mxfp4", 1), ("mxfp4", 2)])
def test_cache_tiny_matches_forward_and_lru(act, T):
    sh = synthdata.TINY
    _log(f"cache tiny {act} T={T}")
    host = synthdata.all_experts_host(sh)
    dev = {w: (torch.from_numpy(host[w][0]).to(DEV), torch.from_numpy(host[w][1]).to(DEV)) for w in host}
    wr_dev = torch.from_numpy(synthdata.router_weight(sh)).to(DEV)
    bias = synthdata.zipf_bias(sh)
    st = _run_trace(sh, dev, _pinned_copy(dev), wr_dev, 4, T, 40, act, bias)
    assert st["hits"] > 0 and st["misses"] > 4  # the trace both reuses and evicts


def test_cache_full_size_experts():
    sh = synthdata.CACHE_E64
    _log("cache: 64 full-size experts, upload ...")
    dev = synthdata.upload_experts(sh, DEV)
    host = _pinned_copy(dev)
    torch.cuda.synchronize()
    wr_dev = torch.from_numpy(synthdata.router_weight(sh)).to(DEV)
    bias = synthdata.zipf_bias(sh)
    _log("cache: 64 full-size experts, 12 steps")
    st = _run_trace(sh, dev, host, wr_dev, 24, 1, 12, "fp32", bias)
    assert st["hits"] > 0 and st["misses"] > 24


def test_cache_reset_empties_and_refuses_oversized_steps():
    sh = synthdata.TINY
    host = synthdata.all_experts_host(sh)
    dev = {w: (torch.from_numpy(host[w][0]).to(DEV), torch.from_numpy(host[w][1]).to(DEV)) for w in host}
    pinned = _pinned_copy(dev)
    wr_dev = torch.from_numpy(synthdata.router_weight(sh)).to(DEV)
    x = torch.from_numpy(synthdata.tokens(sh, 1)).to(DEV)
    cf = k3.CachedForward(x, wr_dev, pinned, 2, sh.k)
    cf()
    st = cf.read()
    assert st["steps"] == 1 and st["misses"] == 2 and sorted(e for e in st["expert_in"]) == sorted(
        cf.route["topk_idx"].cpu().numpy().ravel().tolist())
    cf.reset()
    st = cf.read()
    assert st["steps"] == 0 and st["expert_in"] == [-1, -1] and all(s == -1 for s in st["slot_of"])
    x3 = torch.from_numpy(synthdata.tokens(sh, 3)).to(DEV)
    with pytest.raises(k3.K3MoEError):
        k3.CachedForward(x3, wr_dev, pinned, 4, sh.k)()  # 3 tokens x top-2 = 6 pairs > 4 slots


def test_cache_step_replays_in_a_hip_graph():
    """k3moe_forward_cached enqueues everything in stream order with no host
    synchronisation, so a step can be captured and replayed: after the first
    replay every expert of the (fixed) token is resident, later replays are
    all hits and give the same y as the eager step."""
    sh = synthdata.TINY
    host = synthdata.all_experts_host(sh)
    dev = {w: (torch.from_numpy(host[w][0]).to(DEV), torch.from_numpy(host[w][1]).to(DEV)) for w in host}
    pinned = _pinned_copy(dev)
    wr_dev = torch.from_numpy(synthdata.router_weight(sh)).to(DEV)
    x = torch.from_numpy(synthdata.tokens(sh, 1, first=321)).to(DEV)
    eager = k3.Forward(x, wr_dev, dev, sh.k)
    eager()
    torch.cuda.synchronize()
    y_ref = eager.y.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    cf = k3.CachedForward(x, wr_dev, pinned, 4, sh.k, stream=s)
    with torch.cuda.stream(s):
        cf()  # warm-up call outside the capture
    torch.cuda.synchronize()
    cf.reset()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        cf()
    torch.cuda.synchronize()
    cf.reset()
    torch.cuda.synchronize()
    for rep in range(4):
        cf.y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(cf.y, y_ref), f"replay {rep}: y differs from the eager k3moe_forward"
        st = cf.read()
        assert st["steps"] == rep + 1
        assert st["misses"] == sh.k and st["hits"] == sh.k * rep  # misses on the first replay only
