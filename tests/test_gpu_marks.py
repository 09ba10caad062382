"""Kernel timing marks of the expert-FFN stage (k3moe_set_stage_marks) on the
GPU: the marks name the kernels each path launches, in order, each kernel's
start and end events bracket a positive duration and follow launch order, and
marking changes no output bit."""
import numpy as np
import pytest
import torch

import synthdata

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import mxfp4_routed_expert_softmax_amd as k3  # noqa: E402

DEV = torch.device("cuda:0")


@pytest.fixture(scope="module")
def tiny():
    sh = synthdata.TINY
    host = synthdata.all_experts_host(sh)
    dev = {w: (torch.from_numpy(host[w][0]).to(DEV), torch.from_numpy(host[w][1]).to(DEV)) for w in host}
    return sh, dev, torch.from_numpy(synthdata.router_weight(sh)).to(DEV)


# T, activation mode -> the kernels the stage launches, in order
CASES = [
    (1, "fp32", ["gateup", "down_combine"]),
    (130, "fp32", ["active_list", "gateup", "down", "combine"]),
    (1, "mxfp4", ["quantize", "gateup", "down", "combine"]),
    (65, "mxfp4", ["active_list", "quantize", "gateup", "down", "combine"]),
]


@pytest.mark.parametrize("T,act,kinds", CASES)
def test_marks_name_the_stage_kernels(tiny, T, act, kinds):
    sh, dev, wr = tiny
    print(f"marks T={T} act={act}", flush=True)
    x = torch.from_numpy(synthdata.tokens(sh, T)).to(DEV)
    fw = k3.Forward(x, wr, dev, sh.k, act_mode=act)
    fw.run_route()
    fw.run_ffn()
    torch.cuda.synchronize()
    y0 = fw.y.clone()
    stream = torch.cuda.current_stream()
    marks = k3.StageMarks(k3.MAX_MARKS, stream)
    marks.set()
    try:
        fw.y.fill_(float("nan"))
        fw.run_ffn()
    finally:
        k3.StageMarks.clear()
    torch.cuda.synchronize()
    assert marks.launched == len(kinds)
    assert marks.kinds() == kinds
    assert torch.equal(fw.y, y0), "marking changed the output"
    # every kernel's own duration is positive; each starts after the previous ended
    ev = marks.events
    dur = [marks.kernel_ms(i) for i in range(len(kinds))]
    gaps = [ev[2 * i - 1].elapsed_time(ev[2 * i]) for i in range(1, len(kinds))]
    assert all(v > 0.0 for v in dur), dur
    assert all(g >= 0.0 for g in gaps), gaps
    # cleared: a later call records nothing and leaves the counts alone
    fw.run_ffn()
    torch.cuda.synchronize()
    assert marks.launched == len(kinds)


def test_fewer_marks_than_kernels(tiny):
    sh, dev, wr = tiny
    x = torch.from_numpy(synthdata.tokens(sh, 65)).to(DEV)
    fw = k3.Forward(x, wr, dev, sh.k, act_mode="mxfp4")
    marks = k3.StageMarks(2, torch.cuda.current_stream())
    marks.set()
    try:
        fw()
    finally:
        k3.StageMarks.clear()
    torch.cuda.synchronize()
    assert marks.launched == 5
    assert marks.kinds() == ["active_list", "quantize"]
    assert np.isfinite(fw.y.cpu().numpy()).all()
