"""Host logic of bench.py (no GPU): the per-kernel algorithmic byte counts
and the per-kernel times taken from the stage's mark events."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import synthdata  # noqa: E402


def test_kernel_bytes_of_the_decode_step():
    sh = synthdata.WORKLOADS["k3_decode_t1"].shape
    kb = bench.kernel_bytes(sh, 1, 16, "fp32")
    # per token, 16 experts: gate + up 249,561,088 B, down 124,780,544 B (the
    # MXFP4 size rule: n/2 code bytes + n/32 scale bytes for n weights)
    assert kb["gateup"] == 249_561_088 + 7168 * 4
    assert kb["down_combine"] == 124_780_544 + 7168 * 4
    assert kb["active_list"] is None


def test_kernel_bytes_of_the_mx_prefill():
    sh = synthdata.WORKLOADS["k3_prefill_t4096"].shape
    T, P, d, f = 4096, 4096 * 16, 7168, 2048
    kb = bench.kernel_bytes(sh, T, 896, "mxfp4")
    xq, hq = T * (d // 2 + d // 32), P * (f // 2 + f // 32)
    assert kb["quantize"] == T * d * 4 + xq
    assert kb["gateup"] == 896 * 2 * f * (d // 2 + d // 32) + xq + hq
    assert kb["down"] == 896 * d * (f // 2 + f // 32) + hq + P * d * 4
    assert kb["combine"] == P * d * 4 + T * d * 4


class _Marks:
    def __init__(self, times, kinds):
        self._t = times
        self._k = kinds

    def kinds(self):
        return self._k

    def kernel_ms(self, i):
        return self._t[i]


def test_kernel_times_average_each_kind_over_steps():
    mks = [_Marks([0.040, 0.025], ["gateup", "down_combine"]),
           _Marks([0.050, 0.025], ["gateup", "down_combine"])]
    kt = bench.kernel_times(mks)
    assert abs(kt["gateup"]["avg_ms"] - 0.045) < 1e-12
    assert abs(kt["down_combine"]["avg_ms"] - 0.025) < 1e-12
    assert kt["gateup"]["samples"] == 2


def test_kernels_of_one_kind_in_a_step_add_up():
    # the small-batch gate/up runs as two kernels (one-token experts, then the rest)
    mks = [_Marks([0.8, 1.2, 1.1, 0.01], ["gateup", "gateup", "down", "combine"])]
    kt = bench.kernel_times(mks)
    assert abs(kt["gateup"]["avg_ms"] - 2.0) < 1e-12 and kt["gateup"]["samples"] == 1
