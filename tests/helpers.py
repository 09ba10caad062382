"""Shared helpers of the GPU parity tests: device inputs from the seeded
generators, oracle references, and the comparison rules.

Parity bar (fp32 activations): routing bit-exact (topk_idx, counts, offsets,
perm_pair, row_of_pair), topk_w within 1e-6 relative of the fp64 oracle, and
y with relative L2 error <= 1e-5 and max abs error <= 1e-4 * max|y_oracle|
over the compared rows.  MXFP4 activations: x_q and h_q bit-exact, h and y by
the same tolerance, y computed by the oracle from the device's own h (the
oracle quantises it independently), see the MX tests."""
from __future__ import annotations

import numpy as np

import oracle
import synthdata

RTOL_L2 = 1e-5
RTOL_MAX = 1e-4
RTOL_W = 1e-6


def assert_y_close(y_dev: np.ndarray, y_ref: np.ndarray, what: str = "y"):
    y_dev = np.asarray(y_dev, np.float64)
    y_ref = np.asarray(y_ref, np.float64)
    assert y_dev.shape == y_ref.shape, (y_dev.shape, y_ref.shape)
    diff = y_dev - y_ref
    ref_norm = np.linalg.norm(y_ref)
    ref_max = np.abs(y_ref).max()
    if ref_norm == 0.0:
        assert np.abs(diff).max() == 0.0, f"{what}: expected exact zeros"
        return
    rel_l2 = np.linalg.norm(diff) / ref_norm
    max_abs = np.abs(diff).max()
    assert rel_l2 <= RTOL_L2, f"{what}: relative L2 error {rel_l2:.3e} > {RTOL_L2}"
    assert max_abs <= RTOL_MAX * ref_max, f"{what}: max abs error {max_abs:.3e} > {RTOL_MAX} * {ref_max:.3e}"


def assert_route_equal(dev: dict, ref: dict):
    """dev: dict of torch tensors from the binding; ref: oracle.route()."""
    idx = dev["topk_idx"].cpu().numpy()
    assert np.array_equal(idx, ref["topk_idx"]), "topk_idx differs from the oracle"
    for name in ("counts", "offsets", "perm_pair", "row_of_pair"):
        assert np.array_equal(dev[name].cpu().numpy(), ref[name]), f"{name} differs from the oracle"
    w = dev["topk_w"].cpu().numpy().astype(np.float64)
    assert np.all(np.abs(w - ref["topk_w"]) <= RTOL_W * np.abs(ref["topk_w"]) + 1e-30), "topk_w"


def host_expert_getter(shape, host_experts=None, cache=None):
    """Expert e's MX matrices on the host: from a stacked host copy if given,
    else regenerated from its seeds (cached)."""
    cache = {} if cache is None else cache

    def get(e):
        e = int(e)
        if host_experts is not None:
            return {w: (host_experts[w][0][e], host_experts[w][1][e]) for w in host_experts}
        if e not in cache:
            cache[e] = synthdata.expert(shape, e)
        return cache[e]

    return get


def oracle_y(x: np.ndarray, route: dict, tokens, get, act_mode="fp32", h_override=None):
    """Oracle y rows for the given token ids (fp64)."""
    out = []
    for t in tokens:
        hov = None if h_override is None else h_override(t)
        out.append(oracle.token_forward(x[t], route["topk_idx"][t], route["topk_w"][t], get,
                                        act_mode=act_mode, h_override=hov))
    return np.stack(out)
