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


class SeqExpertGetter:
    """Expert weights regenerated from their seeds in a thread pool and handed
    out in ascending id order, as oracle.layer_forward asks for them (each
    expert generated once, a bounded number held at a time)."""

    def __init__(self, shape, ids, threads: int = 16, ahead: int = 48):
        from collections import deque
        from concurrent.futures import ThreadPoolExecutor
        self.ids = sorted(int(e) for e in ids)
        self.shape = shape
        self.pool = ThreadPoolExecutor(threads)
        self.q = deque()
        self.next = 0
        self.ahead = ahead
        self._fill()

    def _fill(self):
        while self.next < len(self.ids) and len(self.q) < self.ahead:
            e = self.ids[self.next]
            self.q.append((e, self.pool.submit(synthdata.expert, self.shape, e)))
            self.next += 1

    def __call__(self, e):
        e0, fut = self.q.popleft()
        assert e0 == int(e), f"expert {e} asked out of order (next is {e0})"
        out = fut.result()
        self._fill()
        if not self.q:
            self.pool.shutdown()
        return out


def oracle_y_major(x, route, tokens, shape, act_mode="fp32", h_override=None, keep=None, get=None):
    """Oracle y rows of the given tokens, expert-major (oracle.layer_forward),
    with the experts regenerated from their seeds unless ``get`` is given."""
    tokens = [int(t) for t in tokens]
    if get is None:
        ids = {int(e) for t in tokens for e in route["topk_idx"][t]}
        get = SeqExpertGetter(shape, ids)
    return oracle.layer_forward(x, route, tokens, get, act_mode=act_mode, h_override=h_override, keep=keep)


def covering_tokens(route, n_min: int, seed: int, n_heavy: int = 16, pass_rows=(96,)):
    """Token ids chosen so that the rows checked cover the grouped layout:
    every active expert has at least one checked pair; the n_heavy experts
    with the most tokens (lower id first on ties) have their last row checked,
    and their row r for each r in pass_rows below their count; then seeded
    random tokens up to n_min.  Rows of an expert are its tokens in ascending
    order."""
    idx = route["topk_idx"]
    T = idx.shape[0]
    counts, offsets, perm = route["counts"], route["offsets"], route["perm_pair"]
    k = idx.shape[1]
    chosen = set()

    def tok_at(e, r):
        return int(perm[offsets[e] + r]) // k

    heavy = sorted(np.nonzero(counts)[0], key=lambda e: (-int(counts[e]), int(e)))[:n_heavy]
    for e in heavy:
        n = int(counts[e])
        chosen.add(tok_at(e, n - 1))
        for r in pass_rows:
            if n > r:
                chosen.add(tok_at(e, r))
    covered = {int(e) for t in chosen for e in idx[t]}
    active = {int(e) for e in np.nonzero(counts)[0]}
    # greedy cover of the rest: the token with the most uncovered experts, lowest id on ties
    while covered != active:
        gain = np.array([len(set(map(int, idx[t])) - covered) for t in range(T)])
        t = int(np.argmax(gain))
        chosen.add(t)
        covered |= set(map(int, idx[t]))
    rng = np.random.default_rng(seed)
    rest = [t for t in rng.permutation(T) if t not in chosen]
    for t in rest[:max(0, n_min - len(chosen))]:
        chosen.add(int(t))
    return sorted(chosen)
