"""Pins of the oracle's router: fp64 logits, top-k selection with lower-index
ties, renormalised softmax weights, bias modes, expert grouping."""
import numpy as np
import pytest
from scipy.special import softmax

import oracle
import synthdata


def _brute_topk(key, k):
    """Full stable sort by (key descending, expert ascending) -- numpy lexsort."""
    T, E = key.shape
    out = np.empty((T, k), np.int32)
    for t in range(T):
        order = np.lexsort((np.arange(E), -key[t]))
        out[t] = order[:k]
    return out


def test_logits_vs_dense_matmul():
    r = np.random.default_rng(1)
    x = r.standard_normal((5, 192)).astype(np.float32)
    wr = (r.standard_normal((37, 192)) / 14).astype(np.float32)
    got = oracle.router_logits(x, wr)
    ref = x.astype(np.float64) @ wr.astype(np.float64).T
    assert np.allclose(got, ref, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("k", [1, 2, 5, 16, 37])
def test_topk_vs_lexsort_random(k):
    r = np.random.default_rng(k)
    key = r.standard_normal((9, 37))
    assert np.array_equal(oracle.select_topk(key, k), _brute_topk(key, k))


def test_topk_adversarial_ties():
    E, k = 40, 7
    key = np.zeros((1, E))                       # all equal -> experts 0..k-1
    assert np.array_equal(oracle.select_topk(key, k)[0], np.arange(k))
    r = np.random.default_rng(3)
    key = np.round(r.standard_normal((6, E)), 1)  # many exact ties
    assert np.array_equal(oracle.select_topk(key, k), _brute_topk(key, k))
    # duplicated router rows give exactly equal logits -> lower index first
    x = r.standard_normal((3, 64)).astype(np.float32)
    wr = r.standard_normal((E, 64)).astype(np.float32)
    wr[11] = wr[29]
    lg = oracle.router_logits(x, wr)
    assert np.array_equal(lg[:, 11], lg[:, 29])
    assert np.array_equal(oracle.select_topk(lg, E), _brute_topk(lg, E))


def test_weights_closed_forms():
    r = np.random.default_rng(4)
    lg = r.standard_normal((4, 24)) * 3
    # k = E: the renormalised weights are the full softmax
    idx = oracle.select_topk(lg, 24)
    w = oracle.topk_weights(lg, idx)
    ref = np.take_along_axis(softmax(lg, axis=1), idx.astype(np.int64), axis=1)
    assert np.allclose(w, ref, rtol=1e-14, atol=0)
    # k = 1: weight exactly one
    idx1 = oracle.select_topk(lg, 1)
    assert np.all(oracle.topk_weights(lg, idx1) == 1.0)
    # equal logits: 1/k each
    eq = np.full((1, 24), 0.7)
    w = oracle.topk_weights(eq, oracle.select_topk(eq, 8))
    assert np.allclose(w, 1 / 8, rtol=1e-15)
    # general k: equals softmax over the selected logits only, sums to one
    idx5 = oracle.select_topk(lg, 5)
    w5 = oracle.topk_weights(lg, idx5)
    sel = np.take_along_axis(lg, idx5.astype(np.int64), axis=1)
    assert np.allclose(w5, softmax(sel, axis=1), rtol=1e-14)
    assert np.allclose(w5.sum(1), 1.0, rtol=0, atol=2e-15)
    # descending order of weights follows descending logits
    assert np.all(np.diff(w5, axis=1) <= 0)


def test_bias_modes():
    r = np.random.default_rng(6)
    x = r.standard_normal((8, 64)).astype(np.float32)
    wr = (r.standard_normal((30, 64)) / 8).astype(np.float32)
    b = (r.standard_normal(30) * 2).astype(np.float32)
    lg = oracle.router_logits(x, wr)
    a = oracle.route(x, wr, 4, b, oracle.BIAS_LOGITS)
    assert np.array_equal(a["topk_idx"], _brute_topk(lg + b.astype(np.float64), 4))
    s = oracle.route(x, wr, 4, b, oracle.BIAS_SELECT_ONLY)
    assert np.array_equal(s["topk_idx"], a["topk_idx"])  # same selection key
    # selection-only: weights come from the unbiased logits of the chosen experts
    sel = np.take_along_axis(lg, s["topk_idx"].astype(np.int64), axis=1)
    assert np.allclose(s["topk_w"], softmax(sel, axis=1), rtol=1e-14)
    # ... and so do not move when the bias changes but the selection does not
    s2 = oracle.route(x, wr, 4, b + np.float32(0.0), oracle.BIAS_SELECT_ONLY)
    assert np.array_equal(s2["topk_w"], s["topk_w"])
    # a huge bias on one expert forces it in everywhere
    bb = np.zeros(30, np.float32)
    bb[17] = 1e6
    f = oracle.route(x, wr, 4, bb, oracle.BIAS_SELECT_ONLY)
    assert np.all(f["topk_idx"][:, 0] == 17)
    n = oracle.route(x, wr, 4)
    assert np.array_equal(n["topk_idx"], _brute_topk(lg, 4))


def _check_perm(idx, E, p):
    T, k = idx.shape
    counts, offsets, perm, inv = p["counts"], p["offsets"], p["perm_pair"], p["row_of_pair"]
    assert counts.sum() == T * k
    assert offsets[0] == 0 and offsets[-1] == T * k and np.all(np.diff(offsets) == counts)
    assert np.array_equal(np.sort(perm), np.arange(T * k))       # each pair exactly once
    assert np.array_equal(inv[perm], np.arange(T * k))           # inverse map
    # brute force: rows sorted by (expert, token)
    pairs = np.arange(T * k)
    e_of = idx.reshape(-1)
    t_of = pairs // k
    order = np.lexsort((t_of, e_of))
    assert np.array_equal(perm, order.astype(np.int32))
    for e in range(E):
        assert np.array_equal(np.bincount(e_of, minlength=E)[e], counts[e])


@pytest.mark.parametrize("T,E,k", [(1, 16, 2), (7, 16, 16), (64, 896, 16), (33, 40, 3)])
def test_permutation_invariants(T, E, k):
    r = np.random.default_rng(T * 1000 + E)
    idx = np.stack([r.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    _check_perm(idx, E, oracle.permute(idx, E))


def test_permutation_rejects_bad_indices():
    with pytest.raises(ValueError):
        oracle.permute(np.array([[1, 1]], np.int32), 4)
    with pytest.raises(ValueError):
        oracle.permute(np.array([[0, 4]], np.int32), 4)


def test_route_tiny_workload_end_to_end():
    sh = synthdata.TINY
    x = synthdata.tokens(sh, 3)
    wr = synthdata.router_weight(sh)
    r = oracle.route(x, wr, sh.k)
    _check_perm(r["topk_idx"], sh.E, r)
    assert np.allclose(r["topk_w"].sum(1), 1.0, atol=2e-15)


# ------------------------------------------------------------ sigmoid router ---
# The pages' router (fiv.co.kr deep dive, invariant #5 and the MoE-routing
# study-plan row): sigmoid scores, the bias added to the score for selection
# only, weights from the bias-free scores (renormalised here: the reading
# taken).  Pinned against scipy's expit and brute-force sorts.

def test_sigmoid_vs_scipy_expit():
    from scipy.special import expit
    r = np.random.default_rng(11)
    lg = np.concatenate([r.standard_normal(2000) * 4, [0.0, 1e-300, -1e-300, 36.0, -36.0, 709.0, -745.0,
                                                       800.0, -800.0]])[None, :]
    s = oracle.sigmoid(lg)
    assert np.all(np.isfinite(s)) and np.all(s >= 0) and np.all(s <= 1)
    assert np.allclose(s, expit(lg), rtol=2e-16 * 4, atol=1e-300)
    assert s[0, 2000] == 0.5                                   # sigma(0) exactly
    assert np.allclose(s + oracle.sigmoid(-lg), 1.0, rtol=0, atol=2.3e-16)  # symmetry


def test_sigmoid_selection_and_weights():
    from scipy.special import expit
    r = np.random.default_rng(12)
    x = r.standard_normal((6, 64)).astype(np.float32)
    wr = (r.standard_normal((40, 64)) / 8).astype(np.float32)
    lg = oracle.router_logits(x, wr)
    s = oracle.route(x, wr, 5, score_fn=oracle.SCORE_SIGMOID)
    # sigmoid is increasing: without a bias the choice is the logits' choice
    assert np.array_equal(s["topk_idx"], _brute_topk(lg, 5))
    sel = np.take_along_axis(expit(lg), s["topk_idx"].astype(np.int64), axis=1)
    assert np.allclose(s["topk_w"], sel / sel.sum(1, keepdims=True), rtol=1e-14)
    assert np.allclose(s["topk_w"].sum(1), 1.0, rtol=0, atol=2e-15)
    # the weights differ from the softmax ones (a dropped score function fails here)
    m = oracle.route(x, wr, 5)
    assert np.array_equal(m["topk_idx"], s["topk_idx"]) and not np.allclose(m["topk_w"], s["topk_w"])


def test_sigmoid_bias_steers_selection_only():
    from scipy.special import expit
    r = np.random.default_rng(13)
    x = r.standard_normal((8, 64)).astype(np.float32)
    wr = (r.standard_normal((30, 64)) / 8).astype(np.float32)
    b = (r.standard_normal(30) * 0.3).astype(np.float32)
    lg = oracle.router_logits(x, wr)
    s = oracle.route(x, wr, 4, b, oracle.BIAS_SELECT_ONLY, oracle.SCORE_SIGMOID)
    assert np.array_equal(s["topk_idx"], _brute_topk(expit(lg) + b.astype(np.float64), 4))
    sel = np.take_along_axis(expit(lg), s["topk_idx"].astype(np.int64), axis=1)
    assert np.allclose(s["topk_w"], sel / sel.sum(1, keepdims=True), rtol=1e-14)


def test_sigmoid_bias_is_added_to_the_score_not_the_logit():
    # two experts: logits 10 and 0, bias 0.6 on the second.  On the score
    # sigma(10) = 0.99995 < sigma(0) + 0.6 = 1.1, so the second wins; on the
    # logit (the softmax router's selection-only bias) 10 > 0.6 keeps the first.
    x = np.array([[1.0]], np.float32)
    wr = np.array([[10.0], [0.0]], np.float32)
    b = np.array([0.0, 0.6], np.float32)
    s = oracle.route(x, wr, 1, b, oracle.BIAS_SELECT_ONLY, oracle.SCORE_SIGMOID)
    m = oracle.route(x, wr, 1, b, oracle.BIAS_SELECT_ONLY, oracle.SCORE_SOFTMAX)
    assert s["topk_idx"][0, 0] == 1 and m["topk_idx"][0, 0] == 0
    assert s["topk_w"][0, 0] == 1.0


def test_sigmoid_all_ties():
    x = np.zeros((2, 16), np.float32)
    wr = np.ones((12, 16), np.float32)
    s = oracle.route(x, wr, 5, score_fn=oracle.SCORE_SIGMOID)
    assert np.array_equal(s["topk_idx"], np.tile(np.arange(5, dtype=np.int32), (2, 1)))
    assert np.all(s["topk_w"] == 0.2)
