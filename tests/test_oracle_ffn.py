"""Pins of the oracle's expert FFN (SwiGLU on MXFP4 weights) and combine:
a dense fp64 matmul on explicitly dequantised weights, closed forms and
invariants."""
import numpy as np
import pytest
from scipy.special import expit

import oracle
import synthdata


def _bit_decode(codes, scales):
    """Dense fp64 matrix from MX codes/scales using only bit fields (sign bit 3,
    exponent bits 2..1, mantissa bit 0) -- independent of the oracle's table."""
    lo, hi = codes & 15, codes >> 4
    nib = np.stack([lo, hi], axis=-1).reshape(codes.shape[0], -1).astype(np.int64)
    s, e, m = (nib >> 3) & 1, (nib >> 1) & 3, nib & 1
    mag = np.where(e == 0, m / 2.0, 2.0 ** (e - 1) * (1.0 + m / 2.0))
    val = np.where(s == 1, -mag, mag)
    return val * np.repeat(2.0 ** (scales.astype(np.float64) - 127), 32, axis=1)


def _rand_expert(r, d, f, lo=120, hi=124):
    def mat(rows, cols):
        return (r.integers(0, 256, (rows, cols // 2), dtype=np.uint8),
                r.integers(lo, hi + 1, (rows, cols // 32), dtype=np.uint8))
    return {"gate": mat(f, d), "up": mat(f, d), "down": mat(d, f)}


def _dense_ffn(x, ex):
    Wg, Wu, Wd = (_bit_decode(*ex[w]) for w in ("gate", "up", "down"))
    g, u = Wg @ x, Wu @ x
    h = g * expit(g) * u
    return Wd @ h


@pytest.mark.parametrize("d,f", [(256, 128), (1024, 512), (512, 96)])
def test_ffn_vs_dense_matmul(d, f):
    r = np.random.default_rng(d + f)
    ex = _rand_expert(r, d, f)
    x = r.standard_normal(d)
    got = oracle.expert_ffn(x, ex)
    ref = _dense_ffn(x, ex)
    assert np.linalg.norm(got - ref) <= 1e-12 * np.linalg.norm(ref)


def test_gate_and_up_are_not_interchangeable():
    # silu(g)*u != silu(u)*g: the dense check above would catch a swap; make it explicit
    r = np.random.default_rng(2)
    ex = _rand_expert(r, 64, 32)
    x = r.standard_normal(64)
    h, g, u = oracle.gateup(x, ex["gate"], ex["up"], return_gu=True)
    assert np.allclose(h, g * expit(g) * u, rtol=1e-14)
    assert not np.allclose(h, u * expit(u) * g)


def test_silu_stable_and_correct():
    for z in (-800.0, -100.0, -20.0, -1.5, -0.0, 0.0, 1e-300, 0.3, 20.0, 100.0, 800.0):
        got = oracle.silu(z)
        ref = z * expit(z)
        assert np.isfinite(got)
        assert got == pytest.approx(ref, rel=1e-15, abs=1e-300)
    assert oracle.silu(100.0) == 100.0 * expit(100.0)


def test_closed_form_all_ones():
    d, f = 96, 64
    one = lambda rows, cols: (np.full((rows, cols // 2), 0x22, np.uint8), np.full((rows, cols // 32), 127, np.uint8))
    ex = {"gate": one(f, d), "up": one(f, d), "down": one(d, f)}
    x = np.random.default_rng(0).standard_normal(d)
    s = float(np.sum(x))
    h, g, u = oracle.gateup(x, ex["gate"], ex["up"], return_gu=True)
    assert np.allclose(g, s, rtol=1e-13) and np.allclose(u, s, rtol=1e-13)
    o = oracle.down(h, ex["down"])
    assert np.allclose(o, f * s * s * expit(s), rtol=1e-12)


def test_zero_code_block_contributes_nothing():
    r = np.random.default_rng(8)
    d, f = 128, 64
    ex = _rand_expert(r, d, f)
    x = r.standard_normal(d)
    base = None
    for fill in (0x00, 0x88):           # +0 and -0 codes
        for sc in (0, 1, 127, 200, 254):
            e2 = {k: (v[0].copy(), v[1].copy()) for k, v in ex.items()}
            e2["gate"][0][:, 16:32] = fill   # block 1 of every gate row
            e2["gate"][1][:, 1] = sc
            e2["down"][0][:, 0:16] = fill    # block 0 of every down row
            e2["down"][1][:, 0] = sc
            y = oracle.expert_ffn(x, e2)
            if base is None:
                base = y
            assert np.array_equal(y, base)


def test_zero_expert_contributes_nothing():
    r = np.random.default_rng(9)
    d, f = 64, 32
    exs = [_rand_expert(r, d, f) for _ in range(3)]
    exs[1] = {k: (np.zeros_like(v[0]), v[1]) for k, v in exs[1].items()}
    x = r.standard_normal(d).astype(np.float32)
    w = np.array([0.5, 0.3, 0.2])
    y = oracle.token_forward(x, [0, 1, 2], w, lambda e: exs[e])
    y2 = oracle.token_forward(x, [0, 2], w[[0, 2]], lambda e: exs[e])
    assert np.array_equal(y, y2)


def test_k1_weight_one_is_the_single_expert():
    r = np.random.default_rng(10)
    ex = _rand_expert(r, 128, 64)
    x = r.standard_normal(128).astype(np.float32)
    y = oracle.token_forward(x, [0], np.array([1.0]), lambda e: ex)
    assert np.array_equal(y, oracle.expert_ffn(x.astype(np.float64), ex))


@pytest.mark.parametrize("delta", [-3, 1, 5])
def test_down_scale_shift_scales_output_exactly(delta):
    r = np.random.default_rng(11)
    ex = _rand_expert(r, 128, 64)
    x = r.standard_normal(128)
    y = oracle.expert_ffn(x, ex)
    e2 = dict(ex)
    e2["down"] = (ex["down"][0], (ex["down"][1].astype(np.int32) + delta).astype(np.uint8))
    assert np.array_equal(oracle.expert_ffn(x, e2), y * 2.0 ** delta)


def test_relabelling_experts_is_consistent():
    sh = synthdata.TINY
    wr = synthdata.router_weight(sh)
    exs = synthdata.all_experts_host(sh)
    x = synthdata.tokens(sh, 4)
    get = lambda e: {w: (exs[w][0][e], exs[w][1][e]) for w in exs}
    perm = np.random.default_rng(12).permutation(sh.E)          # new id of old expert e = perm[e]
    inv = np.argsort(perm)
    wr2 = wr[inv]
    get2 = lambda e: get(int(inv[e]))
    a, b = oracle.route(x, wr, sh.k), oracle.route(x, wr2, sh.k)
    assert np.array_equal(perm[a["topk_idx"]], b["topk_idx"])   # no ties in these logits
    for t in range(4):
        ya = oracle.token_forward(x[t], a["topk_idx"][t], a["topk_w"][t], get)
        yb = oracle.token_forward(x[t], b["topk_idx"][t], b["topk_w"][t], get2)
        # the softmax normaliser sums over experts in id order, so relabelling
        # only reorders that sum: equal up to its rounding
        assert np.allclose(ya, yb, rtol=1e-14, atol=1e-14 * np.abs(ya).max())


def test_combine_is_weighted_sum_and_batch_invariant():
    sh = synthdata.TINY
    exs = synthdata.all_experts_host(sh)
    get = lambda e: {w: (exs[w][0][e], exs[w][1][e]) for w in exs}
    x = synthdata.tokens(sh, 2)
    e_t, w_t = [3, 9], np.array([0.75, 0.25])
    y = oracle.token_forward(x[0], e_t, w_t, get)
    o3 = oracle.expert_ffn(x[0].astype(np.float64), get(3))
    o9 = oracle.expert_ffn(x[0].astype(np.float64), get(9))
    assert np.array_equal(y, 0.75 * o3 + 0.25 * o9)
    # a token's result does not depend on which other tokens are in the batch
    wr = synthdata.router_weight(sh)
    r1 = oracle.route(x[:1], wr, sh.k)
    r2 = oracle.route(x, wr, sh.k)
    assert np.array_equal(r1["topk_idx"][0], r2["topk_idx"][0])
    assert np.array_equal(r1["topk_w"][0], r2["topk_w"][0])


def test_mx_mode_uses_quantised_activations():
    sh = synthdata.TINY
    exs = synthdata.all_experts_host(sh)
    get = lambda e: {w: (exs[w][0][e], exs[w][1][e]) for w in exs}
    x = synthdata.token(sh, 0)
    keep = {}
    y = oracle.token_forward(x, [1, 2], [0.6, 0.4], get, act_mode="mxfp4", keep=keep)
    xq = oracle.mx_roundtrip(x)
    assert np.array_equal(keep["x_used"], xq)
    ref = np.zeros(sh.d)
    for j, e in enumerate([1, 2]):
        h = oracle.gateup(xq, get(e)["gate"], get(e)["up"])
        ref += [0.6, 0.4][j] * oracle.down(oracle.mx_roundtrip(h), get(e)["down"])
    assert np.array_equal(y, ref)
    y32 = oracle.token_forward(x, [1, 2], [0.6, 0.4], get)
    assert not np.allclose(y, y32, rtol=1e-3)   # a different function, as expected


@pytest.mark.parametrize("act_mode", ["fp32", "mxfp4"])
@pytest.mark.parametrize("override", [False, True])
def test_layer_forward_is_token_forward(act_mode, override):
    """The expert-major evaluation (each expert visited once for all of its
    pairs) forms every token's sum with the same fp64 operations in the same
    order as token_forward, so the two agree bit for bit."""
    sh = synthdata.TINY
    host = synthdata.all_experts_host(sh)
    get = lambda e: {w: (host[w][0][e], host[w][1][e]) for w in host}  # noqa: E731
    x = synthdata.tokens(sh, 40, first=123)
    r = oracle.route(x, synthdata.router_weight(sh), sh.k)
    rng = np.random.default_rng(5)
    hs = rng.standard_normal((40, sh.k, sh.f)).astype(np.float32)
    hov = (lambda t: list(hs[t])) if override else None
    toks = [39, 0, 7, 8, 21]
    seen = []

    def get_logged(e):
        seen.append(e)
        return get(e)

    keep = {}
    got = oracle.layer_forward(x, r, toks, get_logged, act_mode=act_mode, h_override=hov, keep=keep)
    assert seen == sorted(set(seen)), "experts are fetched once each, ascending"
    for i, t in enumerate(toks):
        kt = {}
        ref = oracle.token_forward(x[t], r["topk_idx"][t], r["topk_w"][t], get, act_mode=act_mode,
                                   h_override=None if hov is None else hov(t), keep=kt)
        assert np.array_equal(got[i], ref)
        for j in range(sh.k):
            assert np.array_equal(keep["h"][(t, j)], kt["h"][j])


def test_ffn_vs_dense_matmul_format_edges():
    """The format-edge layer (scale bytes over 0..252, the subnormal 2^-127
    included, and all-zero / all -0 code blocks under any scale byte): the
    oracle's expert FFN still equals the dense fp64 product of the bit-decoded
    weights, and every byte value and both zero-block kinds are present."""
    sh = synthdata.EDGE
    x = synthdata.tokens(sh, 3, first=11).astype(np.float64)
    for e in (0, 5):
        ex = synthdata.expert(sh, e)
        for w in ("gate", "up", "down"):
            c, s = ex[w]
            assert set(np.unique(s)) == set(range(253)), w
            blocks = c.reshape(c.shape[0], -1, 16)
            zero = (blocks == 0).all(-1)
            negz = (blocks == 0x88).all(-1)
            for b in synthdata.EDGE_ZERO_BYTES:
                assert (s[zero] == b).any() and (s[negz] == b).any(), (w, b)
        for t in range(3):
            got = oracle.expert_ffn(x[t], ex)
            ref = _dense_ffn(x[t], ex)
            assert np.all(np.isfinite(ref))
            assert np.linalg.norm(got - ref) <= 1e-12 * np.linalg.norm(ref)
