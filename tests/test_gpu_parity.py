"""GPU parity of the HIP path (through the C ABI) against the fp64 oracle.

Every output is poisoned before each call (y NaN, routing -7, debug outputs
NaN / 0xFF), so nothing the kernels skip can pass.  Small layers are compared
element by element on every token.  The full 896-expert layer (d_model 7168,
d_ff 2048, top-16), in the launch configuration the benchmark times: routing
on every token; y on every token up to 64 tokens and on the 256-token skewed
batch (fp32 activations); in MXFP4 mode x_q and h_q on every pair, and h and
y on tokens chosen so that every active expert has a checked pair and the
heaviest experts' last rows and pass boundaries are checked.  A format-edge
layer puts every E8M0 byte 0..252 and all-zero / -0 code blocks through
every path."""
import numpy as np
import pytest
import torch

import oracle
import synthdata
from helpers import (assert_route_equal, assert_y_close, covering_tokens, host_expert_getter, oracle_y,
                     oracle_y_major)

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import mxfp4_routed_expert_softmax_amd as k3  # noqa: E402

DEV = torch.device("cuda:0")


def _log(msg):
    print(msg, flush=True)


def _to_dev_experts(host):
    return {w: (torch.from_numpy(host[w][0]).to(DEV), torch.from_numpy(host[w][1]).to(DEV)) for w in host}


# ----------------------------------------------------------------- tiny ---
@pytest.fixture(scope="module")
def tiny():
    sh = synthdata.TINY
    host = synthdata.all_experts_host(sh)
    wr = synthdata.router_weight(sh)
    return dict(shape=sh, host=host, dev=_to_dev_experts(host), wr=wr,
                wr_dev=torch.from_numpy(wr).to(DEV), get=host_expert_getter(sh, host))


def _run(x, wr_dev, experts, k, bias=None, bias_mode="none", act="fp32", dbg=None, score="softmax"):
    """k3moe_forward with every output poisoned first (y NaN, routing -7), so
    that a row or pair the kernels never write cannot pass for a computed one."""
    xd = torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
    bd = None if bias is None else torch.from_numpy(bias).to(DEV)
    fw = k3.Forward(xd, wr_dev, experts, k, bd, bias_mode, act, dbg, score_fn=score)
    fw.y.fill_(float("nan"))
    for t in fw.route.values():
        t.fill_(-7)
    fw()
    torch.cuda.synchronize()
    y = fw.y.cpu().numpy()
    assert np.isfinite(y).all(), "y has rows the kernels did not write (or non-finite values)"
    return y, fw.route


@pytest.mark.parametrize("T", [1, 2, 63, 64, 65, 130, 1100])
def test_tiny_fp32_all_tokens(tiny, T):
    sh = tiny["shape"]
    _log(f"tiny fp32 T={T}")
    x = synthdata.tokens(sh, T, first=1000 * T)
    y, route = _run(x, tiny["wr_dev"], tiny["dev"], sh.k)
    ref = oracle.route(x, tiny["wr"], sh.k)
    assert_route_equal(route, ref)
    assert_y_close(y, oracle_y(x, ref, range(T), tiny["get"]))


def test_tiny_decode_reps_deterministic(tiny):
    sh = tiny["shape"]
    for rep in range(3):
        x = synthdata.tokens(sh, 1, first=rep)
        y1, r1 = _run(x, tiny["wr_dev"], tiny["dev"], sh.k)
        y2, r2 = _run(x, tiny["wr_dev"], tiny["dev"], sh.k)
        assert np.array_equal(y1, y2)
        for kname in r1:
            assert torch.equal(r1[kname], r2[kname])


def test_tiny_edge_cases(tiny):
    sh = tiny["shape"]
    # all-zero tokens: every logit is 0 -> experts 0..k-1 (lower id wins), w = 1/k, y = 0
    x = np.zeros((3, sh.d), np.float32)
    y, route = _run(x, tiny["wr_dev"], tiny["dev"], sh.k)
    assert np.array_equal(route["topk_idx"].cpu().numpy(), np.tile(np.arange(sh.k), (3, 1)))
    assert np.all(route["topk_w"].cpu().numpy() == np.float32(1.0 / sh.k))
    assert np.all(y == 0.0)
    # duplicated router rows tie exactly -> the lower id is chosen first
    wr = tiny["wr"].copy()
    x = synthdata.tokens(sh, 8, first=50)
    lg = oracle.router_logits(x, wr)
    top = int(np.argmax(lg[0]))
    wr[(top + 5) % sh.E] = wr[top]
    wrd = torch.from_numpy(wr).to(DEV)
    y, route = _run(x, wrd, tiny["dev"], sh.k)
    ref = oracle.route(x, wr, sh.k)
    assert_route_equal(route, ref)
    assert_y_close(y, oracle_y(x, ref, range(8), tiny["get"]))


@pytest.mark.parametrize("k", [1, 16])
def test_tiny_k_extremes(tiny, k):
    sh = tiny["shape"]
    x = synthdata.tokens(sh, 5, first=77)
    y, route = _run(x, tiny["wr_dev"], tiny["dev"], k)
    ref = oracle.route(x, tiny["wr"], k)
    assert_route_equal(route, ref)
    if k == 1:
        assert np.all(route["topk_w"].cpu().numpy() == 1.0)
    assert_y_close(y, oracle_y(x, ref, range(5), tiny["get"]))


@pytest.mark.parametrize("T", [40, 1100])
@pytest.mark.parametrize("mode", ["logits", "select_only"])
def test_tiny_bias_modes(tiny, mode, T):
    sh = tiny["shape"]
    bias = synthdata.zipf_bias(sh)
    x = synthdata.tokens(sh, T, first=300)
    y, route = _run(x, tiny["wr_dev"], tiny["dev"], sh.k, bias, mode)
    bm = oracle.BIAS_LOGITS if mode == "logits" else oracle.BIAS_SELECT_ONLY
    ref = oracle.route(x, tiny["wr"], sh.k, bias, bm)
    assert_route_equal(route, ref)
    assert_y_close(y, oracle_y(x, ref, range(T), tiny["get"]))


_BM = {"none": 0, "logits": 1, "select_only": 2}


@pytest.mark.parametrize("T", [5, 40, 1100])
@pytest.mark.parametrize("mode", ["none", "logits", "select_only"])
def test_tiny_sigmoid_router(tiny, T, mode):
    """The pages' router: sigmoid scores, bias on the score for selection only
    (T = 1100: logits from the int8 slices, certified selection)."""
    sh = tiny["shape"]
    bias = None if mode == "none" else synthdata.zipf_bias(sh) * np.float32(0.1)
    x = synthdata.tokens(sh, T, first=700 + T)
    y, route = _run(x, tiny["wr_dev"], tiny["dev"], sh.k, bias, mode, score="sigmoid")
    ref = oracle.route(x, tiny["wr"], sh.k, bias, _BM[mode], oracle.SCORE_SIGMOID)
    assert_route_equal(route, ref)
    assert_y_close(y, oracle_y(x, ref, range(T), tiny["get"]))


@pytest.mark.parametrize("score", ["softmax", "sigmoid"])
def test_tiny_int8_router_ties_fall_back(tiny, score):
    """Batches of >= 1024 tokens take logits from int8 slices with a certified
    selection.  Duplicated router rows make exact ties in every token and
    all-zero tokens make every logit equal: neither can be certified, so those
    tokens are recomputed exactly -- and must still match the oracle bit for
    bit, ties to the lower expert index."""
    sh = tiny["shape"]
    wr = tiny["wr"].copy()
    wr[11] = wr[3]
    wr[6] = wr[5]
    wr[15] = wr[0]
    wr_dev = torch.from_numpy(wr).to(DEV)
    T = 1100
    x = synthdata.tokens(sh, T, first=4242)
    x[[0, 17, 1099]] = 0.0
    y, route = _run(x, wr_dev, tiny["dev"], sh.k, score=score)
    ref = oracle.route(x, wr, sh.k, score_fn=oracle.SCORE_SIGMOID if score == "sigmoid" else oracle.SCORE_SOFTMAX)
    assert_route_equal(route, ref)
    assert np.array_equal(ref["topk_idx"][0], np.arange(sh.k))  # all-zero token: the lowest indices
    assert_y_close(y, oracle_y(x, ref, range(T), tiny["get"]))


@pytest.mark.parametrize("partner", [80, 40])
def test_int8_router_near_tie_at_k_plus_one(partner):
    """Certified selection when the k-th and (k+1)-th experts differ by less
    than the int8 slices resolve.  Experts 64..79 score 26, 25, ..., 11 on
    every token (so all 16 winners come from one list of 64); the partner
    scores 11 as well, and the higher-indexed of expert 79 and the partner
    gets a further 2^-45 that the slices truncate away.  The exact logits
    put that expert 16th; the sliced ones tie, so the token must fall back to
    the exact recompute.  partner 80: the (k+1)-th is entry 16 of the
    winners' own list; partner 40: it heads another list."""
    E, d, k, T = 128, 256, 16, 1100
    rng = np.random.default_rng(8080 + partner)
    wr = np.zeros((E, d), dtype=np.float32)
    background = [e for e in range(E) if not 64 <= e <= 79 and e != partner]
    wr[background, 2:] = (0.1 * rng.standard_normal((len(background), d - 2))).astype(np.float32)
    wr[64:80, 0] = np.arange(26, 10, -1, dtype=np.float32)
    wr[partner, 0] = 11.0
    wr[max(79, partner), 1] = np.float32(2.0 ** -45)
    x = rng.standard_normal((T, d)).astype(np.float32)
    x[:, 0] = 1.0
    x[:, 1] = 1.0
    route = k3.k3moe_route(torch.from_numpy(x).to(DEV), torch.from_numpy(wr).to(DEV), k)
    torch.cuda.synchronize()
    ref = oracle.route(x, wr, k)
    expect = list(range(64, 79)) + [max(79, partner)]
    assert all(list(r) == expect for r in ref["topk_idx"])
    assert_route_equal(route, ref)


def test_k3_int8_router_many_uncertified_tokens():
    """The 896-expert router at 300 tokens (int8 slices, K split) with 20
    router rows duplicated: a token whose top 17 holds a duplicated expert has
    an exact tie there and cannot be certified, which is about a third of
    the tokens -- far more than the fallback's four block slots, so its
    kernels loop over the list -- and three all-zero tokens are selected
    directly.  Routing must match the oracle bit for bit."""
    sh = synthdata.K3
    wr = synthdata.router_weight(sh)
    rng = np.random.default_rng(300)
    src = rng.choice(sh.E, 20, replace=False)
    dst = rng.choice(np.setdiff1d(np.arange(sh.E), src), 20, replace=False)
    wr[dst] = wr[src]
    T = 300
    x = synthdata.tokens(sh, T, first=9000)
    x[[0, 150, 299]] = 0.0
    _log("k3 int8 router, 20 duplicated rows, T=300")
    route = k3.k3moe_route(torch.from_numpy(x).to(DEV), torch.from_numpy(wr).to(DEV), sh.k)
    torch.cuda.synchronize()
    ref = oracle.route(x, wr, sh.k)
    tied = sum(bool(set(r) & set(dst.tolist()) or set(r) & set(src.tolist())) for r in ref["topk_idx"])
    assert tied >= 40, tied  # the list is long
    assert_route_equal(route, ref)


def _graph_replays_match_eager(xs, wr_dev, experts, k, act="fp32"):
    """k3moe_forward captured once in a HIP graph, then replayed for each
    input in xs (copied into the captured input buffer), with an eager call
    on another input between replays: every replay must equal an eager call
    on the same input bit for bit (outputs and all routing buffers).  The
    library allocates nothing and issues no memset, so every node is a
    kernel."""
    gx = xs[0].clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    fw = k3.Forward(gx, wr_dev, experts, k, act_mode=act, stream=s)
    with torch.cuda.stream(s):
        fw()  # first call outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        fw()
    torch.cuda.synchronize()
    eager = k3.Forward(xs[0], wr_dev, experts, k, act_mode=act)
    n = len(xs)
    for r in range(n):
        gx.copy_(xs[r])
        g.replay()
        torch.cuda.synchronize()
        y_g = fw.y.clone()
        route_g = {name: t.clone() for name, t in fw.route.items()}
        eager.set_x(xs[(r + 1) % n])
        eager()
        torch.cuda.synchronize()
        eager.set_x(xs[r])
        y_e = eager().clone()
        torch.cuda.synchronize()
        assert torch.equal(y_g, y_e), f"replay {r}: y differs from the eager call"
        for name in route_g:
            assert torch.equal(route_g[name], eager.route[name]), f"replay {r}: {name} differs"


@pytest.mark.parametrize("T,act", [(1, "fp32"), (40, "fp32"), (300, "mxfp4"), (1100, "fp32")])
def test_tiny_graph_replay(tiny, T, act):
    sh = tiny["shape"]
    _log(f"tiny graph replay T={T} {act}")
    xs = [torch.from_numpy(synthdata.tokens(sh, T, first=6000 + 10 * T + r * T)).to(DEV) for r in range(4)]
    _graph_replays_match_eager(xs, tiny["wr_dev"], tiny["dev"], sh.k, act)


def test_t0_is_a_noop(tiny):
    sh = tiny["shape"]
    x = torch.zeros((0, sh.d), dtype=torch.float32, device=DEV)
    y, route = k3.k3moe_forward(x, tiny["wr_dev"], tiny["dev"], sh.k)
    torch.cuda.synchronize()
    assert y.shape == (0, sh.d)


def _dbg_buffers(T, k, d, f):
    """Debug outputs filled with sentinels: h NaN, codes and scales 0xFF (a
    scale byte the quantiser never writes)."""
    u8 = dict(dtype=torch.uint8, device=DEV)
    return dict(x_codes=torch.full((T, d // 2), 0xFF, **u8), x_scales=torch.full((T, d // 32), 0xFF, **u8),
                h=torch.full((T * k, f), float("nan"), dtype=torch.float32, device=DEV),
                h_codes=torch.full((T * k, f // 2), 0xFF, **u8), h_scales=torch.full((T * k, f // 32), 0xFF, **u8))


def _check_mx_split(x, ref, dbg, y, tokens, k, get=None, shape=None):
    """Split-step parity of the MXFP4 path: x_q bit-exact on every token, h_q
    bit-exact on every pair (the oracle's quantiser applied to the device's
    own fp32 h), no sentinel left in any debug output; on the given tokens, h
    against the oracle's h from the quantised x and y against the oracle's
    down + combine of the device's h.  Experts come from ``get`` (host
    copies) or are regenerated from the seeds of ``shape``."""
    # 1. activation quantisation, bit-exact on every token
    xc, xs = oracle.mx_quantize(x)
    assert np.array_equal(dbg["x_codes"].cpu().numpy(), xc), "x_q codes"
    assert np.array_equal(dbg["x_scales"].cpu().numpy(), xs), "x_q scales"
    # 2. h quantisation of the device's own fp32 h, bit-exact on every pair
    h_dev = dbg["h"].cpu().numpy()
    assert not np.isnan(h_dev).any(), "h of some pair was never written"
    hs_dev = dbg["h_scales"].cpu().numpy()
    assert not (hs_dev == 0xFF).any(), "h_q scales of some pair were never written"
    hc, hs = oracle.mx_quantize(h_dev)
    assert np.array_equal(dbg["h_codes"].cpu().numpy(), hc), "h_q codes"
    assert np.array_equal(hs_dev, hs), "h_q scales"
    # 3. + 4. h and y on the chosen tokens, expert-major
    tokens = [int(t) for t in tokens]
    keep = {}
    y_ref = oracle_y_major(x, ref, tokens, shape, act_mode="mxfp4",
                           h_override=lambda t: [h_dev[t * k + j] for j in range(k)], keep=keep, get=get)
    pairs = [(t, j) for t in tokens for j in range(k)]
    assert_y_close(np.stack([h_dev[t * k + j] for t, j in pairs]), np.stack([keep["h"][p] for p in pairs]), "h")
    assert_y_close(y[tokens], y_ref, "y")


@pytest.mark.parametrize("T,k", [(2, 16), (5, 16)])
def test_tiny_mx_k_equals_e(tiny, T, k):
    """k = E: every expert holds all T tokens, more pairs than experts (an
    active list in which every expert has the same passes)."""
    sh = tiny["shape"]
    x = synthdata.tokens(sh, T, first=900 + T)
    dbg = _dbg_buffers(T, k, sh.d, sh.f)
    y, route = _run(x, tiny["wr_dev"], tiny["dev"], k, act="mxfp4", dbg=dbg)
    ref = oracle.route(x, tiny["wr"], k)
    assert_route_equal(route, ref)
    assert np.all(ref["counts"] == T)
    _check_mx_split(x, ref, dbg, y, range(T), k, get=tiny["get"])


@pytest.mark.parametrize("T", [1, 2, 37, 300, 1100, 2000])
def test_tiny_mx_split_step(tiny, T):
    """T = 2000: ~250 tokens per expert, three passes of up to 96 each."""
    sh = tiny["shape"]
    _log(f"tiny mx T={T}")
    x = synthdata.tokens(sh, T, first=5000 + T)
    dbg = _dbg_buffers(T, sh.k, sh.d, sh.f)
    y, route = _run(x, tiny["wr_dev"], tiny["dev"], sh.k, act="mxfp4", dbg=dbg)
    ref = oracle.route(x, tiny["wr"], sh.k)
    assert_route_equal(route, ref)
    toks = range(T) if T <= 300 else range(0, T, 7)
    _check_mx_split(x, ref, dbg, y, toks, sh.k, get=tiny["get"])


# ------------------------------------------------ small d_ff % 512 layers ---
@pytest.fixture(scope="module", params=["small_f1536", "small_f512"])
def small(request):
    sh = {"small_f1536": synthdata.SMALL_F1536, "small_f512": synthdata.SMALL_F512}[request.param]
    host = synthdata.all_experts_host(sh)
    wr = synthdata.router_weight(sh)
    return dict(shape=sh, host=host, dev=_to_dev_experts(host), wr=wr,
                wr_dev=torch.from_numpy(wr).to(DEV), get=host_expert_getter(sh, host))


@pytest.mark.parametrize("T", [1, 7, 32, 40])
def test_small_fp32_all_tokens(small, T):
    """T*k <= 128: gate/up GEMV writing h as MX-FP8 slices, down on the matrix
    cores; T = 40 with k = 4 takes the grouped path."""
    sh = small["shape"]
    _log(f"{sh.name} fp32 T={T}")
    x = synthdata.tokens(sh, T, first=700 + T)
    y, route = _run(x, small["wr_dev"], small["dev"], sh.k)
    ref = oracle.route(x, small["wr"], sh.k)
    assert_route_equal(route, ref)
    assert_y_close(y, oracle_y(x, ref, range(T), small["get"]))
    y2, _ = _run(x, small["wr_dev"], small["dev"], sh.k)
    assert np.array_equal(y, y2), "not bitwise deterministic"


def _forward_vs_split(x, wr_dev, experts, k, bias=None, bias_mode="none"):
    """k3moe_forward against k3moe_route then k3moe_ffn on the same buffers
    (routing outputs poisoned before each): the two must agree bit for bit."""
    xd = torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
    bd = None if bias is None else torch.from_numpy(bias).to(DEV)
    fw = k3.Forward(xd, wr_dev, experts, k, bd, bias_mode)
    for t in fw.route.values():
        t.fill_(-7)
    y1 = fw().clone()
    r1 = {n: t.clone() for n, t in fw.route.items()}
    for t in fw.route.values():
        t.fill_(-7)
    fw.y.fill_(0.0)
    fw.run_route()
    y2 = fw.run_ffn().clone()
    torch.cuda.synchronize()
    for n in r1:
        assert torch.equal(r1[n], fw.route[n]), f"routing output {n} differs"
    assert torch.equal(y1, y2), "y differs between k3moe_forward and route + ffn"
    return y1.cpu().numpy(), {n: t.cpu() for n, t in r1.items()}


@pytest.mark.parametrize("bias_mode", ["none", "logits", "select_only"])
def test_small_forward_one_token(small, bias_mode):
    sh = small["shape"]
    _log(f"{sh.name} one-token forward vs route + ffn, bias {bias_mode}")
    bias = None if bias_mode == "none" else synthdata.zipf_bias(sh)
    for rep in range(4):
        # rep 3: x = 0, every logit 0 -- ties everywhere, the first k experts win
        x = synthdata.tokens(sh, 1, first=4000 + rep) if rep < 3 else np.zeros((1, sh.d), np.float32)
        y, route = _forward_vs_split(x, small["wr_dev"], small["dev"], sh.k, bias, bias_mode)
        bm = {"none": oracle.BIAS_NONE, "logits": oracle.BIAS_LOGITS, "select_only": oracle.BIAS_SELECT_ONLY}[bias_mode]
        ref = oracle.route(x, small["wr"], sh.k, bias, bm)
        assert_route_equal(route, ref)
        assert_y_close(y, oracle_y(x, ref, [0], small["get"]))


@pytest.mark.parametrize("T", [1, 37, 600, 1200])
def test_small_mx_split_step(small, T):
    """MXFP4 activations on layers whose d_model and d_ff are multiples of
    512: the pipelined grouped GEMMs with one, two and three K chunks (512,
    1024, 1536); T = 600 puts more than 96 tokens on an expert (several
    passes per block); T = 1200 puts 200-300 tokens on an expert (three or
    four passes of up to 96)."""
    sh = small["shape"]
    _log(f"{sh.name} mx T={T}")
    x = synthdata.tokens(sh, T, first=9000 + T)
    dbg = _dbg_buffers(T, sh.k, sh.d, sh.f)
    y, route = _run(x, small["wr_dev"], small["dev"], sh.k, act="mxfp4", dbg=dbg)
    ref = oracle.route(x, small["wr"], sh.k)
    assert_route_equal(route, ref)
    toks = range(T) if T <= 300 else range(0, T, 5)
    _check_mx_split(x, ref, dbg, y, toks, sh.k, get=small["get"])


# ------------------------------------------------------ contract limits ---
_LIMIT_SHAPES = {sh.name: sh for sh in (synthdata.LIMIT_E1024, synthdata.WIDE)}
_limit_layers = {}


def _limit_layer(name):
    if name not in _limit_layers:
        sh = _LIMIT_SHAPES[name]
        host = synthdata.all_experts_host(sh)
        wr = synthdata.router_weight(sh)
        _limit_layers[name] = dict(shape=sh, dev=_to_dev_experts(host), wr=wr,
                                   wr_dev=torch.from_numpy(wr).to(DEV), get=host_expert_getter(sh, host))
    return _limit_layers[name]


# 1024 experts: k = 32 (the largest k; fp64 router at every T), k = 31 and 16
# at 1100 tokens (the certified int8 router; k = 31 keeps 32 entries per
# list); T = 8 (256 pairs over 1024 experts: the one-token and the
# several-token gate/up launches of the grouped path side by side).  The
# wide layer: the pair path (T = 1, 3) and the grouped path (T = 70).
@pytest.mark.parametrize("name,k,T", [("limit_e1024", 32, 1), ("limit_e1024", 32, 8), ("limit_e1024", 32, 70),
                                      ("limit_e1024", 32, 1100),
                                      ("limit_e1024", 31, 1100), ("limit_e1024", 16, 1100),
                                      ("wide_d8256", 2, 1), ("wide_d8256", 2, 3), ("wide_d8256", 2, 70)])
def test_limit_fp32(name, k, T):
    L = _limit_layer(name)
    sh = L["shape"]
    _log(f"{name} fp32 k={k} T={T}")
    x = synthdata.tokens(sh, T, first=31 * T + k)
    y, route = _run(x, L["wr_dev"], L["dev"], k)
    ref = oracle.route(x, L["wr"], k)
    assert_route_equal(route, ref)
    toks = range(T) if T <= 128 else range(0, T, 3)
    assert_y_close(y[list(toks)], oracle_y(x, ref, toks, L["get"]))


@pytest.mark.parametrize("T", [3, 70])
def test_wide_mx_split_step(T):
    L = _limit_layer("wide_d8256")
    sh = L["shape"]
    _log(f"{sh.name} mx T={T}")
    x = synthdata.tokens(sh, T, first=77 + T)
    dbg = _dbg_buffers(T, sh.k, sh.d, sh.f)
    y, route = _run(x, L["wr_dev"], L["dev"], sh.k, act="mxfp4", dbg=dbg)
    ref = oracle.route(x, L["wr"], sh.k)
    assert_route_equal(route, ref)
    _check_mx_split(x, ref, dbg, y, range(T), sh.k, get=L["get"])


# ---------------------------------------------------------- format edges ---
@pytest.fixture(scope="module")
def edge():
    sh = synthdata.EDGE
    host = synthdata.all_experts_host(sh)
    wr = synthdata.router_weight(sh)
    return dict(shape=sh, host=host, dev=_to_dev_experts(host), wr=wr,
                wr_dev=torch.from_numpy(wr).to(DEV), get=host_expert_getter(sh, host))


@pytest.mark.parametrize("T", [1, 3, 70, 300])
def test_edge_format_fp32(edge, T):
    """Weights whose scale bytes take every value 0..252 (byte 0: the
    subnormal scale 2^-127), with products of ordinary size, and blocks of
    all-zero and all -0 codes under any scale byte, in gate, up and down:
    T = 1, 3 the pair path (down on the matrix cores), 70 the grouped GEMVs,
    300 also the int8 router (its bound is wide here: every token falls back
    to the fp64 recompute)."""
    sh = edge["shape"]
    _log(f"edge fp32 T={T}")
    x = synthdata.tokens(sh, T, first=40 + T)
    y, route = _run(x, edge["wr_dev"], edge["dev"], sh.k)
    ref = oracle.route(x, edge["wr"], sh.k)
    assert_route_equal(route, ref)
    assert_y_close(y, oracle_y(x, ref, range(T), edge["get"]))


@pytest.mark.parametrize("T", [1, 70, 300])
def test_edge_format_mx_split_step(edge, T):
    sh = edge["shape"]
    _log(f"edge mx T={T}")
    x = synthdata.tokens(sh, T, first=90 + T)
    dbg = _dbg_buffers(T, sh.k, sh.d, sh.f)
    y, route = _run(x, edge["wr_dev"], edge["dev"], sh.k, act="mxfp4", dbg=dbg)
    ref = oracle.route(x, edge["wr"], sh.k)
    assert_route_equal(route, ref)
    _check_mx_split(x, ref, dbg, y, range(T), sh.k, get=edge["get"])


# ------------------------------------------- adversarial MXFP4 pass lists ---
# 1024 experts with 512-wide reduction axes (the pipelined matrix-core GEMMs
# and their per-XCD pass lists), small enough to upload whole
ADV = synthdata.LayerShape("adv_e1024_f512", d=512, f=512, E=1024, k=2, layer=8)


def test_mx_pass_lists_round_robin_fallback():
    """k3moe_ffn on a routing built by hand: expert 1023 holds every token
    (14,200: 148 passes of the GEMMs), experts 0..1022 about 14 each (one pass).
    Eight equal-pass runs would give XCDs 0-6 about 146 experts each, more than
    a table holds (ceil(E / 8) + 8 = 136), so the pass lists are dealt
    round-robin instead.  x_q and h_q on every pair, h and y on a token of
    every expert and on the heavy expert's last rows."""
    sh, T = ADV, 14200
    _log("adversarial pass lists: generating 1024 experts")
    dev = _to_dev_experts(synthdata.all_experts_host(sh))
    x = synthdata.tokens(sh, T)
    idx = np.stack([np.full(T, sh.E - 1), np.arange(T) % (sh.E - 1)], axis=1).astype(np.int32)
    ref = dict(topk_idx=idx, topk_w=np.full((T, 2), 0.5, np.float32))
    ref.update(oracle.permute(idx, sh.E))
    route = {n: torch.from_numpy(np.ascontiguousarray(v)).to(DEV) for n, v in ref.items()}
    dbg = _dbg_buffers(T, sh.k, sh.d, sh.f)
    yd = torch.full((T, sh.d), float("nan"), dtype=torch.float32, device=DEV)
    k3.k3moe_ffn(torch.from_numpy(x).to(DEV), dev, route, act_mode="mxfp4", y=yd, dbg=dbg)
    torch.cuda.synchronize()
    y = yd.cpu().numpy()
    assert np.isfinite(y).all(), "y has rows the kernels did not write"
    toks = list(range(sh.E - 1)) + list(range(T - 120, T))
    _check_mx_split(x, ref, dbg, y, toks, sh.k, shape=sh)


# ----------------------------------------------------------- full layer ---
@pytest.fixture(scope="module")
def k3layer():
    sh = synthdata.K3
    _log("uploading the 896-expert layer ...")
    dev = synthdata.upload_experts(sh, DEV)
    wr = synthdata.router_weight(sh)
    _log("upload done")
    return dict(shape=sh, dev=dev, wr=wr, wr_dev=torch.from_numpy(wr).to(DEV),
                get=host_expert_getter(sh), bias=synthdata.zipf_bias(sh))


def test_k3_decode_forward_vs_split(k3layer):
    sh = k3layer["shape"]
    for rep in (3, 500, -1):
        _log(f"k3 one-token forward vs route + ffn, rep {rep}")
        # rep -1: x = 0 (all 896 logits tie: the first k experts, weights 1/k)
        x = synthdata.tokens(sh, 1, first=rep) if rep >= 0 else np.zeros((1, sh.d), np.float32)
        y, route = _forward_vs_split(x, k3layer["wr_dev"], k3layer["dev"], sh.k)
        ref = oracle.route(x, k3layer["wr"], sh.k)
        assert_route_equal(route, ref)


@pytest.mark.parametrize("T", [1, 64])
def test_k3_sigmoid_router_select_only_bias(k3layer, T):
    sh = k3layer["shape"]
    _log(f"k3 sigmoid router, selection-only bias, T={T}")
    bias = k3layer["bias"] * np.float32(0.05)
    x = synthdata.tokens(sh, T, first=5000 + T)
    y, route = _run(x, k3layer["wr_dev"], k3layer["dev"], sh.k, bias, "select_only", score="sigmoid")
    ref = oracle.route(x, k3layer["wr"], sh.k, bias, oracle.BIAS_SELECT_ONLY, oracle.SCORE_SIGMOID)
    assert_route_equal(route, ref)
    toks = [0] if T == 1 else [0, 17, 63]
    assert_y_close(y[toks], oracle_y(x, ref, toks, k3layer["get"]))


def test_k3_decode_graph_replay(k3layer):
    sh = k3layer["shape"]
    _log("k3 decode graph replay")
    xs = [torch.from_numpy(synthdata.tokens(sh, 1, first=7000 + r)).to(DEV) for r in range(4)]
    _graph_replays_match_eager(xs, k3layer["wr_dev"], k3layer["dev"], sh.k)


def test_k3_decode_t1(k3layer):
    sh = k3layer["shape"]
    for rep in (0, 1, 999):
        _log(f"k3 decode rep {rep}")
        x = synthdata.tokens(sh, 1, first=rep)
        y, route = _run(x, k3layer["wr_dev"], k3layer["dev"], sh.k)
        ref = oracle.route(x, k3layer["wr"], sh.k)
        assert_route_equal(route, ref)
        assert_y_close(y, oracle_y(x, ref, [0], k3layer["get"]))
        y2, _ = _run(x, k3layer["wr_dev"], k3layer["dev"], sh.k)
        assert np.array_equal(y, y2), "decode output is not bitwise deterministic"


def test_k3_small_batch_t8(k3layer):
    """Pair-major path (gate/up per pair, down with the fused gather combine)."""
    sh = k3layer["shape"]
    x = synthdata.tokens(sh, 8, first=20000)
    y, route = _run(x, k3layer["wr_dev"], k3layer["dev"], sh.k)
    ref = oracle.route(x, k3layer["wr"], sh.k)
    assert_route_equal(route, ref)
    assert_y_close(y, oracle_y_major(x, ref, range(8), sh))


def test_k3_batch_t64(k3layer):
    """The 64-token batch (grouped GEMVs): y on every token."""
    sh = k3layer["shape"]
    x = synthdata.tokens(sh, 64)
    y, route = _run(x, k3layer["wr_dev"], k3layer["dev"], sh.k)
    ref = oracle.route(x, k3layer["wr"], sh.k)
    assert_route_equal(route, ref)
    _log(f"k3 T=64: oracle on all 64 tokens ({int((ref['counts'] > 0).sum())} experts)")
    assert_y_close(y, oracle_y_major(x, ref, range(64), sh))


@pytest.mark.parametrize("T", [1, 8, 64])
def test_k3_mx_small_batches(k3layer, T):
    """MXFP4 mode at small batches, where nearly every expert holds one or two
    tokens of a 16-row matrix tile (T = 1 and 8: slots are segment heads;
    T = 64: an active list with the balanced per-XCD pass lists).  x_q and
    h_q on every pair, h and y on every token."""
    sh = k3layer["shape"]
    x = synthdata.tokens(sh, T, first=30000 + T)
    dbg = _dbg_buffers(T, sh.k, sh.d, sh.f)
    y, route = _run(x, k3layer["wr_dev"], k3layer["dev"], sh.k, act="mxfp4", dbg=dbg)
    ref = oracle.route(x, k3layer["wr"], sh.k)
    assert_route_equal(route, ref)
    c = ref["counts"]
    _log(f"k3 mx T={T}: {int((c > 0).sum())} active experts, at most {int(c.max())} tokens each")
    _check_mx_split(x, ref, dbg, y, range(T), sh.k, shape=sh)


def test_k3_prefill_t4096_mx(k3layer):
    """4096-token prefill, MXFP4 activations: routing on every token, x_q and
    h_q on every pair, h and y on >= 128 tokens that give every active expert
    a checked pair and check the last rows of the 16 heaviest experts and
    their row 96 (past the first 96-token pass)."""
    sh = k3layer["shape"]
    T = 4096
    x = synthdata.tokens(sh, T)
    dbg = _dbg_buffers(T, sh.k, sh.d, sh.f)
    y, route = _run(x, k3layer["wr_dev"], k3layer["dev"], sh.k, act="mxfp4", dbg=dbg)
    _log("k3 T=4096 oracle routing")
    ref = oracle.route(x, k3layer["wr"], sh.k)
    assert_route_equal(route, ref)
    toks = covering_tokens(ref, 128, seed=4096)
    _log(f"k3 T=4096 oracle h and y on {len(toks)} tokens")
    _check_mx_split(x, ref, dbg, y, toks, sh.k, shape=sh)


def test_k3_skew_t256(k3layer):
    """Zipf-skewed 256-token batch (bias in the logits): MXFP4 split-step on
    >= 96 tokens covering every active expert and the heavy experts' last
    rows; fp32 activations end to end on every token."""
    sh = k3layer["shape"]
    T = 256
    x = synthdata.tokens(sh, T)
    bias = k3layer["bias"]
    ref = oracle.route(x, k3layer["wr"], sh.k, bias, oracle.BIAS_LOGITS)
    # MXFP4 path (grouped scaled-MFMA GEMM under skew)
    dbg = _dbg_buffers(T, sh.k, sh.d, sh.f)
    y, route = _run(x, k3layer["wr_dev"], k3layer["dev"], sh.k, bias, "logits", act="mxfp4", dbg=dbg)
    assert_route_equal(route, ref)
    counts = ref["counts"]
    toks = covering_tokens(ref, 96, seed=256)
    _log(f"k3 skew: {int((counts > 0).sum())} active experts, max {counts.max()} tokens/expert; "
         f"mx on {len(toks)} tokens")
    _check_mx_split(x, ref, dbg, y, toks, sh.k, shape=sh)
    # fp32 path end to end, every token
    y32, route32 = _run(x, k3layer["wr_dev"], k3layer["dev"], sh.k, bias, "logits")
    assert_route_equal(route32, ref)
    _log("k3 skew fp32: oracle on all 256 tokens")
    assert_y_close(y32, oracle_y_major(x, ref, range(T), sh))


def test_k3_prefill_t32768_mx_sampled(k3layer):
    """The compute-bound prefill shape (32,768 tokens, ~585 per expert):
    routing on every token, x_q and h_q on every pair, h and y on tokens that
    cover every active expert, the heaviest experts' last rows and the rows
    where 128-token passes begin."""
    sh = k3layer["shape"]
    T = 32768
    x = synthdata.tokens(sh, T)
    dbg = _dbg_buffers(T, sh.k, sh.d, sh.f)
    y, route = _run(x, k3layer["wr_dev"], k3layer["dev"], sh.k, act="mxfp4", dbg=dbg)
    _log("k3 T=32768 oracle routing")
    ref = oracle.route(x, k3layer["wr"], sh.k)
    assert_route_equal(route, ref)
    toks = covering_tokens(ref, 80, seed=32768, n_heavy=8, pass_rows=(96, 128, 256, 384, 512))
    _log(f"k3 T=32768 oracle h and y on {len(toks)} tokens")
    _check_mx_split(x, ref, dbg, y, toks, sh.k, shape=sh)
