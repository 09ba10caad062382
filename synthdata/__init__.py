"""Seeded synthetic inputs for the routed-expert MoE layer.

This module only draws random inputs; it holds none of the layer's
arithmetic.  Both the fp64 oracle (tests, CPU baseline) and the HIP path
(tests, benchmark) take their inputs from here.

Shapes and distributions follow the workload the pages describe (896 routed
experts, 16 active per token, single-token greedy decode: fiv.co.kr
"kimi-k3-in-c deep dive", glossary "MoE" row and the cost paragraph;
repolode.com "O que e?").  The pages never state d_model or d_ff; the layer
here uses d_model = 7168 and d_ff = 2048 per expert, and a tiny layer
(256 / 128, 16 experts, top-2) for fast exact checks.

Every tensor is drawn from its own ``SeedSequence([MAGIC, layer, tensor,
index])`` so any single expert or token can be regenerated alone:
``index`` is the expert id for weights and the token / repetition id for x.
"""
from __future__ import annotations

import dataclasses
import math
from concurrent.futures import ThreadPoolExecutor

import numpy as np

MAGIC = 0x4B334D4F

# tensor ids inside the seed sequence
T_ROUTER, T_GATE_CODES, T_GATE_SCALES, T_UP_CODES, T_UP_SCALES = 0, 1, 2, 3, 4
T_DOWN_CODES, T_DOWN_SCALES, T_X, T_RANKING = 5, 6, 7, 8
T_EDGE = 9  # the format-edge layer's extra draws (scale jitter, zero blocks)

SCALE_LO, SCALE_HI = 120, 124  # E8M0 scale bytes drawn uniformly in [120, 124]


@dataclasses.dataclass(frozen=True)
class LayerShape:
    name: str
    d: int        # d_model
    f: int        # d_ff per expert
    E: int        # routed experts
    k: int        # experts per token
    layer: int    # seed-sequence layer id
    fmt: str = "uniform"  # "uniform", or "edge": the format-edge construction below

    @property
    def expert_bytes(self) -> int:
        """MX bytes of one expert: three matrices of d*f params, 4 bits each
        plus one scale byte per 32 params."""
        p = self.d * self.f
        return 3 * (p // 2 + p // 32)


TINY = LayerShape("tiny", d=256, f=128, E=16, k=2, layer=0)
K3 = LayerShape("k3", d=7168, f=2048, E=896, k=16, layer=1)
# Small layers whose d_ff is a multiple of 512 (the small-batch matrix-core
# path): three and one 512-value chunks, fewer experts per token than waves
# per block, an odd k.
SMALL_F1536 = LayerShape("small_f1536", d=1024, f=1536, E=24, k=4, layer=2)
SMALL_F512 = LayerShape("small_f512", d=512, f=512, E=12, k=3, layer=3)
# The contract's limits: 1024 experts (16 top-k lists of 64) with up to 32
# per token; and a wide layer whose d_model exceeds 256 MX blocks (two per
# lane in the gate/up GEMV) and whose d_ff takes two blocks per lane in the
# down GEMVs, neither a multiple of 512.
LIMIT_E1024 = LayerShape("limit_e1024", d=256, f=128, E=1024, k=32, layer=4)
WIDE = LayerShape("wide_d8256", d=8256, f=2560, E=8, k=2, layer=5)
# The format's edges: weight scale bytes over the whole range 0..252 (the
# subnormal scale 2^-127 of byte 0 included) with products of ordinary size,
# and blocks whose codes are all +0 or all -0 under any scale byte.  Column
# block b of x is drawn at 2^-EDGE_XEXP[b], gate/up rows of d_ff block c are
# scaled by 2^EDGE_OEXP[c] (so h by about 2^(2 EDGE_OEXP[c])), and the down
# scales undo that; the router rows carry 2^EDGE_XEXP[b] so logits stay O(1).
EDGE = LayerShape("edge_fmt", d=1024, f=512, E=8, k=2, layer=6, fmt="edge")
# Full-size experts (d_model 7168, d_ff 2048, top-16) but 64 of them: the
# expert-cache tests stream whole experts over the host link without
# generating the 21 GB layer.
CACHE_E64 = LayerShape("cache_e64", d=7168, f=2048, E=64, k=16, layer=7)
EDGE_XEXP = np.round(np.linspace(-77, 73, EDGE.d // 32)).astype(np.int64)
EDGE_OEXP = np.round(np.linspace(-48, 50, EDGE.f // 32)).astype(np.int64)
EDGE_ZERO_BYTES = (0, 1, 251, 252)  # scale bytes forced onto some all-zero-code blocks


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    shape: LayerShape
    T: int
    act_mode: str          # "fp32" or "mxfp4"
    zipf_bias: bool = False
    reps: int = 1


WORKLOADS = {
    "tiny_decode_t1": Workload("tiny_decode_t1", TINY, T=1, act_mode="fp32", reps=1000),
    "k3_decode_t1": Workload("k3_decode_t1", K3, T=1, act_mode="fp32", reps=1000),
    "k3_batch_t64": Workload("k3_batch_t64", K3, T=64, act_mode="fp32", reps=100),
    "k3_prefill_t4096": Workload("k3_prefill_t4096", K3, T=4096, act_mode="mxfp4", reps=20),
    "k3_skew_t256": Workload("k3_skew_t256", K3, T=256, act_mode="mxfp4", zipf_bias=True, reps=100),
    # informational: small MXFP4 batches, where most experts hold one or two
    # tokens (the GEMV side of the tokens-per-expert dispatch)
    "k3_batch_t8_mx": Workload("k3_batch_t8_mx", K3, T=8, act_mode="mxfp4", reps=100),
    "k3_batch_t64_mx": Workload("k3_batch_t64_mx", K3, T=64, act_mode="mxfp4", reps=100),
    # informational: ~585 tokens per expert, past the point where the MXFP4
    # products stop being bound by the weight stream
    "k3_prefill_t32768": Workload("k3_prefill_t32768", K3, T=32768, act_mode="mxfp4", reps=5),
}


def rng(layer: int, tensor: int, index: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([MAGIC, layer, tensor, index]))


def _edge_col_exp(shape: LayerShape) -> np.ndarray:
    return np.repeat(EDGE_XEXP, 32)


def router_weight(shape: LayerShape) -> np.ndarray:
    """W_r fp32 [E, d], entries ~ N(0, 1/d); row e from its own stream (the
    format-edge layer: column block b times 2^EDGE_XEXP[b])."""
    w = np.empty((shape.E, shape.d), dtype=np.float32)
    sd = 1.0 / math.sqrt(shape.d)
    for e in range(shape.E):
        row = rng(shape.layer, T_ROUTER, e).standard_normal(shape.d) * sd
        if shape.fmt == "edge":
            row = np.ldexp(row, _edge_col_exp(shape))
        w[e] = row.astype(np.float32)
    return w


def token(shape: LayerShape, index: int) -> np.ndarray:
    """One activation row, fp32 [d], entries ~ N(0, 1) (the format-edge
    layer: column block b times 2^-EDGE_XEXP[b])."""
    v = rng(shape.layer, T_X, index).standard_normal(shape.d)
    if shape.fmt == "edge":
        v = np.ldexp(v, -_edge_col_exp(shape))
    return v.astype(np.float32)


def tokens(shape: LayerShape, T: int, first: int = 0) -> np.ndarray:
    return np.stack([token(shape, first + t) for t in range(T)]) if T else np.zeros((0, shape.d), np.float32)


def zipf_bias(shape: LayerShape) -> np.ndarray:
    """Per-expert bias 2.0 * ln(1 / rank^1.1) over a seeded random ranking
    (rank 1..E), computed in fp64 and stored fp32: a few experts draw most
    tokens."""
    perm = rng(shape.layer, T_RANKING, 0).permutation(shape.E)
    rank = np.empty(shape.E, dtype=np.float64)
    rank[perm] = np.arange(1, shape.E + 1, dtype=np.float64)
    return (2.0 * np.log(1.0 / rank ** 1.1)).astype(np.float32)


_MATS = {  # which: (codes tensor id, scales tensor id, rows, cols) as functions of the shape
    "gate": (T_GATE_CODES, T_GATE_SCALES, "f", "d"),
    "up": (T_UP_CODES, T_UP_SCALES, "f", "d"),
    "down": (T_DOWN_CODES, T_DOWN_SCALES, "d", "f"),
}


def expert_matrix(shape: LayerShape, e: int, which: str):
    """One MX matrix of expert e: (codes u8 [rows, cols/2], scales u8
    [rows, cols/32]).  Codes are uniform bytes (every 4-bit code equally
    likely, including -0); scale bytes uniform in [120, 124]."""
    tc, ts, r, c = _MATS[which]
    rows, cols = getattr(shape, r), getattr(shape, c)
    codes = rng(shape.layer, tc, e).integers(0, 256, size=(rows, cols // 2), dtype=np.uint8)
    if shape.fmt == "edge":
        return _edge_matrix(shape, e, which, codes)
    scales = rng(shape.layer, ts, e).integers(SCALE_LO, SCALE_HI + 1, size=(rows, cols // 32), dtype=np.uint8)
    return codes, scales


def _edge_matrix(shape: LayerShape, e: int, which: str, codes: np.ndarray):
    """Scale bytes of the format-edge layer (clipped to 0..252):
    gate/up [r][b] = 127 + EDGE_XEXP[b] + EDGE_OEXP[r // 32] + U{-2..2};
    down    [c][b] = 128 - 2 EDGE_OEXP[b] + U{-28..28}.
    Then 5 % of the blocks get all-zero codes and 5 % all -0 codes (byte
    0x88), and the first blocks of each kind carry the scale bytes
    EDGE_ZERO_BYTES."""
    r = rng(shape.layer, T_EDGE, 8 * e + ("gate", "up", "down").index(which))
    rows, nb = codes.shape[0], codes.shape[1] // 16
    if which == "down":
        base = 128 - 2 * EDGE_OEXP[None, :]
        jit = r.integers(-28, 29, size=(rows, nb))
    else:
        base = 127 + EDGE_XEXP[None, :] + EDGE_OEXP[np.arange(rows) // 32][:, None]
        jit = r.integers(-2, 3, size=(rows, nb))
    scales = np.clip(base + jit, 0, 252).astype(np.uint8)
    kind = r.random((rows, nb))
    blocks = codes.reshape(rows, nb, 16)
    blocks[kind < 0.05] = 0x00
    blocks[(kind >= 0.05) & (kind < 0.10)] = 0x88
    for sel in (kind < 0.05, (kind >= 0.05) & (kind < 0.10)):
        rr, bb = np.nonzero(sel)
        n = min(len(rr), len(EDGE_ZERO_BYTES))
        scales[rr[:n], bb[:n]] = EDGE_ZERO_BYTES[:n]
    return codes, scales


def expert(shape: LayerShape, e: int) -> dict:
    return {w: expert_matrix(shape, e, w) for w in ("gate", "up", "down")}


def all_experts_host(shape: LayerShape, threads: int = 8) -> dict:
    """Every expert's matrices stacked: {which: (codes [E, rows, cols/2],
    scales [E, rows, cols/32])}.  Only for small shapes (the full layer is
    21 GB; use ``upload_experts`` for that)."""
    out = {}
    for which in ("gate", "up", "down"):
        _, _, r, c = _MATS[which]
        rows, cols = getattr(shape, r), getattr(shape, c)
        codes = np.empty((shape.E, rows, cols // 2), np.uint8)
        scales = np.empty((shape.E, rows, cols // 32), np.uint8)

        def fill(e, which=which, codes=codes, scales=scales):
            codes[e], scales[e] = expert_matrix(shape, e, which)

        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(fill, range(shape.E)))
        out[which] = (codes, scales)
    return out


def upload_experts(shape: LayerShape, device, threads: int = 16, experts=None) -> dict:
    """Generate every expert on the host, expert by expert in a thread pool,
    and copy each into preallocated device tensors.  Returns {which: (codes,
    scales)} as torch uint8 tensors on ``device`` with shapes
    [E, rows, cols/2] and [E, rows, cols/32].  ``experts`` optionally limits
    generation to a subset (the rest stay zero)."""
    import torch

    out = {}
    for which in ("gate", "up", "down"):
        _, _, r, c = _MATS[which]
        rows, cols = getattr(shape, r), getattr(shape, c)
        out[which] = (torch.zeros((shape.E, rows, cols // 2), dtype=torch.uint8, device=device),
                      torch.zeros((shape.E, rows, cols // 32), dtype=torch.uint8, device=device))
    ids = range(shape.E) if experts is None else sorted(set(int(e) for e in experts))

    def job(e):
        return e, expert(shape, e)

    ids = list(ids)
    with ThreadPoolExecutor(threads) as ex:
        for c0 in range(0, len(ids), 2 * threads):  # bounded host memory
            for e, mats in ex.map(job, ids[c0:c0 + 2 * threads]):
                for which, (cd, sc) in mats.items():
                    out[which][0][e].copy_(torch.from_numpy(cd))
                    out[which][1][e].copy_(torch.from_numpy(sc))
    return out
