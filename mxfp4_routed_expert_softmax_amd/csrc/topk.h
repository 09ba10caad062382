// topk.h -- top-k of one token's fp64 router logits for gfx950 wave64, by a
// whole block: bitonic lists, then one ranking step.  Internal to the HIP
// library.
//
// The selection is the pages' router choice (fiv.co.kr "kimi-k3-in-c deep
// dive", study-plan row "MoE and routing"): the k largest keys, ties to the
// lower expert index, listed by descending key; the weights are the softmax
// over the chosen weight-logits (equal to the full softmax restricted to the
// selection and renormalised).
#pragma once
#include <float.h>
#include "device_common.h"

namespace k3 {

constexpr int kTopkLists = 16;  // E <= 1024: 64 experts per list

// (key, id) order: larger key first, ties to the lower id.  A slot without
// a candidate holds (-inf, INT_MAX) and so sorts after every expert, whose
// id is smaller, even one whose key is -inf.
constexpr int kNoId = 0x7fffffff;

__device__ __forceinline__ bool before(double ka, int ia, double kb, int ib)
{
    // bitwise, not short-circuit: both tests are cheap and a branch per
    // compare-exchange would cost more than them
    return (ka > kb) | ((ka == kb) & (ia < ib));
}

// The value of lane L ^ J.  Inside a 16-lane row the exchange stays on the
// vector unit (DPP; every source lane is inside the row, so no lane takes
// the bound-control zero): J = 1, 2 are quad permutations; J = 4 is a
// half-row mirror (L -> L ^ 7 within 8) followed by a quad reversal
// (L -> L ^ 3); J = 8 is a rotation of the row by 8.  J = 16 and 32 cross
// rows and go through the LDS crossbar.
template <int J>
__device__ __forceinline__ int xchg(int v)
{
    if (J == 1) return __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, true);  // quad_perm [1,0,3,2]
    if (J == 2) return __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, true);  // quad_perm [2,3,0,1]
    if (J == 4) {
        const int m = __builtin_amdgcn_mov_dpp(v, 0x141, 0xF, 0xF, true);  // row_half_mirror
        return __builtin_amdgcn_mov_dpp(m, 0x1B, 0xF, 0xF, true);          // quad_perm [3,2,1,0]
    }
    if (J == 8) return __builtin_amdgcn_mov_dpp(v, 0x128, 0xF, 0xF, true);  // row_ror:8
    if (J < 32) return __builtin_amdgcn_ds_swizzle(v, (J << 10) | 0x1F);
    return __builtin_amdgcn_ds_bpermute(((int)(threadIdx.x & 63) ^ 32) << 2, v);
}

// one compare-exchange step: lanes L and L^J; the lower lane of an
// ascending block keeps the element that comes first
template <int J>
__device__ __forceinline__ void bitonic_step(double& k, int& id, bool asc)
{
    const int lane = threadIdx.x & 63;
    int lo = __double2loint(k), hi = __double2hiint(k);
    int plo = xchg<J>(lo), phi = xchg<J>(hi), pid = xchg<J>(id);
    const double pk = __hiloint2double(phi, plo);
    const bool lower = (lane & J) == 0;
    // the partner's element moves here when it belongs in this lane: it
    // comes first and this is the front lane of the pair, or the reverse
    const bool take = before(pk, pid, k, id) == (lower == asc);
    k = take ? pk : k;
    id = take ? pid : id;
}

template <int S>
__device__ __forceinline__ void bitonic_stage(double& k, int& id)
{
    const bool asc = ((threadIdx.x & 63) & S) == 0 || S == 64;
    if (S > 32) bitonic_step<32>(k, id, asc);
    if (S > 16) bitonic_step<16>(k, id, asc);
    if (S > 8) bitonic_step<8>(k, id, asc);
    if (S > 4) bitonic_step<4>(k, id, asc);
    if (S > 2) bitonic_step<2>(k, id, asc);
    bitonic_step<1>(k, id, asc);
}

__device__ __forceinline__ void bitonic_sort64(double& k, int& id)
{
    bitonic_stage<2>(k, id);
    bitonic_stage<4>(k, id);
    bitonic_stage<8>(k, id);
    bitonic_stage<16>(k, id);
    bitonic_stage<32>(k, id);
    bitonic_stage<64>(k, id);
}

// The pages' router score: a sigmoid of the logit, in the form that never
// overflows (1/(1+e^-l) for l >= 0, e^l/(1+e^l) below), fp64.
__device__ __forceinline__ double sigmoid_f64(double l)
{
    if (l >= 0.0) return 1.0 / (1.0 + exp(-l));
    const double el = exp(l);
    return el / (1.0 + el);
}

// Selection key of one expert: the score (logit, or its sigmoid) plus the
// selection-only bias.
__device__ __forceinline__ double topk_key(double l, const float* bias, int e, int bias_select_only, int sigmoid)
{
    double key = sigmoid ? sigmoid_f64(l) : l;
    if (bias_select_only) key += (double)bias[e];
    return key;
}

// fp64 value of lane L ^ J (J < 32)
template <int J>
__device__ __forceinline__ double xchg_f64(double v)
{
    return __hiloint2double(xchg<J>(__double2hiint(v)), xchg<J>(__double2loint(v)));
}

// Butterflies over the lanes of each half-wave: every lane of lanes 0..31
// ends with the max / the sum over lanes 0..31, in a fixed order.
__device__ __forceinline__ double half_max_f64(double v)
{
    v = fmax(v, xchg_f64<16>(v));
    v = fmax(v, xchg_f64<8>(v));
    v = fmax(v, xchg_f64<4>(v));
    v = fmax(v, xchg_f64<2>(v));
    return fmax(v, xchg_f64<1>(v));
}

__device__ __forceinline__ double half_sum_f64(double v)
{
    v += xchg_f64<16>(v);
    v += xchg_f64<8>(v);
    v += xchg_f64<4>(v);
    v += xchg_f64<2>(v);
    return v + xchg_f64<1>(v);
}

// The k <= 32 winners held by lanes 0..k-1 of one (whole) wave, in order
// (my_e, with its weight-logit wl): their weights -- softmax over the
// selected weight-logits, or (sigmoid) their sigmoid scores renormalised --
// and the outputs (each may be null).  max_first: lane 0's weight-logit is
// the largest (the keys were the weight-logits themselves), so the softmax
// maximum needs no reduction.
__device__ __forceinline__ void topk_finish(int k, int my_e, double wl, int sigmoid, bool max_first,
                                            int* sel_e_out, int32_t* idx_out, float* w_out)
{
    const int lane = threadIdx.x & 63;
    double ex;
    if (sigmoid) {
        ex = (lane < k) ? sigmoid_f64(wl) : 0.0;
    } else {
        double mx;
        if (max_first)
            mx = __hiloint2double(__builtin_amdgcn_readfirstlane(__double2hiint(wl)),
                                  __builtin_amdgcn_readfirstlane(__double2loint(wl)));
        else
            mx = half_max_f64((lane < k) ? wl : -DBL_MAX);
        ex = (lane < k) ? exp(wl - mx) : 0.0;
    }
    const double sum = half_sum_f64(ex);
    if (lane < k) {
        if (idx_out) idx_out[lane] = my_e;
        if (w_out) w_out[lane] = (float)(ex / sum);
        if (sel_e_out) sel_e_out[lane] = my_e;
    }
}

// LDS of block_topk_token: the best KL entries of up to 16 sorted lists,
// then the k winners in order.  An entry is one 16-byte record, read with a
// single LDS load.
struct __attribute__((aligned(16))) TopkEntry {
    double key;
    int id;
    int pad;
};
struct TopkLists {
    TopkEntry list[kTopkLists][32];
    TopkEntry win[32];
    double cmax[kTopkLists];  // certification: per-list max of the bound factors
    int ok;
};

// The rank of every kept entry among all kept entries: its position in its
// own sorted list plus, for every other list, how many of that list's KL
// entries come before it -- a binary search, since the entries that come
// before it form a prefix of the sorted list.  Lane (group g, slot p) of
// wave w holds entry p of list w and searches lists g, g + G, ...; the
// groups' counts are then summed.  An entry of the overall top k is in the
// top KL of its list, and so is every entry that beats it: its rank among
// the kept entries is its rank among all experts.  Entries ranked below k
// are written to L.win in rank order.
template <int KL>
__device__ __forceinline__ void rank_winners(int nl, int k, TopkLists& L)
{
    constexpr int G = 64 / KL;            // lane groups per wave
    constexpr int MAXL = kTopkLists / G;  // lists each group searches
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int pos = lane % KL, grp = lane / KL;
    const TopkEntry c = L.list[wave][pos];
    int cnt[MAXL];
    bool live[MAXL];
    int src[MAXL];
#pragma unroll
    for (int j = 0; j < MAXL; ++j) {
        const int l = grp + G * j;
        live[j] = l < nl && l != wave;
        src[j] = live[j] ? l : 0;  // a harmless in-range list when idle
        cnt[j] = 0;
    }
#pragma unroll
    for (int st = KL / 2; st >= 1; st >>= 1) {
#pragma unroll
        for (int j = 0; j < MAXL; ++j) {
            const TopkEntry t = L.list[src[j]][cnt[j] + st - 1];
            cnt[j] += before(t.key, t.id, c.key, c.id) ? st : 0;
        }
    }
    int r = grp == 0 ? pos : 0;
#pragma unroll
    for (int j = 0; j < MAXL; ++j) {
        const TopkEntry t = L.list[src[j]][cnt[j]];  // cnt <= KL - 1 here
        const int n = cnt[j] + (before(t.key, t.id, c.key, c.id) ? 1 : 0);
        r += live[j] ? n : 0;
    }
    if (G == 4) r += __builtin_amdgcn_ds_swizzle(r, (16 << 10) | 0x1F);
    r += __builtin_amdgcn_ds_bpermute((lane ^ 32) << 2, r);
    if (grp == 0 && r < k) L.win[r] = c;
}

// Top-k of one token by a whole block of at least E/64 waves: the experts
// fall in lists of 64; each list is sorted by a 64-lane bitonic network
// (DPP / swizzle exchanges) and its best KL (>= the winners needed) are
// kept; one ranking step (rank_winners) then orders the winners.  Wave 0
// writes the k winners in order to sel_e_out (LDS, may be null), idx_out and
// w_out (global, may be null).  Ends with a block barrier.
//
// Certified form (wc non-null, k < E): the keys are approximations, key e
// within xscale * wc[e] of the exact one; with bound = xscale * max_e wc[e]
// the selection is kept only if every gap among the best k + 1 keys exceeds
// twice the bound (and a relative 2^-40 for the fp64 rounding of the keys
// themselves) -- then the exact keys have the same winners in the same
// order.  Otherwise nothing is written and false comes back (block-uniform).
// The (k+1)-th key, for k <= 16 with 16 entries kept per list: it is either
// kept (and then ranked k among the kept entries) or it is entry 16 of its
// list (all k winners came from that list), so it is the best of the kept
// rank-k entry and every list's entry 16.
__device__ __forceinline__ bool block_topk_token(int E, int k, const double* __restrict__ lrow,
                                                 const float* __restrict__ bias, int bias_select_only, int sigmoid,
                                                 TopkLists& L, int* sel_e_out, int32_t* idx_out, float* w_out,
                                                 const double* __restrict__ wc = nullptr, double xscale = 0.0)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const bool cert = wc != nullptr;
    const int KL = k <= 16 ? 16 : 32;
    const int nk = cert ? k + 1 : k;      // ranks written to L.win
    const bool extra = cert && KL == 16;  // entry 16 of every list kept too
    const int nl = (E + 63) / 64;  // <= waves (E <= 64 * waves): list w is wave w's
    if (wave < nl) {
        const int e = 64 * wave + lane;
        double key = -__builtin_inf();
        int id = kNoId;
        double c = 0.0;
        if (e < E) {
            key = topk_key(lrow[e], bias, e, bias_select_only, sigmoid);
            id = e;
            if (cert) c = wc[e];
        }
        bitonic_sort64(key, id);
        if (lane < KL + (extra ? 1 : 0)) L.list[wave][lane] = TopkEntry{key, id, 0};
        if (cert) {
            c = half_max_f64(c);
            c = fmax(c, xchg_f64<32>(c));
            if (lane == 0) L.cmax[wave] = c;
        }
    }
    if (cert && threadIdx.x == 0) L.win[k] = TopkEntry{-__builtin_inf(), kNoId, 0};
    __syncthreads();
    if (wave < nl) {
        if (KL == 16)
            rank_winners<16>(nl, nk, L);
        else
            rank_winners<32>(nl, nk, L);
    }
    __syncthreads();
    bool ok = true;
    if (wave == 0) {
        const TopkEntry w = L.win[lane & 31];
        if (cert) {
            // lanes 0..15: the bound, and the best candidate for the (k+1)-th key
            double c = lane < nl ? L.cmax[lane] : 0.0;
            TopkEntry nx = (extra && lane < nl) ? L.list[lane][16] : TopkEntry{-__builtin_inf(), kNoId, 0};
            if (lane == 0 && before(L.win[k].key, L.win[k].id, nx.key, nx.id)) nx = L.win[k];
#define K3_NEXT_STEP(J)                                                 \
    {                                                                   \
        c = fmax(c, xchg_f64<J>(c));                                    \
        const double pk = xchg_f64<J>(nx.key);                          \
        const int pid = xchg<J>(nx.id);                                 \
        const bool tk = before(pk, pid, nx.key, nx.id);                 \
        nx.key = tk ? pk : nx.key;                                      \
        nx.id = tk ? pid : nx.id;                                       \
    }
            K3_NEXT_STEP(8)
            K3_NEXT_STEP(4)
            K3_NEXT_STEP(2)
            K3_NEXT_STEP(1)
#undef K3_NEXT_STEP
            const double bound = xscale * __shfl(c, 0, 64);
            const double nxk = __shfl(nx.key, 0, 64);
            const double b = __shfl(w.key, (lane + 1) & 63, 64);  // key of winner lane + 1
            const double bb = lane + 1 < k ? b : nxk;
            const bool bad = (lane < k) & !(w.key - bb > 2.0 * bound + 0x1p-40 * (fabs(w.key) + fabs(bb)));
            ok = __ballot(bad) == 0;
            if (lane == 0) L.ok = ok ? 1 : 0;
        }
        if (ok) {
            // softmax without a selection-only bias: the key is the weight-logit itself
            const int my_e = (lane < k) ? w.id : 0;
            const double wl = (lane < k) ? ((bias_select_only || sigmoid) ? lrow[my_e] : w.key) : 0.0;
            topk_finish(k, my_e, wl, sigmoid, !(bias_select_only || sigmoid), sel_e_out, idx_out, w_out);
        }
    }
    __syncthreads();
    return cert ? L.ok != 0 : true;
}

}  // namespace k3
