// topk.h -- top-k of one token's fp64 router logits for gfx950 wave64, by a
// whole block (bitonic lists and merges) or by one wave (k rounds of a wave
// argmax).  Internal to the HIP library.
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

constexpr int kCoopMaxT = 8;  // tokens per batch up to which a block cooperates per token
constexpr int kTopkLists = 16;  // E <= 1024: 64 experts per list

// (key, id) order: larger key first, ties to the lower id; id INT_MAX is
// "no candidate" and sorts last.
__device__ __forceinline__ bool before(double ka, int ia, double kb, int ib)
{
    if (ia == 0x7fffffff) return false;
    if (ib == 0x7fffffff) return true;
    return ka > kb || (ka == kb && ia < ib);
}

template <int J>
__device__ __forceinline__ int xchg(int v)
{
    if (J == 1) return __builtin_amdgcn_update_dpp(v, v, 0xB1, 0xF, 0xF, false);  // quad_perm [1,0,3,2]
    if (J == 2) return __builtin_amdgcn_update_dpp(v, v, 0x4E, 0xF, 0xF, false);  // quad_perm [2,3,0,1]
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
    double pk = __hiloint2double(phi, plo);
    const bool lower = (lane & J) == 0;
    const bool mine_first = before(k, id, pk, pid);
    const bool keep_mine = (lower == asc) ? mine_first : !mine_first;
    if (!keep_mine) {
        k = pk;
        id = pid;
    }
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

// The k winners held by lanes 0..k-1 of one wave, in order (my_e, with its
// weight-logit wl): their weights -- softmax over the selected
// weight-logits, or (sigmoid) their sigmoid scores renormalised; a fixed
// butterfly for the max and the sum -- and the outputs (each may be null).
__device__ __forceinline__ void topk_finish(int k, int my_e, double wl, int sigmoid, int* sel_e_out,
                                            int32_t* idx_out, float* w_out)
{
    const int lane = threadIdx.x & 63;
    double ex;
    if (sigmoid) {
        ex = (lane < k) ? sigmoid_f64(wl) : 0.0;
    } else {
        double mx = (lane < k) ? wl : -DBL_MAX;
        for (int m = 32; m >= 1; m >>= 1) mx = fmax(mx, __shfl_xor(mx, m, 64));
        ex = (lane < k) ? exp(wl - mx) : 0.0;
    }
    double sum = ex;
    for (int m = 32; m >= 1; m >>= 1) sum += __shfl_xor(sum, m, 64);
    if (lane < k) {
        if (idx_out) idx_out[lane] = my_e;
        if (w_out) w_out[lane] = (float)(ex / sum);
        if (sel_e_out) sel_e_out[lane] = my_e;
    }
}

// LDS of block_topk_token: two banks of up to 16 sorted lists of 32 slots
// (the merge tree reads one bank and writes the other).
struct TopkLists {
    double key[2][kTopkLists][32];
    int id[2][kTopkLists][32];
};

// Top-k of one token by a whole block of at least E/64 waves: the experts
// fall in lists of 64; each list is sorted by a 64-lane bitonic network
// (DPP / swizzle exchanges) and its best KL (>= k) are kept; a tree of
// pairwise bitonic merges reduces the lists to one.  Wave 0 then writes the
// k winners in order to sel_e_out (LDS, may be null), idx_out and w_out
// (global, may be null).  Ends with a block barrier.
__device__ __forceinline__ void block_topk_token(int E, int k, const double* __restrict__ lrow,
                                                 const float* __restrict__ bias, int bias_select_only, int sigmoid,
                                                 TopkLists& L, int* sel_e_out, int32_t* idx_out, float* w_out)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
    const int KL = k <= 16 ? 16 : 32;
    int nl = (E + 63) / 64;  // <= nw lists (E <= 64 * waves): list w is wave w's
    if (wave < nl) {
        const int e = 64 * wave + lane;
        double key = 0.0;
        int id = 0x7fffffff;
        if (e < E) {
            key = topk_key(lrow[e], bias, e, bias_select_only, sigmoid);
            id = e;
        }
        bitonic_sort64(key, id);
        if (lane < KL) {
            L.key[0][wave][lane] = key;
            L.id[0][wave][lane] = id;
        }
    }
    __syncthreads();
    int bank = 0;
    while (nl > 1) {
        const int half = (nl + 1) / 2;
        for (int m = wave; m < half; m += nw) {
            // lanes [0, KL): list 2m ascending; lanes [KL, 2KL): list 2m+1 reversed
            const int a = 2 * m, b = 2 * m + 1;
            double mk = 0.0;
            int mid = 0x7fffffff;
            if (lane < KL) {
                mk = L.key[bank][a][lane];
                mid = L.id[bank][a][lane];
            } else if (lane < 2 * KL && b < nl) {
                mk = L.key[bank][b][2 * KL - 1 - lane];
                mid = L.id[bank][b][2 * KL - 1 - lane];
            }
            // bitonic merge of the 2*KL lanes (ascending everywhere)
            if (KL == 32) bitonic_step<32>(mk, mid, true);
            bitonic_step<16>(mk, mid, true);
            bitonic_step<8>(mk, mid, true);
            bitonic_step<4>(mk, mid, true);
            bitonic_step<2>(mk, mid, true);
            bitonic_step<1>(mk, mid, true);
            if (lane < KL) {
                L.key[bank ^ 1][m][lane] = mk;
                L.id[bank ^ 1][m][lane] = mid;
            }
        }
        __syncthreads();
        bank ^= 1;
        nl = half;
    }
    if (wave == 0) {
        // softmax without a selection-only bias: the sorted key is the weight-logit itself
        const int my_e = (lane < k) ? L.id[bank][0][lane] : 0;
        const double wl =
            (lane < k) ? ((bias_select_only || sigmoid) ? lrow[my_e] : L.key[bank][0][lane]) : 0.0;
        topk_finish(k, my_e, wl, sigmoid, sel_e_out, idx_out, w_out);
    }
    __syncthreads();
}

// Top-k of one token held by one wave (sel_e_out, idx_out, w_out may be
// null): lane l owns experts l, l+64, ...
// (E <= 1024 -> at most 16 per lane).  k rounds of a wave-wide
// (key max, index min) reduction; the winning lane retires its entry.  The
// weight logits of the k winners are read back at the end (they equal the
// keys unless the bias steers the selection only).
constexpr int kMaxPerLane = 16;

// (key, expert) of the better candidate: larger key, ties to the lower id;
// be == INT_MAX marks "no candidate".
__device__ __forceinline__ bool better(double ok, int oe, double bk, int be)
{
    return (oe != 0x7fffffff) && (be == 0x7fffffff || ok > bk || (ok == bk && oe < be));
}

// One exchange step of the wave argmax through a DPP lane pattern (VALU
// latency, no LDS round trip).
template <int CTRL>
__device__ __forceinline__ void argmax_dpp(double& bk, int& be)
{
    int lo = __double2loint(bk), hi = __double2hiint(bk);
    int olo = __builtin_amdgcn_update_dpp(lo, lo, CTRL, 0xF, 0xF, false);
    int ohi = __builtin_amdgcn_update_dpp(hi, hi, CTRL, 0xF, 0xF, false);
    int oe = __builtin_amdgcn_update_dpp(be, be, CTRL, 0xF, 0xF, false);
    double ok = __hiloint2double(ohi, olo);
    if (better(ok, oe, bk, be)) {
        bk = ok;
        be = oe;
    }
}

// Wave-wide argmax: within each row of 16 lanes by DPP (quad swaps, then
// rotations by 4 and 8), then the four row winners compared as uniform values.
__device__ __forceinline__ void wave_argmax(double& bk, int& be)
{
    argmax_dpp<0xB1>(bk, be);   // quad_perm [1,0,3,2]
    argmax_dpp<0x4E>(bk, be);   // quad_perm [2,3,0,1]
    argmax_dpp<0x124>(bk, be);  // row_ror:4
    argmax_dpp<0x128>(bk, be);  // row_ror:8
    int lo = __double2loint(bk), hi = __double2hiint(bk);
    double rk = bk;
    int re = be;
    rk = __hiloint2double(__builtin_amdgcn_readlane(hi, 0), __builtin_amdgcn_readlane(lo, 0));
    re = __builtin_amdgcn_readlane(be, 0);
#pragma unroll
    for (int r = 1; r < 4; ++r) {
        double ok = __hiloint2double(__builtin_amdgcn_readlane(hi, 16 * r),
                                     __builtin_amdgcn_readlane(lo, 16 * r));
        int oe = __builtin_amdgcn_readlane(be, 16 * r);
        if (better(ok, oe, rk, re)) {
            rk = ok;
            re = oe;
        }
    }
    bk = rk;
    be = re;
}

__device__ __forceinline__ void wave_topk(int E, int k, const double* __restrict__ lrow,
                          const float* __restrict__ bias, int bias_select_only, int sigmoid,
                          int* sel_e_out, int32_t* idx_out, float* w_out)
{
    const int lane = threadIdx.x & 63;
    // branch-free loads (clamped index) so all of them are in flight at once
    double key[kMaxPerLane];
    uint32_t taken = 0;
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i) {
        const int e = lane + 64 * i;
        key[i] = lrow[min(e, E - 1)];
        if (e >= E) taken |= 1u << i;
    }
    if (sigmoid) {
#pragma unroll
        for (int i = 0; i < kMaxPerLane; ++i) key[i] = sigmoid_f64(key[i]);
    }
    if (bias_select_only) {
        float b[kMaxPerLane];
#pragma unroll
        for (int i = 0; i < kMaxPerLane; ++i) b[i] = bias[min(lane + 64 * i, E - 1)];
#pragma unroll
        for (int i = 0; i < kMaxPerLane; ++i) key[i] += (double)b[i];
    }
    int my_e = 0;
    for (int j = 0; j < k; ++j) {
        double bk = 0.0;
        int be = 0x7fffffff;
#pragma unroll
        for (int i = 0; i < kMaxPerLane; ++i) {
            // ascending expert id inside the lane: strict > keeps the lower id
            if (!((taken >> i) & 1u) && (be == 0x7fffffff || key[i] > bk)) {
                bk = key[i];
                be = lane + 64 * i;
            }
        }
        wave_argmax(bk, be);
        if ((be & 63) == lane) taken |= 1u << (be >> 6);
        if (lane == j) my_e = be;
    }
    topk_finish(k, my_e, (lane < k) ? lrow[my_e] : 0.0, sigmoid, sel_e_out, idx_out, w_out);
}

}  // namespace k3
