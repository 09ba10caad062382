// gemv.hip -- fp32-activation expert FFN on MXFP4 weights for gfx950:
// grouped gate/up GEMV with fused SwiGLU, grouped down GEMV, deterministic
// gate-weighted combine.
//
// Weights are consumed as packed 4-bit codes straight from HBM and decoded in
// registers, never expanded in memory (fiv.co.kr "kimi-k3-in-c deep dive",
// "four reductions", MXFP4 paragraph: multiply on the nibbles, because
// expanding would multiply the bytes moved; yunpan.plus section 02, direct
// MXFP4 computation).  Each active expert's rows are read once per step and
// applied to every token routed to it.
//
// Work mapping: a group of G lanes owns a few weight rows and splits the
// reduction axis; every lane streams one 32-element MX block (16 code bytes,
// one 128-bit load, plus its scale byte) per row per step, so a group reads
// G*16 contiguous bytes of each row per step.  The gfx950 scaled convert
// turns two codes into two fp32 values with the block's power-of-two scale
// applied, exactly.  Partial sums are reduced across the group by shuffles.
#include "device_common.h"
#include "kernels.h"

namespace k3 {

// Which expert does this block's slot serve?  Either the slot-th entry of the
// active list, or (no list) slot = a sorted row that must head its expert's
// segment.  Returns false for idle slots.
__device__ __forceinline__ bool slot_expert(const FfnArgs& a, int slot, int& e, int& r_beg, int& n_e)
{
    if (a.active) {
        if (slot >= a.active[a.E]) return false;
        e = a.active[slot];
    } else {
        if (slot >= a.P) return false;
        e = a.topk_idx[a.perm_pair[slot]];
        if (a.offsets[e] != slot) return false;
    }
    r_beg = a.offsets[e];
    n_e = a.offsets[e + 1] - r_beg;
    return n_e > 0;
}

// ---------------------------------------------------------------------------
// gate/up: block = 8 groups of 32 lanes; group g owns gate rows r0..r0+3 and
// the same up rows.  h[row][r] = silu(g_r) * u_r for every token row of the
// expert, TCH tokens per pass over the weights.
template <int TCH>
__global__ __launch_bounds__(256) void gateup_gemv_kernel(FfnArgs a, float* __restrict__ h)
{
    constexpr int R = 4;
    int e, r_beg, n_e;
    if (!slot_expert(a, blockIdx.y, e, r_beg, n_e)) return;
    const int lane = threadIdx.x & 31, grp = threadIdx.x >> 5;
    const int r0 = (blockIdx.x * 8 + grp) * R;
    if (r0 >= a.f) return;
    const int d = a.d, nb = d >> 5;
    const size_t crow = (size_t)(d >> 1), srow = (size_t)nb;
    const size_t wrow0 = (size_t)e * a.f + r0;
    const uint8_t* gcp = a.gc + wrow0 * crow;
    const uint8_t* ucp = a.uc + wrow0 * crow;
    const uint8_t* gsp = a.gs + wrow0 * srow;
    const uint8_t* usp = a.us + wrow0 * srow;

    for (int t0 = 0; t0 < n_e; t0 += TCH) {
        const float* xr[TCH];
#pragma unroll
        for (int tt = 0; tt < TCH; ++tt) {
            int m = min(t0 + tt, n_e - 1);
            int tok = a.perm_pair[r_beg + m] / a.k;
            xr[tt] = a.x + (size_t)tok * d;
        }
        float ag[TCH][R], au[TCH][R];
#pragma unroll
        for (int tt = 0; tt < TCH; ++tt)
#pragma unroll
            for (int i = 0; i < R; ++i) { ag[tt][i] = 0.f; au[tt][i] = 0.f; }

        for (int blk = lane; blk < nb; blk += 32) {
            uint4 qg[R], qu[R];
            float sg[R], su[R];
#pragma unroll
            for (int i = 0; i < R; ++i) {
                qg[i] = ldg16(gcp + i * crow + (size_t)blk * 16);
                qu[i] = ldg16(ucp + i * crow + (size_t)blk * 16);
                sg[i] = e8m0_f32(gsp[i * srow + blk]);
                su[i] = e8m0_f32(usp[i * srow + blk]);
            }
#pragma unroll
            for (int tt = 0; tt < TCH; ++tt) {
                if (t0 + tt < n_e) {
                    float xs[32];
                    load32f(xr[tt] + (size_t)blk * 32, xs);
#pragma unroll
                    for (int i = 0; i < R; ++i) {
                        ag[tt][i] = dot32_fp4(qg[i], sg[i], xs, ag[tt][i]);
                        au[tt][i] = dot32_fp4(qu[i], su[i], xs, au[tt][i]);
                    }
                }
            }
        }
#pragma unroll
        for (int tt = 0; tt < TCH; ++tt) {
            if (t0 + tt >= n_e) break;
#pragma unroll
            for (int i = 0; i < R; ++i) {
                float g = ag[tt][i], u = au[tt][i];
#pragma unroll
                for (int m = 16; m >= 1; m >>= 1) {
                    g += shfl_xor(g, m, 32);
                    u += shfl_xor(u, m, 32);
                }
                if (lane == i) h[(size_t)(r_beg + t0 + tt) * a.f + r0 + i] = silu_f32(g) * u;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// down: block = 16 groups of 16 lanes; group g owns down rows c0..c0+7.
// o[row][c] = Wd_e[c,:] . h[row] for every token row of the expert.
template <int TCH>
__global__ __launch_bounds__(256) void down_gemv_kernel(FfnArgs a, const float* __restrict__ h,
                                                        float* __restrict__ o)
{
    constexpr int R = 8;
    int e, r_beg, n_e;
    if (!slot_expert(a, blockIdx.y, e, r_beg, n_e)) return;
    const int lane = threadIdx.x & 15, grp = threadIdx.x >> 4;
    const int c0 = (blockIdx.x * 16 + grp) * R;
    if (c0 >= a.d) return;
    const int f = a.f, nb = f >> 5;
    const size_t crow = (size_t)(f >> 1), srow = (size_t)nb;
    const size_t wrow0 = (size_t)e * a.d + c0;
    const uint8_t* dcp = a.dc + wrow0 * crow;
    const uint8_t* dsp = a.ds + wrow0 * srow;

    for (int t0 = 0; t0 < n_e; t0 += TCH) {
        float acc[TCH][R];
#pragma unroll
        for (int tt = 0; tt < TCH; ++tt)
#pragma unroll
            for (int i = 0; i < R; ++i) acc[tt][i] = 0.f;
        for (int blk = lane; blk < nb; blk += 16) {
            uint4 q[R];
            float sc[R];
#pragma unroll
            for (int i = 0; i < R; ++i) {
                q[i] = ldg16(dcp + i * crow + (size_t)blk * 16);
                sc[i] = e8m0_f32(dsp[i * srow + blk]);
            }
#pragma unroll
            for (int tt = 0; tt < TCH; ++tt) {
                if (t0 + tt < n_e) {
                    float hs[32];
                    load32f(h + (size_t)(r_beg + t0 + tt) * f + (size_t)blk * 32, hs);
#pragma unroll
                    for (int i = 0; i < R; ++i) acc[tt][i] = dot32_fp4(q[i], sc[i], hs, acc[tt][i]);
                }
            }
        }
#pragma unroll
        for (int tt = 0; tt < TCH; ++tt) {
            if (t0 + tt >= n_e) break;
#pragma unroll
            for (int i = 0; i < R; ++i) {
                float v = acc[tt][i];
#pragma unroll
                for (int m = 8; m >= 1; m >>= 1) v += shfl_xor(v, m, 16);
                if (lane == i) o[(size_t)(r_beg + t0 + tt) * a.d + c0 + i] = v;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// y[t] = sum_j w[t,j] * o[row_of_pair[t*k+j]], j ascending (deterministic).
__global__ __launch_bounds__(256) void combine_kernel(FfnArgs a, const float* __restrict__ o,
                                                      float* __restrict__ y)
{
    const int t = blockIdx.x;
    const int c4 = blockIdx.y * 256 + threadIdx.x;
    const int d4 = a.d >> 2;
    if (c4 >= d4) return;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j = 0; j < a.k; ++j) {
        const int p = t * a.k + j;
        const float w = a.topk_w[p];
        const float4 v = reinterpret_cast<const float4*>(o + (size_t)a.row_of_pair[p] * a.d)[c4];
        acc.x = __builtin_fmaf(w, v.x, acc.x);
        acc.y = __builtin_fmaf(w, v.y, acc.y);
        acc.z = __builtin_fmaf(w, v.z, acc.z);
        acc.w = __builtin_fmaf(w, v.w, acc.w);
    }
    reinterpret_cast<float4*>(y + (size_t)t * a.d)[c4] = acc;
}

void launch_gateup_gemv(const FfnArgs& a, float* h, hipStream_t s)
{
    dim3 grid((a.f + 31) / 32, a.nslots);
    if (a.T == 1)
        gateup_gemv_kernel<1><<<grid, dim3(256), 0, s>>>(a, h);
    else
        gateup_gemv_kernel<4><<<grid, dim3(256), 0, s>>>(a, h);
}

void launch_down_gemv(const FfnArgs& a, const float* h, float* o, hipStream_t s)
{
    dim3 grid((a.d + 127) / 128, a.nslots);
    if (a.T == 1)
        down_gemv_kernel<1><<<grid, dim3(256), 0, s>>>(a, h, o);
    else
        down_gemv_kernel<4><<<grid, dim3(256), 0, s>>>(a, h, o);
}

void launch_combine(const FfnArgs& a, const float* o, float* y, hipStream_t s)
{
    dim3 grid(a.T, (a.d / 4 + 255) / 256);
    combine_kernel<<<grid, dim3(256), 0, s>>>(a, o, y);
}

}  // namespace k3
