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
// Work mapping (both GEMVs): the reduction axis is split over the lanes of a
// workgroup, one 32-element MX block per lane (BPL blocks if the axis is
// longer than the group), so each lane keeps its slice of the activation in
// registers for the whole kernel and no activation is re-read per row.  A
// wave then streams rows: per row a lane loads 16 code bytes (one 128-bit
// load; 64 lanes read 1 KB of the row contiguously) and one scale byte, and
// the gfx950 scaled convert turns two codes at a time into fp32 with the
// block's power-of-two scale applied exactly.  Sixteen rows are issued
// together, then reduced across the wave with a transposed shuffle
// reduction (17 swizzles for 16 rows) and, when several waves share a row,
// across waves through LDS in a fixed order -- deterministic sums.
#include "device_common.h"
#include "kernels.h"
#include "launch.h"
#include "slices.h"

namespace k3 {

// xor-swizzle inside 32-lane halves (ds_swizzle bitmask mode, no LDS access)
template <int M>
__device__ __forceinline__ float swz_xor(float v)
{
    static_assert(M > 0 && M < 32, "swizzle masks reach 31");
    return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), (M << 10) | 0x1F));
}

__device__ __forceinline__ float xor32(float v)
{
    const int lane = threadIdx.x & 63;
    return __int_as_float(__builtin_amdgcn_ds_bpermute((lane ^ 32) << 2, __float_as_int(v)));
}

// 16 partial sums per lane -> lane l holds the wave-wide sum of acc[l & 15].
// Step by step the lane whose bit is set keeps the upper half and sends the
// lower half to its partner; the order of additions is fixed.
// First step for the pair (acc[i], acc[i + 8]).
__device__ __forceinline__ float transpose_step8(float lo, float hi)
{
    const bool b3 = (threadIdx.x & 63) & 8;
    const float keep = b3 ? hi : lo, send = b3 ? lo : hi;
    return keep + swz_xor<8>(send);
}

// The remaining steps, from the eight first-step results.
__device__ __forceinline__ float wave_transpose_sum_from8(const float (&a8)[8])
{
    const int lane = threadIdx.x & 63;
    float a4[4], a2[2];
    const bool b2 = lane & 4, b1 = lane & 2, b0 = lane & 1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float keep = b2 ? a8[i + 4] : a8[i], send = b2 ? a8[i] : a8[i + 4];
        a4[i] = keep + swz_xor<4>(send);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        float keep = b1 ? a4[i + 2] : a4[i], send = b1 ? a4[i] : a4[i + 2];
        a2[i] = keep + swz_xor<2>(send);
    }
    float keep = b0 ? a2[1] : a2[0], send = b0 ? a2[0] : a2[1];
    float s = keep + swz_xor<1>(send);
    s += swz_xor<16>(s);
    s += xor32(s);
    return s;
}

__device__ __forceinline__ float wave_transpose_sum16(const float (&acc)[16])
{
    float a8[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) a8[i] = transpose_step8(acc[i], acc[i + 8]);
    return wave_transpose_sum_from8(a8);
}

// Which expert does this block's slot serve?  Either the slot-th entry of the
// active list, or (no list) slot = a grouped row that must head its expert's
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

// Load the lane's activation slice (BPL blocks of 32) of one row, zeros past
// the end of the reduction axis.
template <int BPL>
__device__ __forceinline__ void load_act(const float* row, int blk0, int stride_blk, int nb,
                                         float (&xr)[BPL][32])
{
#pragma unroll
    for (int b = 0; b < BPL; ++b) {
        int blk = blk0 + b * stride_blk;
        if (blk < nb) {
            load32f(row + (size_t)blk * 32, xr[b]);
        } else {
#pragma unroll
            for (int i = 0; i < 32; ++i) xr[b][i] = 0.f;
        }
    }
}

// Make the compiler treat v as redefined here: stops loop-invariant code
// motion from hoisting the decode of a weight block out of a token loop
// (which would keep every decoded value of a batch live at once).
__device__ __forceinline__ void opaque(uint4& v)
{
    asm volatile("" : "+v"(v.x), "+v"(v.y), "+v"(v.z), "+v"(v.w));
}

// acc[tt] += (one 32-element MX block: 16 code bytes q, scale sc) . xs[tt][0..31]
// for TCH token rows; every code pair is decoded once and used by all rows.
template <int TCH>
__device__ __forceinline__ void dot32_multi(uint4 q, float sc, const float (&xs)[TCH][32], float (&acc)[TCH])
{
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        f32x2 p0 = fp4x2_scaled<0>(w[k], sc);
        f32x2 p1 = fp4x2_scaled<1>(w[k], sc);
        f32x2 p2 = fp4x2_scaled<2>(w[k], sc);
        f32x2 p3 = fp4x2_scaled<3>(w[k], sc);
#pragma unroll
        for (int tt = 0; tt < TCH; ++tt) {
            const float* x = xs[tt] + 8 * k;
            float s = acc[tt];
            s = __builtin_fmaf(p0.x, x[0], s);
            s = __builtin_fmaf(p0.y, x[1], s);
            s = __builtin_fmaf(p1.x, x[2], s);
            s = __builtin_fmaf(p1.y, x[3], s);
            s = __builtin_fmaf(p2.x, x[4], s);
            s = __builtin_fmaf(p2.y, x[5], s);
            s = __builtin_fmaf(p3.x, x[6], s);
            s = __builtin_fmaf(p3.y, x[7], s);
            acc[tt] = s;
        }
    }
}

// ---------------------------------------------------------------------------
// Partial sums of a batch: acc[tt * R + i] = row i of the batch for token tt,
// R = 16 / TCH rows per batch, so one transposed reduction serves the batch.

// gate/up.  Block = 4 waves; the 256 lanes split the d axis (lane = block,
// BPL blocks per lane).  The block walks kGuRows row pairs of one expert in
// batches of R rows (R/2 gate rows + the same R/2 up rows); each wave reduces
// a batch with one transposed reduction and parks the sums in LDS; one
// fixed-order cross-wave sum per token pass gives g and u, and
// h = silu(g) * u is written per token row of the expert.
constexpr int kGuRows = 32;  // row pairs per block

// PAIR: the pair-major variant for small batches -- block y serves pair
// p = t*k + j alone (expert topk_idx[p], token t, h row p), no grouping.
// 4 waves per SIMD on the pair path: all four blocks a CU receives at
// d_model 7168 are resident at once.  The grouped form (token loop, expert
// lookups) does not fit 128 registers without spilling; it runs at 3 (its
// scratch traffic cost more than the fourth wave gains).
// SL (pair path only): h is written as its kSlices MX-FP8 slices (the
// block's 32 rows are exactly one 32-value block of h) instead of fp32.
// SEL (grouped path): kSelAll, or only the slots whose expert has exactly one
// token (kSelOne: with the token loop gone it fits 128 registers like the
// pair form and runs at four waves per SIMD), or only those with two or more
// (kSelMulti, two tokens per pass: four waves per SIMD with two registers
// spilled outside the row loop, 2.08 -> 2.03 ms at 64 tokens against three).
constexpr int kSelAll = 0, kSelOne = 1, kSelMulti = 2;

template <int TCH, int BPL, bool PAIR, bool SL = false, int SEL = kSelAll>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(
    BPL == 1 && TCH == 1 ? ((PAIR || SEL == kSelOne) ? 4 : 3) : (SEL == kSelMulti ? 4 : 1), 8)))
void gateup_gemv_kernel(FfnArgs a, float* __restrict__ h, uint8_t* __restrict__ hs_codes = nullptr,
                        uint8_t* __restrict__ hs_scales = nullptr)
{
    constexpr int R = 16 / TCH, HALF = R / 2;
    __shared__ float part[TCH][4][kGuRows * 2];  // [tt][wave][gate rows | up rows]
    int e, r_beg, n_e;
    if (PAIR) {
        r_beg = blockIdx.y;
        e = a.pair_w[r_beg];  // weight index (the expert, or its cache slot)
        n_e = 1;
    } else if (!slot_expert(a, blockIdx.y, e, r_beg, n_e)) {
        return;
    } else {
        if (SEL == kSelOne) {
            if (n_e != 1) return;
            n_e = 1;
        }
        if (SEL == kSelMulti && n_e < 2) return;
        e = wslot(a, e);
    }
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r0 = blockIdx.x * kGuRows;
    const int d = a.d, nb = d >> 5;
    const size_t crow = (size_t)(d >> 1), srow = (size_t)nb;
    const size_t wrow0 = (size_t)e * a.f + r0;
    const int npairs = min(kGuRows, a.f - r0);  // multiple of 8 (f % 32 == 0)
    const __amdgpu_buffer_rsrc_t rg = weight_rsrc(a.gc + wrow0 * crow);
    const __amdgpu_buffer_rsrc_t ru = weight_rsrc(a.uc + wrow0 * crow);
    const __amdgpu_buffer_rsrc_t rgs = weight_rsrc(a.gs + wrow0 * srow);
    const __amdgpu_buffer_rsrc_t rus = weight_rsrc(a.us + wrow0 * srow);
    uint32_t coff[BPL], soffl[BPL];
#pragma unroll
    for (int b = 0; b < BPL; ++b) {
        const int blk = tid + 256 * b;
        coff[b] = blk < nb ? (uint32_t)blk * 16u : kOff;
        soffl[b] = blk < nb ? (uint32_t)blk : kOff;
    }

    for (int t0 = 0; t0 < n_e; t0 += TCH) {
        float xr[BPL][TCH][32];
#pragma unroll
        for (int tt = 0; tt < TCH; ++tt) {
            int m = min(t0 + tt, n_e - 1);
            int tok = (PAIR ? r_beg : a.perm_pair[r_beg + m]) / a.k;
            float tmp[BPL][32];
            load_act<BPL>(a.x + (size_t)tok * d, tid, 256, nb, tmp);
#pragma unroll
            for (int b = 0; b < BPL; ++b)
#pragma unroll
                for (int i = 0; i < 32; ++i) xr[b][tt][i] = tmp[b][i];
        }
        for (int pb = 0; pb < npairs; pb += HALF) {
            uint4 q[R][BPL];
            uint32_t sb[R][BPL];
#pragma unroll
            for (int i = 0; i < R; ++i) {
                const uint32_t row = (uint32_t)(pb + (i % HALF));
#pragma unroll
                for (int b = 0; b < BPL; ++b) {
                    q[i][b] = ld_stream(i < HALF ? rg : ru, coff[b], row * (uint32_t)crow);
                    sb[i][b] = ld_scale(i < HALF ? rgs : rus, soffl[b], row * (uint32_t)srow);
                }
            }
            float acc[16];
#pragma unroll
            for (int i = 0; i < R; ++i) {
                float s[TCH];
#pragma unroll
                for (int tt = 0; tt < TCH; ++tt) s[tt] = 0.f;
#pragma unroll
                for (int b = 0; b < BPL; ++b) dot32_multi<TCH>(q[i][b], e8m0_f32(sb[i][b]), xr[b], s);
#pragma unroll
                for (int tt = 0; tt < TCH; ++tt) acc[tt * R + i] = s[tt];
            }
            const float v = wave_transpose_sum16(acc);
            if (lane < 16) {
                const int tt = lane / R, i = lane % R;
                // gate row pb + i -> slot pb + i; up row pb + i - HALF -> kGuRows + pb + i - HALF
                part[tt][wave][i < HALF ? pb + i : kGuRows + pb + i - HALF] = v;
            }
        }
        __syncthreads();
        if (SL) {  // PAIR, TCH == 1, npairs == 32: half-wave 0 holds one MX block of h
            static_assert(!SL || (PAIR && TCH == 1), "slices output is a pair-path option");
            if (tid < 32) {
                float g = 0.f, u = 0.f;
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    g += part[0][w][tid];
                    u += part[0][w][kGuRows + tid];
                }
                uint32_t code[kSlices], sbyte[kSlices];
                split_block(silu_f32(g) * u, code, sbyte);
                store_block(tid, r0 >> 5, a.f, hs_codes + (size_t)r_beg * kSlices * a.f,
                            hs_scales + (size_t)r_beg * kSlices * (a.f >> 5), code, sbyte);
            }
            continue;  // one token pass: the loop ends here
        }
        // fixed-order cross-wave sum; thread (tt, r) finishes row r of token tt
        for (int i = tid; i < TCH * npairs; i += 256) {
            const int tt = i / npairs, r = i - tt * npairs;
            if (t0 + tt < n_e) {
                float g = 0.f, u = 0.f;
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    g += part[tt][w][r];
                    u += part[tt][w][kGuRows + r];
                }
                h[(size_t)(r_beg + t0 + tt) * a.f + r0 + r] = silu_f32(g) * u;
            }
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// down.  Block = 4 waves; NK waves split the f axis (one block per lane, BPL
// per lane beyond 64*NK blocks), 4/NK teams of waves take different rows.
// Each team owns kDnRows rows of the expert, walked in batches of R rows;
// the weights of a batch are loaded once and applied to every token pass
// (their scale bytes kept four to a register, and partial sums paired by the
// first reduction step as they appear, so the d_ff = 2048 form fits 128
// registers: four waves per SIMD without spilling).
constexpr int kDnRows = 16;  // rows per team

template <int TCH, int NK, int BPL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(TCH == 1 && NK == 1 && BPL == 1 ? 4 : 1, 8)))
void down_gemv_kernel(FfnArgs a, const float* __restrict__ hbuf,
                                                        float* __restrict__ o)
{
    constexpr int TEAMS = 4 / NK, R = 16 / TCH;
    __shared__ float part[NK > 1 ? 4 : 1][16];
    int e, r_beg, n_e;
    if (!slot_expert(a, blockIdx.y, e, r_beg, n_e)) return;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int team = wave / NK, kw = wave % NK;
    const int kl = kw * 64 + lane;  // lane index along the f axis
    const int c0 = (blockIdx.x * TEAMS + team) * kDnRows;
    const int f = a.f, nb = f >> 5;
    const size_t crow = (size_t)(f >> 1), srow = (size_t)nb;
    const bool live = c0 < a.d;  // d % 16 == 0: a team's rows are all in or all out
    const size_t wrow0 = (size_t)wslot(a, e) * a.d + (live ? c0 : 0);
    const __amdgpu_buffer_rsrc_t rd = weight_rsrc(a.dc + wrow0 * crow);
    const __amdgpu_buffer_rsrc_t rds = weight_rsrc(a.ds + wrow0 * srow);
    uint32_t coff[BPL], soffl[BPL];
#pragma unroll
    for (int b = 0; b < BPL; ++b) {
        const int blk = kl + 64 * NK * b;
        coff[b] = blk < nb ? (uint32_t)blk * 16u : kOff;
        soffl[b] = blk < nb ? (uint32_t)blk : kOff;
    }

    for (int rb = 0; rb < kDnRows; rb += R) {
        uint4 q[R][BPL];
        uint32_t sbp[R / 4][BPL];  // scale bytes four to a register (held across tokens)
#pragma unroll
        for (int b = 0; b < BPL; ++b) {
            uint32_t sb[R];
#pragma unroll
            for (int i = 0; i < R; ++i) {
                q[i][b] = ld_stream(rd, coff[b], (uint32_t)(rb + i) * (uint32_t)crow);
                sb[i] = ld_scale(rds, soffl[b], (uint32_t)(rb + i) * (uint32_t)srow);
            }
#pragma unroll
            for (int j = 0; j < R / 4; ++j)
                sbp[j][b] = sb[4 * j] | (sb[4 * j + 1] << 8) | (sb[4 * j + 2] << 16) | (sb[4 * j + 3] << 24);
        }
        for (int t0 = 0; t0 < n_e; t0 += TCH) {
            float hr[BPL][TCH][32];
#pragma unroll
            for (int tt = 0; tt < TCH; ++tt) {
                int m = min(t0 + tt, n_e - 1);
                float tmp[BPL][32];
                load_act<BPL>(hbuf + (size_t)(r_beg + m) * f, kl, 64 * NK, nb, tmp);
#pragma unroll
                for (int b = 0; b < BPL; ++b)
#pragma unroll
                    for (int i = 0; i < 32; ++i) hr[b][tt][i] = tmp[b][i];
            }
            auto row_dot = [&](int i, float (&s)[TCH]) {
#pragma unroll
                for (int tt = 0; tt < TCH; ++tt) s[tt] = 0.f;
#pragma unroll
                for (int b = 0; b < BPL; ++b) {
                    uint4 qq = q[i][b];
                    uint32_t sp = sbp[i >> 2][b];
                    opaque(qq);
                    asm volatile("" : "+v"(sp));
                    dot32_multi<TCH>(qq, e8m0_f32((sp >> (8 * (i & 3))) & 0xffu), hr[b], s);
                }
            };
            float a8[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                float lo, hi;
                if (TCH == 1) {
                    float s0[TCH], s1[TCH];
                    row_dot(j, s0);
                    row_dot(j + 8, s1);
                    lo = s0[0];
                    hi = s1[TCH - 1];
                } else {
                    float s2[TCH];
                    row_dot(j, s2);
                    lo = s2[0];
                    hi = s2[TCH - 1];
                }
                a8[j] = transpose_step8(lo, hi);
            }
            const float v = wave_transpose_sum_from8(a8);
            const int tt = (lane & 15) / R, i = (lane & 15) % R;
            if (NK == 1) {
                if (live && lane < 16 && t0 + tt < n_e)
                    o[(size_t)(r_beg + t0 + tt) * a.d + c0 + rb + i] = v;
            } else {
                if (lane < 16) part[wave][lane] = v;
                __syncthreads();
                if (kw == 0 && lane < 16 && live && t0 + tt < n_e) {
                    float sum = 0.f;
#pragma unroll
                    for (int w = 0; w < NK; ++w) sum += part[team * NK + w][lane];
                    o[(size_t)(r_beg + t0 + tt) * a.d + c0 + rb + i] = sum;
                }
                __syncthreads();
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Pair-major down with the combine fused, for small batches: block (x, t)
// owns RW rows [RW*x, RW*x+RW) of y[t] (RW = d/256 when that divides, so
// every CU gets the same share); wave w streams those rows of the experts
// j = w, w+8, ... of token t (one f-wide row per lane, BPL blocks per lane)
// in batches of 16 rows, reduces each batch with one transposed reduction
// and accumulates w[t,j] * o in j order; the eight waves' partial sums are
// added in wave order.  Deterministic, and no per-pair output is written.
constexpr int kGatherWaves = 8;

template <int RW, int BPL>
__global__ __launch_bounds__(64 * kGatherWaves) void down_gather_kernel(FfnArgs a, const float* __restrict__ hbuf,
                                                                        float* __restrict__ y)
{
    constexpr int NBT = (RW + 15) / 16;
    __shared__ float part[kGatherWaves][RW];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int t = blockIdx.y, c0 = blockIdx.x * RW;
    const int f = a.f, nb = f >> 5, k = a.k;
    const size_t crow = (size_t)(f >> 1), srow = (size_t)nb;
    uint32_t coff[BPL], soffl[BPL];
#pragma unroll
    for (int b = 0; b < BPL; ++b) {
        const int blk = lane + 64 * b;
        coff[b] = blk < nb ? (uint32_t)blk * 16u : kOff;
        soffl[b] = blk < nb ? (uint32_t)blk : kOff;
    }
    float yacc[NBT];
#pragma unroll
    for (int bt = 0; bt < NBT; ++bt) yacc[bt] = 0.f;
    for (int j = wave; j < k; j += kGatherWaves) {
        const int p = t * k + j;
        const int e = a.pair_w[p];  // weight index (the expert, or its cache slot)
        const float w = a.topk_w[p];
        const size_t wrow0 = (size_t)e * a.d + c0;
        const __amdgpu_buffer_rsrc_t rd = weight_rsrc(a.dc + wrow0 * crow);
        const __amdgpu_buffer_rsrc_t rds = weight_rsrc(a.ds + wrow0 * srow);
        float hr[BPL][1][32];
        {
            float tmp[BPL][32];
            load_act<BPL>(hbuf + (size_t)p * f, lane, 64, nb, tmp);
#pragma unroll
            for (int b = 0; b < BPL; ++b)
#pragma unroll
                for (int i = 0; i < 32; ++i) hr[b][0][i] = tmp[b][i];
        }
#pragma unroll
        for (int bt = 0; bt < NBT; ++bt) {
            uint4 q[16][BPL];
            uint32_t sb[16][BPL];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int row = 16 * bt + i;
#pragma unroll
                for (int b = 0; b < BPL; ++b) {
                    if (row < RW) {
                        q[i][b] = ld_stream(rd, coff[b], (uint32_t)row * (uint32_t)crow);
                        sb[i][b] = ld_scale(rds, soffl[b], (uint32_t)row * (uint32_t)srow);
                    } else {
                        q[i][b] = make_uint4(0u, 0u, 0u, 0u);
                        sb[i][b] = 127u;
                    }
                }
            }
            float acc[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float s1[1] = {0.f};
#pragma unroll
                for (int b = 0; b < BPL; ++b) dot32_multi<1>(q[i][b], e8m0_f32(sb[i][b]), hr[b], s1);
                acc[i] = s1[0];
            }
            const float v = wave_transpose_sum16(acc);
            yacc[bt] = __builtin_fmaf(w, v, yacc[bt]);
        }
    }
#pragma unroll
    for (int bt = 0; bt < NBT; ++bt)
        if (lane < 16 && 16 * bt + lane < RW) part[wave][16 * bt + lane] = yacc[bt];
    __syncthreads();
    if (tid < RW) {
        float sum = 0.f;
#pragma unroll
        for (int w = 0; w < kGatherWaves; ++w) sum += part[w][tid];
        y[(size_t)t * a.d + c0 + tid] = sum;
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
    const float4* o4 = reinterpret_cast<const float4*>(o);
    for (int j0 = 0; j0 < a.k; j0 += 4) {
        // four pairs at a time, indices clamped so every load is in flight;
        // the weights of pairs past k are zero and add nothing
        int row[4];
        float w[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int p = t * a.k + min(j0 + u, a.k - 1);
            row[u] = a.row_of_pair[p];
            w[u] = (j0 + u < a.k) ? a.topk_w[p] : 0.0f;
        }
        float4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            if (a.o_stream) {  // rows too large for the caches: read once, non-temporal
                const f32x4 t = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(o4 + (size_t)row[u] * d4 + c4));
                v[u] = make_float4(t[0], t[1], t[2], t[3]);
            } else {
                v[u] = o4[(size_t)row[u] * d4 + c4];
            }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            acc.x = __builtin_fmaf(w[u], v[u].x, acc.x);
            acc.y = __builtin_fmaf(w[u], v[u].y, acc.y);
            acc.z = __builtin_fmaf(w[u], v[u].z, acc.z);
            acc.w = __builtin_fmaf(w[u], v[u].w, acc.w);
        }
    }
    reinterpret_cast<float4*>(y + (size_t)t * a.d)[c4] = acc;
}

// ---------------------------------------------------------------------------
// Tokens per pass of the grouped GEMVs: one for small batches (about two
// tokens per active expert; in gate/up the experts with a single token run
// without the token loop at four waves per SIMD, the others two tokens per
// pass), two once experts hold many tokens (each decoded weight then serves
// two activation rows).
static int tokens_per_pass(const FfnArgs& a) { return a.T <= 64 ? 1 : 2; }

template <int TCH, bool PAIR>
static void gateup_dispatch(const FfnArgs& a, float* h, hipStream_t s)
{
    const int nb = a.d / 32;
    dim3 grid((a.f + kGuRows - 1) / kGuRows, PAIR ? a.P : a.nslots);
    if (nb <= 256)
        k3_launch(gateup_gemv_kernel<TCH, 1, PAIR>, grid, dim3(256), s, a, h, static_cast<uint8_t*>(nullptr), static_cast<uint8_t*>(nullptr));
    else
        k3_launch(gateup_gemv_kernel<TCH, 2, PAIR>, grid, dim3(256), s, a, h, static_cast<uint8_t*>(nullptr), static_cast<uint8_t*>(nullptr));  // d <= kMaxDim: wider rows are refused by the ABI
}

bool use_pair_path(const FfnArgs& a) { return a.P <= kPairMajorMax && a.f <= 8192; }

void launch_gateup_gemv_slices(const FfnArgs& a, uint8_t* hs_codes, uint8_t* hs_scales, hipStream_t s)
{
    const dim3 grid(a.f / kGuRows, a.P);
    if (a.d / 32 <= 256)
        k3_launch(gateup_gemv_kernel<1, 1, true, true>, grid, dim3(256), s, a, static_cast<float*>(nullptr), hs_codes, hs_scales);
    else
        k3_launch(gateup_gemv_kernel<1, 2, true, true>, grid, dim3(256), s, a, static_cast<float*>(nullptr), hs_codes, hs_scales);
}

void launch_gateup_gemv(const FfnArgs& a, float* h, hipStream_t s)
{
    if (use_pair_path(a)) {
        gateup_dispatch<1, true>(a, h, s);
    } else if (tokens_per_pass(a) == 1 && a.d / 32 <= 256) {
        // experts with one token at four waves per SIMD, then the others two tokens
        // per pass, each decoded weight serving both (about half of the active
        // experts each at 64 tokens of uniform routing)
        const dim3 grid((a.f + kGuRows - 1) / kGuRows, a.nslots);
        k3_launch(gateup_gemv_kernel<1, 1, false, false, kSelOne>, grid, dim3(256), s, a, h, static_cast<uint8_t*>(nullptr), static_cast<uint8_t*>(nullptr));
        k3_launch(gateup_gemv_kernel<2, 1, false, false, kSelMulti>, grid, dim3(256), s, a, h, static_cast<uint8_t*>(nullptr), static_cast<uint8_t*>(nullptr));
    } else if (tokens_per_pass(a) == 1) {
        gateup_dispatch<1, false>(a, h, s);
    } else
        gateup_dispatch<2, false>(a, h, s);
}

template <int RW>
static void down_gather_dispatch(const FfnArgs& a, const float* h, float* y, hipStream_t s)
{
    const int nb = a.f / 32;
    dim3 grid(a.d / RW, a.T);
    if (nb <= 64)
        k3_launch(down_gather_kernel<RW, 1>, grid, dim3(64 * kGatherWaves), s, a, h, y);
    else if (nb <= 128)
        k3_launch(down_gather_kernel<RW, 2>, grid, dim3(64 * kGatherWaves), s, a, h, y);
    else
        k3_launch(down_gather_kernel<RW, 4>, grid, dim3(64 * kGatherWaves), s, a, h, y);
}

void launch_down_gather(const FfnArgs& a, const float* h, float* y, hipStream_t s)
{
    // 28 rows per block gives exactly one block per CU at d_model 7168
    if (a.d % 28 == 0 && a.d / 28 >= 256)
        down_gather_dispatch<28>(a, h, y, s);
    else
        down_gather_dispatch<16>(a, h, y, s);
}

template <int TCH, int NK>
static void down_dispatch_nk(const FfnArgs& a, const float* h, float* o, hipStream_t s)
{
    const int nb = a.f / 32;
    constexpr int TEAMS = 4 / NK;
    dim3 grid((a.d + TEAMS * kDnRows - 1) / (TEAMS * kDnRows), a.nslots);
    if (nb <= 64 * NK)
        k3_launch(down_gemv_kernel<TCH, NK, 1>, grid, dim3(256), s, a, h, o);
    else
        k3_launch(down_gemv_kernel<TCH, NK, 2>, grid, dim3(256), s, a, h, o);  // f <= kMaxDim: wider rows are refused by the ABI
}

template <int TCH>
static void down_dispatch(const FfnArgs& a, const float* h, float* o, hipStream_t s)
{
    const int nb = a.f / 32;
    if (nb <= 64)
        down_dispatch_nk<TCH, 1>(a, h, o, s);
    else if (nb <= 128)
        down_dispatch_nk<TCH, 2>(a, h, o, s);
    else
        down_dispatch_nk<TCH, 4>(a, h, o, s);
}

void launch_down_gemv(const FfnArgs& a, const float* h, float* o, hipStream_t s)
{
    if (tokens_per_pass(a) == 1)
        down_dispatch<1>(a, h, o, s);
    else
        down_dispatch<2>(a, h, o, s);
}

void launch_combine(const FfnArgs& a, const float* o, float* y, hipStream_t s)
{
    dim3 grid(a.T, (a.d / 4 + 255) / 256);
    k3_launch(combine_kernel, grid, dim3(256), s, a, o, y);
}

}  // namespace k3
