// mx.hip -- MXFP4-activation expert FFN for gfx950: activation quantiser,
// grouped gate/up GEMM with fused SwiGLU + h quantiser, grouped down GEMM with
// fused gate-weighted scatter-add combine.  Both GEMMs run on the CDNA4
// scaled matrix cores (V_MFMA_SCALE_F32_16X16X128_F8F6F4, FP4 x FP4 with
// E8M0 block scales, fp32 accumulate).
//
// Weights stay in the pages' format: 4-bit E2M1 codes with one E8M0 scale per
// 32 values along the reduction axis (fiv.co.kr "kimi-k3-in-c deep dive",
// "four reductions", MXFP4 note).  The matrix core consumes exactly that
// format, so neither the weights nor the quantised activations are expanded.
//
// Operand layout of one 16x16x128 step (lane l = 16*g + i, g = 0..3): the
// lane supplies 32 consecutive K-values of row i (A) / column i (B) as 16
// code bytes, low nibble first, plus that block's scale byte.  Because the
// dot product is invariant to a permutation of K applied to both operands,
// a lane here takes the 4 blocks [128g, 128g+128) of a 512-wide K chunk as one
// 64-byte contiguous run and feeds block s of it to step s; the four scale
// bytes of those blocks arrive in one 32-bit word, and step s selects byte s.
#include "device_common.h"
#include "kernels.h"

namespace k3 {

// ---------------------------------------------------------------------------
// MX quantiser (OCP MX rule): scale byte = clamp(floor(log2 amax) - 2 + 127,
// 0, 254), 0 for an all-zero block; |v| / 2^(byte-127) rounded to the nearest
// E2M1 magnitude, ties to the even code, saturating at 6; sign bit kept.
// Every step is exact in fp32.
__device__ __forceinline__ uint32_t mx_scale_byte(float amax)
{
    if (!(amax > 0.0f)) return 0u;
    uint32_t b = __float_as_uint(amax);
    uint32_t ef = b >> 23;
    int fl = ef ? (int)ef - 127 : (31 - __clz((int)b)) - 149;  // floor(log2 amax)
    int byte = fl - 2 + 127;
    return (uint32_t)min(max(byte, 0), 254);
}

// 2^(127 - byte); byte <= 252 for any finite fp32 amax, so this is normal.
__device__ __forceinline__ float mx_inv_scale(uint32_t byte)
{
    return __uint_as_float((254u - byte) << 23);
}

__device__ __forceinline__ uint32_t e2m1_encode(float v, float inv_scale)
{
    float m = fabsf(v) * inv_scale;
    // midpoints 0.25 0.75 1.25 1.75 2.5 3.5 5: a tie moves up only when the
    // upper neighbour has the even code
    uint32_t idx = (m > 0.25f) + (m >= 0.75f) + (m > 1.25f) + (m >= 1.75f) +
                   (m > 2.5f) + (m >= 3.5f) + (m > 5.0f);
    return ((__float_as_uint(v) >> 31) << 3) | idx;
}

// 8 lanes per 32-element block, 4 values per lane.
__global__ __launch_bounds__(256) void quantize_rows_kernel(long nblocks, const float* __restrict__ v,
                                                            uint8_t* __restrict__ codes,
                                                            uint8_t* __restrict__ scales)
{
    const long gid = (long)blockIdx.x * 256 + threadIdx.x;
    const long blk = gid >> 3;
    const int sub = (int)(gid & 7);
    if (blk >= nblocks) return;  // whole 8-lane group leaves together
    float4 q = reinterpret_cast<const float4*>(v)[blk * 8 + sub];
    float amax = fmaxf(fmaxf(fabsf(q.x), fabsf(q.y)), fmaxf(fabsf(q.z), fabsf(q.w)));
    amax = fmaxf(amax, __shfl_xor(amax, 4, 8));
    amax = fmaxf(amax, __shfl_xor(amax, 2, 8));
    amax = fmaxf(amax, __shfl_xor(amax, 1, 8));
    uint32_t byte = mx_scale_byte(amax);
    float inv = mx_inv_scale(byte);
    uint32_t c0 = e2m1_encode(q.x, inv), c1 = e2m1_encode(q.y, inv);
    uint32_t c2 = e2m1_encode(q.z, inv), c3 = e2m1_encode(q.w, inv);
    uint16_t packed = (uint16_t)(c0 | (c1 << 4) | (c2 << 8) | (c3 << 12));
    reinterpret_cast<uint16_t*>(codes)[blk * 8 + sub] = packed;
    if (sub == 0) scales[blk] = (uint8_t)byte;
}

void launch_quantize_rows(long nblocks, const float* v, uint8_t* codes, uint8_t* scales,
                          hipStream_t s)
{
    long threads = nblocks * 8;
    quantize_rows_kernel<<<dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s>>>(
        nblocks, v, codes, scales);
}

__global__ __launch_bounds__(256) void zero_kernel(float4* __restrict__ p, size_t n4)
{
    size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n4) p[i] = make_float4(0.f, 0.f, 0.f, 0.f);
}

void launch_zero(float* y, size_t n, hipStream_t s)
{
    size_t n4 = n / 4;  // n is a multiple of 32
    zero_kernel<<<dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, s>>>(
        reinterpret_cast<float4*>(y), n4);
}

// ---------------------------------------------------------------------------
// Slot -> expert (same rule as the fp32 path).
__device__ __forceinline__ bool mx_slot_expert(const FfnArgs& a, int slot, int& e, int& r_beg, int& n_e)
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

__device__ __forceinline__ i32x8 op4(uint4 q)
{
    i32x8 r = {(int)q.x, (int)q.y, (int)q.z, (int)q.w, 0, 0, 0, 0};
    return r;
}

template <int SEL>
__device__ __forceinline__ f32x4 mfma_fp4(uint4 a, uint4 b, uint32_t sa, uint32_t sb, f32x4 c)
{
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(op4(a), op4(b), c, 4, 4, SEL, (int)sa,
                                                            SEL, (int)sb);
}

// One operand row-lane's share of a K chunk: CH512 -> 64 code bytes (4 blocks)
// and their 4 scale bytes in one word; else one 128-wide step: 16 bytes and
// one scale byte (zeros past the row end contribute nothing).
struct Frag512 {
    uint4 q[4];
    uint32_t s;
};

__device__ __forceinline__ void load_frag512(const uint8_t* crow, const uint8_t* srow, int kc, int g,
                                             Frag512& f)
{
    const uint8_t* cp = crow + (kc >> 1) + 64 * g;
#pragma unroll
    for (int i = 0; i < 4; ++i) f.q[i] = ldg16(cp + 16 * i);
    f.s = *reinterpret_cast<const uint32_t*>(srow + (kc >> 5) + 4 * g);
}

__device__ __forceinline__ void load_frag128(const uint8_t* crow, const uint8_t* srow, int kc, int g,
                                             int K, uint4& q, uint32_t& s)
{
    int blk = (kc >> 5) + g;
    if (blk < (K >> 5)) {
        q = ldg16(crow + 16 * (size_t)blk);
        s = srow[blk];
    } else {
        q = make_uint4(0u, 0u, 0u, 0u);
        s = 127u;
    }
}

// ---------------------------------------------------------------------------
// gate/up GEMM: block = 4 waves, wave w owns f rows [n0 + 32w, +32) as two
// 16-row subtiles of both gate and up; M = the expert's tokens in tiles of
// 16, MT tiles per pass.  Epilogue: h = silu(g) * u in fp32, then the MX
// quantiser over each token's 32 consecutive f values (exactly the wave's
// two subtiles), written to h_q rows in grouped order.
constexpr int kMT = 8;

__global__ __launch_bounds__(256) void gateup_mfma_kernel(FfnArgs a, const uint8_t* __restrict__ xqc,
                                                          const uint8_t* __restrict__ xqs,
                                                          uint8_t* __restrict__ hqc,
                                                          uint8_t* __restrict__ hqs,
                                                          float* __restrict__ dbg_h,
                                                          uint8_t* __restrict__ dbg_hc,
                                                          uint8_t* __restrict__ dbg_hs)
{
    int e, r_beg, n_e;
    if (!mx_slot_expert(a, blockIdx.y, e, r_beg, n_e)) return;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int li = lane & 15, g = lane >> 4;
    const int nw = blockIdx.x * 128 + wave * 32;
    if (nw >= a.f) return;
    const int K = a.d;
    const size_t crow = (size_t)(K >> 1), srow = (size_t)(K >> 5);
    const bool ch512 = (K % 512) == 0;
    // B rows this lane feeds: gate/up rows nw + 16*s + li
    const uint8_t *bgc[2], *bgs[2], *buc[2], *bus[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        size_t wr = (size_t)e * a.f + nw + 16 * s + li;
        bgc[s] = a.gc + wr * crow;
        bgs[s] = a.gs + wr * srow;
        buc[s] = a.uc + wr * crow;
        bus[s] = a.us + wr * srow;
    }
    for (int m0 = 0; m0 < n_e; m0 += 16 * kMT) {
        const int mt_n = min(kMT, (n_e - m0 + 15) >> 4);
        // A rows this lane feeds: token of grouped row r_beg + m0 + 16*mt + li (clamped)
        const uint8_t *axc[kMT], *axs[kMT];
#pragma unroll
        for (int mt = 0; mt < kMT; ++mt) {
            int m = min(m0 + 16 * mt + li, n_e - 1);
            int tok = a.perm_pair[r_beg + m] / a.k;
            axc[mt] = xqc + (size_t)tok * crow;
            axs[mt] = xqs + (size_t)tok * srow;
        }
        f32x4 cg[kMT][2], cu[kMT][2];
#pragma unroll
        for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                cg[mt][s] = (f32x4){0.f, 0.f, 0.f, 0.f};
                cu[mt][s] = (f32x4){0.f, 0.f, 0.f, 0.f};
            }
        int kc = 0;
        if (ch512) {
            for (; kc < K; kc += 512) {
                Frag512 fg[2], fu[2];
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    load_frag512(bgc[s], bgs[s], kc, g, fg[s]);
                    load_frag512(buc[s], bus[s], kc, g, fu[s]);
                }
#pragma unroll
                for (int mt = 0; mt < kMT; ++mt) {
                    if (mt < mt_n) {
                        Frag512 fa;
                        load_frag512(axc[mt], axs[mt], kc, g, fa);
#pragma unroll
                        for (int s = 0; s < 2; ++s) {
                            cg[mt][s] = mfma_fp4<0>(fa.q[0], fg[s].q[0], fa.s, fg[s].s, cg[mt][s]);
                            cu[mt][s] = mfma_fp4<0>(fa.q[0], fu[s].q[0], fa.s, fu[s].s, cu[mt][s]);
                            cg[mt][s] = mfma_fp4<1>(fa.q[1], fg[s].q[1], fa.s, fg[s].s, cg[mt][s]);
                            cu[mt][s] = mfma_fp4<1>(fa.q[1], fu[s].q[1], fa.s, fu[s].s, cu[mt][s]);
                            cg[mt][s] = mfma_fp4<2>(fa.q[2], fg[s].q[2], fa.s, fg[s].s, cg[mt][s]);
                            cu[mt][s] = mfma_fp4<2>(fa.q[2], fu[s].q[2], fa.s, fu[s].s, cu[mt][s]);
                            cg[mt][s] = mfma_fp4<3>(fa.q[3], fg[s].q[3], fa.s, fg[s].s, cg[mt][s]);
                            cu[mt][s] = mfma_fp4<3>(fa.q[3], fu[s].q[3], fa.s, fu[s].s, cu[mt][s]);
                        }
                    }
                }
            }
        } else {
            for (; kc < K; kc += 128) {
                uint4 qg[2], qu[2];
                uint32_t sg[2], su[2];
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    load_frag128(bgc[s], bgs[s], kc, g, K, qg[s], sg[s]);
                    load_frag128(buc[s], bus[s], kc, g, K, qu[s], su[s]);
                }
#pragma unroll
                for (int mt = 0; mt < kMT; ++mt) {
                    if (mt < mt_n) {
                        uint4 qa;
                        uint32_t sa;
                        load_frag128(axc[mt], axs[mt], kc, g, K, qa, sa);
#pragma unroll
                        for (int s = 0; s < 2; ++s) {
                            cg[mt][s] = mfma_fp4<0>(qa, qg[s], sa, sg[s], cg[mt][s]);
                            cu[mt][s] = mfma_fp4<0>(qa, qu[s], sa, su[s], cu[mt][s]);
                        }
                    }
                }
            }
        }
        // epilogue: lane (li, g) holds rows m = 4g + v, column li of each subtile
#pragma unroll
        for (int mt = 0; mt < kMT; ++mt) {
            if (mt >= mt_n) break;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int m = m0 + 16 * mt + 4 * g + v;
                float h0 = silu_f32(cg[mt][0][v]) * cu[mt][0][v];
                float h1 = silu_f32(cg[mt][1][v]) * cu[mt][1][v];
                float amax = fmaxf(fabsf(h0), fabsf(h1));
                amax = fmaxf(amax, __shfl_xor(amax, 8, 16));
                amax = fmaxf(amax, __shfl_xor(amax, 4, 16));
                amax = fmaxf(amax, __shfl_xor(amax, 2, 16));
                amax = fmaxf(amax, __shfl_xor(amax, 1, 16));
                uint32_t byte = mx_scale_byte(amax);
                float inv = mx_inv_scale(byte);
                uint32_t q0 = e2m1_encode(h0, inv), q1 = e2m1_encode(h1, inv);
                uint32_t p0 = __shfl_xor(q0, 1, 16), p1 = __shfl_xor(q1, 1, 16);
                if (m < n_e) {
                    const size_t r = (size_t)(r_beg + m);
                    const int blk = nw >> 5;
                    const size_t fcb = (size_t)(a.f >> 1), fsb = (size_t)(a.f >> 5);
                    int pair = -1;
                    if (dbg_h || dbg_hc || dbg_hs) pair = a.perm_pair[r];
                    if ((li & 1) == 0) {
                        uint8_t b0 = (uint8_t)(q0 | (p0 << 4)), b1 = (uint8_t)(q1 | (p1 << 4));
                        hqc[r * fcb + 16 * blk + (li >> 1)] = b0;
                        hqc[r * fcb + 16 * blk + 8 + (li >> 1)] = b1;
                        if (dbg_hc) {
                            dbg_hc[(size_t)pair * fcb + 16 * blk + (li >> 1)] = b0;
                            dbg_hc[(size_t)pair * fcb + 16 * blk + 8 + (li >> 1)] = b1;
                        }
                    }
                    if (li == 0) {
                        hqs[r * fsb + blk] = (uint8_t)byte;
                        if (dbg_hs) dbg_hs[(size_t)pair * fsb + blk] = (uint8_t)byte;
                    }
                    if (dbg_h) {
                        dbg_h[(size_t)pair * a.f + nw + li] = h0;
                        dbg_h[(size_t)pair * a.f + nw + 16 + li] = h1;
                    }
                }
            }
        }
    }
}

void launch_gateup_mfma(const FfnArgs& a, const uint8_t* xq_codes, const uint8_t* xq_scales,
                        uint8_t* hq_codes, uint8_t* hq_scales, float* dbg_h, uint8_t* dbg_hc,
                        uint8_t* dbg_hs, hipStream_t s)
{
    dim3 grid((a.f + 127) / 128, a.nslots);
    gateup_mfma_kernel<<<grid, dim3(256), 0, s>>>(a, xq_codes, xq_scales, hq_codes, hq_scales, dbg_h,
                                                  dbg_hc, dbg_hs);
}

// ---------------------------------------------------------------------------
// down GEMM: block = 4 waves, wave w owns d rows [n0 + 64w, +64) as four
// 16-row subtiles; A = the expert's h_q rows (contiguous in grouped order).
// Epilogue: y[t][c] += w[t,j] * o[c], fp32 atomic add (the combine).
__global__ __launch_bounds__(256) void down_mfma_kernel(FfnArgs a, const uint8_t* __restrict__ hqc,
                                                        const uint8_t* __restrict__ hqs,
                                                        float* __restrict__ y)
{
    int e, r_beg, n_e;
    if (!mx_slot_expert(a, blockIdx.y, e, r_beg, n_e)) return;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int li = lane & 15, g = lane >> 4;
    const int nw = blockIdx.x * 256 + wave * 64;
    if (nw >= a.d) return;
    const int K = a.f;
    const size_t crow = (size_t)(K >> 1), srow = (size_t)(K >> 5);
    const bool ch512 = (K % 512) == 0;
    const uint8_t *bc[4], *bs[4];
    bool sub_ok[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        int n = nw + 16 * s;
        sub_ok[s] = n < a.d;
        size_t wr = (size_t)e * a.d + (sub_ok[s] ? n : nw) + li;
        bc[s] = a.dc + wr * crow;
        bs[s] = a.ds + wr * srow;
    }
    for (int m0 = 0; m0 < n_e; m0 += 16 * kMT) {
        const int mt_n = min(kMT, (n_e - m0 + 15) >> 4);
        const uint8_t *ac[kMT], *as[kMT];
#pragma unroll
        for (int mt = 0; mt < kMT; ++mt) {
            size_t r = (size_t)(r_beg + min(m0 + 16 * mt + li, n_e - 1));
            ac[mt] = hqc + r * crow;
            as[mt] = hqs + r * srow;
        }
        f32x4 c[kMT][4];
#pragma unroll
        for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
            for (int s = 0; s < 4; ++s) c[mt][s] = (f32x4){0.f, 0.f, 0.f, 0.f};
        if (ch512) {
            for (int kc = 0; kc < K; kc += 512) {
                Frag512 fb[4];
#pragma unroll
                for (int s = 0; s < 4; ++s) load_frag512(bc[s], bs[s], kc, g, fb[s]);
#pragma unroll
                for (int mt = 0; mt < kMT; ++mt) {
                    if (mt < mt_n) {
                        Frag512 fa;
                        load_frag512(ac[mt], as[mt], kc, g, fa);
#pragma unroll
                        for (int s = 0; s < 4; ++s) {
                            c[mt][s] = mfma_fp4<0>(fa.q[0], fb[s].q[0], fa.s, fb[s].s, c[mt][s]);
                            c[mt][s] = mfma_fp4<1>(fa.q[1], fb[s].q[1], fa.s, fb[s].s, c[mt][s]);
                            c[mt][s] = mfma_fp4<2>(fa.q[2], fb[s].q[2], fa.s, fb[s].s, c[mt][s]);
                            c[mt][s] = mfma_fp4<3>(fa.q[3], fb[s].q[3], fa.s, fb[s].s, c[mt][s]);
                        }
                    }
                }
            }
        } else {
            for (int kc = 0; kc < K; kc += 128) {
                uint4 qb[4];
                uint32_t sb[4];
#pragma unroll
                for (int s = 0; s < 4; ++s) load_frag128(bc[s], bs[s], kc, g, K, qb[s], sb[s]);
#pragma unroll
                for (int mt = 0; mt < kMT; ++mt) {
                    if (mt < mt_n) {
                        uint4 qa;
                        uint32_t sa;
                        load_frag128(ac[mt], as[mt], kc, g, K, qa, sa);
#pragma unroll
                        for (int s = 0; s < 4; ++s) c[mt][s] = mfma_fp4<0>(qa, qb[s], sa, sb[s], c[mt][s]);
                    }
                }
            }
        }
#pragma unroll
        for (int mt = 0; mt < kMT; ++mt) {
            if (mt >= mt_n) break;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int m = m0 + 16 * mt + 4 * g + v;
                if (m < n_e) {
                    const int pair = a.perm_pair[r_beg + m];
                    const int t = pair / a.k;
                    const float w = a.topk_w[pair];
                    float* yr = y + (size_t)t * a.d + nw + li;
#pragma unroll
                    for (int s = 0; s < 4; ++s)
                        if (sub_ok[s]) unsafeAtomicAdd(yr + 16 * s, w * c[mt][s][v]);
                }
            }
        }
    }
}

void launch_down_mfma(const FfnArgs& a, const uint8_t* hq_codes, const uint8_t* hq_scales, float* y,
                      hipStream_t s)
{
    dim3 grid((a.d + 255) / 256, a.nslots);
    down_mfma_kernel<<<grid, dim3(256), 0, s>>>(a, hq_codes, hq_scales, y);
}

}  // namespace k3
