// route.hip -- router logits (fp64), softmax top-k, and the grouping of
// token-expert pairs by expert, for gfx950.
//
// The pages' router (k3_router, fiv.co.kr "kimi-k3-in-c deep dive", study-plan
// row "MoE and routing") scores every expert, picks 16 of 896 per token
// (glossary row "MoE") and hands the chosen experts to k3_moe.  Here the
// scores are fp64-accumulated logits, the choice is the top-k with ties to the
// lower expert index, and the weights are the softmax over all experts
// restricted to the chosen ones and renormalised (equal to a softmax over the
// chosen logits).  The grouping is a deterministic counting sort: per
// 64-token chunk a bitmask per expert, a prefix over chunks and experts, and a
// rank inside the chunk by popcount -- no atomics decide an order.
#include <float.h>
#include "device_common.h"
#include "kernels.h"
#include "launch.h"
#include "topk.h"

namespace k3 {

// ---------------------------------------------------------------------------
// Router logits, small T: one 256-thread block per expert row; the threads
// split d (float4 per thread per step, all of a thread's loads in flight at
// once), every token of the batch accumulated while the row streams through.
// fp32 x fp32 products are exact in fp64; the sums are fp64, reduced in a
// fixed order (wave shuffles, then the four waves through LDS).
constexpr int kGemvTok = 8;
constexpr int kRouterPerThread = 8;  // float4 steps per thread: d <= 8192 in one pass

__device__ __forceinline__ double shfl_xor_d(double v, int m)
{
    return __shfl_xor(v, m, 64);
}

// R consecutive expert rows per block: the token slice a thread loads is
// reused for all R rows.
template <int R>
__global__ __launch_bounds__(256) void router_gemv_kernel(
    int T, int E, int d, const float* __restrict__ x, const float* __restrict__ wr,
    const float* __restrict__ bias, int bias_in_logits, double* __restrict__ logits)
{
    __shared__ double part[R][kGemvTok][4];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int e0 = blockIdx.x * R;
    const int n4 = d >> 2;
    double acc[R][kGemvTok];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int t = 0; t < kGemvTok; ++t) acc[r][t] = 0.0;
    for (int base = 0; base < n4; base += 256 * kRouterPerThread) {
        // branch-free (clamped) loads; lanes past the end multiply by zero
        float4 w[R][kRouterPerThread];
        float live[kRouterPerThread];
#pragma unroll
        for (int j = 0; j < kRouterPerThread; ++j) {
            const int i = base + tid + 256 * j;
            live[j] = (i < n4) ? 1.0f : 0.0f;
#pragma unroll
            for (int r = 0; r < R; ++r)
                w[r][j] = reinterpret_cast<const float4*>(wr + (size_t)min(e0 + r, E - 1) * d)[min(i, n4 - 1)];
        }
#pragma unroll
        for (int t = 0; t < kGemvTok; ++t) {
            if (t < T) {
                const float4* x4 = reinterpret_cast<const float4*>(x + (size_t)t * d);
                float4 v[kRouterPerThread];
#pragma unroll
                for (int j = 0; j < kRouterPerThread; ++j) v[j] = x4[min(base + tid + 256 * j, n4 - 1)];
#pragma unroll
                for (int r = 0; r < R; ++r) {
#pragma unroll
                    for (int j = 0; j < kRouterPerThread; ++j) {
                        const double m = (double)live[j];
                        acc[r][t] = fma((double)w[r][j].x * m, (double)v[j].x, acc[r][t]);
                        acc[r][t] = fma((double)w[r][j].y * m, (double)v[j].y, acc[r][t]);
                        acc[r][t] = fma((double)w[r][j].z * m, (double)v[j].z, acc[r][t]);
                        acc[r][t] = fma((double)w[r][j].w * m, (double)v[j].w, acc[r][t]);
                    }
                }
            }
        }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
#pragma unroll
        for (int t = 0; t < kGemvTok; ++t) {
            if (t < T) {
                double v = acc[r][t];
                for (int m = 32; m >= 1; m >>= 1) v += shfl_xor_d(v, m);
                if (lane == 0) part[r][t][wave] = v;
            }
        }
    }
    __syncthreads();
    if (tid < R * T) {
        const int r = tid / T, t = tid - r * T, e = e0 + r;
        if (e < E) {
            double v = ((part[r][t][0] + part[r][t][1]) + part[r][t][2]) + part[r][t][3];
            if (bias_in_logits) v += (double)bias[e];
            logits[(size_t)t * E + e] = v;
        }
    }
}

// Router logits, larger T: fp64 matrix cores (V_MFMA_F64_16X16X4_F64), 64
// tokens x 64 experts per 256-thread block (each wave a 32 x 32 corner as
// 2 x 2 MFMA tiles), x and W_r staged through LDS as fp32 and widened at the
// operand (exact).  Lane l supplies A[l%16][l/16] and B[l/16][l%16]; it
// receives D[l/16 + 4v][l%16].  Small batches split K over gridDim.z; the
// partial logits are then added in split order.
typedef double f64x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void router_mfma_kernel(int T, int E, int d, int kslice,
                                                          const float* __restrict__ x,
                                                          const float* __restrict__ wr,
                                                          double* __restrict__ out)
{
    constexpr int BK = 32;
    // two LDS buffers: the next K step is fetched into registers while this
    // one is on the matrix cores, then stored to the other buffer
    __shared__ float xs[2][64][BK + 1];
    __shared__ float ws[2][64][BK + 1];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave & 1, wn = wave >> 1;
    const int t0 = blockIdx.y * 64, e0 = blockIdx.x * 64;
    const int kb = blockIdx.z * kslice, ke = kb + kslice;
    f64x4 acc[2][2];
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) acc[mi][ni] = (f64x4){0.0, 0.0, 0.0, 0.0};
    float xr[8], wv[8];
    auto fetch = [&](int k0) {
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int idx = tid + q * 256;
            const int r = idx >> 5, c = idx & 31;
            const int tr = t0 + r, er = e0 + r;
            xr[q] = (tr < T) ? x[(size_t)tr * d + k0 + c] : 0.0f;
            wv[q] = (er < E) ? wr[(size_t)er * d + k0 + c] : 0.0f;
        }
    };
    auto stash = [&](int b) {
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int idx = tid + q * 256;
            const int r = idx >> 5, c = idx & 31;
            xs[b][r][c] = xr[q];
            ws[b][r][c] = wv[q];
        }
    };
    fetch(kb);
    stash(0);
    __syncthreads();
    int buf = 0;
    for (int k0 = kb; k0 < ke; k0 += BK) {
        const bool more = k0 + BK < ke;
        if (more) fetch(k0 + BK);
#pragma unroll
        for (int kk = 0; kk < BK / 4; ++kk) {
            const int kcol = 4 * kk + (lane >> 4);
            double av[2], bv[2];
#pragma unroll
            for (int mi = 0; mi < 2; ++mi) av[mi] = (double)xs[buf][32 * wm + 16 * mi + (lane & 15)][kcol];
#pragma unroll
            for (int ni = 0; ni < 2; ++ni) bv[ni] = (double)ws[buf][32 * wn + 16 * ni + (lane & 15)][kcol];
#pragma unroll
            for (int mi = 0; mi < 2; ++mi)
#pragma unroll
                for (int ni = 0; ni < 2; ++ni)
                    acc[mi][ni] = __builtin_amdgcn_mfma_f64_16x16x4f64(av[mi], bv[ni], acc[mi][ni], 0, 0, 0);
        }
        if (more) stash(buf ^ 1);
        __syncthreads();
        buf ^= 1;
    }
    double* o = out + (size_t)blockIdx.z * T * E;
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int t = t0 + 32 * wm + 16 * mi + (lane >> 4) + 4 * v;
                const int e = e0 + 32 * wn + 16 * ni + (lane & 15);
                if (t < T && e < E) o[(size_t)t * E + e] = acc[mi][ni][v];
            }
}

// logits = sum of the nsplit partial logits, in split order (+ bias)
__global__ __launch_bounds__(256) void router_reduce_kernel(int nsplit, long n, int E, const double* __restrict__ part,
                                                            const float* __restrict__ bias, int bias_in_logits,
                                                            double* __restrict__ logits)
{
    const long i = (long)blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    double v = 0.0;
    for (int sp = 0; sp < nsplit; ++sp) v += part[(size_t)sp * n + i];
    if (bias_in_logits) v += (double)bias[i % E];
    logits[i] = v;
}

// bias added in place (unsplit MFMA path)
__global__ __launch_bounds__(256) void router_bias_kernel(long n, int E, const float* __restrict__ bias,
                                                          double* __restrict__ logits)
{
    const long i = (long)blockIdx.x * 256 + threadIdx.x;
    if (i < n) logits[i] += (double)bias[i % E];
}

// ---------------------------------------------------------------------------
// Router logits for large batches on the int8 matrix cores, certified.
//
// Error-free splitting of the operands (the scheme of Ozaki, Ogita, Oishi and
// Rump for matrix products, in its integer form): every row v of x and of
// W_r is scaled by 2^-a, a its exponent (max |v| < 2^a), and cut by
// truncation into kSl signed 7-bit slices, v = 2^a (sum_p V_p 2^-7(p+1) +
// r 2^-7kSl) with |r| < 1 -- each step exact in fp32.  The logit x.w is then
// taken as the slice pairs with p + q <= kSl - 1 (kSl (kSl + 1) / 2 of the
// kSl^2: 15 of 25 at five slices), each an int8 dot product summed exactly in
// int32 on the matrix cores, combined in fp64.
// Against the exact x.w this is off by less than
//   2^(a_x - 7 kSl) (kSl d 2^a_w + |w|_1)
// (truncation of x after kSl slices, and for each slice p of x the
// truncation of w after kSl - p slices).  The fp64 sums add at most
// (2 d + 128 + 32 S) 2^-53 2^a_x |w|_1 more, S = the K slices: the oracle's
// sequential sum of d exact products errs by at most (d - 1) 2^-53 2^a_x
// |w|_1; every slice of ours adds kSl exact level terms, each at most (l + 1)
// 2^a_x |w|_1 over the slice (truncated slices never exceed the value), so
// its kSl - 1 roundings err by at most (kSl - 1) kSl (kSl + 1) / 2 2^-53
// times that (60 at five slices, 105 at six), and adding the S slice results
// by at most kSl (kSl + 1) / 2 (S - 1) 2^-53 2^a_x |w|_1 (15 or 21 per add).
// wc[e] holds that bound's factor of 2^a_x for row e; the top-k of each token
// then checks that every gap among its best k + 1 keys exceeds twice the
// token's bound.  A token that fails (ties, near-ties) goes to a list whose
// logits router_exact_kernel recomputes in fp64 and topk_fail_kernel
// selects from; an all-zero token's logits are exact already (0, plus the
// bias).  Five slices leave the bound at ~5e-7 of logits of unit scale at the
// 896-expert layer: about one token in 2,000 of random inputs goes to the list.
constexpr int kSl = kRouterSlices;  // slices per operand
constexpr int kZeroRow = -100000;  // exponent marker of an all-zero row

// One row per block (x rows first, then W_r rows): its exponent, its slices
// ([kSl][rows][d] int8) and, for W_r rows, the bound factor.
// Block 0 also empties the list of uncertified tokens for this call.
__global__ __launch_bounds__(256) void router_slice_kernel(int T, int E, int d, int nsplit, const float* __restrict__ x,
                                                           const float* __restrict__ wr, int8_t* __restrict__ xs,
                                                           int8_t* __restrict__ wsl, int* __restrict__ xe,
                                                           int* __restrict__ we, double* __restrict__ wc,
                                                           int* __restrict__ fail)
{
    if (blockIdx.x == 0 && threadIdx.x == 0) fail[0] = 0;
    __shared__ float redm[4];
    __shared__ double redn[4];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const bool isx = (int)blockIdx.x < T;
    const int r = isx ? (int)blockIdx.x : (int)blockIdx.x - T, rows = isx ? T : E;
    const float* v = (isx ? x : wr) + (size_t)r * d;
    int8_t* out = (isx ? xs : wsl) + (size_t)r * d;
    const size_t pstride = (size_t)rows * d;
    float m = 0.f;
    double n1 = 0.0;
    for (int i = 4 * tid; i < d; i += 1024) {
        const float4 f = *reinterpret_cast<const float4*>(v + i);
        m = fmaxf(m, fmaxf(fmaxf(fabsf(f.x), fabsf(f.y)), fmaxf(fabsf(f.z), fabsf(f.w))));
        n1 += ((double)fabsf(f.x) + (double)fabsf(f.y)) + ((double)fabsf(f.z) + (double)fabsf(f.w));
    }
    for (int o = 32; o >= 1; o >>= 1) {
        m = fmaxf(m, __shfl_xor(m, o, 64));
        n1 += __shfl_xor(n1, o, 64);
    }
    if (lane == 0) {
        redm[wave] = m;
        redn[wave] = n1;
    }
    __syncthreads();
    m = fmaxf(fmaxf(redm[0], redm[1]), fmaxf(redm[2], redm[3]));
    n1 = (redn[0] + redn[1]) + (redn[2] + redn[3]);
    int a = kZeroRow;
    if (m > 0.f) (void)frexpf(m, &a);  // m < 2^a
    const int sh = m > 0.f ? -a : 0;
    for (int i = 4 * tid; i < d; i += 1024) {
        const float4 f = *reinterpret_cast<const float4*>(v + i);
        float u[4] = {ldexpf(f.x, sh), ldexpf(f.y, sh), ldexpf(f.z, sh), ldexpf(f.w, sh)};
#pragma unroll
        for (int p = 0; p < kSl; ++p) {
            uint32_t packed = 0u;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float t = u[j] * 128.0f;
                const float q = truncf(t);  // |q| <= 127
                u[j] = t - q;               // exact: the fraction of t
                packed |= ((uint32_t)(int)q & 0xffu) << (8 * j);
            }
            *reinterpret_cast<uint32_t*>(out + (size_t)p * pstride + i) = packed;
        }
    }
    if (tid == 0) {
        if (isx) {
            xe[r] = a;
        } else {
            we[r] = a;
            // |w|_1 rounded up (the fp64 sum of d exact terms is within d 2^-53 of it)
            const double w1 = n1 * (1.0 + 0x1p-30);
            const double c = ldexp((double)kSl * d * ldexp(1.0, m > 0.f ? a : -1000) + w1, -7 * kSl) +
                             (2.0 * d + 128.0 + 32.0 * nsplit) * 0x1p-53 * w1;
            wc[r] = c * (1.0 + 0x1p-20);
        }
    }
}

// Logits of a 64-token x 64-expert tile: four waves, each a 32 x 32 corner as
// 2 x 2 tiles of V_MFMA_I32_16X16X64_I8, one int32 accumulator set per slice
// level p + q.  Per 64-wide K step the kSl slices of both operands go through
// LDS (rows padded to 80 bytes: the 16 rows of a fragment read fall on
// distinct banks), the next step's slices already in flight in registers.
// Lane l supplies A[l%16][16(l/16) .. +15] and B[same][l%16]; it receives
// D[4(l/16) + v][l%16].
constexpr int kI8Row = 80;

typedef int i32x4v __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void router_i8_kernel(
    int T, int E, int d, const int8_t* __restrict__ xs, const int8_t* __restrict__ wsl, const int* __restrict__ xe,
    const int* __restrict__ we, const float* __restrict__ bias, int bias_in_logits, double* __restrict__ logits,
    int nsplit, double* __restrict__ part)
{
    __shared__ __attribute__((aligned(16))) int8_t As[kSl][64 * kI8Row];
    __shared__ __attribute__((aligned(16))) int8_t Bs[kSl][64 * kI8Row];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave & 1, wn = wave >> 1, li = lane & 15, g = lane >> 4;
    // blocks go round-robin over the 8 XCDs; XCD x takes a contiguous run of
    // tiles (token tile major), so the ~64 blocks resident on one XCD share
    // a few x tiles and every W tile through its L2
    // (the K slices of one tile are adjacent items)
    const int ET = (E + 63) / 64, total = ET * ((T + 63) / 64) * nsplit, per = (total + 7) / 8;
    const int id = (int)(blockIdx.x & 7) * per + (int)(blockIdx.x >> 3);
    if (id >= total) return;
    const int tile = id / nsplit, split = id - tile * nsplit;
    const int t0 = (tile / ET) * 64, e0 = (tile % ET) * 64;
    const int kc = d / nsplit, kb = split * kc;  // this block's K slice: [kb, kb + kc)
    // staging: thread -> (row, 16-byte piece c) of every slice; rows past the
    // end repeat the last row (their results are discarded)
    const int srow = tid >> 2, sc = tid & 3;
    const size_t xoff = (size_t)min(t0 + srow, T - 1) * d + 16 * sc + kb;
    const size_t woff = (size_t)min(e0 + srow, E - 1) * d + 16 * sc + kb;
    const size_t xps = (size_t)T * d, wps = (size_t)E * d;
    const int8_t* xsrc = xs + xoff;
    const int8_t* wsrc = wsl + woff;
    i32x4v acc[kSl][2][2];
#pragma unroll
    for (int l = 0; l < kSl; ++l)
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
#pragma unroll
            for (int ni = 0; ni < 2; ++ni) acc[l][mi][ni] = (i32x4v){0, 0, 0, 0};
    i32x4v ra[kSl], rb[kSl];
#pragma unroll
    for (int p = 0; p < kSl; ++p) {
        ra[p] = *reinterpret_cast<const i32x4v*>(xsrc + p * xps);
        rb[p] = *reinterpret_cast<const i32x4v*>(wsrc + p * wps);
    }
    for (int k0 = 0; k0 < kc; k0 += 64) {
        __syncthreads();  // every wave is done with the previous step's LDS
#pragma unroll
        for (int p = 0; p < kSl; ++p) {
            *reinterpret_cast<i32x4v*>(&As[p][srow * kI8Row + 16 * sc]) = ra[p];
            *reinterpret_cast<i32x4v*>(&Bs[p][srow * kI8Row + 16 * sc]) = rb[p];
        }
        __syncthreads();
        {
            // the next step's slices, in flight during this step's matrix work
            // (the last step fetches its own chunk again: branch-free)
            const int kn = min(k0 + 64, kc - 64);
#pragma unroll
            for (int p = 0; p < kSl; ++p) {
                ra[p] = *reinterpret_cast<const i32x4v*>(xsrc + p * xps + kn);
                rb[p] = *reinterpret_cast<const i32x4v*>(wsrc + p * wps + kn);
            }
        }
        i32x4v bf[kSl][2];
#pragma unroll
        for (int q = 0; q < kSl; ++q)
#pragma unroll
            for (int ni = 0; ni < 2; ++ni)
                bf[q][ni] = *reinterpret_cast<const i32x4v*>(&Bs[q][(32 * wn + 16 * ni + li) * kI8Row + 16 * g]);
#pragma unroll
        for (int p = 0; p < kSl; ++p) {
            i32x4v af[2];
#pragma unroll
            for (int mi = 0; mi < 2; ++mi)
                af[mi] = *reinterpret_cast<const i32x4v*>(&As[p][(32 * wm + 16 * mi + li) * kI8Row + 16 * g]);
#pragma unroll
            for (int q = 0; q + p < kSl; ++q)
#pragma unroll
                for (int mi = 0; mi < 2; ++mi)
#pragma unroll
                    for (int ni = 0; ni < 2; ++ni)
                        acc[p + q][mi][ni] =
                            __builtin_amdgcn_mfma_i32_16x16x64_i8(af[mi], bf[q][ni], acc[p + q][mi][ni], 0, 0, 0);
        }
    }
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int t = t0 + 32 * wm + 16 * mi + 4 * g + v;
                const int e = e0 + 32 * wn + 16 * ni + li;
                if (t < T && e < E) {
                    double sum = 0.0;  // level l = p + q carries 2^-7(l+2); every term exact
#pragma unroll
                    for (int l = kSl - 1; l >= 0; --l) sum += ldexp((double)acc[l][mi][ni][v], -7 * (l + 2));
                    const int ax = xe[t], aw = we[e];
                    double lg = (ax == kZeroRow || aw == kZeroRow) ? 0.0 : ldexp(sum, ax + aw);
                    if (nsplit > 1) {  // partial logit of this K slice, added up in slice order later
                        part[((size_t)split * T + t) * E + e] = lg;
                    } else {
                        if (bias_in_logits) lg += (double)bias[e];
                        logits[(size_t)t * E + e] = lg;
                    }
                }
            }
}

bool use_router_i8(int T, int E, int k, int d)
{
    return T >= kRouterI8MinT && k < 32 && k < E && d % 64 == 0 && d <= kMaxDim && E <= 1024;
}

// K slices of the int8 router: the smallest power of two that gives the
// grid about 512 blocks (at most 8; every slice whole 64-wide K steps)
int router_i8_splits(int T, int E, int d)
{
    const int tiles = ((E + 63) / 64) * ((T + 63) / 64);
    int ns = 1;
    while (tiles * ns < 512 && ns < 8 && (d / 64) % (2 * ns) == 0) ns *= 2;
    return ns;
}

void launch_router_i8(int T, int E, int d, const float* x, const float* wr, const float* bias, int bias_in_logits,
                      int8_t* xs, int8_t* wsl, int* xe, int* we, double* wc, double* logits, double* partials,
                      int* fail, hipStream_t s)
{
    const int ns = router_i8_splits(T, E, d);
    router_slice_kernel<<<dim3(T + E), dim3(256), 0, s>>>(T, E, d, ns, x, wr, xs, wsl, xe, we, wc, fail);
    const int total = ((E + 63) / 64) * ((T + 63) / 64) * ns;
    router_i8_kernel<<<dim3(8 * ((total + 7) / 8)), dim3(256), 0, s>>>(T, E, d, xs, wsl, xe, we, bias, bias_in_logits,
                                                                       logits, ns, partials);
    if (ns > 1) {
        const long n = (long)T * E;
        router_reduce_kernel<<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s>>>(ns, n, E, partials, bias,
                                                                                    bias_in_logits, logits);
    }
}

int router_splits(int T, int E, int d)
{
    if (T <= kGemvTok) return 1;
    const int tiles = ((E + 63) / 64) * ((T + 63) / 64);
    int ns = 1;
    // split K while the grid is small; each slice a multiple of 32 columns
    while (tiles * ns < 256 && ns < 16 && (d / 32) % (2 * ns) == 0) ns *= 2;
    return ns;
}

void launch_router_logits(int T, int E, int d, const float* x, const float* wr,
                          const float* bias, int bias_in_logits, double* logits,
                          double* partials, hipStream_t s)
{
    if (T <= kGemvTok) {
        if (T <= 2 && E >= 512)  // two rows per block still leave > 256 blocks
            router_gemv_kernel<2><<<dim3((E + 1) / 2), dim3(256), 0, s>>>(T, E, d, x, wr, bias, bias_in_logits,
                                                                         logits);
        else
            router_gemv_kernel<1><<<dim3(E), dim3(256), 0, s>>>(T, E, d, x, wr, bias, bias_in_logits, logits);
        return;
    }
    const int ns = router_splits(T, E, d);
    const long n = (long)T * E;
    dim3 grid((E + 63) / 64, (T + 63) / 64, ns);
    if (ns == 1) {
        router_mfma_kernel<<<grid, dim3(256), 0, s>>>(T, E, d, d, x, wr, logits);
        if (bias_in_logits)
            router_bias_kernel<<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s>>>(n, E, bias, logits);
    } else {
        router_mfma_kernel<<<grid, dim3(256), 0, s>>>(T, E, d, d / ns, x, wr, partials);
        router_reduce_kernel<<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s>>>(ns, n, E, partials, bias,
                                                                                  bias_in_logits, logits);
    }
}

// ---------------------------------------------------------------------------
// Block-wide exclusive scan over blockDim.x (multiple of 64, <= 1024) ints.
__device__ int block_exclusive_scan(int v, int* wave_tot, int* total)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
    int inc = v;
    for (int m = 1; m < 64; m <<= 1) {
        int o = __shfl_up(inc, m, 64);
        if (lane >= m) inc += o;
    }
    if (lane == 63) wave_tot[wave] = inc;
    __syncthreads();
    if (threadIdx.x == 0) {
        int run = 0;
        for (int w = 0; w < nw; ++w) {
            int tmp = wave_tot[w];
            wave_tot[w] = run;
            run += tmp;
        }
        wave_tot[nw] = run;
    }
    __syncthreads();
    int excl = wave_tot[wave] + inc - v;
    *total = wave_tot[nw];
    __syncthreads();
    return excl;
}

// Top-k of one token per block (16 waves): the selection and the weights of
// token blockIdx.x.  With xe (logits from the int8 slices): the selection is
// certified against the token's bound 2^a_x max_e wc[e]; a token that fails
// is appended to the fail list (its selection follows in topk_fail_kernel,
// from logits that router_exact_kernel recomputes).  An all-zero token's
// logits are exact (0, plus the bias): selected directly.
__global__ __launch_bounds__(1024) void topk_token_kernel(int E, int k, const double* __restrict__ logits,
                                                          const float* __restrict__ bias, int bias_select_only,
                                                          int sigmoid, int32_t* __restrict__ topk_idx,
                                                          float* __restrict__ topk_w, const int* __restrict__ xe,
                                                          const double* __restrict__ wc, int* __restrict__ fail)
{
    __shared__ TopkLists lists;
    const int t = blockIdx.x;
    const double* lrow = logits + (size_t)t * E;
    int32_t* idx = topk_idx + (size_t)t * k;
    float* w = topk_w + (size_t)t * k;
    if (xe && xe[t] != kZeroRow) {
        const double xscale = ldexp(1.0, xe[t]);
        if (!block_topk_token(E, k, lrow, bias, bias_select_only, sigmoid, lists, nullptr, idx, w, wc, xscale) &&
            threadIdx.x == 0)
            fail[1 + atomicAdd(fail, 1)] = t;
        return;
    }
    block_topk_token(E, k, lrow, bias, bias_select_only, sigmoid, lists, nullptr, idx, w);
}

// Exact logits of the tokens on the fail list: block (b, j) forms expert rows
// 2b and 2b + 1 of list entries j, j + gridDim.y, ... as fp64 sums of the
// exact fp32 x fp32 products (per thread a strided partial, then a fixed
// tree: within ~d 2^-53 max|x||w| of the exact dot product, equal rows give
// equal logits), plus the bias where it belongs in the logits.
constexpr int kFailSlots = 4;

__global__ __launch_bounds__(256) void router_exact_kernel(int E, int d, const float* __restrict__ x,
                                                           const float* __restrict__ wr, const float* __restrict__ bias,
                                                           int bias_in_logits, const int* __restrict__ fail,
                                                           double* __restrict__ logits)
{
    __shared__ double part[2][4];
    const int n = fail[0];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int e0 = 2 * (int)blockIdx.x, n4 = d >> 2;
    const float4* w0 = reinterpret_cast<const float4*>(wr + (size_t)e0 * d);
    const float4* w1 = reinterpret_cast<const float4*>(wr + (size_t)min(e0 + 1, E - 1) * d);
    for (int j = blockIdx.y; j < n; j += gridDim.y) {
        const int t = fail[1 + j];
        const float4* x4 = reinterpret_cast<const float4*>(x + (size_t)t * d);
        double a0 = 0.0, a1 = 0.0;
        for (int i = tid; i < n4; i += 256) {
            const float4 v = x4[i], p = w0[i], q = w1[i];
            a0 = fma((double)p.x, (double)v.x, a0);
            a0 = fma((double)p.y, (double)v.y, a0);
            a0 = fma((double)p.z, (double)v.z, a0);
            a0 = fma((double)p.w, (double)v.w, a0);
            a1 = fma((double)q.x, (double)v.x, a1);
            a1 = fma((double)q.y, (double)v.y, a1);
            a1 = fma((double)q.z, (double)v.z, a1);
            a1 = fma((double)q.w, (double)v.w, a1);
        }
        for (int m = 32; m >= 1; m >>= 1) {
            a0 += shfl_xor_d(a0, m);
            a1 += shfl_xor_d(a1, m);
        }
        if (lane == 0) {
            part[0][wave] = a0;
            part[1][wave] = a1;
        }
        __syncthreads();
        if (tid < 2 && e0 + tid < E) {
            double v = ((part[tid][0] + part[tid][1]) + part[tid][2]) + part[tid][3];
            if (bias_in_logits) v += (double)bias[e0 + tid];
            logits[(size_t)t * E + e0 + tid] = v;
        }
        __syncthreads();  // part is reused by the next entry
    }
}

// The selection of the fail-list tokens from their exact logits: block j
// takes entries j, j + gridDim.x, ...
__global__ __launch_bounds__(1024) void topk_fail_kernel(int E, int k, const double* __restrict__ logits,
                                                         const float* __restrict__ bias, int bias_select_only,
                                                         int sigmoid, int32_t* __restrict__ topk_idx,
                                                         float* __restrict__ topk_w, const int* __restrict__ fail)
{
    __shared__ TopkLists lists;
    const int n = fail[0];
    for (int j = blockIdx.x; j < n; j += gridDim.x) {
        const int t = fail[1 + j];
        // ends with a block barrier: the lists are free for the next entry
        block_topk_token(E, k, logits + (size_t)t * E, bias, bias_select_only, sigmoid, lists, nullptr,
                         topk_idx + (size_t)t * k, topk_w + (size_t)t * k);
    }
}

// Grouping, one block per 64-token chunk, 16 waves.  ONE: a single token,
// selected here too (the one-token step in one launch).  Otherwise the
// selection is read from topk_idx; the kernel writes the chunk's per-expert
// token masks and counts, and a single-chunk batch (T <= 64) also finishes
// the grouping: counts, offsets, perm_pair, row_of_pair.
template <bool ONE>
__global__ __launch_bounds__(1024) void topk_group_kernel(
    int T, int E, int k, const double* __restrict__ logits, const float* __restrict__ bias,
    int bias_select_only, int sigmoid, int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
    uint64_t* __restrict__ chunk_masks, int32_t* __restrict__ chunk_cnt,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ perm_pair, int32_t* __restrict__ row_of_pair)
{
    __shared__ unsigned long long mask[1024];
    __shared__ int sel[kChunk * 32];
    __shared__ int offs[1025];
    __shared__ int wave_tot[17];
    __shared__ TopkLists lists;
    const int tid = threadIdx.x;
    const int c = blockIdx.x, t0 = c * kChunk;
    const int nt = min(kChunk, T - t0);
    if (ONE) {
        // one token: each expert's count is 0 or 1, its offset the number of
        // chosen experts below it, a pair's row the rank of its expert
        block_topk_token(E, k, logits, bias, bias_select_only, sigmoid, lists, sel, topk_idx, topk_w);
        for (int e = tid; e <= E; e += blockDim.x) {
            int below = 0, hit = 0;
            for (int j = 0; j < k; ++j) {
                below += sel[j] < e;
                hit += sel[j] == e;
            }
            offsets[e] = below;
            if (e < E) counts[e] = hit;
        }
        if (tid < k) {
            int rank = 0;
            for (int i = 0; i < k; ++i) rank += sel[i] < sel[tid];
            perm_pair[rank] = tid;
            row_of_pair[tid] = rank;
        }
        return;
    }
    for (int i = tid; i < nt * k; i += blockDim.x) {
        const int tl = i / k, j = i - tl * k;
        sel[tl * 32 + j] = topk_idx[(size_t)(t0 + tl) * k + j];
    }
    for (int e = tid; e < E; e += blockDim.x) mask[e] = 0ull;
    __syncthreads();
    for (int i = tid; i < nt * k; i += blockDim.x) {
        int tl = i / k, j = i - tl * k;
        atomicOr(&mask[sel[tl * 32 + j]], 1ull << tl);
    }
    __syncthreads();
    if (gridDim.x > 1) {
        for (int e = tid; e < E; e += blockDim.x) {
            chunk_masks[(size_t)c * E + e] = mask[e];
            chunk_cnt[(size_t)c * E + e] = __popcll(mask[e]);
        }
        return;
    }
    // single chunk: finish the grouping in this block
    int cnt = (tid < E) ? __popcll(mask[tid]) : 0;
    int total;
    int excl = block_exclusive_scan(cnt, wave_tot, &total);
    if (tid < E) {
        counts[tid] = cnt;
        offsets[tid] = excl;
        offs[tid] = excl;
    }
    if (tid == 0) offsets[E] = total;
    __syncthreads();
    for (int i = tid; i < nt * k; i += blockDim.x) {
        int tl = i / k, j = i - tl * k;
        int e = sel[tl * 32 + j];
        int row = offs[e] + __popcll(mask[e] & ((1ull << tl) - 1ull));
        int p = (t0 + tl) * k + j;
        perm_pair[row] = p;
        row_of_pair[p] = row;
    }
}

// Multi-chunk grouping, step 2: per expert, prefix over chunks; then a
// block-wide prefix over experts.  One block of 1024 threads (E <= 1024).
__global__ __launch_bounds__(1024) void group_scan_kernel(
    int nch, int E, int P, const int32_t* chunk_cnt, int32_t* chunk_base,  // may alias
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets)
{
    __shared__ int wave_tot[17];
    const int e = threadIdx.x;
    int run = 0;
    if (e < E) {
        for (int c = 0; c < nch; ++c) {
            int v = chunk_cnt[(size_t)c * E + e];
            chunk_base[(size_t)c * E + e] = run;
            run += v;
        }
    }
    int total;
    int excl = block_exclusive_scan(e < E ? run : 0, wave_tot, &total);
    if (e < E) {
        counts[e] = run;
        offsets[e] = excl;
    }
    if (e == 0) offsets[E] = P;
}

// Multi-chunk grouping, step 3: each pair's row = expert offset + rows of the
// expert in earlier chunks + earlier tokens of the same chunk (popcount).
__global__ __launch_bounds__(256) void group_scatter_kernel(
    int P, int E, int k, const int32_t* __restrict__ topk_idx,
    const uint64_t* __restrict__ chunk_masks, const int32_t* __restrict__ chunk_base,
    const int32_t* __restrict__ offsets, int32_t* __restrict__ perm_pair,
    int32_t* __restrict__ row_of_pair)
{
    int p = blockIdx.x * 256 + threadIdx.x;
    if (p >= P) return;
    int t = p / k;
    int e = topk_idx[p];
    int c = t / kChunk, tl = t - c * kChunk;
    size_t ce = (size_t)c * E + e;
    int row = offsets[e] + chunk_base[ce] + __popcll(chunk_masks[ce] & ((1ull << tl) - 1ull));
    perm_pair[row] = p;
    row_of_pair[p] = row;
}

void launch_topk_group(int T, int E, int k, double* logits, const float* bias,
                       int bias_select_only, int sigmoid, int32_t* topk_idx, float* topk_w,
                       uint64_t* chunk_masks, int32_t* chunk_base, int32_t* counts,
                       int32_t* offsets, int32_t* perm_pair, int32_t* row_of_pair,
                       const TopkCert& cert, hipStream_t s)
{
    const int nch = (T + kChunk - 1) / kChunk;
    // chunk_base doubles as the per-chunk count array before the scan
    if (T == 1) {
        topk_group_kernel<true><<<dim3(1), dim3(1024), 0, s>>>(T, E, k, logits, bias, bias_select_only, sigmoid,
                                                               topk_idx, topk_w, chunk_masks, chunk_base, counts,
                                                               offsets, perm_pair, row_of_pair);
        return;
    }
    topk_token_kernel<<<dim3(T), dim3(1024), 0, s>>>(E, k, logits, bias, bias_select_only, sigmoid, topk_idx,
                                                     topk_w, cert.xe, cert.wc, cert.fail);
    if (cert.xe) {
        router_exact_kernel<<<dim3((E + 1) / 2, kFailSlots), dim3(256), 0, s>>>(E, cert.d, cert.x, cert.wr, bias,
                                                                               cert.bias_in_logits, cert.fail, logits);
        topk_fail_kernel<<<dim3(kFailSlots), dim3(1024), 0, s>>>(E, k, logits, bias, bias_select_only, sigmoid,
                                                                topk_idx, topk_w, cert.fail);
    }
    topk_group_kernel<false><<<dim3(nch), dim3(1024), 0, s>>>(T, E, k, logits, bias, bias_select_only, sigmoid,
                                                              topk_idx, topk_w, chunk_masks, chunk_base, counts,
                                                              offsets, perm_pair, row_of_pair);
    if (nch > 1) {
        const int P = T * k;
        group_scan_kernel<<<dim3(1), dim3(1024), 0, s>>>(nch, E, P, chunk_base, chunk_base,
                                                          counts, offsets);
        group_scatter_kernel<<<dim3((P + 255) / 256), dim3(256), 0, s>>>(
            P, E, k, topk_idx, chunk_masks, chunk_base, offsets, perm_pair, row_of_pair);
    }
}

// ---------------------------------------------------------------------------
// Active experts in ascending id (those with at least one token); the count
// goes to active[E].  With mt > 0 also the MXFP4 pass lists: each active
// expert needs ceil(tiles / mt) passes of the GEMMs.  The experts are cut, in
// list order, into eight runs of near-equal total passes (an expert goes to
// XCD floor(8 * passes before it / all passes)), so each XCD's share is within
// one expert's passes of an eighth however the load is skewed (dealing the
// experts round-robin put 1.6 times the mean on one XCD of the skewed
// 256-token batch).  Per XCD x: pslot[x * pstride + j] = its j-th slot,
// passes[x * pstride + j] = passes before it (the XCD's total after the
// last), passes[8 * pstride + x] = its slot count (at most pstride - 1).
__global__ __launch_bounds__(1024) void active_list_kernel(int E, const int32_t* __restrict__ offsets,
                                                           int32_t* __restrict__ active, int mt,
                                                           int32_t* __restrict__ passes,
                                                           int32_t* __restrict__ pslot, int pstride)
{
    __shared__ int wave_tot[17];
    __shared__ int first[8], base[8], cnt[8], sum[8];
    __shared__ int np_of[1024];  // passes of each slot
    const int e = threadIdx.x;
    const int n = (e < E) ? offsets[e + 1] - offsets[e] : 0;
    const int flag = n > 0;
    int total;
    const int pos = block_exclusive_scan(flag, wave_tot, &total);
    if (flag) active[pos] = e;
    if (e == 0) active[E] = total;
    if (mt <= 0) return;
    const int np = flag ? (((n + 15) >> 4) + mt - 1) / mt : 0;
    int ptot;
    const int pre = block_exclusive_scan(np, wave_tot, &ptot);
    if (e < 8) {
        first[e] = 0x7fffffff;
        base[e] = 0x7fffffff;
        cnt[e] = 0;
        sum[e] = 0;
    }
    __syncthreads();
    const int x = flag ? (int)min((8LL * pre) / ptot, 7LL) : 0;
    if (flag) {
        np_of[pos] = np;
        atomicMin(&first[x], pos);
        atomicMin(&base[x], pre);
        atomicAdd(&cnt[x], 1);
        atomicAdd(&sum[x], np);
    }
    __syncthreads();
    // the tables hold pstride - 1 = ceil(E / 8) + 8 slots per XCD; a routing
    // that would put more on one XCD (a few huge experts among many one-pass
    // ones) is dealt round-robin instead
    bool fits = true;
#pragma unroll
    for (int i = 0; i < 8; ++i) fits = fits && cnt[i] <= pstride - 1;
    if (fits) {
        if (flag) {  // an XCD's slots are consecutive
            pslot[x * pstride + pos - first[x]] = pos;
            passes[x * pstride + pos - first[x]] = pre - base[x];
        }
        if (e < 8) {
            passes[e * pstride + cnt[e]] = sum[e];
            passes[8 * pstride + e] = cnt[e];
        }
    } else if (e < 8) {
        int c = 0, j = 0;
        for (; 8 * j + e < total; ++j) {
            pslot[e * pstride + j] = 8 * j + e;
            passes[e * pstride + j] = c;
            c += np_of[8 * j + e];
        }
        passes[e * pstride + j] = c;
        passes[8 * pstride + e] = j;
    }
}

// ceil(E / 8) + 8 slots per XCD (the passes-balanced runs exceed an eighth of
// the experts by a few when all are active), and the total after them
int pass_stride(int E) { return (E + 7) / 8 + 9; }

void launch_active_list(int E, const int32_t* offsets, int32_t* active, int mt, int32_t* passes, int32_t* pslot,
                        int pstride, hipStream_t s)
{
    k3_launch(active_list_kernel, dim3(1), dim3(1024), s, E, offsets, active, mt, passes, pslot, pstride);
}

}  // namespace k3
