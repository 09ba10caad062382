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
// Tile order: the hardware deals consecutive workgroups round-robin to the 8
// XCDs, each with its own L2.  Experts go round-robin to XCDs (slot s -> XCD
// s % 8) and each XCD receives the n-tiles of one expert back to back, so an
// expert's activation rows are read from HBM once and from that XCD's L2 by
// its other tiles; busy and idle experts spread evenly over the XCDs.
constexpr int kXcds = 8;

__device__ __forceinline__ bool xcd_tile(int bid, int nslots, int ntiles, int& slot, int& tile)
{
    const int x = bid % kXcds, pos = bid / kXcds;
    slot = x + kXcds * (pos / ntiles);
    tile = pos % ntiles;
    return slot < nslots;
}

static int xcd_grid(int nslots, int ntiles)
{
    return kXcds * ((nslots + kXcds - 1) / kXcds) * ntiles;
}

// ---------------------------------------------------------------------------
// Grouped scaled-MFMA GEMM building blocks.  A = activation rows of one
// expert (x_q rows of its tokens, or its h_q rows), staged per 512-wide K
// chunk in LDS: row m holds 256 code bytes then the chunk's 16 scale bytes
// (272-byte stride, which also spreads rows over the LDS banks); two buffers,
// the next chunk is fetched into registers while the current one is used.
// B = weight rows, loaded straight into registers (each weight byte is used
// by exactly one wave), also one chunk ahead.
constexpr int kMT = 8;             // 16-token tiles per pass (M <= 128)
constexpr int kARow = 272;         // LDS bytes per staged activation row
constexpr int kAStage = 16 * kMT * kARow;

// Stage the A chunk kc into an LDS buffer with the gfx950 direct
// global->LDS load (lane l of a wave instruction lands at M0 + 16*l): item
// it = 17*r + c (16 code pieces then the scale piece of row r) goes to LDS
// byte 16*it, i.e. row r at r*kARow.  Rows past the expert's tokens repeat its
// last row; their outputs are discarded.
__device__ __forceinline__ void a_issue(const uint8_t* const* rows_c, const uint8_t* const* rows_s, int nrows,
                                        int mt_n, int kc, uint8_t* dst)
{
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int n_items = 16 * mt_n * 17;  // a multiple of 64 when mt_n is even; else the tail is masked
#pragma unroll
    for (int i = 0; i < 9; ++i) {
        const int base = 256 * i + 64 * wave;
        if (base >= n_items) break;
        const int it = base + lane;
        if (it < n_items) {
            const int r = min(it / 17, nrows - 1), c = it - (it / 17) * 17;
            const uint8_t* src = c < 16 ? rows_c[r] + (kc >> 1) + 16 * c : rows_s[r] + (kc >> 5);
            __builtin_amdgcn_global_load_lds(src, dst + 16 * base, 16, 0, 0);
        }
    }
}

// A fragment of M-tile mt for this lane (row 16*mt + li, quarter g)
__device__ __forceinline__ void a_frag(const uint8_t* lds, int mt, int li, int g, Frag512& f)
{
    const uint8_t* row = lds + (16 * mt + li) * kARow;
#pragma unroll
    for (int i = 0; i < 4; ++i) f.q[i] = *reinterpret_cast<const uint4*>(row + 64 * g + 16 * i);
    f.s = *reinterpret_cast<const uint32_t*>(row + 256 + 4 * g);
}

template <int NB>
__device__ __forceinline__ void b_fetch(Frag512 (&F)[NB], const uint8_t* const (&bc)[NB],
                                        const uint8_t* const (&bs)[NB], int kc, int g)
{
#pragma unroll
    for (int s = 0; s < NB; ++s) load_frag512(bc[s], bs[s], kc, g, F[s]);
}

// M-tiles one at a time, the next tile's A fragment read from LDS while the
// current one is on the matrix cores (keeps at most two fragments live)
template <int NB>
__device__ __forceinline__ void mma_chunk(const Frag512 (&F)[NB], const uint8_t* lds, int mt_n, int li, int g,
                                          f32x4 (&c)[kMT][NB])
{
    Frag512 fa, fn;
    a_frag(lds, 0, li, g, fa);
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt) {
        if (mt < mt_n) {
            if (mt + 1 < mt_n) a_frag(lds, mt + 1, li, g, fn);
#pragma unroll
            for (int s = 0; s < NB; ++s) {
                c[mt][s] = mfma_fp4<0>(fa.q[0], F[s].q[0], fa.s, F[s].s, c[mt][s]);
                c[mt][s] = mfma_fp4<1>(fa.q[1], F[s].q[1], fa.s, F[s].s, c[mt][s]);
                c[mt][s] = mfma_fp4<2>(fa.q[2], F[s].q[2], fa.s, F[s].s, c[mt][s]);
                c[mt][s] = mfma_fp4<3>(fa.q[3], F[s].q[3], fa.s, F[s].s, c[mt][s]);
            }
            fa = fn;
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}

// The K loop of one M pass (K % 512 == 0): LDS double buffer for A filled by
// DMA one chunk ahead; the B fragments of a chunk are loaded at its start
// (their latency overlaps the other resident waves' matrix work).
template <int NB>
__device__ __forceinline__ void gemm_pass512(const uint8_t* const* rows_c, const uint8_t* const* rows_s, int nrows,
                                             const uint8_t* const (&bc)[NB], const uint8_t* const (&bs)[NB],
                                             int K, int mt_n, int li, int g, uint8_t* lds, f32x4 (&c)[kMT][NB])
{
    Frag512 F[NB];
    a_issue(rows_c, rows_s, nrows, mt_n, 0, lds);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    int buf = 0;
    for (int kc = 0; kc < K; kc += 512) {
        b_fetch<NB>(F, bc, bs, kc, g);
        const bool more = kc + 512 < K;
        if (more) a_issue(rows_c, rows_s, nrows, mt_n, kc + 512, lds + (buf ^ 1) * kAStage);
        mma_chunk<NB>(F, lds + buf * kAStage, mt_n, li, g, c);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();  // next buffer landed; every wave is done with this one
        buf ^= 1;
    }
}

// 128-wide K steps for reduction axes that are not a multiple of 512 (small
// layers); A straight from global memory.
template <int NB>
__device__ __forceinline__ void gemm_pass128(const uint8_t* const* rows_c, const uint8_t* const* rows_s, int nrows,
                                             const uint8_t* const (&bc)[NB], const uint8_t* const (&bs)[NB],
                                             int K, int mt_n, int li, int g, f32x4 (&c)[kMT][NB])
{
    for (int kc = 0; kc < K; kc += 128) {
        uint4 qb[NB];
        uint32_t sb[NB];
#pragma unroll
        for (int s = 0; s < NB; ++s) load_frag128(bc[s], bs[s], kc, g, K, qb[s], sb[s]);
#pragma unroll
        for (int mt = 0; mt < kMT; ++mt) {
            if (mt < mt_n) {
                const int r = min(16 * mt + li, nrows - 1);
                uint4 qa;
                uint32_t sa;
                load_frag128(rows_c[r], rows_s[r], kc, g, K, qa, sa);
#pragma unroll
                for (int s = 0; s < NB; ++s) c[mt][s] = mfma_fp4<0>(qa, qb[s], sa, sb[s], c[mt][s]);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// gate/up GEMM: block = 4 waves, n-tile = 64 f rows; wave w owns gate rows
// and up rows [n0 + 16w, +16).  M = the expert's tokens, up to 128 per pass.
// Epilogue: h = silu(g) * u in fp32; the MX quantiser runs over each token's
// 32 consecutive f values, held by two neighbouring waves' subtiles, so the
// block exchanges h through LDS once per pass.
constexpr int kGuTile = 64;

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void gateup_mfma_kernel(FfnArgs a, const uint8_t* __restrict__ xqc,
                                                          const uint8_t* __restrict__ xqs,
                                                          uint8_t* __restrict__ hqc,
                                                          uint8_t* __restrict__ hqs,
                                                          float* __restrict__ dbg_h,
                                                          uint8_t* __restrict__ dbg_hc,
                                                          uint8_t* __restrict__ dbg_hs)
{
    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * kAStage];
    __shared__ const uint8_t* rows_c[16 * kMT];
    __shared__ const uint8_t* rows_s[16 * kMT];
    const int ntiles = (a.f + kGuTile - 1) / kGuTile;
    int slot, ftile;
    if (!xcd_tile(blockIdx.x, a.nslots, ntiles, slot, ftile)) return;
    int e, r_beg, n_e;
    if (!mx_slot_expert(a, slot, e, r_beg, n_e)) return;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int li = lane & 15, g = lane >> 4;
    const int n0 = ftile * kGuTile;
    const int nrow_w = min(n0 + 16 * wave, a.f - 16);  // f % 32 == 0: a partial tile repeats rows, masked below
    const int K = a.d;
    const size_t crow = (size_t)(K >> 1), srow = (size_t)(K >> 5);
    const uint8_t* bc[2];
    const uint8_t* bs[2];
    {
        const size_t wr = (size_t)e * a.f + nrow_w + li;
        bc[0] = a.gc + wr * crow;
        bs[0] = a.gs + wr * srow;
        bc[1] = a.uc + wr * crow;
        bs[1] = a.us + wr * srow;
    }
    float* hx = reinterpret_cast<float*>(lds);  // h exchange after the K loop: [128][64] fp32 = 32 KB
    for (int m0 = 0; m0 < n_e; m0 += 16 * kMT) {
        const int nrows = min(16 * kMT, n_e - m0);
        const int mt_n = (nrows + 15) >> 4;
        if (threadIdx.x < 16 * kMT) {
            const int m = min(m0 + (int)threadIdx.x, n_e - 1);
            const int tok = a.perm_pair[r_beg + m] / a.k;
            rows_c[threadIdx.x] = xqc + (size_t)tok * crow;
            rows_s[threadIdx.x] = xqs + (size_t)tok * srow;
        }
        __syncthreads();
        f32x4 c[kMT][2];
#pragma unroll
        for (int mt = 0; mt < kMT; ++mt) {
            c[mt][0] = (f32x4){0.f, 0.f, 0.f, 0.f};
            c[mt][1] = (f32x4){0.f, 0.f, 0.f, 0.f};
        }
        if ((K % 512) == 0)
            gemm_pass512<2>(rows_c, rows_s, nrows, bc, bs, K, mt_n, li, g, lds, c);
        else
            gemm_pass128<2>(rows_c, rows_s, nrows, bc, bs, K, mt_n, li, g, c);
        // h of this wave's 16 columns -> LDS [m][16*wave + col]
#pragma unroll
        for (int mt = 0; mt < kMT; ++mt) {
            if (mt < mt_n) {
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int m = 16 * mt + 4 * g + v;
                    hx[m * kGuTile + 16 * wave + li] = silu_f32(c[mt][0][v]) * c[mt][1][v];
                }
            }
        }
        __syncthreads();
        // quantise: one thread per (token row, 32-column block): 128 x 2 items
        for (int it = threadIdx.x; it < nrows * (kGuTile / 32); it += 256) {
            const int m = it >> 1, hb = it & 1;
            const int col0 = n0 + 32 * hb;
            if (col0 < a.f) {
                const float* hv = hx + m * kGuTile + 32 * hb;
                float amax = 0.f;
#pragma unroll
                for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(hv[i]));
                const uint32_t byte = mx_scale_byte(amax);
                const float inv = mx_inv_scale(byte);
                uint32_t w4[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    uint32_t wv = 0;
#pragma unroll
                    for (int i = 0; i < 8; ++i) wv |= e2m1_encode(hv[8 * q + i], inv) << (4 * i);
                    w4[q] = wv;
                }
                const size_t r = (size_t)(r_beg + m0 + m);
                const size_t fcb = (size_t)(a.f >> 1), fsb = (size_t)(a.f >> 5);
                const int blk = col0 >> 5;
                *reinterpret_cast<uint4*>(hqc + r * fcb + 16 * blk) = make_uint4(w4[0], w4[1], w4[2], w4[3]);
                hqs[r * fsb + blk] = (uint8_t)byte;
                if (dbg_h || dbg_hc || dbg_hs) {
                    const int pair = a.perm_pair[r];
                    if (dbg_hc) *reinterpret_cast<uint4*>(dbg_hc + (size_t)pair * fcb + 16 * blk) = make_uint4(w4[0], w4[1], w4[2], w4[3]);
                    if (dbg_hs) dbg_hs[(size_t)pair * fsb + blk] = (uint8_t)byte;
                    if (dbg_h) {
#pragma unroll
                        for (int i = 0; i < 32; ++i) dbg_h[(size_t)pair * a.f + col0 + i] = hv[i];
                    }
                }
            }
        }
        __syncthreads();
    }
}

void launch_gateup_mfma(const FfnArgs& a, const uint8_t* xq_codes, const uint8_t* xq_scales,
                        uint8_t* hq_codes, uint8_t* hq_scales, float* dbg_h, uint8_t* dbg_hc,
                        uint8_t* dbg_hs, hipStream_t s)
{
    const int grid = xcd_grid(a.nslots, (a.f + kGuTile - 1) / kGuTile);
    gateup_mfma_kernel<<<dim3(grid), dim3(256), 0, s>>>(a, xq_codes, xq_scales, hq_codes, hq_scales, dbg_h,
                                                        dbg_hc, dbg_hs);
}

// ---------------------------------------------------------------------------
// down GEMM: block = 4 waves, n-tile = 128 d rows; wave w owns rows
// [n0 + 32w, +32) as two 16-row subtiles; A = the expert's h_q rows
// (contiguous in grouped order).  Epilogue: y[t][c] += w[t,j] * o[c], fp32
// atomic add (the combine).
constexpr int kDnTile = 128;

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void down_mfma_kernel(FfnArgs a, const uint8_t* __restrict__ hqc,
                                                        const uint8_t* __restrict__ hqs,
                                                        float* __restrict__ y, float* __restrict__ o)
{
    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * kAStage];
    __shared__ const uint8_t* rows_c[16 * kMT];
    __shared__ const uint8_t* rows_s[16 * kMT];
    const int ntiles = (a.d + kDnTile - 1) / kDnTile;
    int slot, dtile;
    if (!xcd_tile(blockIdx.x, a.nslots, ntiles, slot, dtile)) return;
    int e, r_beg, n_e;
    if (!mx_slot_expert(a, slot, e, r_beg, n_e)) return;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int li = lane & 15, g = lane >> 4;
    const int nw = dtile * kDnTile + wave * 32;
    const int K = a.f;
    const size_t crow = (size_t)(K >> 1), srow = (size_t)(K >> 5);
    const uint8_t* bc[2];
    const uint8_t* bs[2];
    bool sub_ok[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        const int n = nw + 16 * s;
        sub_ok[s] = n < a.d;  // d % 32 == 0: 16-row subtiles are whole
        const size_t wr = (size_t)e * a.d + (sub_ok[s] ? n : 0) + li;
        bc[s] = a.dc + wr * crow;
        bs[s] = a.ds + wr * srow;
    }
    for (int m0 = 0; m0 < n_e; m0 += 16 * kMT) {
        const int nrows = min(16 * kMT, n_e - m0);
        const int mt_n = (nrows + 15) >> 4;
        if (threadIdx.x < 16 * kMT) {
            const size_t r = (size_t)(r_beg + min(m0 + (int)threadIdx.x, n_e - 1));
            rows_c[threadIdx.x] = hqc + r * crow;
            rows_s[threadIdx.x] = hqs + r * srow;
        }
        __syncthreads();
        f32x4 c[kMT][2];
#pragma unroll
        for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
            for (int s = 0; s < 2; ++s) c[mt][s] = (f32x4){0.f, 0.f, 0.f, 0.f};
        if ((K % 512) == 0)
            gemm_pass512<2>(rows_c, rows_s, nrows, bc, bs, K, mt_n, li, g, lds, c);
        else
            gemm_pass128<2>(rows_c, rows_s, nrows, bc, bs, K, mt_n, li, g, c);
#pragma unroll
        for (int mt = 0; mt < kMT; ++mt) {
            if (mt >= mt_n) break;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int m = m0 + 16 * mt + 4 * g + v;
                if (m < n_e) {
                    if (o) {
                        // per-pair output row (grouped order); the combine kernel gathers
                        float* orow = o + (size_t)(r_beg + m) * a.d + nw + li;
#pragma unroll
                        for (int s = 0; s < 2; ++s)
                            if (sub_ok[s]) orow[16 * s] = c[mt][s][v];
                    } else {
                        const int pair = a.perm_pair[r_beg + m];
                        const int t = pair / a.k;
                        const float w = a.topk_w[pair];
                        float* yr = y + (size_t)t * a.d + nw + li;
#pragma unroll
                        for (int s = 0; s < 2; ++s)
                            if (sub_ok[s]) unsafeAtomicAdd(yr + 16 * s, w * c[mt][s][v]);
                    }
                }
            }
        }
        __syncthreads();  // rows_c / rows_s reused by the next pass
    }
}

void launch_down_mfma(const FfnArgs& a, const uint8_t* hq_codes, const uint8_t* hq_scales, float* y,
                      float* o, hipStream_t s)
{
    const int grid = xcd_grid(a.nslots, (a.d + kDnTile - 1) / kDnTile);
    down_mfma_kernel<<<dim3(grid), dim3(256), 0, s>>>(a, hq_codes, hq_scales, y, o);
}

}  // namespace k3
