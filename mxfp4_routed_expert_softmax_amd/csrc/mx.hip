// mx.hip -- MXFP4-activation expert FFN for gfx950: activation quantiser,
// grouped gate/up GEMM with fused SwiGLU + h quantiser, grouped down GEMM
// writing one fp32 output row per token-expert pair (the gate-weighted
// combine of those rows is combine_kernel, a deterministic gather).  Both
// GEMMs run on the CDNA4 scaled matrix cores (V_MFMA_SCALE_F32_16X16X128_F8F6F4,
// FP4 x FP4 with E8M0 block scales, fp32 accumulate).
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
#include "launch.h"

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
    k3_launch(quantize_rows_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), s, nblocks, v, codes,
              scales);
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

// One operand row-lane's share of a 512-wide K chunk: for each of the four
// 128-wide matrix steps i, the 16 code bytes of block 4i + g (lane quarter
// g), and the four blocks' scale bytes in one word (byte i for step i).
struct Frag512 {
    uint4 q[4];
    uint32_t s;
};

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
// XCDs, each with its own L2.  Without pass lists (few pairs: slots are
// segment heads) experts go round-robin to XCDs (slot s -> XCD s % 8) and
// each XCD receives the n-tiles of one expert back to back, so an expert's
// activation rows are read from HBM once and from that XCD's L2 by its other
// tiles.  With an active list, the pass lists place the experts instead
// (active_list_kernel: eight runs of equal passes).
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
// Epilogues shared by both GEMM forms.  Accumulator c[mt][s] of lane
// (g, li) holds row (token) 16*mt + 4*g + v, column li of subtile s.
constexpr int kMT = 8;  // 16-token tiles per pass (M <= 128)

// Eight values -> eight E2M1 codes in one word (element 2i in the low
// nibble of byte i): the gfx950 convert rounds to nearest even and
// saturates at 6, keeping the sign (the OCP rule above); the scale is
// applied beforehand as an exact power-of-two product.
__device__ __forceinline__ uint32_t e2m1_pack8(const float* v, float inv)
{
    uint32_t w = 0u;
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[0] * inv, v[1] * inv, 1.0f, 0);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[2] * inv, v[3] * inv, 1.0f, 1);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[4] * inv, v[5] * inv, 1.0f, 2);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[6] * inv, v[7] * inv, 1.0f, 3);
    return w;
}

// gate/up: h = silu(g) * u of this wave's 16 columns -> LDS hx [m][64] (row
// stride 65 words, so that the quantiser's per-row reads fall on distinct
// banks), then the MX quantiser over each token's 32 consecutive f values
// (held by two neighbouring waves), one thread per (row, 32-column block).
constexpr int kHxStride = 65;

template <int MT>
__device__ __forceinline__ void gateup_epilogue(const FfnArgs& a, const f32x4 (&c)[MT][2], float* hx, int mt_n,
                                                int nrows, int m0, int r_beg, int n0, int wave, int li, int g,
                                                uint8_t* __restrict__ hqc, uint8_t* __restrict__ hqs,
                                                float* __restrict__ dbg_h, uint8_t* __restrict__ dbg_hc,
                                                uint8_t* __restrict__ dbg_hs)
{
    constexpr int kW = 64;  // f columns per block
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        if (mt < mt_n) {
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int m = 16 * mt + 4 * g + v;
                hx[m * kHxStride + 16 * wave + li] = silu_f32(c[mt][0][v]) * c[mt][1][v];
            }
        }
    }
    __syncthreads();
    for (int it = threadIdx.x; it < nrows * (kW / 32); it += 256) {
        const int m = it >> 1, hb = it & 1;
        const int col0 = n0 + 32 * hb;
        if (col0 < a.f) {
            float hv[32];
#pragma unroll
            for (int i = 0; i < 32; ++i) hv[i] = hx[m * kHxStride + 32 * hb + i];
            float amax = 0.f;
#pragma unroll
            for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(hv[i]));
            const uint32_t byte = mx_scale_byte(amax);
            const float inv = mx_inv_scale(byte);
            const uint4 w4 = make_uint4(e2m1_pack8(hv, inv), e2m1_pack8(hv + 8, inv), e2m1_pack8(hv + 16, inv),
                                        e2m1_pack8(hv + 24, inv));
            const size_t r = (size_t)(r_beg + m0 + m);
            const size_t fcb = (size_t)(a.f >> 1), fsb = (size_t)(a.f >> 5);
            const int blk = col0 >> 5;
            *reinterpret_cast<uint4*>(hqc + r * fcb + 16 * blk) = w4;
            hqs[r * fsb + blk] = (uint8_t)byte;
            if (dbg_h || dbg_hc || dbg_hs) {
                const int pair = a.perm_pair[r];
                if (dbg_hc) *reinterpret_cast<uint4*>(dbg_hc + (size_t)pair * fcb + 16 * blk) = w4;
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

// down: per-pair fp32 rows o (grouped order) for the deterministic combine;
// subtile s of this wave covers d rows nw + 16*s .. +15
template <int MT, bool NT>
__device__ __forceinline__ void down_epilogue(const FfnArgs& a, const f32x4 (&c)[MT][2], int mt_n, int m0,
                                              int n_e, int r_beg, int nw, const bool (&sub_ok)[2], int li, int g,
                                              float* __restrict__ o)
{
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        if (mt >= mt_n) break;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int m = m0 + 16 * mt + 4 * g + v;
            if (m < n_e) {
                float* orow = o + (size_t)(r_beg + m) * a.d + nw + li;
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    if (sub_ok[s]) {
                        if (NT)  // rows written once and read once (FfnArgs::o_stream)
                            __builtin_nontemporal_store(c[mt][s][v], orow + 16 * s);
                        else
                            orow[16 * s] = c[mt][s][v];
                    }
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Any K (a multiple of 32; the small layers): 128-wide K steps, both
// operands straight from global memory, zeros past the row end.
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

// gate/up GEMM: block = 4 waves, n-tile = 64 f rows; wave w owns gate rows
// and up rows [n0 + 16w, +16).  M = the expert's tokens, up to 128 per pass.
constexpr int kGuTile = 64;

__global__ __launch_bounds__(256) void gateup_mfma_kernel(FfnArgs a, const uint8_t* __restrict__ xqc,
                                                          const uint8_t* __restrict__ xqs,
                                                          uint8_t* __restrict__ hqc,
                                                          uint8_t* __restrict__ hqs,
                                                          float* __restrict__ dbg_h,
                                                          uint8_t* __restrict__ dbg_hc,
                                                          uint8_t* __restrict__ dbg_hs)
{
    __shared__ float hx[16 * kMT * kHxStride];
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
        const size_t wr = (size_t)wslot(a, e) * a.f + nrow_w + li;
        bc[0] = a.gc + wr * crow;
        bs[0] = a.gs + wr * srow;
        bc[1] = a.uc + wr * crow;
        bs[1] = a.us + wr * srow;
    }
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
        gemm_pass128<2>(rows_c, rows_s, nrows, bc, bs, K, mt_n, li, g, c);
        gateup_epilogue<kMT>(a, c, hx, mt_n, nrows, m0, r_beg, n0, wave, li, g, hqc, hqs, dbg_h, dbg_hc, dbg_hs);
    }
}

// down GEMM: block = 4 waves, n-tile = 128 d rows; wave w owns rows
// [n0 + 32w, +32) as two 16-row subtiles; A = the expert's h_q rows
// (contiguous in grouped order).
constexpr int kDnTile = 128;

__global__ __launch_bounds__(256) void down_mfma_kernel(FfnArgs a, const uint8_t* __restrict__ hqc,
                                                        const uint8_t* __restrict__ hqs, float* __restrict__ o)
{
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
        const size_t wr = (size_t)wslot(a, e) * a.d + (sub_ok[s] ? n : 0) + li;
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
        gemm_pass128<2>(rows_c, rows_s, nrows, bc, bs, K, mt_n, li, g, c);
        if (a.o_stream)
            down_epilogue<kMT, true>(a, c, mt_n, m0, n_e, r_beg, nw, sub_ok, li, g, o);
        else
            down_epilogue<kMT, false>(a, c, mt_n, m0, n_e, r_beg, nw, sub_ok, li, g, o);
        __syncthreads();  // rows_c / rows_s reused by the next pass
    }
}

// ---------------------------------------------------------------------------
// K % 512 == 0 (the layer's d_model and d_ff): a pipelined form.
//
// A = the expert's activation rows (x_q rows of its tokens, or its h_q
// rows), copied per 512-wide K chunk into LDS by direct global->LDS copies;
// two stages, chunk i+1 is copied while chunk i is used.  Stage layout (up to
// 96 rows): row r's 16 code pieces of 16 bytes at 256*r + 16*(p ^ (r & 15))
// -- the XOR puts the 16 rows of one fragment read on distinct LDS banks --
// then the rows' 16 chunk scale bytes at kACodes + 16*r.
//
// B = weight rows.  Their codes are buffer-loaded straight into registers
// (each byte is used by exactly one wave) one chunk ahead of the matrix
// work; matrix step i takes K range [128i, 128i + 128) of the chunk, so one
// load instruction reads 64 contiguous bytes of each of 16 rows (measured
// ~9 % faster than 16-byte pieces at a 64-byte stride, which touch twice the
// cache lines per instruction); their E8M0 scales -- 16 bytes per row and chunk, which as separate
// loads would cost as many cache-line requests as the codes -- are copied
// into LDS once per block (the block's rows are contiguous, so the copy is
// one contiguous run per weight matrix) and read from there.
constexpr int kPassMT = 6;  // 16-token tiles per pass (the register budget of two blocks per CU)
constexpr int kACodes = 256 * 16 * kPassMT;
constexpr int kAStage = kACodes + 16 * 16 * kPassMT;
constexpr int kBLoads = 8;          // B code loads per chunk (two subtiles x 4)
constexpr int kBScaleBytes = 28672; // LDS for the block's weight scales: 128 rows x K/32 (K <= 7168)
constexpr int kMxLds = 2 * kAStage + kBScaleBytes;

// Weight codes of one wave's two 16-row subtiles: buffer resources on the
// subtiles' first rows and a per-lane offset (row li, quarter g); the
// lane's scale words are at LDS offset bso[s] + kc/32.
struct BSrc {
    __amdgpu_buffer_rsrc_t rc[2];
    uint32_t voc;
    uint32_t bso[2];
};

__device__ __forceinline__ void b_fetch(const BSrc& b, int kc, Frag512 (&F)[2])
{
#pragma unroll
    for (int s = 0; s < 2; ++s) {
#pragma unroll
        for (int i = 0; i < 4; ++i) F[s].q[i] = ld_codes(b.rc[s], b.voc + 64u * i, (uint32_t)(kc >> 1));
    }
}


// Per-thread copy offsets of the A stage, fixed over the K loop: code copy q
// of wave w moves rows 4*(4q+w) .. +3, one 16-byte piece per lane; wave 0
// copies the scale pieces of rows 0..63, wave 1 those of rows 64..95.  Rows
// past the expert's tokens repeat its last row (their outputs are discarded).
struct ASrc {
    uint32_t oc[kPassMT], os;
};

__device__ __forceinline__ void a_offsets(const uint32_t* rowtok, int nrows, uint32_t crow, uint32_t srow, ASrc& A)
{
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
    for (int q = 0; q < kPassMT; ++q) {
        const int r = 4 * (4 * q + wave) + (lane >> 4), p = lane & 15;
        A.oc[q] = rowtok[min(r, nrows - 1)] * crow + 16u * (uint32_t)(p ^ (r & 15));
    }
    A.os = rowtok[min(64 * (wave & 1) + lane, nrows - 1)] * srow;
}

// Copy A chunk kc into an LDS stage (assembly copies, awaited explicitly)
__device__ __forceinline__ void a_issue(const ASrc& A, const uint8_t* cbase, const uint8_t* sbase, int kc,
                                        uint32_t dst)
{
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const uint8_t* cb = cbase + (kc >> 1);
#pragma unroll
    for (int q = 0; q < kPassMT; ++q) dma16(cb, A.oc[q], dst + 1024u * (uint32_t)(4 * q + wave));
    if (wave < 2 && 64 * wave + lane < 16 * kPassMT)
        dma16(sbase + (kc >> 5), A.os, dst + (uint32_t)kACodes + 1024u * (uint32_t)wave);
}

// This lane's LDS read offsets within a stage for M-tile 0: code pieces
// 4g+i of row li (XOR-swizzled) and the scale word of quarter g; tile mt adds
// 4096*mt (256*mt for the scales) -- immediate offsets of the LDS reads.
struct AOffs {
    uint32_t q[4], s, sel;
};

// The lane's four block scales (blocks g, 4+g, 8+g, 12+g of the chunk, one
// per 128-wide step) out of the row's 16 chunk scale bytes w, as one word
__device__ __forceinline__ uint32_t gather_scales(uint4 w, uint32_t sel)
{
    const uint32_t lo = __builtin_amdgcn_perm(w.y, w.x, sel);
    const uint32_t hi = __builtin_amdgcn_perm(w.w, w.z, sel);
    return __builtin_amdgcn_perm(hi, lo, 0x05040100u);
}

__device__ __forceinline__ AOffs a_read_offsets(int li, int g)
{
    AOffs o;
#pragma unroll
    for (int i = 0; i < 4; ++i) o.q[i] = (uint32_t)(256 * li + 16 * ((4 * i + g) ^ li));
    o.s = (uint32_t)(kACodes + 16 * li);
    o.sel = (uint32_t)g | ((uint32_t)(4 + g) << 8) | 0x0c0c0000u;
    return o;
}

// A fragment of M-tile MT_ (row 16*MT_ + li, quarter g) from stage st
template <int MT_>
__device__ __forceinline__ void a_frag(const uint8_t* st, const AOffs& o, Frag512& f)
{
#pragma unroll
    for (int i = 0; i < 4; ++i) f.q[i] = *reinterpret_cast<const uint4*>(st + o.q[i] + 4096 * MT_);
    f.s = gather_scales(*reinterpret_cast<const uint4*>(st + o.s + 256 * MT_), o.sel);
}

template <int MT_, int MT>
__device__ __forceinline__ void mma_tiles(const Frag512 (&F)[2], const uint32_t (&sb)[2], const uint8_t* st,
                                          const AOffs& o, const Frag512& fa, f32x4 (&c)[MT][2])
{
    Frag512 fn;
    if constexpr (MT_ + 1 < MT) a_frag<MT_ + 1>(st, o, fn);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        c[MT_][s] = mfma_fp4<0>(fa.q[0], F[s].q[0], fa.s, sb[s], c[MT_][s]);
        c[MT_][s] = mfma_fp4<1>(fa.q[1], F[s].q[1], fa.s, sb[s], c[MT_][s]);
        c[MT_][s] = mfma_fp4<2>(fa.q[2], F[s].q[2], fa.s, sb[s], c[MT_][s]);
        c[MT_][s] = mfma_fp4<3>(fa.q[3], F[s].q[3], fa.s, sb[s], c[MT_][s]);
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (MT_ + 1 < MT) mma_tiles<MT_ + 1, MT>(F, sb, st, o, fn, c);
}

// The MT M-tiles of chunk kc from stage st, one at a time, the next tile's A
// fragment read from LDS while the current one is on the matrix cores
template <int MT>
__device__ __forceinline__ void mma_chunk(const Frag512 (&F)[2], const BSrc& B, const uint8_t* lds, int kc,
                                          const uint8_t* st, const AOffs& o, f32x4 (&c)[MT][2])
{
    const uint8_t* bsc = lds + 2 * kAStage + (kc >> 5);
    const uint32_t sb[2] = {gather_scales(*reinterpret_cast<const uint4*>(bsc + B.bso[0]), o.sel),
                            gather_scales(*reinterpret_cast<const uint4*>(bsc + B.bso[1]), o.sel)};
    Frag512 fa;
    a_frag<0>(st, o, fa);
    mma_tiles<0, MT>(F, sb, st, o, fa, c);
    // keep the matrix work here: without a use, the compiler may sink it
    // past the copies and the barrier that follow
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        asm volatile("" : "+v"(c[mt][0]));
        asm volatile("" : "+v"(c[mt][1]));
    }
}

// Chunk i < nk-1, its A stage BUF = i & 1: fetch B chunk i+1 into Fn; wait
// until only those loads are in flight (B chunk i, and every copy issued
// before it -- the A copy of chunk i -- have landed); barrier (every wave's
// part of A chunk i is visible, and every wave is done with the other stage);
// copy A chunk i+1 into the other stage; run chunk i.  B is in flight one
// chunk ahead, about two chunks of every wave's weight stream at the wait.
template <int BUF, int MT>
__device__ __forceinline__ void gemm_step(const ASrc& A, const BSrc& B, const uint8_t* cbase, const uint8_t* sbase,
                                          int i, const AOffs& o, uint8_t* lds, const Frag512 (&Fc)[2],
                                          Frag512 (&Fn)[2], f32x4 (&c)[MT][2])
{
    b_fetch(B, 512 * (i + 1), Fn);
    __builtin_amdgcn_sched_barrier(0);
    vm_wait<kBLoads>();
    __syncthreads();
    a_issue(A, cbase, sbase, 512 * (i + 1), lds_addr(lds) + (uint32_t)((BUF ^ 1) * kAStage));
    __builtin_amdgcn_sched_barrier(0);
    mma_chunk<MT>(Fc, B, lds, 512 * i, lds + BUF * kAStage, o, c);
    __builtin_amdgcn_sched_barrier(0);
}

// the last chunk: nothing left to fetch; the closing barrier frees the LDS
// for the epilogue
template <int BUF, int MT>
__device__ __forceinline__ void gemm_last(const BSrc& B, int i, const AOffs& o, uint8_t* lds,
                                          const Frag512 (&Fc)[2], f32x4 (&c)[MT][2])
{
    vm_wait<0>();
    __syncthreads();
    mma_chunk<MT>(Fc, B, lds, 512 * i, lds + BUF * kAStage, o, c);
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
}

// One M pass of MT tiles over the whole K axis (nk = K/512 chunks): two B
// register sets and the two A stages swap roles every chunk (the loop body
// holds two chunks, so no register copies).  On entry every wave has issued
// the copies the first chunk needs (weight scales, if this is the block's
// first pass); they land before the first wait returns.
template <int MT>
__device__ __forceinline__ void gemm_pass512(const ASrc& A, const BSrc& B, const uint8_t* cbase,
                                             const uint8_t* sbase, int K, const AOffs& o, uint8_t* lds,
                                             f32x4 (&c)[MT][2])
{
    const int nk = K >> 9;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        c[mt][0] = (f32x4){0.f, 0.f, 0.f, 0.f};
        c[mt][1] = (f32x4){0.f, 0.f, 0.f, 0.f};
    }
    Frag512 F0[2], F1[2];
    a_issue(A, cbase, sbase, 0, lds_addr(lds));
    b_fetch(B, 0, F0);
    __builtin_amdgcn_sched_barrier(0);
    int i = 0;
    for (; i + 1 < nk; i += 2) {
        gemm_step<0, MT>(A, B, cbase, sbase, i, o, lds, F0, F1, c);
        if (i + 2 >= nk) {
            gemm_last<1, MT>(B, i + 1, o, lds, F1, c);
            return;
        }
        gemm_step<1, MT>(A, B, cbase, sbase, i + 1, o, lds, F1, F0, c);
    }
    gemm_last<0, MT>(B, i, o, lds, F0, c);
}

template <int MT>
__device__ __forceinline__ void gateup_pass(const FfnArgs& a, const ASrc& A, const BSrc& B, const uint8_t* xqc,
                                            const uint8_t* xqs, int mt_n, int nrows, int m0, int r_beg, int n0,
                                            int wave, int li, int g, uint8_t* lds, uint8_t* hqc, uint8_t* hqs,
                                            float* dbg_h, uint8_t* dbg_hc, uint8_t* dbg_hs)
{
    f32x4 c[MT][2];
    gemm_pass512<MT>(A, B, xqc, xqs, a.d, a_read_offsets(li, g), lds, c);
    gateup_epilogue<MT>(a, c, reinterpret_cast<float*>(lds), mt_n, nrows, m0, r_beg, n0, wave, li, g, hqc, hqs,
                        dbg_h, dbg_hc, dbg_hs);
}

template <int MT>
__device__ __forceinline__ void down_pass(const FfnArgs& a, const ASrc& A, const BSrc& B, const uint8_t* cbase,
                                          const uint8_t* sbase, int mt_n, int m0, int n_e, int r_beg, int nw,
                                          const bool (&sub_ok)[2], int li, int g, uint8_t* lds, float* o)
{
    f32x4 c[MT][2];
    gemm_pass512<MT>(A, B, cbase, sbase, a.f, a_read_offsets(li, g), lds, c);
    if (a.o_stream)
        down_epilogue<MT, true>(a, c, mt_n, m0, n_e, r_beg, nw, sub_ok, li, g, o);
    else
        down_epilogue<MT, false>(a, c, mt_n, m0, n_e, r_beg, nw, sub_ok, li, g, o);
}

// Every pass runs kPassMT tiles (a fixed set of accumulator registers;
// tiles past the pass's rows compute on repeated rows and are discarded).
// Shapes: d_model and d_ff multiples of 512 and at most 7168 (the weight
// scales of a block fit the LDS), d_ff a multiple of 64 (whole gate/up
// tiles) and d_model a multiple of 128 (whole down tiles).
bool use_mx512(const FfnArgs& a)
{
    return a.d % 512 == 0 && a.f % 512 == 0 && a.d <= 7168 && a.f <= 7168 && a.f % kGuTile == 0 &&
           a.d % kDnTile == 0;
}

// Passes p0 .. p1-1 of expert e (rows r_beg .., n_e tokens) against f tile
// ftile: the block's weight scales to LDS, then one GEMM pass per <= kPassMT
// token tiles (balanced tile counts).
__device__ __forceinline__ void gateup_mx_item(const FfnArgs& a, int e, int r_beg, int n_e, int ftile, int p0,
                                               int p1, uint8_t* lds, uint32_t* rowtok,
                                               const uint8_t* __restrict__ xqc, const uint8_t* __restrict__ xqs,
                                               uint8_t* __restrict__ hqc, uint8_t* __restrict__ hqs,
                                               float* __restrict__ dbg_h, uint8_t* __restrict__ dbg_hc,
                                               uint8_t* __restrict__ dbg_hs)
{
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int li = lane & 15, g = lane >> 4;
    const int n0 = ftile * kGuTile;
    const uint32_t crow = (uint32_t)(a.d >> 1), srow = (uint32_t)(a.d >> 5);
    // the block's weight scales: gate rows n0.. (64 rows), then up rows
    {
        const size_t r0 = (size_t)wslot(a, e) * a.f + n0;
        const int nb = kGuTile * (int)srow;
        lds_copy(a.gs + r0 * srow, lds_addr(lds) + 2u * kAStage, nb);
        lds_copy(a.us + r0 * srow, lds_addr(lds) + 2u * kAStage + (uint32_t)nb, nb);
    }
    BSrc B;
    {
        const size_t wr = (size_t)wslot(a, e) * a.f + (size_t)(n0 + 16 * wave);
        B.rc[0] = weight_rsrc(a.gc + wr * crow);
        B.rc[1] = weight_rsrc(a.uc + wr * crow);
        B.voc = (uint32_t)li * crow + 16u * (uint32_t)g;
        B.bso[0] = (uint32_t)(16 * wave + li) * srow;
        B.bso[1] = B.bso[0] + (uint32_t)kGuTile * srow;
    }
    const int tiles = (n_e + 15) >> 4, npass = (tiles + kPassMT - 1) / kPassMT;
    for (int p = p0; p < p1; ++p) {
        // passes of near-equal tile counts (<= kPassMT)
        const int t0 = p * tiles / npass, t1 = (p + 1) * tiles / npass;
        const int m0 = 16 * t0, nrows = min(16 * t1, n_e) - m0, mt_n = t1 - t0;
        if (threadIdx.x < 16 * kPassMT) {
            const int m = m0 + min((int)threadIdx.x, nrows - 1);
            rowtok[threadIdx.x] = (uint32_t)(a.perm_pair[r_beg + m] / a.k);
        }
        __syncthreads();
        ASrc A;
        a_offsets(rowtok, nrows, crow, srow, A);
        gateup_pass<kPassMT>(a, A, B, xqc, xqs, mt_n, nrows, m0, r_beg, n0, wave, li, g, lds, hqc, hqs, dbg_h,
                             dbg_hc, dbg_hs);
    }
}

// Passes p0 .. p1-1 of expert e against d tile dtile.
__device__ __forceinline__ void down_mx_item(const FfnArgs& a, int e, int r_beg, int n_e, int dtile, int p0,
                                             int p1, uint8_t* lds, uint32_t* rowtok,
                                             const uint8_t* __restrict__ hqc, const uint8_t* __restrict__ hqs,
                                             float* __restrict__ o)
{
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int li = lane & 15, g = lane >> 4;
    const int nw = dtile * kDnTile + wave * 32;
    const uint32_t crow = (uint32_t)(a.f >> 1), srow = (uint32_t)(a.f >> 5);
    // the block's weight scales: d rows dtile*128 .. +127
    lds_copy(a.ds + ((size_t)wslot(a, e) * a.d + (size_t)dtile * kDnTile) * srow, lds_addr(lds) + 2u * kAStage,
             kDnTile * (int)srow);
    const bool sub_ok[2] = {true, true};  // d % 128 == 0
    BSrc B;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        const size_t wr = (size_t)wslot(a, e) * a.d + (size_t)(nw + 16 * s);
        B.rc[s] = weight_rsrc(a.dc + wr * crow);
        B.bso[s] = (uint32_t)(32 * wave + 16 * s + li) * srow;
    }
    B.voc = (uint32_t)li * crow + 16u * (uint32_t)g;
    // h_q rows of the expert are contiguous: the copy bases start at its first row
    const uint8_t* cbase = hqc + (size_t)r_beg * crow;
    const uint8_t* sbase = hqs + (size_t)r_beg * srow;
    const int tiles = (n_e + 15) >> 4, npass = (tiles + kPassMT - 1) / kPassMT;
    for (int p = p0; p < p1; ++p) {
        const int t0 = p * tiles / npass, t1 = (p + 1) * tiles / npass;
        const int m0 = 16 * t0, nrows = min(16 * t1, n_e) - m0, mt_n = t1 - t0;
        if (threadIdx.x < 16 * kPassMT) rowtok[threadIdx.x] = (uint32_t)(m0 + min((int)threadIdx.x, nrows - 1));
        __syncthreads();
        ASrc A;
        a_offsets(rowtok, nrows, crow, srow, A);
        down_pass<kPassMT>(a, A, B, cbase, sbase, mt_n, m0, n_e, r_beg, nw, sub_ok, li, g, lds, o);
        __syncthreads();  // rowtok reused by the next pass
    }
}

// Work of one gate/up block.  Without pass lists: the (slot, tile) of
// xcd_tile and all of the slot's passes.  With them, every (slot, tile,
// pass) is an item: the items of XCD x are its slots (pslot, balanced over
// the XCDs by passes) in order, each as tiles x passes with the passes
// innermost, so the passes of one (slot, tile) -- the same weight rows,
// streamed for different tokens -- run side
// by side on one XCD and share its L2; a heavy expert's passes no longer run
// one after another in a single block.  Block b takes its XCD's items b/8,
// b/8 + cap, ... (cap = the grid's blocks per XCD, sized from an estimate of
// the count).  The down GEMM keeps one block per (slot, tile): its items are
// a quarter as long (K = d_ff), and per-pass items measured slower there.
constexpr int kMaxPassList = 1024 / kXcds + 10;  // pass_stride(1024) + 1 entries

template <typename Body>
__device__ __forceinline__ void mx_items(const FfnArgs& a, int ntiles, int* scum, Body body)
{
    if (!a.passes) {
        int slot, tile, e, r_beg, n_e;
        if (!xcd_tile(blockIdx.x, a.nslots, ntiles, slot, tile)) return;
        if (!mx_slot_expert(a, slot, e, r_beg, n_e)) return;
        const int tiles = (n_e + 15) >> 4;
        body(e, r_beg, n_e, tile, 0, (tiles + kPassMT - 1) / kPassMT);
        return;
    }
    const int x = blockIdx.x % kXcds, pos0 = blockIdx.x / kXcds, cap = gridDim.x / kXcds;
    const int nx = a.passes[kXcds * a.pstride + x];
    for (int i = threadIdx.x; i <= nx; i += blockDim.x) scum[i] = a.passes[x * a.pstride + i];
    __syncthreads();
    const int total = scum[nx] * ntiles;
    for (int pos = pos0; pos < total; pos += cap) {
        int lo = 0, hi = nx - 1;  // the slot j with scum[j] * ntiles <= pos < scum[j + 1] * ntiles
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (scum[mid] * ntiles <= pos)
                lo = mid;
            else
                hi = mid - 1;
        }
        const int npass = scum[lo + 1] - scum[lo], r = pos - scum[lo] * ntiles;
        const int tile = r / npass, pass = r - tile * npass;
        int e, r_beg, n_e;
        mx_slot_expert(a, a.pslot[x * a.pstride + lo], e, r_beg, n_e);  // an active slot
        __syncthreads();  // the previous item is done with the LDS
        body(e, r_beg, n_e, tile, pass, pass + 1);
    }
}

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void gateup_mx512_kernel(
    FfnArgs a, const uint8_t* __restrict__ xqc, const uint8_t* __restrict__ xqs, uint8_t* __restrict__ hqc,
    uint8_t* __restrict__ hqs, float* __restrict__ dbg_h, uint8_t* __restrict__ dbg_hc,
    uint8_t* __restrict__ dbg_hs)
{
    __shared__ __attribute__((aligned(16))) uint8_t lds[kMxLds];
    __shared__ uint32_t rowtok[16 * kPassMT];
    __shared__ int scum[kMaxPassList];
    mx_items(a, a.f / kGuTile, scum, [&](int e, int r_beg, int n_e, int tile, int p0, int p1) {
        gateup_mx_item(a, e, r_beg, n_e, tile, p0, p1, lds, rowtok, xqc, xqs, hqc, hqs, dbg_h, dbg_hc, dbg_hs);
    });
}

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void down_mx512_kernel(
    FfnArgs a, const uint8_t* __restrict__ hqc, const uint8_t* __restrict__ hqs, float* __restrict__ o)
{
    __shared__ __attribute__((aligned(16))) uint8_t lds[kMxLds];
    __shared__ uint32_t rowtok[16 * kPassMT];
    int slot, tile, e, r_beg, n_e;
    if (a.pslot) {
        // the gate/up GEMM's balanced slot lists: XCD x takes the d tiles of
        // its slots, one block running all of a slot's passes
        const int x = blockIdx.x % kXcds, pos = blockIdx.x / kXcds, nt = a.d / kDnTile;
        if (pos / nt >= a.passes[kXcds * a.pstride + x]) return;
        slot = a.pslot[x * a.pstride + pos / nt];
        tile = pos % nt;
    } else if (!xcd_tile(blockIdx.x, a.nslots, a.d / kDnTile, slot, tile)) {
        return;
    }
    if (!mx_slot_expert(a, slot, e, r_beg, n_e)) return;
    const int tiles = (n_e + 15) >> 4;
    down_mx_item(a, e, r_beg, n_e, tile, 0, (tiles + kPassMT - 1) / kPassMT, lds, rowtok, hqc, hqs, o);
}

int mx_tiles_per_pass() { return kPassMT; }

// Grid of the MXFP4 gate/up GEMM: one block per (slot, tile) without pass
// lists; with them, per XCD its slots plus an estimate of the extra passes
// (blocks loop over the rest).
static int mx_grid(const FfnArgs& a, int ntiles)
{
    if (!a.passes) return xcd_grid(a.nslots, ntiles);
    const int extra = (a.P + 16 * kPassMT * kXcds - 1) / (16 * kPassMT * kXcds);
    return kXcds * ntiles * ((a.nslots + kXcds - 1) / kXcds + extra + 2);
}

void launch_gateup_mfma(const FfnArgs& a, const uint8_t* xq_codes, const uint8_t* xq_scales,
                        uint8_t* hq_codes, uint8_t* hq_scales, float* dbg_h, uint8_t* dbg_hc,
                        uint8_t* dbg_hs, hipStream_t s)
{
    const int grid = use_mx512(a) ? mx_grid(a, a.f / kGuTile) : xcd_grid(a.nslots, (a.f + kGuTile - 1) / kGuTile);
    if (use_mx512(a))
        k3_launch(gateup_mx512_kernel, dim3(grid), dim3(256), s, a, xq_codes, xq_scales, hq_codes, hq_scales, dbg_h,
                  dbg_hc, dbg_hs);
    else
        k3_launch(gateup_mfma_kernel, dim3(grid), dim3(256), s, a, xq_codes, xq_scales, hq_codes, hq_scales, dbg_h,
                  dbg_hc, dbg_hs);
}

void launch_down_mfma(const FfnArgs& a, const uint8_t* hq_codes, const uint8_t* hq_scales, float* o,
                      hipStream_t s)
{
    // with the balanced slot lists an XCD takes up to pstride - 1 slots
    const int grid = use_mx512(a) && a.pslot ? kXcds * (a.pstride - 1) * (a.d / kDnTile)
                                             : xcd_grid(a.nslots, (a.d + kDnTile - 1) / kDnTile);
    if (use_mx512(a))
        k3_launch(down_mx512_kernel, dim3(grid), dim3(256), s, a, hq_codes, hq_scales, o);
    else
        k3_launch(down_mfma_kernel, dim3(grid), dim3(256), s, a, hq_codes, hq_scales, o);
}

}  // namespace k3
