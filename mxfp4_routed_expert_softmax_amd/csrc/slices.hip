// slices.hip -- the down product of the small-batch fp32-activation path on
// the gfx950 scaled matrix cores, with the gate-weighted combine fused:
// V_MFMA_SCALE_F32_16X16X128_F8F6F4 with an expert's MXFP4 down weights as the
// FP4 A operand and the pair's h, carried as six MX-FP8 slices (slices.h), as
// the FP8 B operand.
//
// The weights are never decoded by vector instructions (fiv.co.kr
// "kimi-k3-in-c deep dive", "four reductions", MXFP4 note: compute on the
// packed nibbles).  The six slices sit in six B columns; one matrix
// instruction gives the dot products of 16 weight rows with all of them, and
// the sum over the columns (a fixed butterfly) is the row's dot product with
// the fp32 h.  Accumulation is fp32.
//
// Step layout (lane l = 16*g + i): A lane = weight row i, B lane = slice i
// (lanes i >= 6 feed zeros).  Within a 512-value chunk c, step s assigns MX
// block 16c + 4g + s to K-block g of the instruction, so lane group g of A
// uses four consecutive blocks of its row across the four steps and one
// 32-bit word of their scale bytes (step s selects byte s).  The dot product
// does not depend on this K order.  The matrix core takes a 32-value K-block
// of an FP4 operand from one lane group, but an FP8 operand's K-block g from
// two: lane group g' carries the 16-value half (g' & 1) of K-blocks g'/2
// (bytes 0-15) and 2 + g'/2 (bytes 16-31), while the E8M0 scale of K-block g
// still comes from lane group g.
#include "slices.h"
#include "launch.h"

namespace k3 {

namespace {

// Sum over the 16 lanes of a row group (same value in all 16; fixed tree).
__device__ __forceinline__ float sum16(float v)
{
    v += sl_xor<1>(v);
    v += sl_xor<2>(v);
    v += sl_xor<4>(v);
    v += sl_xor<8>(v);
    return v;
}

__device__ __forceinline__ i32x8 a_op(uint4 q)
{
    i32x8 r = {(int)q.x, (int)q.y, (int)q.z, (int)q.w, 0, 0, 0, 0};
    return r;
}

// FP4 A (weights) x FP8 E4M3 B (slices), step SEL of a chunk
template <int SEL>
__device__ __forceinline__ f32x4 mma(uint4 a, i32x8 b, uint32_t sa, uint32_t sb, f32x4 c)
{
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a_op(a), b, c, 4, 0, SEL, (int)sa, SEL, (int)sb);
}

// One lane's B fragment of a chunk: per step the 32 slice bytes in the FP8
// operand order (halves of two K-blocks), and the scale word of K-block g.
struct BFrag {
    i32x8 v[4];  // step s: bytes 0-15 = lo half-block, 16-31 = hi half-block
    uint32_t s;
};

// One lane's A fragment of a chunk for one 16-row tile: 64 code bytes + 4 scales.
struct AFrag {
    uint4 q[4];
    uint32_t s;
};

__device__ __forceinline__ f32x4 mma_chunk(const AFrag& a, const BFrag& b, f32x4 acc)
{
    acc = mma<0>(a.q[0], b.v[0], a.s, b.s, acc);
    acc = mma<1>(a.q[1], b.v[1], a.s, b.s, acc);
    acc = mma<2>(a.q[2], b.v[2], a.s, b.s, acc);
    acc = mma<3>(a.q[3], b.v[3], a.s, b.s, acc);
    return acc;
}

// ---- LDS-staged weights --------------------------------------------------
// A 16-row tile of one 512-value chunk is copied into an LDS stage with the
// gfx950 direct global->LDS load (lane l of an instruction lands at M0 +
// 16*l), so every instruction reads whole 256-byte row runs of HBM; the
// matrix-core fragments are then read from LDS.  Stage layout: row r's
// K-block b (16 code bytes) at 256*r + 16*(b ^ r) -- the XOR spreads the 16
// rows of one fragment read over distinct LDS banks -- and its 16 chunk scale
// bytes at 4096 + 16*r.
constexpr int kStage = 4096 + 256;
constexpr int kStageLoads = 5;  // load instructions per stage (4 code + 1 scale)

// Per-lane offsets of a tile-chunk copy (tile rows past rmax repeat row rmax,
// their results are discarded): code pieces j = 0..3 and the scale piece.
struct TileOffs {
    uint32_t c[4], s;
};

__device__ __forceinline__ TileOffs tile_offs(uint32_t rowbytes, int nb, int rmax)
{
    const int lane = threadIdx.x & 63, p = lane & 15;
    TileOffs o;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int r = 4 * j + (lane >> 4);
        o.c[j] = (uint32_t)min(r, rmax) * rowbytes + 16u * (uint32_t)(p ^ r);
    }
    o.s = (uint32_t)(min(lane, rmax) * nb);
    return o;
}

// codes / scales: the tile's first row; c: chunk
__device__ __forceinline__ void stage_tile(const uint8_t* codes, const uint8_t* scales, const TileOffs& o, int c,
                                           uint32_t st)
{
    const uint8_t* cb = codes + 256 * c;
#pragma unroll
    for (int j = 0; j < 4; ++j) dma16(cb, o.c[j], st + 1024 * j);
    if ((threadIdx.x & 63) < 16) dma16(scales + 16 * c, o.s, st + 4096);
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// The lane's A fragment of a staged tile-chunk (4 code runs + the scale
// word), read and waited for in one block.
__device__ __forceinline__ void stage_frag(uint32_t st, int g, int i, AFrag& a)
{
    u32x4 q0, q1, q2, q3;
    uint32_t sc;
    const uint32_t row = st + 256 * i;
    asm volatile(
        "ds_read_b128 %0, %5\n\t"
        "ds_read_b128 %1, %6\n\t"
        "ds_read_b128 %2, %7\n\t"
        "ds_read_b128 %3, %8\n\t"
        "ds_read_b32 %4, %9\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(q0), "=&v"(q1), "=&v"(q2), "=&v"(q3), "=&v"(sc)
        : "v"(row + 16 * ((4 * g + 0) ^ i)), "v"(row + 16 * ((4 * g + 1) ^ i)), "v"(row + 16 * ((4 * g + 2) ^ i)),
          "v"(row + 16 * ((4 * g + 3) ^ i)), "v"(st + 4096 + 16 * i + 4 * g)
        : "memory");
    a.q[0] = make_uint4(q0.x, q0.y, q0.z, q0.w);
    a.q[1] = make_uint4(q1.x, q1.y, q1.z, q1.w);
    a.q[2] = make_uint4(q2.x, q2.y, q2.z, q2.w);
    a.q[3] = make_uint4(q3.x, q3.y, q3.z, q3.w);
    a.s = sc;
}

// A B chunk (the kSlices slice rows of one 512-value chunk, 512 bytes each,
// and their 16 scale bytes each) staged like the weights: slice row j at
// 512*j with its 16-byte unit u at position u ^ 2j (spreads the six rows of
// one fragment read over the LDS banks), scales at 3072 + 16*j.  Issues
// kStageLoads instructions like stage_tile (the scale copy is repeated once).
struct BOffs {
    uint32_t c[3], s;
};

__device__ __forceinline__ BOffs b_offs(uint32_t rowbytes, int nb)
{
    const int lane = threadIdx.x & 63, upos = lane & 31;
    BOffs o;
#pragma unroll
    for (int J = 0; J < 3; ++J) {
        const int j = 2 * J + (lane >> 5);
        o.c[J] = (uint32_t)j * rowbytes + 16u * (uint32_t)(upos ^ (2 * j));
    }
    o.s = (uint32_t)(min(lane, kSlices - 1) * nb);
    return o;
}

// codes / scales: slice row 0 of the token or pair; c: chunk
__device__ __forceinline__ void stage_b(const uint8_t* codes, const uint8_t* scales, const BOffs& o, int c,
                                        uint32_t st)
{
    const uint8_t* cb = codes + 512 * c;
#pragma unroll
    for (int J = 0; J < 3; ++J) dma16(cb, o.c[J], st + 1024 * J);
    if ((threadIdx.x & 63) < kSlices) {
        dma16(scales + 16 * c, o.s, st + 3072);
        dma16(scales + 16 * c, o.s, st + 3072);
    }
}

// The lane's B fragment from a staged B chunk (lanes i >= kSlices get zeros).
__device__ __forceinline__ void stage_bfrag(uint32_t st, int g, int i, BFrag& b)
{
    const int j = min(i, kSlices - 1);
    const uint32_t row = st + 512 * j;
    uint32_t lo[4], hi[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const uint32_t u = 2 * (4 * (g >> 1) + s) + (g & 1);
        lo[s] = row + 16 * (u ^ (2 * j));
        hi[s] = row + 16 * ((u + 16) ^ (2 * j));
    }
    u32x4 r[8];
    uint32_t sc;
    asm volatile(
        "ds_read_b128 %0, %9\n\t"
        "ds_read_b128 %1, %10\n\t"
        "ds_read_b128 %2, %11\n\t"
        "ds_read_b128 %3, %12\n\t"
        "ds_read_b128 %4, %13\n\t"
        "ds_read_b128 %5, %14\n\t"
        "ds_read_b128 %6, %15\n\t"
        "ds_read_b128 %7, %16\n\t"
        "ds_read_b32 %8, %17\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7]),
          "=&v"(sc)
        : "v"(lo[0]), "v"(hi[0]), "v"(lo[1]), "v"(hi[1]), "v"(lo[2]), "v"(hi[2]), "v"(lo[3]), "v"(hi[3]),
          "v"(st + 3072 + 16 * j + 4 * g)
        : "memory");
    const int live = i < kSlices ? -1 : 0;  // lanes past the slices feed zeros
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const u32x4 l = r[2 * s], h = r[2 * s + 1];
        b.v[s] = (i32x8){(int)l.x & live, (int)l.y & live, (int)l.z & live, (int)l.w & live,
                         (int)h.x & live, (int)h.y & live, (int)h.z & live, (int)h.w & live};
    }
    b.s = sc;
}

// Wait until at most n stage copies issued after the one about to be read
// are still in flight (loads complete in issue order; other loads issued in
// between only make the wait stricter).
__device__ __forceinline__ void wait_stages(int n)
{
    if (n >= 3) vm_wait<3 * kStageLoads>();
    else if (n == 2) vm_wait<2 * kStageLoads>();
    else if (n == 1) vm_wait<kStageLoads>();
    else vm_wait<0>();
}

}  // namespace

// LDS-staged variant (f = 512 .. 2048, a multiple of 512): wave w runs the
// pairs j = w, w+8, ...; per pair it streams the nch B items (the h slices,
// kept in registers for the whole pair) and then, tile by tile, the nch
// tile-chunks of every tile -- whole weight rows -- through its private ring
// of NS LDS stages, NS - 1 copies ahead, across pairs.
template <int RW, int NS>
__global__ __launch_bounds__(512) void down_slices_staged_kernel(FfnArgs a, const uint8_t* __restrict__ hs_codes,
                                                                 const uint8_t* __restrict__ hs_scales,
                                                                 float* __restrict__ y)
{
    constexpr int NT = (RW + 15) / 16;
    __shared__ __attribute__((aligned(16))) uint8_t ring_mem[8][NS][kStage];
    __shared__ float part[8][16 * NT];
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, i = lane & 15;
    const int t = blockIdx.y, c0 = blockIdx.x * RW;
    const int f = a.f, nb = f >> 5, nch = nb >> 4, k = a.k;  // nch <= 4
    const uint32_t crow = (uint32_t)(f >> 1);
    const int npair = wave < k ? (k - wave + 7) / 8 : 0;
    const int per = nch * (1 + NT), n = npair * per;
    const uint32_t ring = __builtin_amdgcn_readfirstlane(lds_addr(&ring_mem[wave][0][0]));
    TileOffs to[NT];
#pragma unroll
    for (int q = 0; q < NT; ++q) to[q] = tile_offs(crow, nb, min(15, RW - 1 - 16 * q));
    const BOffs bo = b_offs((uint32_t)f, nb);
    // the wave's experts and weights (k <= 32: at most 4 pairs), read before
    // any copy is in flight so that no wait on them drains the ring later
    int ex[4];
    float wt[4];  // bit patterns via readfirstlane
#pragma unroll
    for (int mm = 0; mm < 4; ++mm) {
        const int pp = t * k + min(wave + 8 * mm, k - 1);
        ex[mm] = __builtin_amdgcn_readfirstlane(a.pair_w[pp]);  // weight index (the expert, or its cache slot)
        wt[mm] = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(a.topk_w[pp])));
    }
    auto pick = [&](const int (&v)[4], int m) { return m == 0 ? v[0] : m == 1 ? v[1] : m == 2 ? v[2] : v[3]; };
    auto issue = [&](int it) {
        const int m = it / per, r = it - m * per;
        const int p = t * k + wave + 8 * m;
        const uint32_t st = ring + (it % NS) * kStage;
        if (r < nch) {
            stage_b(hs_codes + (size_t)p * kSlices * f, hs_scales + (size_t)p * kSlices * nb, bo, r, st);
        } else {
            const int q = (r - nch) / nch, c = (r - nch) - q * nch;
            const size_t row0 = (size_t)pick(ex, m) * a.d + c0 + 16 * q;
            // NT <= 2: pick the tile's offsets without indexing registers at run time
            stage_tile(a.dc + row0 * crow, a.ds + row0 * nb, (NT == 1 || q == 0) ? to[0] : to[NT - 1], c, st);
        }
    };
    for (int it = 0; it < NS - 1 && it < n; ++it) issue(it);
    auto next = [&](int it) {  // issue the copy NS - 1 ahead, then wait for item it
        if (it + NS - 1 < n) issue(it + NS - 1);
        wait_stages(min(NS - 1, n - 1 - it));
    };
    float yacc[NT][4];
#pragma unroll
    for (int q = 0; q < NT; ++q)
#pragma unroll
        for (int v = 0; v < 4; ++v) yacc[q][v] = 0.f;
    for (int m = 0; m < npair; ++m) {
        const int base = m * per;
        BFrag fb0, fb1, fb2, fb3;  // separate objects: never indexed at run time
        next(base);
        stage_bfrag(ring + (base % NS) * kStage, g, i, fb0);
        if (nch > 1) { next(base + 1); stage_bfrag(ring + ((base + 1) % NS) * kStage, g, i, fb1); }
        if (nch > 2) { next(base + 2); stage_bfrag(ring + ((base + 2) % NS) * kStage, g, i, fb2); }
        if (nch > 3) { next(base + 3); stage_bfrag(ring + ((base + 3) % NS) * kStage, g, i, fb3); }
        f32x4 acc[NT];
#pragma unroll
        for (int q = 0; q < NT; ++q) {
            acc[q] = (f32x4){0.f, 0.f, 0.f, 0.f};
            auto step = [&](int c, const BFrag& fb) {
                const int it = base + nch + q * nch + c;
                next(it);
                AFrag fa;
                stage_frag(ring + (it % NS) * kStage, g, i, fa);
                acc[q] = mma_chunk(fa, fb, acc[q]);
                __builtin_amdgcn_sched_barrier(0);  // keep one fragment live at a time
            };
            step(0, fb0);
            if (nch > 1) step(1, fb1);
            if (nch > 2) step(2, fb2);
            if (nch > 3) step(3, fb3);
        }
        const float w = m == 0 ? wt[0] : m == 1 ? wt[1] : m == 2 ? wt[2] : wt[3];
#pragma unroll
        for (int q = 0; q < NT; ++q)
#pragma unroll
            for (int v = 0; v < 4; ++v) yacc[q][v] = __builtin_fmaf(w, sum16(acc[q][v]), yacc[q][v]);
    }
    if (i == 0) {
#pragma unroll
        for (int q = 0; q < NT; ++q)
#pragma unroll
            for (int v = 0; v < 4; ++v) part[wave][16 * q + 4 * g + v] = yacc[q][v];
    }
    __syncthreads();
    if (tid < RW) {
        float sum = 0.f;
#pragma unroll
        for (int w = 0; w < 8; ++w) sum += part[w][tid];
        y[(size_t)t * a.d + c0 + tid] = sum;
    }
}

// The staged copies move 16-byte pieces of the scale rows, so the scale
// array must be 16-byte aligned.
bool use_slices_path(const FfnArgs& a)
{
    return use_pair_path(a) && a.f % 512 == 0 && a.f <= 2048 && reinterpret_cast<uintptr_t>(a.ds) % 16 == 0;
}

void launch_down_slices(const FfnArgs& a, const uint8_t* hs_codes, const uint8_t* hs_scales, float* y,
                        hipStream_t s)
{
    // 28 rows per block gives exactly one block per CU at d_model 7168
    if (a.d % 28 == 0 && a.d / 28 >= 256)
        k3_launch(down_slices_staged_kernel<28, 4>, dim3(a.d / 28, a.T), dim3(512), s, a, hs_codes, hs_scales, y);
    else
        k3_launch(down_slices_staged_kernel<16, 4>, dim3(a.d / 16, a.T), dim3(512), s, a, hs_codes, hs_scales, y);
}

}  // namespace k3
