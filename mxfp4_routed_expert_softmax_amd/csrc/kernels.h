// kernels.h -- host-side launchers of the gfx950 kernels (internal to the HIP
// library; the public surface is include/k3moe.h).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace k3 {

// Tokens per permutation chunk: one bit per token in a 64-bit mask.
constexpr int kChunk = 64;
// Largest d_model and d_ff: the GEMVs cover 512 MX blocks of a row.
constexpr int kMaxDim = 16384;

// Workspace carve-up (byte offsets from the 256-aligned workspace base).
struct WsLayout {
    size_t logits;       // double [T][E]            router logits (+bias)
    size_t partials;     // double [nsplit][T][E]    split-K router partial sums
    size_t chunk_masks;  // uint64 [nch][E]          which chunk tokens chose e
    size_t chunk_base;   // int32  [nch][E]          rows of e before chunk c
    size_t active;       // int32  [E + 1]           active experts, count last
    size_t passes;       // int32  [16*pstride + 8]  MXFP4 GEMMs: pass lists per XCD, their counts, then their slots
    size_t rsl_x;        // int8   [kRouterSlices][T][d]  int8 router: slices of x
    size_t rsl_w;        // int8   [kRouterSlices][E][d]  int8 router: slices of W_r
    size_t rsl_xe;       // int32  [T]               int8 router: row exponents of x
    size_t rsl_we;       // int32  [E]               int8 router: row exponents of W_r
    size_t rsl_wc;       // double [E]               int8 router: bound factors
    size_t rsl_fail;     // int32  [1 + T]           int8 router: tokens left uncertified (count, ids)
    size_t route_total;  // bytes the routing calls need (a prefix of the rest)
    size_t h;            // fp32   [T*k][f]          fp32 mode: SwiGLU output
    size_t o;            // fp32   [T*k][d]          fp32 mode: per-pair down
    size_t hs_codes;     // uint8  [T*k][6][f]       fp32 pair mode: h slices
    size_t hs_scales;    // uint8  [T*k][6][f/32]
    size_t xq_codes;     // uint8  [T][d/2]          mx mode: MX(x)
    size_t xq_scales;    // uint8  [T][d/32]
    size_t hq_codes;     // uint8  [T*k][f/2]        mx mode: MX(h)
    size_t hq_scales;    // uint8  [T*k][f/32]
    size_t total;
};

WsLayout ws_layout(int T, int E, int k, int d, int f, int act_mode);

// ---- routing ------------------------------------------------------------
// partials: [router_splits()][T][E] fp64 scratch (unused when it returns 1)
int router_splits(int T, int E, int d);
void launch_router_logits(int T, int E, int d, const float* x, const float* wr,
                          const float* bias, int bias_in_logits, double* logits,
                          double* partials, hipStream_t s);
// Large batches: logits from int8 slices of x and W_r (exact int32 products,
// fp64 combination) with a rigorous per-token bound, for the certified
// top-k.  The workspace regions rsl_* above; below ~1024 tokens the K axis is
// split over router_i8_splits() blocks whose fp64 partial logits go to
// partials and are added in split order.  Below 256 tokens slicing W_r costs
// more than the fp64 matrix-core router takes.
constexpr int kRouterI8MinT = 256;
constexpr int kRouterSlices = 5;  // int8 slices per operand (7 bits each)
bool use_router_i8(int T, int E, int k, int d);
int router_i8_splits(int T, int E, int d);
void launch_router_i8(int T, int E, int d, const float* x, const float* wr, const float* bias, int bias_in_logits,
                      int8_t* xs, int8_t* wsl, int* xe, int* we, double* wc, double* logits, double* partials,
                      int* fail, hipStream_t s);
// What the top-k needs to certify int8 logits (xe null: exact fp64 logits)
struct TopkCert {
    const int* xe;
    const double* wc;
    const float* x;
    const float* wr;
    int d;
    int bias_in_logits;
    int* fail;  // [1 + T]: the tokens whose selection was not certified (count first)
};
// top-k + weights + per-chunk masks; for T <= 64 also the whole grouping
// (logits: rewritten for a token whose certification fails)
void launch_topk_group(int T, int E, int k, double* logits, const float* bias,
                       int bias_select_only, int sigmoid, int32_t* topk_idx, float* topk_w,
                       uint64_t* chunk_masks, int32_t* chunk_base, int32_t* counts,
                       int32_t* offsets, int32_t* perm_pair, int32_t* row_of_pair,
                       const TopkCert& cert, hipStream_t s);
// active list; with mt > 0 also the per-XCD pass lists of FfnArgs::passes
// and ::pslot (mt token tiles of 16 per pass)
void launch_active_list(int E, const int32_t* offsets, int32_t* active, int mt, int32_t* passes, int32_t* pslot,
                        int pstride, hipStream_t s);
int pass_stride(int E);
int mx_tiles_per_pass();

// ---- fp32-activation expert path (GEMV family) ----------------------------
struct FfnArgs {
    int T, E, k, d, f, P;
    const float* x;
    const uint8_t *gc, *gs, *uc, *us, *dc, *ds;
    const int32_t* topk_idx;
    const float* topk_w;
    const int32_t* offsets;
    const int32_t* perm_pair;
    const int32_t* row_of_pair;
    const int32_t* active;  // null: slots are sorted rows (segment heads)
    int nslots;
    // MXFP4 GEMMs with an active list: per XCD x, pslot[x * pstride + j] =
    // that XCD's j-th slot (the slots balanced over the XCDs by passes),
    // passes[x * pstride + j] = passes of token tiles before it, the total
    // last; passes[8 * pstride + x] = the XCD's slot count.  Null: one block
    // per (slot, tile) running all of the slot's passes.
    const int32_t* passes;
    const int32_t* pslot;
    int pstride;
    // HBM expert cache: weights of expert e sit at slot slot_of[e] of the
    // weight arrays (null: at e itself)
    const int32_t* slot_of;
    // per-pair rows o of the grouped paths take non-temporal stores and loads
    // (set when they outgrow the 256 MB last-level cache: written once, read
    // once by the combine; smaller ones stay cached between the two kernels)
    int o_stream;
    // weight index of pair p for the pair-major kernels: topk_idx itself, or
    // (expert cache) the slot of that pair's expert -- one load, no branch, in
    // kernels that run at the edge of their register budget
    const int32_t* pair_w;
};

// Index of expert e's weights in the weight arrays
__device__ __forceinline__ int wslot(const FfnArgs& a, int e)
{
    // e is block-uniform everywhere this is used: keep the lookup scalar
    return __builtin_amdgcn_readfirstlane(a.slot_of ? a.slot_of[e] : e);
}
// Batches with at most kPairMajorMax token-expert pairs (and d_ff <= 8192)
// take the pair-major path: gate/up per pair, then down with the combine
// fused (launch_down_gather); larger ones are grouped by expert.
constexpr int kPairMajorMax = 128;
bool use_pair_path(const FfnArgs& a);
void launch_gateup_gemv(const FfnArgs& a, float* h, hipStream_t s);
void launch_down_gather(const FfnArgs& a, const float* h, float* y, hipStream_t s);
void launch_down_gemv(const FfnArgs& a, const float* h, float* o, hipStream_t s);
void launch_combine(const FfnArgs& a, const float* o, float* y, hipStream_t s);

// ---- fp32-activation pair path on the scaled matrix cores ------------------
// h of a pair is carried as kSlices MX-FP8 (E4M3) slices (slices.h): codes
// [P][kSlices][f] bytes, scales [P][kSlices][f/32].  Taken when the pair path
// is (d_ff a multiple of 512, at most 2048, down scales 16-byte aligned):
// gate/up GEMV writing h as slices, then down on the matrix cores with the
// combine fused.
constexpr int kSlices = 6;
bool use_slices_path(const FfnArgs& a);
void launch_gateup_gemv_slices(const FfnArgs& a, uint8_t* hs_codes, uint8_t* hs_scales, hipStream_t s);
void launch_down_slices(const FfnArgs& a, const uint8_t* hs_codes, const uint8_t* hs_scales, float* y,
                        hipStream_t s);

// ---- MXFP4-activation expert path (scaled-MFMA family) --------------------
void launch_quantize_rows(long nblocks, const float* v, uint8_t* codes, uint8_t* scales,
                          hipStream_t s);
void launch_gateup_mfma(const FfnArgs& a, const uint8_t* xq_codes, const uint8_t* xq_scales,
                        uint8_t* hq_codes, uint8_t* hq_scales, float* dbg_h,
                        uint8_t* dbg_hc, uint8_t* dbg_hs, hipStream_t s);
void launch_zero(float* y, size_t n, hipStream_t s);
// per-pair rows into o [T*k][d] (grouped order) for launch_combine
void launch_down_mfma(const FfnArgs& a, const uint8_t* hq_codes, const uint8_t* hq_scales, float* o,
                      hipStream_t s);

// ---- HBM expert cache (cache.hip) -------------------------------------------
struct CacheLayout {
    size_t hdr;        // int64 [4]: steps, hits, misses, misses of the last step
    size_t slot_of;    // int32 [E]: slot of expert e, -1 when not resident
    size_t expert_in;  // int32 [S]: expert in slot s, -1 when empty
    size_t order;      // int32 [S]: slots, least recently used first
    size_t miss_e;     // int32 [S]: the last step's missed experts (ascending id)
    size_t miss_s;     // int32 [S]: the slot each of them took
    size_t pair_slot;  // int32 [S]: the last step's slot of each pair's expert (P <= S)
    size_t total;
};
struct CacheState {
    int E, S;
    int64_t* hdr;
    int32_t *slot_of, *expert_in, *order, *miss_e, *miss_s, *pair_slot;
};
// where to copy a missed expert from and to: six segments (gate codes, gate
// scales, up codes, up scales, down codes, down scales) of seg_bytes[j] per
// expert, expert e at src[j] + e * seg_bytes[j], slot s at dst[j] + s * seg_bytes[j]
struct CacheCopy {
    const uint8_t* src[6];
    uint8_t* dst[6];
    size_t seg_bytes[6];
};
CacheLayout cache_layout(int E, int S);
size_t cache_state_bytes(int E, int S);
CacheState cache_state_view(void* base, int E, int S);
void launch_cache_reset(const CacheState& c, hipStream_t s);
void launch_cache_update(const CacheState& c, int P, const int32_t* topk_idx, hipStream_t s);
void launch_cache_fill(const CacheState& c, const CacheCopy& cp, int max_miss, hipStream_t s);

}  // namespace k3
