// api.hip -- the C ABI (include/k3moe.h): host-side argument checks,
// workspace carve-up and the launch sequence of the routed-expert MoE layer.
//
// Arguments are refused, never defaulted, when they are out of contract (the
// pages' configuration reader likewise refuses unknown fields instead of
// guessing: fiv.co.kr "kimi-k3-in-c deep dive", the study-plan row on
// correctness and reproducibility).  All checks run before the first HIP call.
#include <string.h>
#include <atomic>
#include <mutex>
#include "k3moe.h"
#include "kernels.h"
#include "launch.h"

namespace k3 {

static size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

WsLayout ws_layout(int T, int E, int k, int d, int f, int act_mode)
{
    WsLayout L{};
    const size_t P = (size_t)T * k;
    const size_t nch = ((size_t)T + kChunk - 1) / kChunk;
    size_t off = 0;
    auto take = [&](size_t bytes) { size_t at = off; off = align256(off + bytes); return at; };
    L.logits = take((size_t)T * E * sizeof(double));
    {
        // K splits of whichever router these dimensions take
        const int ns = use_router_i8(T, E, k, d) ? router_i8_splits(T, E, d) : router_splits(T, E, d);
        L.partials = take(ns > 1 ? (size_t)ns * T * E * sizeof(double) : 0);
    }
    L.chunk_masks = take(nch * E * sizeof(uint64_t));
    L.chunk_base = take(nch * E * sizeof(int32_t));
    L.active = take(((size_t)E + 1) * sizeof(int32_t));
    L.passes = take((16 * (size_t)pass_stride(E) + 8) * sizeof(int32_t));
    {
        const bool i8 = use_router_i8(T, E, k, d);
        L.rsl_x = take(i8 ? (size_t)kRouterSlices * T * d : 0);
        L.rsl_w = take(i8 ? (size_t)kRouterSlices * E * d : 0);
        L.rsl_xe = take(i8 ? (size_t)T * sizeof(int) : 0);
        L.rsl_we = take(i8 ? (size_t)E * sizeof(int) : 0);
        L.rsl_wc = take(i8 ? (size_t)E * sizeof(double) : 0);
        L.rsl_fail = take(i8 ? ((size_t)T + 1) * sizeof(int) : 0);
    }
    L.route_total = off;
    if (act_mode == K3MOE_ACT_FP32) {
        L.h = take(P * f * sizeof(float));
        L.o = take(P * d * sizeof(float));
        const bool pairs = P <= (size_t)kPairMajorMax;  // the slices path is a pair-path variant
        L.hs_codes = take(pairs ? P * kSlices * f : 0);
        L.hs_scales = take(pairs ? P * kSlices * (f / 32) : 0);
    } else {
        L.xq_codes = take((size_t)T * d / 2);
        L.xq_scales = take((size_t)T * d / 32);
        L.hq_codes = take(P * f / 2);
        L.hq_scales = take(P * f / 32);
        L.o = take(P * d * sizeof(float));
    }
    L.total = off;
    return L;
}

}  // namespace k3

using namespace k3;

static thread_local int g_last_hip_error = 0;

static bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

static int check_dims(const k3moe_dims* dm)
{
    if (!dm) return K3MOE_EINVAL;
    if (dm->T < 0 || dm->E < 1 || dm->k < 1 || dm->k > dm->E) return K3MOE_EINVAL;
    if (dm->d_model <= 0 || dm->d_ff <= 0 || dm->d_model % 32 || dm->d_ff % 32) return K3MOE_EINVAL;
    if ((int64_t)dm->T * dm->k > INT32_MAX) return K3MOE_EINVAL;
    if ((int64_t)dm->T * dm->k * (int64_t)(dm->d_model > dm->d_ff ? dm->d_model : dm->d_ff) >
        ((int64_t)1 << 40))
        return K3MOE_EINVAL;  // row offsets must fit the kernels' index arithmetic
    if (dm->E > 1024 || dm->k > 32) return K3MOE_ENOTSUP;
    // the fp32-activation GEMVs give each lane at most two MX blocks of a
    // row (256 lanes x 2 x 32 values): wider reduction axes are refused
    if (dm->d_model > kMaxDim || dm->d_ff > kMaxDim) return K3MOE_ENOTSUP;
    return K3MOE_OK;
}

static int check_mode_act(int act_mode)
{
    return (act_mode == K3MOE_ACT_FP32 || act_mode == K3MOE_ACT_MXFP4) ? K3MOE_OK : K3MOE_ENOTSUP;
}

static int check_score(int score_fn)
{
    return (score_fn == K3MOE_SCORE_SOFTMAX || score_fn == K3MOE_SCORE_SIGMOID) ? K3MOE_OK : K3MOE_ENOTSUP;
}

static int check_mode_bias(int bias_mode, const float* bias)
{
    if (bias_mode != K3MOE_BIAS_NONE && bias_mode != K3MOE_BIAS_LOGITS &&
        bias_mode != K3MOE_BIAS_SELECT_ONLY)
        return K3MOE_ENOTSUP;
    if (bias_mode != K3MOE_BIAS_NONE && !bias) return K3MOE_EINVAL;
    return K3MOE_OK;
}

// act_mode < 0: only the routing part of the workspace is needed
static int check_ws(const k3moe_dims* dm, int act_mode, const void* ws, size_t ws_bytes)
{
    WsLayout L = ws_layout(dm->T, dm->E, dm->k, dm->d_model, dm->d_ff,
                           act_mode < 0 ? K3MOE_ACT_MXFP4 : act_mode);
    size_t need = act_mode < 0 ? L.route_total : L.total;
    if (!ws || ws_bytes < need) return K3MOE_EWORKSPACE;
    if (!aligned(ws, 256)) return K3MOE_EINVAL;
    return K3MOE_OK;
}

static int check_mx(const k3moe_mx& m)
{
    if (!m.codes || !m.scales) return K3MOE_EINVAL;
    if (!aligned(m.codes, 16) || !aligned(m.scales, 4)) return K3MOE_EINVAL;
    return K3MOE_OK;
}

// Cached per device: 1 = gfx950, -1 = other, 0 = unknown yet.
static std::atomic<int> g_is_gfx950[64];

static int check_device()
{
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) {
        g_last_hip_error = (int)err;
        return K3MOE_EHIP;
    }
    if (dev < 0 || dev >= 64) return K3MOE_ENOTSUP;
    int v = g_is_gfx950[dev].load(std::memory_order_relaxed);
    if (v == 0) {
        hipDeviceProp_t prop;
        err = hipGetDeviceProperties(&prop, dev);
        if (err != hipSuccess) {
            g_last_hip_error = (int)err;
            return K3MOE_EHIP;
        }
        v = (strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : -1;
        g_is_gfx950[dev].store(v, std::memory_order_relaxed);
    }
    return v == 1 ? K3MOE_OK : K3MOE_ENOTSUP;
}

static int finish_launches()
{
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) {
        g_last_hip_error = (int)err;
        return K3MOE_EHIP;
    }
    return K3MOE_OK;
}

// ---------------------------------------------------------------- checks ---
static int validate_route(const k3moe_dims* dm, const float* x, const float* w_router,
                          const float* bias, int bias_mode, int score_fn, int32_t* topk_idx, float* topk_w,
                          int32_t* counts, int32_t* offsets, int32_t* perm_pair,
                          int32_t* row_of_pair, void* ws, size_t ws_bytes, int act_mode_for_ws)
{
    int rc = check_dims(dm);
    if (rc) return rc;
    if ((rc = check_mode_bias(bias_mode, bias))) return rc;
    if ((rc = check_score(score_fn))) return rc;
    if (dm->T == 0) return K3MOE_OK;
    if (!x || !w_router || !topk_idx || !topk_w || !counts || !offsets || !perm_pair || !row_of_pair)
        return K3MOE_EINVAL;
    if (!aligned(x, 16) || !aligned(w_router, 16)) return K3MOE_EINVAL;
    return check_ws(dm, act_mode_for_ws, ws, ws_bytes);
}

static int validate_ffn(const k3moe_dims* dm, const float* x, const k3moe_experts* ex,
                        const int32_t* topk_idx, const float* topk_w, const int32_t* counts,
                        const int32_t* offsets, const int32_t* perm_pair, const int32_t* row_of_pair,
                        int act_mode, float* y, void* ws, size_t ws_bytes)
{
    int rc = check_dims(dm);
    if (rc) return rc;
    if ((rc = check_mode_act(act_mode))) return rc;
    if (dm->T == 0) return K3MOE_OK;
    if (!x || !ex || !topk_idx || !topk_w || !counts || !offsets || !perm_pair || !row_of_pair || !y)
        return K3MOE_EINVAL;
    if (!aligned(x, 16) || !aligned(y, 16)) return K3MOE_EINVAL;
    if ((rc = check_mx(ex->gate)) || (rc = check_mx(ex->up)) || (rc = check_mx(ex->down))) return rc;
    return check_ws(dm, act_mode, ws, ws_bytes);
}

// --------------------------------------------------------------- enqueue ---
static void enqueue_route(const k3moe_dims* dm, const float* x, const float* w_router,
                          const float* bias, int bias_mode, int score_fn, int32_t* topk_idx, float* topk_w,
                          int32_t* counts, int32_t* offsets, int32_t* perm_pair,
                          int32_t* row_of_pair, char* ws, const WsLayout& L, hipStream_t s)
{
    double* logits = reinterpret_cast<double*>(ws + L.logits);
    const int bias_in_logits = bias_mode == K3MOE_BIAS_LOGITS;
    TopkCert cert{nullptr, nullptr, x, w_router, dm->d_model, bias_in_logits, nullptr};
    if (use_router_i8(dm->T, dm->E, dm->k, dm->d_model)) {  // x, w_router 16-B aligned: checked above
        int* xe = reinterpret_cast<int*>(ws + L.rsl_xe);
        double* wc = reinterpret_cast<double*>(ws + L.rsl_wc);
        int* fail = reinterpret_cast<int*>(ws + L.rsl_fail);
        launch_router_i8(dm->T, dm->E, dm->d_model, x, w_router, bias, bias_in_logits,
                         reinterpret_cast<int8_t*>(ws + L.rsl_x), reinterpret_cast<int8_t*>(ws + L.rsl_w), xe,
                         reinterpret_cast<int*>(ws + L.rsl_we), wc, logits,
                         reinterpret_cast<double*>(ws + L.partials), fail, s);
        cert.xe = xe;
        cert.wc = wc;
        cert.fail = fail;
    } else {
        launch_router_logits(dm->T, dm->E, dm->d_model, x, w_router, bias, bias_in_logits, logits,
                             reinterpret_cast<double*>(ws + L.partials), s);
    }
    launch_topk_group(dm->T, dm->E, dm->k, logits, bias, bias_mode == K3MOE_BIAS_SELECT_ONLY,
                      score_fn == K3MOE_SCORE_SIGMOID,
                      topk_idx, topk_w, reinterpret_cast<uint64_t*>(ws + L.chunk_masks),
                      reinterpret_cast<int32_t*>(ws + L.chunk_base), counts, offsets, perm_pair,
                      row_of_pair, cert, s);
}

// Timing marks of the expert-FFN stage (a measurement aid, per host thread):
// while a stage is enqueued with marks set, every kernel launched through
// k3_launch times its own dispatch with the next pair of events.
thread_local StageMarkState k3::g_stage_marks{};
static_assert(kMaxMarks == K3MOE_MAX_MARKS, "one limit on marked kernels");

struct MarkScope {
    MarkScope()
    {
        g_stage_marks.active = g_stage_marks.n > 0;
        g_stage_marks.i = 0;
    }
    void kind(int k) { g_stage_marks.kind = k; }  // of the kernels launched next
    ~MarkScope()
    {
        if (g_stage_marks.active && g_stage_marks.launched) *g_stage_marks.launched = g_stage_marks.i;
        g_stage_marks.active = false;
    }
};

static int enqueue_ffn(const k3moe_dims* dm, const float* x, const k3moe_experts* ex,
                        const int32_t* topk_idx, const float* topk_w, const int32_t* offsets,
                        const int32_t* perm_pair, const int32_t* row_of_pair, int act_mode,
                        float* y, const k3moe_debug* dbg, char* ws, const WsLayout& L,
                        hipStream_t s, const int32_t* slot_of = nullptr, const int32_t* pair_slot = nullptr)
{
    FfnArgs a{};
    a.T = dm->T;
    a.E = dm->E;
    a.k = dm->k;
    a.d = dm->d_model;
    a.f = dm->d_ff;
    a.P = dm->T * dm->k;
    a.x = x;
    a.gc = ex->gate.codes;
    a.gs = ex->gate.scales;
    a.uc = ex->up.codes;
    a.us = ex->up.scales;
    a.dc = ex->down.codes;
    a.ds = ex->down.scales;
    a.topk_idx = topk_idx;
    a.topk_w = topk_w;
    a.offsets = offsets;
    a.perm_pair = perm_pair;
    a.row_of_pair = row_of_pair;
    a.slot_of = slot_of;
    a.pair_w = pair_slot ? pair_slot : topk_idx;
    a.o_stream = (size_t)a.P * a.d * sizeof(float) > ((size_t)128 << 20) ? 1 : 0;
    const bool pair_path = act_mode == K3MOE_ACT_FP32 && use_pair_path(a);
    MarkScope mark;
    if (pair_path) {
        a.active = nullptr;  // slots are pairs
        a.nslots = a.P;
    } else if (a.P <= a.E) {
        // few pairs: a slot per grouped row, the segment heads do the work
        a.active = nullptr;
        a.nslots = a.P;
    } else {
        int32_t* active = reinterpret_cast<int32_t*>(ws + L.active);
        const bool mx = act_mode != K3MOE_ACT_FP32;
        int32_t* passes = reinterpret_cast<int32_t*>(ws + L.passes);
        a.pstride = pass_stride(a.E);
        mark.kind(K3MOE_KERNEL_ACTIVE_LIST);
        int32_t* pslot = passes + 8 * a.pstride + 8;
        launch_active_list(a.E, offsets, active, mx ? mx_tiles_per_pass() : 0, passes, pslot, a.pstride, s);
        a.active = active;
        a.nslots = a.E;
        a.passes = mx ? passes : nullptr;
        a.pslot = mx ? pslot : nullptr;
    }
    if (act_mode == K3MOE_ACT_FP32) {
        float* h = reinterpret_cast<float*>(ws + L.h);
        float* o = reinterpret_cast<float*>(ws + L.o);
        if (pair_path && use_slices_path(a)) {
            uint8_t* hsc = reinterpret_cast<uint8_t*>(ws + L.hs_codes);
            uint8_t* hss = reinterpret_cast<uint8_t*>(ws + L.hs_scales);
            mark.kind(K3MOE_KERNEL_GATEUP);
            launch_gateup_gemv_slices(a, hsc, hss, s);
            mark.kind(K3MOE_KERNEL_DOWN_COMBINE);
            launch_down_slices(a, hsc, hss, y, s);
        } else if (pair_path) {
            mark.kind(K3MOE_KERNEL_GATEUP);
            launch_gateup_gemv(a, h, s);
            mark.kind(K3MOE_KERNEL_DOWN_COMBINE);
            launch_down_gather(a, h, y, s);
        } else {
            mark.kind(K3MOE_KERNEL_GATEUP);
            launch_gateup_gemv(a, h, s);
            mark.kind(K3MOE_KERNEL_DOWN);
            launch_down_gemv(a, h, o, s);
            mark.kind(K3MOE_KERNEL_COMBINE);
            launch_combine(a, o, y, s);
        }
    } else {
        uint8_t* xqc = reinterpret_cast<uint8_t*>(ws + L.xq_codes);
        uint8_t* xqs = reinterpret_cast<uint8_t*>(ws + L.xq_scales);
        uint8_t* hqc = reinterpret_cast<uint8_t*>(ws + L.hq_codes);
        uint8_t* hqs = reinterpret_cast<uint8_t*>(ws + L.hq_scales);
        mark.kind(K3MOE_KERNEL_QUANTIZE);
        launch_quantize_rows((long)a.T * (a.d / 32), x, xqc, xqs, s);
        hipError_t err = hipSuccess;
        if (dbg && dbg->x_codes && err == hipSuccess)
            err = hipMemcpyAsync(dbg->x_codes, xqc, (size_t)a.T * a.d / 2, hipMemcpyDeviceToDevice, s);
        if (dbg && dbg->x_scales && err == hipSuccess)
            err = hipMemcpyAsync(dbg->x_scales, xqs, (size_t)a.T * a.d / 32, hipMemcpyDeviceToDevice, s);
        if (err != hipSuccess) {
            g_last_hip_error = (int)err;
            return K3MOE_EHIP;
        }
        mark.kind(K3MOE_KERNEL_GATEUP);
        launch_gateup_mfma(a, xqc, xqs, hqc, hqs, dbg ? dbg->h : nullptr,
                           dbg ? dbg->h_codes : nullptr, dbg ? dbg->h_scales : nullptr, s);
        float* o = reinterpret_cast<float*>(ws + L.o);
        mark.kind(K3MOE_KERNEL_DOWN);
        launch_down_mfma(a, hqc, hqs, o, s);
        mark.kind(K3MOE_KERNEL_COMBINE);
        launch_combine(a, o, y, s);
    }
    return K3MOE_OK;
}

extern "C" {

int k3moe_set_stage_marks(void* const* events, int n, int* kinds, int* launched)
{
    if (n < 0 || n > K3MOE_MAX_MARKS || (n > 0 && !events)) return K3MOE_EINVAL;
    for (int i = 0; i < 2 * n; ++i)
        if (!events[i]) return K3MOE_EINVAL;
    for (int i = 0; i < 2 * n; ++i) g_stage_marks.ev[i] = static_cast<hipEvent_t>(events[i]);
    g_stage_marks.n = n;
    g_stage_marks.kinds = n > 0 ? kinds : nullptr;
    g_stage_marks.launched = n > 0 ? launched : nullptr;
    return K3MOE_OK;
}

int k3moe_workspace_size(const k3moe_dims* dims, int act_mode, size_t* bytes)
{
    int rc = check_dims(dims);
    if (rc) return rc;
    if ((rc = check_mode_act(act_mode))) return rc;
    if (!bytes) return K3MOE_EINVAL;
    *bytes = ws_layout(dims->T, dims->E, dims->k, dims->d_model, dims->d_ff, act_mode).total;
    return K3MOE_OK;
}

int k3moe_route(const k3moe_dims* dims, const float* x, const float* w_router, const float* bias,
                int bias_mode, int score_fn, int32_t* topk_idx, float* topk_w, int32_t* counts, int32_t* offsets,
                int32_t* perm_pair, int32_t* row_of_pair, void* ws, size_t ws_bytes,
                hipStream_t stream)
{
    // the routing part of the workspace is identical in both activation modes
    int rc = validate_route(dims, x, w_router, bias, bias_mode, score_fn, topk_idx, topk_w, counts, offsets,
                            perm_pair, row_of_pair, ws, ws_bytes, -1);
    if (rc || dims->T == 0) return rc;
    if ((rc = check_device())) return rc;
    WsLayout L = ws_layout(dims->T, dims->E, dims->k, dims->d_model, dims->d_ff, K3MOE_ACT_MXFP4);
    enqueue_route(dims, x, w_router, bias, bias_mode, score_fn, topk_idx, topk_w, counts, offsets, perm_pair,
                  row_of_pair, static_cast<char*>(ws), L, stream);
    return finish_launches();
}

int k3moe_ffn(const k3moe_dims* dims, const float* x, const k3moe_experts* experts,
              const int32_t* topk_idx, const float* topk_w, const int32_t* counts,
              const int32_t* offsets, const int32_t* perm_pair, const int32_t* row_of_pair,
              int act_mode, float* y, const k3moe_debug* dbg, void* ws, size_t ws_bytes,
              hipStream_t stream)
{
    int rc = validate_ffn(dims, x, experts, topk_idx, topk_w, counts, offsets, perm_pair, row_of_pair,
                          act_mode, y, ws, ws_bytes);
    if (rc || dims->T == 0) return rc;
    if ((rc = check_device())) return rc;
    WsLayout L = ws_layout(dims->T, dims->E, dims->k, dims->d_model, dims->d_ff, act_mode);
    rc = enqueue_ffn(dims, x, experts, topk_idx, topk_w, offsets, perm_pair, row_of_pair, act_mode, y,
                     act_mode == K3MOE_ACT_MXFP4 ? dbg : nullptr, static_cast<char*>(ws), L, stream);
    return rc ? rc : finish_launches();
}

int k3moe_forward(const k3moe_dims* dims, const float* x, const float* w_router, const float* bias,
                  int bias_mode, int score_fn, const k3moe_experts* experts, int act_mode, int32_t* topk_idx,
                  float* topk_w, int32_t* counts, int32_t* offsets, int32_t* perm_pair,
                  int32_t* row_of_pair, float* y, const k3moe_debug* dbg, void* ws, size_t ws_bytes,
                  hipStream_t stream)
{
    int rc = check_dims(dims);
    if (rc) return rc;
    if ((rc = check_mode_act(act_mode))) return rc;
    rc = validate_route(dims, x, w_router, bias, bias_mode, score_fn, topk_idx, topk_w, counts, offsets,
                        perm_pair, row_of_pair, ws, ws_bytes, act_mode);
    if (rc) return rc;
    rc = validate_ffn(dims, x, experts, topk_idx, topk_w, counts, offsets, perm_pair, row_of_pair,
                      act_mode, y, ws, ws_bytes);
    if (rc || dims->T == 0) return rc;
    if ((rc = check_device())) return rc;
    WsLayout L = ws_layout(dims->T, dims->E, dims->k, dims->d_model, dims->d_ff, act_mode);
    char* w = static_cast<char*>(ws);
    enqueue_route(dims, x, w_router, bias, bias_mode, score_fn, topk_idx, topk_w, counts, offsets, perm_pair,
                  row_of_pair, w, L, stream);
    rc = enqueue_ffn(dims, x, experts, topk_idx, topk_w, offsets, perm_pair, row_of_pair, act_mode, y,
                     act_mode == K3MOE_ACT_MXFP4 ? dbg : nullptr, w, L, stream);
    return rc ? rc : finish_launches();
}

// Scratch of k3moe_forward_noalloc: one array per device in the library's
// own device memory.  Host code never uses the array's name as an address
// (on the host it names a stand-in, not device memory): the device address
// is looked up once per device with hipGetSymbolAddress and kept here.
static __device__ __align__(256) uint8_t scratch[K3MOE_NOALLOC_SCRATCH_BYTES];

static std::mutex g_scratch_mu;
static void* g_scratch_ptr[64];
static int g_scratch_err[64];  // hipError_t of a failed lookup, kept so a retry reports it

static int scratch_ptr(void** out)
{
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) {
        g_last_hip_error = (int)err;
        return K3MOE_EHIP;
    }
    if (dev < 0 || dev >= 64) return K3MOE_ENOTSUP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev] && !g_scratch_err[dev]) {
        void* p = nullptr;
        err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));  // with device dev current
        if (err != hipSuccess || !p)
            g_scratch_err[dev] = err != hipSuccess ? (int)err : (int)hipErrorInvalidSymbol;
        else
            g_scratch_ptr[dev] = p;
    }
    if (g_scratch_err[dev]) {
        g_last_hip_error = g_scratch_err[dev];
        return K3MOE_EHIP;
    }
    *out = g_scratch_ptr[dev];
    return K3MOE_OK;
}

int k3moe_forward_noalloc(const k3moe_dims* dims, const float* x, const float* w_router, const float* bias,
                          int bias_mode, int score_fn, const k3moe_experts* experts, int act_mode,
                          int32_t* topk_idx, float* topk_w, int32_t* counts, int32_t* offsets,
                          int32_t* perm_pair, int32_t* row_of_pair, float* y, const k3moe_debug* dbg,
                          hipStream_t stream)
{
    int rc = check_dims(dims);
    if (rc) return rc;
    if ((rc = check_mode_act(act_mode))) return rc;
    if (dims->T == 0) return K3MOE_OK;
    const size_t need = ws_layout(dims->T, dims->E, dims->k, dims->d_model, dims->d_ff, act_mode).total;
    if (need > K3MOE_NOALLOC_SCRATCH_BYTES) return K3MOE_EWORKSPACE;
    // the remaining checks are k3moe_forward's, on a stand-in workspace
    // address (aligned, never dereferenced) before the first HIP call
    void* const probe = reinterpret_cast<void*>((uintptr_t)256);
    rc = validate_route(dims, x, w_router, bias, bias_mode, score_fn, topk_idx, topk_w, counts, offsets,
                        perm_pair, row_of_pair, probe, K3MOE_NOALLOC_SCRATCH_BYTES, act_mode);
    if (rc) return rc;
    rc = validate_ffn(dims, x, experts, topk_idx, topk_w, counts, offsets, perm_pair, row_of_pair, act_mode, y,
                      probe, K3MOE_NOALLOC_SCRATCH_BYTES);
    if (rc) return rc;
    if ((rc = check_device())) return rc;
    void* ws = nullptr;
    if ((rc = scratch_ptr(&ws))) return rc;
    return k3moe_forward(dims, x, w_router, bias, bias_mode, score_fn, experts, act_mode, topk_idx, topk_w, counts,
                         offsets, perm_pair, row_of_pair, y, dbg, ws, K3MOE_NOALLOC_SCRATCH_BYTES, stream);
}

// ------------------------------------------------------- expert cache ---
static int check_cache_dims(int E, int n_slots)
{
    if (E < 1 || n_slots < 1 || n_slots > E) return K3MOE_EINVAL;
    if (E > 1024) return K3MOE_ENOTSUP;  // the policy kernel is one 1024-thread block
    return K3MOE_OK;
}

int k3moe_cache_state_bytes(int E, int n_slots, size_t* bytes)
{
    int rc = check_cache_dims(E, n_slots);
    if (rc) return rc;
    if (!bytes) return K3MOE_EINVAL;
    *bytes = cache_state_bytes(E, n_slots);
    return K3MOE_OK;
}

int k3moe_cache_reset(void* cache_state, int E, int n_slots, hipStream_t stream)
{
    int rc = check_cache_dims(E, n_slots);
    if (rc) return rc;
    if (!cache_state || !aligned(cache_state, 256)) return K3MOE_EINVAL;
    if ((rc = check_device())) return rc;
    launch_cache_reset(cache_state_view(cache_state, E, n_slots), stream);
    return finish_launches();
}

static int check_cache_experts(const k3moe_experts* e)
{
    if (!e) return K3MOE_EINVAL;
    int rc;
    if ((rc = check_mx(e->gate)) || (rc = check_mx(e->up)) || (rc = check_mx(e->down))) return rc;
    // the copy moves 16-byte pieces of every array
    if (!aligned(e->gate.scales, 16) || !aligned(e->up.scales, 16) || !aligned(e->down.scales, 16))
        return K3MOE_EINVAL;
    return K3MOE_OK;
}

int k3moe_forward_cached(const k3moe_dims* dims, const float* x, const float* w_router, const float* bias,
                         int bias_mode, int score_fn, const k3moe_experts* host_experts,
                         const k3moe_experts* slot_experts, int n_slots, void* cache_state, int act_mode,
                         int32_t* topk_idx, float* topk_w, int32_t* counts, int32_t* offsets, int32_t* perm_pair,
                         int32_t* row_of_pair, float* y, void* ws, size_t ws_bytes, hipStream_t stream)
{
    int rc = check_dims(dims);
    if (rc) return rc;
    if ((rc = check_mode_act(act_mode))) return rc;
    if ((rc = check_cache_dims(dims->E, n_slots))) return rc;
    if ((int64_t)dims->T * dims->k > n_slots) return K3MOE_EINVAL;  // a step's experts must all fit
    if (!cache_state || !aligned(cache_state, 256)) return K3MOE_EINVAL;
    if ((rc = check_cache_experts(host_experts)) || (rc = check_cache_experts(slot_experts))) return rc;
    rc = validate_route(dims, x, w_router, bias, bias_mode, score_fn, topk_idx, topk_w, counts, offsets,
                        perm_pair, row_of_pair, ws, ws_bytes, act_mode);
    if (rc) return rc;
    rc = validate_ffn(dims, x, slot_experts, topk_idx, topk_w, counts, offsets, perm_pair, row_of_pair,
                      act_mode, y, ws, ws_bytes);
    if (rc || dims->T == 0) return rc;
    if ((rc = check_device())) return rc;
    const int E = dims->E, d = dims->d_model, f = dims->d_ff;
    WsLayout L = ws_layout(dims->T, E, dims->k, d, f, act_mode);
    char* w = static_cast<char*>(ws);
    const CacheState cs = cache_state_view(cache_state, E, n_slots);
    CacheCopy cp{};
    const k3moe_mx* hs[3] = {&host_experts->gate, &host_experts->up, &host_experts->down};
    const k3moe_mx* ds[3] = {&slot_experts->gate, &slot_experts->up, &slot_experts->down};
    for (int m = 0; m < 3; ++m) {
        // the device's address of each host array (pinned host memory is
        // mapped for the device; anything else is refused here, before any
        // kernel could touch it)
        for (int q = 0; q < 2; ++q) {
            const uint8_t* hp = q ? hs[m]->scales : hs[m]->codes;
            void* dp = nullptr;
            const hipError_t err = hipHostGetDevicePointer(&dp, const_cast<uint8_t*>(hp), 0);
            if (err != hipSuccess || !dp) {
                g_last_hip_error = err != hipSuccess ? (int)err : (int)hipErrorInvalidValue;
                return K3MOE_EHIP;
            }
            cp.src[2 * m + q] = static_cast<const uint8_t*>(dp);
        }
        cp.dst[2 * m] = const_cast<uint8_t*>(ds[m]->codes);
        cp.dst[2 * m + 1] = const_cast<uint8_t*>(ds[m]->scales);
        cp.seg_bytes[2 * m] = (size_t)d * f / 2;
        cp.seg_bytes[2 * m + 1] = (size_t)d * f / 32;
    }
    const int P = dims->T * dims->k;
    enqueue_route(dims, x, w_router, bias, bias_mode, score_fn, topk_idx, topk_w, counts, offsets, perm_pair,
                  row_of_pair, w, L, stream);
    launch_cache_update(cs, P, topk_idx, stream);
    launch_cache_fill(cs, cp, P < n_slots ? P : n_slots, stream);
    rc = enqueue_ffn(dims, x, slot_experts, topk_idx, topk_w, offsets, perm_pair, row_of_pair, act_mode, y, nullptr,
                     w, L, stream, cs.slot_of, cs.pair_slot);
    return rc ? rc : finish_launches();
}

int k3moe_cache_read(const void* cache_state, int E, int n_slots, int64_t* stats, int32_t* slot_of,
                     int32_t* expert_in, hipStream_t stream)
{
    int rc = check_cache_dims(E, n_slots);
    if (rc) return rc;
    if (!cache_state || !aligned(cache_state, 256)) return K3MOE_EINVAL;
    if ((rc = check_device())) return rc;
    const CacheState cs = cache_state_view(const_cast<void*>(cache_state), E, n_slots);
    hipError_t err = hipSuccess;
    if (stats) err = hipMemcpyAsync(stats, cs.hdr, 4 * sizeof(int64_t), hipMemcpyDeviceToHost, stream);
    if (slot_of && err == hipSuccess)
        err = hipMemcpyAsync(slot_of, cs.slot_of, (size_t)E * sizeof(int32_t), hipMemcpyDeviceToHost, stream);
    if (expert_in && err == hipSuccess)
        err = hipMemcpyAsync(expert_in, cs.expert_in, (size_t)n_slots * sizeof(int32_t), hipMemcpyDeviceToHost,
                             stream);
    if (err == hipSuccess) err = hipStreamSynchronize(stream);
    if (err != hipSuccess) {
        g_last_hip_error = (int)err;
        return K3MOE_EHIP;
    }
    return K3MOE_OK;
}

const char* k3moe_status_string(int status)
{
    switch (status) {
        case K3MOE_OK: return "ok";
        case K3MOE_EINVAL: return "invalid argument (dimension, null or misaligned pointer)";
        case K3MOE_EWORKSPACE: return "workspace missing or too small (k3moe_forward_noalloc: the dimensions need more than its fixed scratch)";
        case K3MOE_ENOTSUP: return "not supported (mode, E > 1024, k > 32, d_model or d_ff > 16384, or device is not gfx950)";
        case K3MOE_EHIP: return "HIP error (see k3moe_last_hip_error)";
        default: return "unknown status";
    }
}

int k3moe_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
