/*
 * k3moe.h -- C ABI of the MI355X (gfx950) routed-expert MoE layer.
 *
 * The layer (the routed-expert half of one MoE layer of the pages' 2.78T
 * model; fiv.co.kr "kimi-k3-in-c deep dive", sections "four reductions" and
 * the glossary rows "MoE" and "MXFP4"):
 *
 *   route:   l[t,e] = x[t] . Wr[e]  (fp64 accumulation)           (+ bias)
 *            S_t    = the k experts with the largest selection key,
 *                     ties to the lower expert index, listed in that order
 *            w[t,j] = softmax over all experts, restricted to S_t and
 *                     renormalised to sum to one
 *            grouping of the T*k token-expert pairs by expert
 *   ffn:     for each pair (t, e = S_t[j]):
 *              h = silu(Wg_e x_t) * (Wu_e x_t)      (SwiGLU, d -> f)
 *              o = Wd_e h                           (f -> d)
 *            y[t] = sum_j w[t,j] * o_{t,j}
 *
 * computed directly on MXFP4 weights: 4-bit E2M1 codes with one E8M0 scale
 * per 32 consecutive values, value = E2M1[code] * 2^(scale - 127)
 * (fiv.co.kr deep dive, "four reductions", MXFP4 note; the weights are never
 * expanded to a wider format in memory).
 *
 * Conventions for every entry point:
 *  - Pointers named as device pointers must be device memory of the current
 *    HIP device (e.g. torch tensors); the caller owns all of them.  The
 *    library allocates nothing at run time.  Between calls it keeps only a
 *    per-device record of "is this device gfx950" and, for
 *    k3moe_forward_noalloc, its fixed per-device scratch array (part of the
 *    loaded library); the expert cache's state is caller-owned memory.
 *  - Calls only enqueue work on `stream` and never synchronise; outputs are
 *    valid once the stream has completed that work.  Calls that share a
 *    workspace must be ordered on one stream.
 *  - Every argument is checked on the host before any HIP call or launch;
 *    errors are returned as negative K3MOE_E* codes, never thrown.  Unknown
 *    enumeration values are refused, never defaulted.
 *  - T == 0 is a valid no-op that returns K3MOE_OK.
 */
#ifndef K3MOE_H
#define K3MOE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
#define K3MOE_OK          0
#define K3MOE_EINVAL     -1  /* bad dimension, null or misaligned pointer    */
#define K3MOE_EWORKSPACE -2  /* workspace missing or smaller than required   */
#define K3MOE_ENOTSUP    -3  /* unknown mode, E > 1024, k > 32, d_model or
                                d_ff > 16384, not gfx950                     */
#define K3MOE_EHIP       -4  /* a HIP call or launch failed; see last_hip_error */

/* ---- modes --------------------------------------------------------------- */
/* Router bias.  The pages' router steers only the *selection* with its bias
 * and weights the chosen experts by unbiased scores (fiv.co.kr deep dive,
 * invariant #5).  K3MOE_BIAS_LOGITS instead adds the bias to the logits, so it
 * moves both the choice and the weights. */
#define K3MOE_BIAS_NONE         0  /* bias ignored (may be NULL)             */
#define K3MOE_BIAS_LOGITS       1  /* l += b: selection and weights          */
#define K3MOE_BIAS_SELECT_ONLY  2  /* key = l + b for selection; weights from l */

/* Router score.  The workload's router scores experts by softmax over the
 * logits (selection on the logits, weights = softmax restricted to the
 * chosen experts and renormalised).  The pages' own router scores each
 * expert by a sigmoid of its logit and weights the chosen experts by their
 * bias-free sigmoid scores (fiv.co.kr deep dive, invariant #5 and the
 * MoE-routing study-plan row); here those weights are renormalised to sum to
 * one (the pages do not say; this is the reading taken).
 *   SOFTMAX: key = l (+ b under SELECT_ONLY); w_j = e^{l_j} / sum_sel e^{l}
 *   SIGMOID: s = 1/(1+e^{-l}); key = s (+ b under SELECT_ONLY);
 *            w_j = s_j / sum_sel s
 * (under BIAS_LOGITS, l already includes the bias). */
#define K3MOE_SCORE_SOFTMAX  0
#define K3MOE_SCORE_SIGMOID  1

/* Activation precision inside the expert FFN. */
#define K3MOE_ACT_FP32   0  /* x and h stay fp32; weights decoded on the fly  */
#define K3MOE_ACT_MXFP4  1  /* x quantised per token, h per pair, to MXFP4 (OCP
                               MX rule: scale 2^(floor(log2 amax) - 2), codes
                               round-to-nearest-even, saturating at 6), then
                               scaled-MXFP4 matrix-core products            */

/* ---- shapes ------------------------------------------------------------ */
typedef struct {
    int32_t T;        /* tokens, >= 0                                         */
    int32_t E;        /* routed experts, 1..1024                              */
    int32_t k;        /* experts per token, 1..min(E, 32)                     */
    int32_t d_model;  /* 32..16384, multiple of 32 (above 16384: ENOTSUP)     */
    int32_t d_ff;     /* 32..16384, multiple of 32 (above 16384: ENOTSUP)     */
} k3moe_dims;

/* One MX matrix [rows][cols] (blocks of 32 along cols, the reduction axis):
 *   codes  : uint8 [rows][cols/2], element 2i in the low nibble of byte i,
 *            element 2i+1 in the high nibble; 16-byte aligned
 *   scales : uint8 [rows][cols/32], E8M0 scale bytes 0..252
 * Rows are contiguous with no padding: a matrix of P values takes
 * P/2 + P/32 bytes (0.53125 B/param, the pages' per-expert byte count).
 * Scale bytes 253 and 254 are outside the contract: the kernels decode and
 * accumulate in fp32, where code 6 at 2^126 or 2^127 (and the sums of such
 * values) overflow; byte 255 is the format's NaN.  Byte 0 is the subnormal
 * scale 2^-127 and is decoded exactly.  Nothing checks the bytes on the
 * device: out-of-contract weights give unspecified y. */
typedef struct {
    const uint8_t *codes;
    const uint8_t *scales;
} k3moe_mx;

/* All experts, stacked along a leading expert axis:
 *   gate, up : [E][d_ff][d_model]   (h = silu(gate x) * up x)
 *   down     : [E][d_model][d_ff]                                          */
typedef struct {
    k3moe_mx gate, up, down;
} k3moe_experts;

/* Optional intermediates of the MXFP4 activation path (all device memory,
 * any field may be NULL; ignored in K3MOE_ACT_FP32 mode).  Pair index
 * p = t*k + j.
 *   x_codes  [T][d_model/2], x_scales [T][d_model/32] : MX(x) per token
 *   h        [T*k][d_ff] fp32 : silu(g)*u before quantisation, per pair
 *   h_codes  [T*k][d_ff/2], h_scales [T*k][d_ff/32]   : MX(h) per pair     */
typedef struct {
    uint8_t *x_codes;
    uint8_t *x_scales;
    float   *h;
    uint8_t *h_codes;
    uint8_t *h_scales;
} k3moe_debug;

/* Bytes of device workspace the calls need for these dimensions and
 * activation mode (a pure host computation; no HIP call).  One workspace of
 * this size serves k3moe_route, k3moe_ffn and k3moe_forward. */
int k3moe_workspace_size(const k3moe_dims *dims, int act_mode, size_t *bytes);

/* Router and grouping (all device pointers):
 *   x         fp32 [T][d_model]           (16-byte aligned)
 *   w_router  fp32 [E][d_model]           (16-byte aligned)
 *   bias      fp32 [E] or NULL (required unless bias_mode == BIAS_NONE)
 *   bias_mode K3MOE_BIAS_*, score_fn K3MOE_SCORE_* (unknown values: ENOTSUP)
 * outputs (bit-deterministic):
 *   topk_idx    int32 [T][k]  chosen experts, descending key, ties -> lower id
 *   topk_w      fp32  [T][k]  renormalised weights (sum to 1), per score_fn
 *   counts      int32 [E]     tokens per expert
 *   offsets     int32 [E+1]   exclusive prefix sum of counts
 *   perm_pair   int32 [T*k]   row -> pair t*k+j; rows grouped by expert in
 *                             ascending expert id, tokens ascending inside
 *   row_of_pair int32 [T*k]   inverse of perm_pair
 * The selection is the one the fp64 router makes: logits are fp64 sums of
 * the exact fp32 x fp32 products (within ~d 2^-53 max|x||w| of the exact dot
 * product; equal router rows give equal logits), plus the bias.  Batches of
 * 256 tokens or more (k < 32, k < E, d_model % 64 == 0) take the logits from
 * int8 slices of x and w_router with a rigorous per-token error bound; a
 * token whose best k + 1 keys are not separated by more than twice that
 * bound has its logits recomputed in fp64 before selecting (one wave per
 * expert row: the same guarantee, another summation order), so exact ties
 * still resolve to the lower expert index.  topk_w is then computed from the
 * sliced logits (within ~1e-8 relative of the exact-logit weights).
 * ws: device workspace of at least k3moe_workspace_size() bytes, 256-aligned. */
int k3moe_route(const k3moe_dims *dims, const float *x, const float *w_router,
                const float *bias, int bias_mode, int score_fn,
                int32_t *topk_idx, float *topk_w, int32_t *counts,
                int32_t *offsets, int32_t *perm_pair, int32_t *row_of_pair,
                void *ws, size_t ws_bytes, hipStream_t stream);

/* Expert FFN and combine, from the outputs of k3moe_route (device pointers).
 *   y  fp32 [T][d_model], fully overwritten.
 *   dbg optional (NULL or a host struct of device pointers), MXFP4 mode only.
 * y is bit-deterministic in both modes: the combine adds the k expert
 * outputs of a token in a fixed order (no atomics). */
int k3moe_ffn(const k3moe_dims *dims, const float *x, const k3moe_experts *experts,
              const int32_t *topk_idx, const float *topk_w, const int32_t *counts,
              const int32_t *offsets, const int32_t *perm_pair,
              const int32_t *row_of_pair, int act_mode, float *y,
              const k3moe_debug *dbg, void *ws, size_t ws_bytes,
              hipStream_t stream);

/* k3moe_route followed by k3moe_ffn on the same stream and workspace; every
 * routing output is still written (the caller owns those buffers). */
int k3moe_forward(const k3moe_dims *dims, const float *x, const float *w_router,
                  const float *bias, int bias_mode, int score_fn, const k3moe_experts *experts,
                  int act_mode, int32_t *topk_idx, float *topk_w,
                  int32_t *counts, int32_t *offsets, int32_t *perm_pair,
                  int32_t *row_of_pair, float *y, const k3moe_debug *dbg,
                  void *ws, size_t ws_bytes, hipStream_t stream);

/* k3moe_forward without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The scratch it needs comes from a
 * fixed array of K3MOE_NOALLOC_SCRATCH_BYTES in the library's own device
 * memory, one per device, reserved when the library's code is loaded on that
 * device and held until the process ends; its address is looked up once per
 * device on the first call.  Dimensions whose workspace
 * (k3moe_workspace_size) exceeds that size are refused with
 * K3MOE_EWORKSPACE before any HIP call: at the 896-expert layer (d_model
 * 7168, d_ff 2048, top-16) that admits single-token decode and batches of up
 * to about 90 tokens.  This call allocates nothing and frees nothing.  All
 * calls on one device share its array and leave their contents in it (the
 * kernels write every scratch byte they read before reading it): calls that
 * overlap in time on one device -- on different streams or threads -- race
 * and give undefined results; calls ordered on one stream do not.  Other
 * arguments, outputs and errors as k3moe_forward. */
#define K3MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int k3moe_forward_noalloc(const k3moe_dims *dims, const float *x, const float *w_router,
                          const float *bias, int bias_mode, int score_fn,
                          const k3moe_experts *experts, int act_mode, int32_t *topk_idx,
                          float *topk_w, int32_t *counts, int32_t *offsets,
                          int32_t *perm_pair, int32_t *row_of_pair, float *y,
                          const k3moe_debug *dbg, hipStream_t stream);

/* ---- HBM cache of experts in front of a host-memory store ----------------
 * For layers whose experts do not all stay in HBM: the pages' engine keeps
 * hot experts in a bounded memory with least-recently-used eviction and
 * fetches a step's missing experts together before its matrix work
 * (fiv.co.kr "kimi-k3-in-c deep dive", "four reductions", expert LRU cache
 * paragraph).  Here every expert lives in host memory that the GPU can read
 * (hipHostMalloc'd), n_slots experts' worth of HBM holds the resident ones,
 * and the policy runs on the GPU in stream order (no host synchronisation):
 *   - a step needs the distinct experts of its selection; resident ones hit;
 *   - misses, in ascending expert id, take the slots that come first in
 *     recency order among the slots the step does not hit (empty slots
 *     first, lowest index first, then least recently used);
 *   - every slot the step touches becomes most recent, those of one step
 *     ordered by slot index.
 * cache_state: device memory of k3moe_cache_state_bytes(E, n_slots) bytes,
 * 256-byte aligned, owned by the caller, set up by k3moe_cache_reset (all
 * slots empty); each k3moe_forward_cached call updates it.  One cache state
 * serves one stream at a time.  E <= 1024, 1 <= n_slots <= E (else EINVAL /
 * ENOTSUP). */
int k3moe_cache_state_bytes(int E, int n_slots, size_t *bytes);
int k3moe_cache_reset(void *cache_state, int E, int n_slots, hipStream_t stream);

/* k3moe_forward with the experts behind the cache:
 *   host_experts  all E experts (layout of k3moe_experts) in pinned host
 *                 memory (hipHostMalloc'd, which the device reads over the
 *                 host link; other memory: K3MOE_EHIP before any launch);
 *                 never written
 *   slot_experts  n_slots experts' worth of device memory in the same layout
 *                 (slot s where expert s would be); the library writes it
 *   cache_state   as above, for this E and n_slots
 * Every array of both must be 16-byte aligned.  T * k <= n_slots (a step's
 * experts must fit at once: EINVAL otherwise).  Per call: routing as
 * k3moe_route; the policy update; a copy of the step's missed experts from
 * host_experts into their slots over the host link; the expert FFN on the
 * slots.  y and every routing output equal k3moe_forward's on host_experts'
 * weights bit for bit.  No dbg.  ws as k3moe_forward. */
int k3moe_forward_cached(const k3moe_dims *dims, const float *x, const float *w_router,
                         const float *bias, int bias_mode, int score_fn,
                         const k3moe_experts *host_experts, const k3moe_experts *slot_experts,
                         int n_slots, void *cache_state, int act_mode, int32_t *topk_idx,
                         float *topk_w, int32_t *counts, int32_t *offsets, int32_t *perm_pair,
                         int32_t *row_of_pair, float *y, void *ws, size_t ws_bytes,
                         hipStream_t stream);

/* Copy the cache state to host memory (each output may be NULL) and wait
 * for the stream: stats int64[4] = steps, hits, misses, misses of the last
 * step; slot_of int32[E] (slot of each expert, -1 if not resident);
 * expert_in int32[n_slots] (expert in each slot, -1 if empty). */
int k3moe_cache_read(const void *cache_state, int E, int n_slots, int64_t *stats, int32_t *slot_of,
                     int32_t *expert_in, hipStream_t stream);

/* Kernel timing marks, a measurement aid (not part of the method): per host
 * thread, every later expert-FFN stage (k3moe_ffn and the FFN half of
 * k3moe_forward, k3moe_forward_noalloc, k3moe_forward_cached) launches its
 * i-th kernel, for i < n, with events[2i] and events[2i+1] attached to the
 * dispatch itself (hipExtLaunchKernel): they take that kernel's start and end
 * time, so their interval is the kernel's own duration, with nothing added
 * to the stream.  kinds[i] receives the kernel's kind (K3MOE_KERNEL_*) and
 * *launched the number of kernels the stage launched (kinds and launched are
 * host memory, either may be NULL, and must stay valid while marks are set).
 * events are 2n hipEvent_t created by the caller; do not set marks while
 * capturing a graph.  n == 0 switches marking off.  Errors: K3MOE_EINVAL for
 * n < 0, n > K3MOE_MAX_MARKS or a NULL event (the marks are then unchanged);
 * launch errors surface as K3MOE_EHIP from the FFN call, as without marks. */
#define K3MOE_MAX_MARKS 8
#define K3MOE_KERNEL_ACTIVE_LIST  1  /* active experts (and MXFP4 pass lists)   */
#define K3MOE_KERNEL_QUANTIZE     2  /* MXFP4 activation quantiser               */
#define K3MOE_KERNEL_GATEUP       3  /* gate/up product with SiLU(g)*u          */
#define K3MOE_KERNEL_DOWN         4  /* down product into per-pair rows         */
#define K3MOE_KERNEL_DOWN_COMBINE 5  /* down product with the combine fused     */
#define K3MOE_KERNEL_COMBINE      6  /* gate-weighted combine of per-pair rows  */
int k3moe_set_stage_marks(void *const *events, int n, int *kinds, int *launched);

/* Human-readable text of a status code (static storage). */
const char *k3moe_status_string(int status);

/* hipError_t of the last K3MOE_EHIP returned on this host thread (0 if none). */
int k3moe_last_hip_error(void);

#ifdef __cplusplus
}
#endif
#endif /* K3MOE_H */
