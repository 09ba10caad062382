// cache.hip -- an HBM cache of experts in front of a host-memory expert
// store: the GPU analog of the pages' expert cache (fiv.co.kr "kimi-k3-in-c
// deep dive", "four reductions", expert LRU cache paragraph: hot experts kept
// in a bounded memory, least recently used evicted, a step's missing experts
// fetched together before its matrix work).  Every expert of a layer sits in
// host memory the GPU can read (pinned); n_slots of them are resident in HBM.
// Per step one single-block kernel updates the policy state from the step's
// selection and lists the misses; a copy kernel pulls the missed experts over
// the host link into their slots; the expert FFN then reads weights through
// the expert -> slot map.
//
// Policy (step-batched LRU): the experts a step needs are its distinct
// selected ids.  Resident ones are hits.  Misses, in ascending expert id, take
// the slots that come first in recency order among the slots the step does
// not hit (empty slots first, lowest index first; then least recently used).
// Every slot the step touches (hits and refills) becomes most recent, those
// of one step ordered by slot index.  State: order[S] (slot indices, least
// recent first), slot_of[E] (-1 = not resident), expert_in[S] (-1 = empty).
#include "device_common.h"
#include "kernels.h"

namespace k3 {

namespace {

constexpr int kCacheThreads = 1024;  // one block; E <= 1024 and S <= 1024

// exclusive scan of v over the block (1024 threads), *total = the sum
__device__ __forceinline__ int cache_scan(int v, int* wsum, int* total)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int incl = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(incl, o, 64);
        if (lane >= o) incl += t;
    }
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    if (threadIdx.x == 0) {
        int run = 0;
        for (int w = 0; w < kCacheThreads / 64; ++w) {
            const int t = wsum[w];
            wsum[w] = run;
            run += t;
        }
        wsum[kCacheThreads / 64] = run;
    }
    __syncthreads();
    const int ex = wsum[wave] + incl - v;
    *total = wsum[kCacheThreads / 64];
    __syncthreads();  // wsum is reused by the next scan
    return ex;
}

__global__ __launch_bounds__(kCacheThreads) void cache_reset_kernel(CacheState c)
{
    const int i = threadIdx.x;
    if (i < c.E) c.slot_of[i] = -1;
    if (i < c.S) {
        c.expert_in[i] = -1;
        c.order[i] = i;
    }
    if (i < 4) c.hdr[i] = 0;
    if (i < c.S) c.miss_e[i] = -1, c.miss_s[i] = -1;
}

__global__ __launch_bounds__(kCacheThreads) void cache_update_kernel(CacheState c, int P,
                                                                     const int32_t* __restrict__ topk_idx)
{
    __shared__ uint8_t need[1024];
    __shared__ uint8_t hit[1024];
    __shared__ uint8_t touched[1024];
    __shared__ int victim[1024];
    __shared__ int fslot[1024];  // slot of each needed expert after the step
    __shared__ int wsum[kCacheThreads / 64 + 1];
    const int i = threadIdx.x;
    const int E = c.E, S = c.S;
    need[i] = 0;
    hit[i] = 0;
    touched[i] = 0;
    __syncthreads();
    for (int p = i; p < P; p += kCacheThreads) need[topk_idx[p]] = 1;
    __syncthreads();
    // hits and misses by expert id
    int is_miss = 0, nh_local = 0, my_slot = -1;
    if (i < E && need[i]) {
        my_slot = c.slot_of[i];
        if (my_slot >= 0) {
            hit[my_slot] = 1;
            nh_local = 1;
        } else {
            is_miss = 1;
        }
    }
    int nm, nh;
    const int r_miss = cache_scan(is_miss, wsum, &nm);
    (void)cache_scan(nh_local, wsum, &nh);
    // victims: the first nm slots of the recency order that the step does not hit
    const int o = i < S ? c.order[i] : 0;
    const int nonhit = (i < S && !hit[o]) ? 1 : 0;
    int nnh;
    const int q = cache_scan(nonhit, wsum, &nnh);
    if (nonhit && q < nm) {
        victim[q] = o;
        touched[o] = 1;
    }
    if (i < S && hit[i]) touched[i] = 1;
    __syncthreads();
    // refills: miss rank r takes victim r (nm <= nnh: the caller keeps the
    // step's distinct experts <= S, and every hit is one of them)
    if (i < E && need[i] && !is_miss) fslot[i] = my_slot;
    if (is_miss && r_miss < nnh) {
        const int s = victim[r_miss];
        fslot[i] = s;
        const int old = c.expert_in[s];
        if (old >= 0) c.slot_of[old] = -1;  // old is not needed by this step (a needed resident is a hit)
        c.slot_of[i] = s;
        c.expert_in[s] = i;
        c.miss_e[r_miss] = i;
        c.miss_s[r_miss] = s;
    }
    // new recency order: untouched slots in their old order, then the
    // touched ones by slot index
    const int untouched = (i < S && !touched[o]) ? 1 : 0;
    int nu;
    const int pu = cache_scan(untouched, wsum, &nu);
    const int tt = (i < S && touched[i]) ? 1 : 0;
    int ntt;
    const int pt = cache_scan(tt, wsum, &ntt);
    // every thread has read its old order entry (before the scans' barriers)
    if (untouched) c.order[pu] = o;
    if (tt) c.order[nu + pt] = i;
    // fslot is complete (written before the scans' barriers): each pair's slot
    for (int p = i; p < P; p += kCacheThreads) c.pair_slot[p] = fslot[topk_idx[p]];
    if (i == 0) {
        c.hdr[0] += 1;   // steps
        c.hdr[1] += nh;  // hits
        c.hdr[2] += nm;  // misses
        c.hdr[3] = nm;   // misses of this step (the copy kernel's count)
    }
}

// One expert's bytes as six segments (gate codes, gate scales, up codes, up
// scales, down codes, down scales), each a multiple of 16 bytes.
struct Seg {
    const uint8_t* src;
    uint8_t* dst;
    size_t n;
};

__device__ __forceinline__ Seg seg_of(const CacheCopy& cp, int j, int e, int s)
{
    const size_t n = cp.seg_bytes[j];
    return Seg{cp.src[j] + (size_t)e * n, cp.dst[j] + (size_t)s * n, n};
}

// Block (chunk, miss i): a 1/gridDim.x share of each segment of miss i.
__global__ __launch_bounds__(256) void cache_fill_kernel(CacheState c, CacheCopy cp)
{
    const int i = blockIdx.y;
    if (i >= (int)c.hdr[3]) return;
    const int e = c.miss_e[i], s = c.miss_s[i];
#pragma unroll 1
    for (int j = 0; j < 6; ++j) {
        const Seg g = seg_of(cp, j, e, s);
        const size_t n16 = g.n / 16;
        const size_t per = (n16 + gridDim.x - 1) / gridDim.x;
        const size_t b = (size_t)blockIdx.x * per, end = min(b + per, n16);
        const uint4* src = reinterpret_cast<const uint4*>(g.src);
        uint4* dst = reinterpret_cast<uint4*>(g.dst);
        size_t t = b + threadIdx.x;
        for (; t + 3 * 256 < end; t += 4 * 256) {
            const uint4 v0 = src[t], v1 = src[t + 256], v2 = src[t + 512], v3 = src[t + 768];
            dst[t] = v0;
            dst[t + 256] = v1;
            dst[t + 512] = v2;
            dst[t + 768] = v3;
        }
        for (; t < end; t += 256) dst[t] = src[t];
    }
}

}  // namespace

size_t cache_state_bytes(int E, int S)
{
    CacheLayout L = cache_layout(E, S);
    return L.total;
}

CacheLayout cache_layout(int E, int S)
{
    CacheLayout L{};
    size_t off = 0;
    auto take = [&](size_t bytes) { size_t at = off; off = (off + bytes + 255) & ~(size_t)255; return at; };
    L.hdr = take(4 * sizeof(int64_t));
    L.slot_of = take((size_t)E * sizeof(int32_t));
    L.expert_in = take((size_t)S * sizeof(int32_t));
    L.order = take((size_t)S * sizeof(int32_t));
    L.miss_e = take((size_t)S * sizeof(int32_t));
    L.miss_s = take((size_t)S * sizeof(int32_t));
    L.pair_slot = take((size_t)S * sizeof(int32_t));
    L.total = off;
    return L;
}

CacheState cache_state_view(void* base, int E, int S)
{
    const CacheLayout L = cache_layout(E, S);
    char* b = static_cast<char*>(base);
    CacheState c;
    c.E = E;
    c.S = S;
    c.hdr = reinterpret_cast<int64_t*>(b + L.hdr);
    c.slot_of = reinterpret_cast<int32_t*>(b + L.slot_of);
    c.expert_in = reinterpret_cast<int32_t*>(b + L.expert_in);
    c.order = reinterpret_cast<int32_t*>(b + L.order);
    c.miss_e = reinterpret_cast<int32_t*>(b + L.miss_e);
    c.miss_s = reinterpret_cast<int32_t*>(b + L.miss_s);
    c.pair_slot = reinterpret_cast<int32_t*>(b + L.pair_slot);
    return c;
}

void launch_cache_reset(const CacheState& c, hipStream_t s)
{
    cache_reset_kernel<<<dim3(1), dim3(kCacheThreads), 0, s>>>(c);
}

void launch_cache_update(const CacheState& c, int P, const int32_t* topk_idx, hipStream_t s)
{
    cache_update_kernel<<<dim3(1), dim3(kCacheThreads), 0, s>>>(c, P, topk_idx);
}

void launch_cache_fill(const CacheState& c, const CacheCopy& cp, int max_miss, hipStream_t s)
{
    // 256 blocks per missed expert: at 16 misses, 4,096 blocks stream the
    // host link; blocks past the step's miss count leave at once
    cache_fill_kernel<<<dim3(256, max_miss), dim3(256), 0, s>>>(c, cp);
}

}  // namespace k3
