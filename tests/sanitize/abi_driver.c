/* Drives the C ABI's host-side checks with out-of-contract arguments, for a
 * build of the library whose host code carries AddressSanitizer and
 * UndefinedBehaviorSanitizer (tests/test_sanitize.py).  Every call here is
 * refused before any HIP call, so no GPU is needed; the run fails on a wrong
 * status or on any sanitizer report.  Test infrastructure only. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "k3moe.h"

#define CHECK(c)                                                          \
    do {                                                                  \
        if (!(c)) {                                                       \
            fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); \
            return 1;                                                     \
        }                                                                 \
    } while (0)

static int ws_rc(int T, int E, int k, int d, int f, int mode, size_t *n)
{
    k3moe_dims dm = {T, E, k, d, f};
    return k3moe_workspace_size(&dm, mode, n);
}

int main(void)
{
    size_t n = 0;
    /* dimensions */
    CHECK(ws_rc(1, 16, 2, 256, 128, 0, &n) == K3MOE_OK && n > 0);
    CHECK(ws_rc(0, 16, 2, 256, 128, 0, &n) == K3MOE_OK);
    CHECK(ws_rc(-1, 16, 2, 256, 128, 0, &n) == K3MOE_EINVAL);
    CHECK(ws_rc(1, 0, 1, 256, 128, 0, &n) == K3MOE_EINVAL);
    CHECK(ws_rc(1, 16, 17, 256, 128, 0, &n) == K3MOE_EINVAL);
    CHECK(ws_rc(1, 16, 2, 250, 128, 0, &n) == K3MOE_EINVAL);
    CHECK(ws_rc(1, 2048, 2, 256, 128, 0, &n) == K3MOE_ENOTSUP);
    CHECK(ws_rc(1, 64, 33, 256, 128, 0, &n) == K3MOE_ENOTSUP);
    CHECK(ws_rc(1, 16, 2, 16416, 128, 0, &n) == K3MOE_ENOTSUP);
    CHECK(ws_rc(1, 16, 2, 256, 128, 7, &n) == K3MOE_ENOTSUP);
    CHECK(ws_rc(32768, 896, 16, 7168, 2048, 1, &n) == K3MOE_OK && n > ((size_t)1 << 30));
    CHECK(ws_rc(1, 16, 2, 256, 128, 0, NULL) == K3MOE_EINVAL);
    CHECK(k3moe_workspace_size(NULL, 0, &n) == K3MOE_EINVAL);

    /* route: fake device pointers, never dereferenced (the checks refuse first) */
    k3moe_dims dm = {4, 16, 2, 256, 128};
    float *fx = (float *)(uintptr_t)0x10000;
    int32_t *fi = (int32_t *)(uintptr_t)0x10000;
    float *ff = (float *)(uintptr_t)0x10000;
    void *fw = (void *)(uintptr_t)0x10000;
    CHECK(k3moe_route(&dm, NULL, fx, NULL, 0, 0, fi, ff, fi, fi, fi, fi, fw, (size_t)1 << 30, NULL) ==
          K3MOE_EINVAL);
    CHECK(k3moe_route(&dm, fx, fx, NULL, K3MOE_BIAS_LOGITS, 0, fi, ff, fi, fi, fi, fi, fw, (size_t)1 << 30, NULL) ==
          K3MOE_EINVAL);
    CHECK(k3moe_route(&dm, fx, fx, NULL, 9, 0, fi, ff, fi, fi, fi, fi, fw, (size_t)1 << 30, NULL) == K3MOE_ENOTSUP);
    CHECK(k3moe_route(&dm, fx, fx, NULL, 0, 2, fi, ff, fi, fi, fi, fi, fw, (size_t)1 << 30, NULL) == K3MOE_ENOTSUP);
    CHECK(k3moe_route(&dm, fx, fx, NULL, 0, 0, fi, ff, fi, fi, fi, fi, fw, 16, NULL) == K3MOE_EWORKSPACE);
    CHECK(k3moe_route(&dm, (float *)(uintptr_t)0x10004, fx, NULL, 0, 0, fi, ff, fi, fi, fi, fi, fw, (size_t)1 << 30,
                      NULL) == K3MOE_EINVAL);
    k3moe_dims z = {0, 16, 2, 256, 128};
    CHECK(k3moe_route(&z, NULL, NULL, NULL, 0, 0, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL) == K3MOE_OK);

    /* ffn / forward / no-alloc / cached */
    k3moe_mx mx = {(const uint8_t *)(uintptr_t)0x10000, (const uint8_t *)(uintptr_t)0x10000};
    k3moe_experts ex = {mx, mx, mx};
    k3moe_experts bad = ex;
    bad.gate.codes = (const uint8_t *)(uintptr_t)0x10008;  /* not 16-byte aligned */
    CHECK(k3moe_ffn(&dm, fx, &ex, fi, ff, fi, fi, fi, fi, 5, ff, NULL, fw, (size_t)1 << 34, NULL) == K3MOE_ENOTSUP);
    CHECK(k3moe_ffn(&dm, fx, &bad, fi, ff, fi, fi, fi, fi, 0, ff, NULL, fw, (size_t)1 << 34, NULL) == K3MOE_EINVAL);
    CHECK(k3moe_ffn(&dm, fx, &ex, fi, ff, fi, fi, fi, fi, 0, NULL, NULL, fw, (size_t)1 << 34, NULL) == K3MOE_EINVAL);
    CHECK(k3moe_forward(&dm, fx, fx, NULL, 0, 0, &ex, 7, fi, ff, fi, fi, fi, fi, ff, NULL, fw, (size_t)1 << 34,
                        NULL) == K3MOE_ENOTSUP);
    k3moe_dims big = {4096, 896, 16, 7168, 2048};
    CHECK(k3moe_forward_noalloc(&big, fx, fx, NULL, 0, 0, &ex, 0, fi, ff, fi, fi, fi, fi, ff, NULL, NULL) ==
          K3MOE_EWORKSPACE);
    size_t cb = 0;
    CHECK(k3moe_cache_state_bytes(896, 256, &cb) == K3MOE_OK && cb > 0);
    CHECK(k3moe_cache_state_bytes(896, 0, &cb) == K3MOE_EINVAL);
    CHECK(k3moe_cache_state_bytes(896, 897, &cb) == K3MOE_EINVAL);
    k3moe_dims one = {1, 896, 16, 7168, 2048};
    CHECK(k3moe_forward_cached(&one, fx, fx, NULL, 0, 0, &ex, &ex, 15, fw, 0, fi, ff, fi, fi, fi, fi, ff, fw,
                               (size_t)1 << 34, NULL) == K3MOE_EINVAL); /* 16 experts in 15 slots */

    /* stage marks */
    void *ev[4] = {fw, fw, fw, NULL};
    CHECK(k3moe_set_stage_marks(ev, -1, NULL, NULL) == K3MOE_EINVAL);
    CHECK(k3moe_set_stage_marks(ev, K3MOE_MAX_MARKS + 1, NULL, NULL) == K3MOE_EINVAL);
    CHECK(k3moe_set_stage_marks(ev, 2, NULL, NULL) == K3MOE_EINVAL);
    CHECK(k3moe_set_stage_marks(NULL, 0, NULL, NULL) == K3MOE_OK);

    for (int rc = -5; rc <= 1; ++rc) CHECK(k3moe_status_string(rc) != NULL && strlen(k3moe_status_string(rc)) > 0);
    CHECK(k3moe_last_hip_error() == 0);
    printf("abi driver ok\n");
    return 0;
}
