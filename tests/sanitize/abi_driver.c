/*
 * Drives the host side of the C ABI (include/mil_ssm.h) under AddressSanitizer and
 * UndefinedBehaviorSanitizer without a GPU: every query and every argument check that
 * returns before work is enqueued.  A descriptor is made with mil_ssm_cache_attach on
 * a 256-byte aligned address that is never dereferenced (attach reads and enqueues
 * nothing); each call below must fail its checks and return the documented status
 * without touching the device.  Test infrastructure: built and run by
 * tests/test_sanitizers.py on the CPU.
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "mil_ssm.h"

static int fails = 0;
#define EXPECT(call, want)                                                              \
    do {                                                                               \
        int got_ = (int)(call);                                                        \
        if (got_ != (want)) {                                                          \
            printf("line %d: %s -> %d, expected %d\n", __LINE__, #call, got_, (want)); \
            ++fails;                                                                   \
        }                                                                              \
    } while (0)

int main(void)
{
    const mil_ssm_dims d = {4, 8, 64, 128, 2};
    mil_ssm_layout lay;
    EXPECT(mil_ssm_cache_layout(&d, 8, MIL_BF16, &lay), MIL_OK);
    EXPECT(lay.bytes % 256, 0);
    EXPECT(mil_ssm_cache_bytes(&d, 8, MIL_BF16) == (size_t)lay.bytes, 1);
    EXPECT(mil_ssm_cache_bytes(&d, 0, MIL_BF16), 0);
    EXPECT(mil_ssm_cache_bytes(&d, MIL_KMAX_LIMIT + 1, MIL_BF16), 0);
    EXPECT(mil_ssm_cache_bytes(NULL, 8, MIL_BF16), 0);
    mil_ssm_dims bad = d;
    bad.ngroups = 3;
    EXPECT(mil_ssm_supported(&bad, MIL_BF16), MIL_E_INVALID);
    bad = d;
    bad.headdim = 48;
    EXPECT(mil_ssm_supported(&bad, MIL_BF16), MIL_E_UNSUPPORTED);
    EXPECT(mil_ssm_supported(&d, 7), MIL_E_INVALID);
    EXPECT(mil_ssm_supported(&d, MIL_F32), MIL_OK);
    EXPECT(mil_ssm_prefill_workspace_bytes(&d, 2, 1000, 256) > 0, 1);
    EXPECT(mil_ssm_prefill_workspace_bytes(&d, 2, 1000, 100), 0);
    EXPECT(mil_ssm_greedy_workspace_bytes(&d, 4, 32000) > 0, 1);
    EXPECT(mil_ssm_greedy_workspace_bytes(&d, 0, 32000), 0);
    EXPECT(mil_ssm_project_workspace_bytes(&d, 16, 4096) < ((size_t)1 << 40), 1);
    for (int s = -1; s <= 7; ++s) EXPECT(mil_status_string(s) != NULL, 1);

    /* a descriptor over an address that is never read or written */
    void *fake = (void *)(uintptr_t)0x7f0000000000ull;
    mil_ssm_cache c;
    memset(&c, 0, sizeof c);
    EXPECT(mil_ssm_cache_phase(&c), 0);
    EXPECT(mil_ssm_cache_attach(&c, &d, 8, MIL_BF16, (char *)fake + 128, (size_t)lay.bytes), MIL_E_ALIGN);
    EXPECT(mil_ssm_cache_attach(&c, &d, 8, MIL_BF16, fake, (size_t)lay.bytes - 1), MIL_E_INVALID);
    EXPECT(mil_ssm_cache_attach(&c, &d, 8, MIL_BF16, fake, (size_t)lay.bytes), MIL_OK);
    EXPECT(mil_ssm_cache_phase(&c), 1);
    const void *p = (const void *)(uintptr_t)0x7f1000000000ull; /* 256-aligned stand-ins, never read */
    float *f = (float *)(uintptr_t)0x7f2000000000ull;
    void *ws = (void *)(uintptr_t)0x7f3000000000ull;
    const size_t wsb = mil_ssm_prefill_workspace_bytes(&d, 2, 1000, 256);
    /* prefill: every check before a launch */
    EXPECT(mil_ssm_prefill(&c, 0, 2, 1000, 256, p, p, p, p, f, f, f, ws, wsb, 2u, NULL), MIL_E_INVALID);
    EXPECT(mil_ssm_prefill(&c, 3, 2, 1000, 256, p, p, p, p, f, f, f, ws, wsb, 0, NULL), MIL_E_INVALID);
    EXPECT(mil_ssm_prefill(&c, 0, 2, 0, 256, p, p, p, p, f, f, f, ws, wsb, 0, NULL), MIL_E_INVALID);
    EXPECT(mil_ssm_prefill(&c, 0, 2, 1000, 96, p, p, p, p, f, f, f, ws, wsb, 0, NULL), MIL_E_INVALID);
    EXPECT(mil_ssm_prefill(&c, 0, 2, 1000, 256, NULL, p, p, p, f, f, f, ws, wsb, 0, NULL), MIL_E_INVALID);
    EXPECT(mil_ssm_prefill(&c, 0, 2, 1000, 256, (char *)p + 1, p, p, p, f, f, f, ws, wsb, 0, NULL), MIL_E_ALIGN);
    EXPECT(mil_ssm_prefill(&c, 0, 2, 1000, 256, p, p, p, p, f, f, f, ws, wsb - 1, 0, NULL), MIL_E_WORKSPACE);
    EXPECT(mil_ssm_prefill(&c, 0, 2, 1000, 256, p, p, p, p, f, f, f, NULL, wsb, 0, NULL), MIL_E_WORKSPACE);
    EXPECT(mil_ssm_prefill(&c, 0, 2, 1000, 256, p, p, p, p, f, f, f, (char *)ws + 64, wsb, 0, NULL),
           MIL_E_ALIGN);
    /* verify / commit / tree / greedy: argument and order checks */
    EXPECT(mil_ssm_verify(&c, 0, p, p, p, p, f, f, f, NULL), MIL_E_INVALID);
    EXPECT(mil_ssm_verify(&c, 9, p, p, p, p, f, f, f, NULL), MIL_E_INVALID);
    EXPECT(mil_ssm_verify(&c, 4, p, p, p, p, f, f, NULL, NULL), MIL_E_INVALID);
    EXPECT(mil_ssm_verify(&c, 4, p, p, p, p, f, f, (float *)((char *)f + 2), NULL), MIL_E_ALIGN);
    EXPECT(mil_ssm_verify_tree(&c, 4, NULL, p, p, p, p, f, f, f, NULL), MIL_E_INVALID);
    const int32_t *acc = (const int32_t *)p;
    EXPECT(mil_ssm_commit(&c, 4, acc, p, p, p, f, f, 0, NULL), MIL_E_ORDER);
    EXPECT(mil_ssm_commit_tree(&c, 4, acc, acc, p, p, p, f, f, 0, NULL), MIL_E_ORDER);
    EXPECT(mil_ssm_commit_greedy(&c, 4, acc, p, 100, MIL_BF16, (int32_t *)f, NULL, p, p, p, f, f, ws, 4096, 0,
                                 NULL),
           MIL_E_ORDER);
    /* the multi-layer commit: every check before anything is enqueued */
    {
        mil_ssm_cache c2;
        memset(&c2, 0, sizeof c2);
        EXPECT(mil_ssm_cache_attach(&c2, &d, 8, MIL_BF16, fake, (size_t)lay.bytes), MIL_OK);
        mil_ssm_cache *two[2] = {&c, &c2}, *same[2] = {&c, &c};
        const void *ptrs[2] = {p, p}, *holes[2] = {p, NULL};
        EXPECT(mil_ssm_commit_layers(NULL, 2, 4, acc, ptrs, ptrs, ptrs, NULL), MIL_E_INVALID);
        EXPECT(mil_ssm_commit_layers(two, 0, 4, acc, ptrs, ptrs, ptrs, NULL), MIL_E_INVALID);
        EXPECT(mil_ssm_commit_layers(two, 2, 4, NULL, ptrs, ptrs, ptrs, NULL), MIL_E_INVALID);
        EXPECT(mil_ssm_commit_layers(two, 2, 4, acc, holes, ptrs, ptrs, NULL), MIL_E_INVALID);
        EXPECT(mil_ssm_commit_layers(same, 2, 4, acc, ptrs, ptrs, ptrs, NULL), MIL_E_INVALID);
        EXPECT(mil_ssm_commit_layers(two, 2, 4, acc, ptrs, ptrs, ptrs, NULL), MIL_E_ORDER);
        EXPECT(mil_ssm_cache_phase(&c2), 1);
    }
    /* project: shapes and pointers */
    EXPECT(mil_ssm_project(&d, 16, 4000, p, p, p, p, p, NULL, MIL_BF16, f, f, f, f, ws, 1 << 20, NULL),
           MIL_E_UNSUPPORTED);
    EXPECT(mil_ssm_project(&d, 0, 4096, p, p, p, p, p, NULL, MIL_BF16, f, f, f, f, ws, 1 << 20, NULL),
           MIL_E_INVALID);
    EXPECT(mil_ssm_project(&d, 16, 4096, NULL, p, p, p, p, NULL, MIL_BF16, f, f, f, f, ws, 1 << 20, NULL),
           MIL_E_INVALID);
    EXPECT(mil_ssm_project(&d, 16, 4096, p, p, p, p, p, NULL, 9, f, f, f, f, ws, 1 << 20, NULL), MIL_E_INVALID);
    /* status, trace and kernel queries */
    EXPECT(mil_ssm_cache_status(&c, NULL, 0, NULL), MIL_E_INVALID);
    EXPECT(mil_ssm_cache_trace(&c, 99, NULL, NULL), MIL_E_INVALID);
    EXPECT(mil_ssm_cache_trace(&c, MIL_TRACE_OFF, NULL, NULL), MIL_OK);
    EXPECT(mil_ssm_prefill_kernels(&c, 2, 1024, 256) != 0, 1);
    EXPECT(mil_ssm_prefill_kernels(&c, 5, 1024, 256), 0);
    EXPECT(mil_ssm_prefill_kernels(NULL, 2, 1024, 256), 0);
    EXPECT(mil_ssm_cache_phase(&c), 1);
    printf(fails ? "FAIL %d\n" : "OK\n", fails);
    return fails ? 1 : 0;
}
