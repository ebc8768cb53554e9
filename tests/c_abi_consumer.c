/*
 * A plain C consumer of include/repops.h.  tests/test_abi_c_consumer.py
 * compiles it as C99 and as C++17 with warnings as errors, links it against
 * librepops.so and runs it.  It calls only the entry points that touch no
 * device (validation, variant selection, names, the contributor order and
 * the workspace size), so it runs on a machine without a GPU.  The matrix
 * addresses are fake and never dereferenced: validation only compares them.
 */
#include "repops.h"

#include <stdint.h>
#include <stdio.h>
#include <string.h>

static int failures = 0;

#define CHECK(cond)                                                   \
    do {                                                              \
        if (!(cond)) {                                                \
            printf("FAIL %s:%d: %s\n", __FILE__, __LINE__, #cond);    \
            ++failures;                                               \
        }                                                             \
    } while (0)

static const float* fake(uintptr_t a) { return (const float*)a; }

/* Row-major A (M x K), B (K x N) and C (M x N) at disjoint fake addresses. */
static repops_status check(const float* C, int64_t c_rs, int64_t c_cs, int64_t M, int64_t N,
                           int64_t K, int variant) {
    return repops_check_args_f32(fake(0x10000000u), K, 1, fake(0x20000000u), N, 1, C, c_rs,
                                 c_cs, M, N, K, 0, 0, variant);
}

int main(void) {
    const float* C = fake(0x30000000u);
    const int n = repops_variant_count();
    int v;

    CHECK(n > 0);
    for (v = 0; v < n; ++v) CHECK(repops_variant_name(v) && strlen(repops_variant_name(v)) > 0);
    CHECK(strcmp(repops_variant_name(n), "?") == 0);
    CHECK(strcmp(repops_variant_name(-1), "?") == 0);
    for (v = REPOPS_OK; v <= REPOPS_ERR_SCRATCH; ++v)
        CHECK(strlen(repops_strerror((repops_status)v)) > 0);
    CHECK(strstr(repops_build_manifest(), "gfx950") != NULL);

    /* Argument validation, as repops_matmul_f32_ex would see it. */
    CHECK(check(C, 64, 1, 48, 64, 32, -1) == REPOPS_OK);
    CHECK(check(C, 64, 1, 48, 64, 32, n - 1) == REPOPS_OK);
    CHECK(check(C, 64, 1, 48, 64, 32, n) == REPOPS_ERR_VARIANT);
    CHECK(check(C, 64, 1, -1, 64, 32, -1) == REPOPS_ERR_DIM);
    CHECK(check(NULL, 64, 1, 48, 64, 32, -1) == REPOPS_ERR_NULL);
    CHECK(check(C, 0, 1, 48, 64, 32, -1) == REPOPS_ERR_STRIDE);
    CHECK(check(fake(0x10000000u + 64), 64, 1, 48, 64, 32, -1) == REPOPS_ERR_ALIAS);
    CHECK(check(NULL, 64, 1, 0, 64, 32, -1) == REPOPS_OK); /* M == 0: nothing to do */

    v = repops_pick_variant_f32(fake(0x10000000u), 4096, 1, fake(0x20000000u), 14336, 1, 4096,
                                14336, 4096, 0, 0);
    CHECK(v >= 0 && v < n);
    CHECK(repops_pick_variant_f32(fake(0x10000000u), 4096, 1, fake(0x20000000u), 14336, 1, -5,
                                  14336, 4096, 0, 0) == -1);

    /* Contributor identities "b", "a", "ab" sort as "a" < "ab" < "b". */
    {
        const uint8_t* dids[3] = {(const uint8_t*)"b", (const uint8_t*)"a",
                                  (const uint8_t*)"ab"};
        const int64_t lens[3] = {1, 1, 2};
        int64_t order[3] = {-1, -1, -1};
        CHECK(repops_canonical_order(dids, lens, 3, order) == REPOPS_OK);
        CHECK(order[0] == 1 && order[1] == 2 && order[2] == 0);
        dids[2] = (const uint8_t*)"a";
        {
            const int64_t dup_lens[3] = {1, 1, 1};
            CHECK(repops_canonical_order(dids, dup_lens, 3, order) == REPOPS_ERR_DUPLICATE);
        }
    }

    /* Workspace of the tensor hash: none for one workgroup's tree. */
    CHECK(repops_merkle_workspace_bytes(256 * 1024, 1024) == 0);
    CHECK(repops_merkle_workspace_bytes(257 * 1024, 1024) > 0);
    CHECK(repops_merkle_workspace_bytes(6, 4) == -1);

    if (failures) return 1;
    printf("c consumer ok: %d variants\n", n);
    return 0;
}
