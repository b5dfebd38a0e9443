// Host-only check of the C ABI's argument validation (csrc/pasa_validate.hpp),
// built with the host compiler's address and undefined-behaviour sanitizers by
// tests/test_sanitize_cpu.py.  It drives every validator with edge-case sizes --
// zero, negative, INT_MAX, products that overflow 32 or 64 bits, slabs past the
// 4 GiB buffer-descriptor bound, non-finite scales -- and checks the documented
// status codes; under the sanitizers any signed overflow, out-of-bounds access
// or other undefined behaviour in the checks ends the run with an error.
#include <limits.h>
#include <math.h>
#include <stdio.h>
#include <stdlib.h>

#include "../precision_flashattention_numerics_amd/csrc/pasa_validate.hpp"

namespace V = pasa::validate;

static int failures = 0;

#define EXPECT(cond)                                                     \
    do {                                                                 \
        if (!(cond)) {                                                   \
            fprintf(stderr, "FAILED line %d: %s\n", __LINE__, #cond);    \
            ++failures;                                                  \
        }                                                                \
    } while (0)

static const int kEdge[] = {INT_MIN, -65504, -1, 0, 1, 2, 7, 31, 32, 33, 63, 64, 65, 127, 128,
                            255, 256, 257, 65503, 65504, 65505, 1 << 20, 1 << 30, INT_MAX - 1,
                            INT_MAX};
static const float kScales[] = {0.0f, -1.0f, 1e-30f, 0.125f, 1.0f, 1e30f, INFINITY, -INFINITY,
                                NAN};

int main() {
    char buf[512];
    void* P = buf;                       // any non-null pointer: validators never dereference
    void* A = (void*)(((uintptr_t)buf + 255) & ~(uintptr_t)255);   // 256-byte aligned
    const int tbl[1] = {0};

    // ---- targeted cases with their documented status
    EXPECT(V::fwd(P, P, P, P, 1, 8, 8, 2, 1, 64, 0.125f, 0) == PASA_OK);
    EXPECT(V::fwd(nullptr, P, P, P, 1, 8, 8, 2, 1, 64, 0.125f, 0) == PASA_ERR_INVALID);
    EXPECT(V::fwd(P, P, P, P, 0, 8, 8, 2, 1, 64, 0.125f, 0) == PASA_ERR_INVALID);
    EXPECT(V::fwd(P, P, P, P, 1, 8, 8, 3, 2, 64, 0.125f, 0) == PASA_ERR_INVALID);
    EXPECT(V::fwd(P, P, P, P, 1, 8, 8, 2, 1, 96, 0.125f, 0) == PASA_ERR_UNSUPPORTED);
    EXPECT(V::fwd(P, P, P, P, 1, 8, 8, 2, 1, 64, NAN, 0) == PASA_ERR_UNSUPPORTED);
    EXPECT(V::fwd(P, P, P, P, 1, 8, 8, 2, 1, 64, 0.0f, 0) == PASA_ERR_UNSUPPORTED);
    EXPECT(V::fwd(P, P, P, P, 1, 8, 8, 2, 1, 64, 0.125f, 2) == PASA_ERR_INVALID);
    // a K/V slab of one head beyond 4 GiB
    EXPECT(V::fwd(P, P, P, P, 1, 8, INT_MAX, 1, 1, 128, 0.125f, 0) == PASA_ERR_UNSUPPORTED);
    EXPECT(V::fwd(P, P, P, P, 1, 8, 1 << 24, 1, 1, 128, 0.125f, 0) == PASA_ERR_UNSUPPORTED);
    // query rows past the int range of a work item's last row
    EXPECT(V::fwd(P, P, P, P, 1, INT_MAX - 100, 8, 1, 1, 64, 0.125f, 0) == PASA_ERR_UNSUPPORTED);
    EXPECT(V::fwd(P, P, P, P, 1, INT_MAX - 511, 8, 1, 1, 64, 0.125f, 0) == PASA_OK);
    // element counts beyond 64-bit indexing
    EXPECT(V::fwd(P, P, P, P, INT_MAX, INT_MAX, 8, INT_MAX, 1, 128, 0.125f, 0) ==
           PASA_ERR_UNSUPPORTED);
    // more than 2^31 - 1 prefill work items
    EXPECT(V::fwd(P, P, P, P, 1 << 20, 1 << 20, 8, 1 << 10, 1, 64, 0.125f, 0) ==
           PASA_ERR_UNSUPPORTED);

    EXPECT(V::fp8_scales(1.0f, 1.0f, 0.125f) == PASA_OK);
    EXPECT(V::fp8_scales(0.0f, 1.0f, 0.125f) == PASA_ERR_UNSUPPORTED);
    EXPECT(V::fp8_scales(1e30f, 1e30f, 0.125f) == PASA_ERR_UNSUPPORTED);   // product overflows
    EXPECT(V::fp8_scales(1e-30f, 1e-30f, 0.125f) == PASA_ERR_UNSUPPORTED); // product underflows

    EXPECT(V::decode_splits(64, 8192, 28, 7, 128) == 2);
    EXPECT(V::decode_splits(64, 8192, 28, 7, 96) == 0);
    EXPECT(V::decode_splits(1, 1, 1, 1, 64) == 1);
    EXPECT(V::decode_splits(INT_MAX, INT_MAX, INT_MAX, 1, 128) >= 1);
    EXPECT(V::fwd_key_split_query(1, 2048, 2048, 32, 128, 1, 256) == 1);
    EXPECT(V::fwd_key_split_query(1, 4096, 4096, 28, 128, 1, 256) == 0);
    EXPECT(V::fwd_key_split_query(2, 9216, 9216, 5, 64, 0, 256) == 1);
    EXPECT(V::fwd_key_split_query(1, 64, 64, 1, 96, 0, 256) == PASA_ERR_UNSUPPORTED);
    EXPECT(V::fwd_key_split_query(1, 64, 64, 1, 128, 0, 65537) == PASA_ERR_INVALID);
    // the largest unit count: a causal problem of 8 * 65536 split items is simulated
    EXPECT(V::fwd_key_split_query(1, 1 << 20, 1 << 20, 64, 64, 1, 65536) >= 0);
    EXPECT(V::workspace_bytes(0, 1, 1, 1) == 0);
    EXPECT(V::workspace_bytes(1, 1, 128, 1) == 512 + 256);

    int n = -7;
    EXPECT(V::decode(P, P, P, P, 64, 8192, 28, 7, 128, 0.088f, 0, &n) == PASA_OK && n == 2);
    EXPECT(V::decode(P, P, P, P, 1, 100, 1, 1, 128, 0.088f, 1000, &n) == PASA_OK && n == 4);
    EXPECT(V::decode(P, P, P, P, 1, 100, 1, 1, 128, 0.088f, -1, &n) == PASA_ERR_INVALID);
    // one split over a million keys: the running sum is folded into fp32 per segment
    EXPECT(V::decode(P, P, P, P, 1, 1 << 20, 1, 1, 128, 0.088f, 1, &n) == PASA_OK && n == 1);
    EXPECT(V::fwd(P, P, P, P, 1, 8, 131072, 8, 1, 128, 0.088f, 1) == PASA_OK);
    EXPECT(V::decode_workspace(nullptr, 1 << 20, 1, 1, 128, 1) == PASA_ERR_WORKSPACE);
    EXPECT(V::decode_workspace((char*)A + 4, 1 << 20, 1, 1, 128, 1) == PASA_ERR_WORKSPACE);
    EXPECT(V::decode_workspace(A, 767, 1, 1, 128, 1) == PASA_ERR_WORKSPACE);
    EXPECT(V::decode_workspace(A, 768, 1, 1, 128, 1) == PASA_OK);

    EXPECT(V::decode_paged(P, P, P, tbl, tbl, P, 2, 8, 4, 64, 64, 10, 4, 0.125f, 0, &n) == PASA_OK);
    EXPECT(V::decode_paged(P, P, P, nullptr, tbl, P, 2, 8, 4, 64, 64, 10, 4, 0.125f, 0, &n) ==
           PASA_ERR_INVALID);
    EXPECT(V::decode_paged(P, P, P, tbl, tbl, P, 2, 8, 4, 64, 48, 10, 4, 0.125f, 0, &n) ==
           PASA_ERR_UNSUPPORTED);
    EXPECT(V::decode_paged(P, P, P, tbl, tbl, P, 2, 8, 4, 64, 1 << 20, 10, 1 << 20, 0.125f, 0,
                           &n) == PASA_ERR_UNSUPPORTED);   // page_size * max_pages > 2^31 - 1

    EXPECT(V::combine((const float*)P, (const float*)P, P, 1, 1, 64, 3) == PASA_OK);
    EXPECT(V::combine(nullptr, (const float*)P, P, 1, 1, 64, 3) == PASA_ERR_INVALID);
    EXPECT(V::combine((const float*)P, (const float*)P, P, 1, 1, 32, 3) == PASA_ERR_UNSUPPORTED);

    // ---- every validator over a grid of edge values: no undefined behaviour,
    // and a status from the documented set
    long long calls = 0;
    for (int a : kEdge)
        for (int b : kEdge)
            for (int c : kEdge) {
                const int dims[] = {64, 128, 96, c};
                for (int d : dims)
                    for (float s : kScales) {
                        const int r1 = V::fwd(P, P, P, P, a, b, c, a, 1, d, s, 1);
                        const int r2 = V::fwd(P, P, P, P, 1, a, b, c, c > 0 ? c : 1, d, s, 0);
                        int m = 0;
                        const int r3 = V::decode(P, P, P, P, a, b, c, 1, d, s, a, &m);
                        const int r4 = V::decode_paged(P, P, P, tbl, tbl, P, a, c, 1, d, b, a, c,
                                                       s, b, &m);
                        const int r5 = V::combine((const float*)P, (const float*)P, P, a, b, d, c);
                        for (int r : {r1, r2, r3, r4, r5})
                            EXPECT(r == PASA_OK || r == PASA_ERR_INVALID ||
                                   r == PASA_ERR_UNSUPPORTED);
                        if (r3 == PASA_OK) EXPECT(m >= 1 && m <= 65535);
                        calls += 5;
                    }
                (void)V::decode_splits(a, b, c, 1, 128);
                for (int cu : {1, 256})
                    for (int causal : {0, 1}) {
                        const int r = V::fwd_key_split_query(1, a, b, c > 0 ? c % 1024 + 1 : c, 128,
                                                             causal, cu);
                        EXPECT(r == 0 || r == 1 || r == PASA_ERR_INVALID);
                    }
                (void)V::workspace_bytes(a, b, 128, c);
                (void)V::decode_workspace(A, (size_t)(unsigned)b, a, c, 64, 1);
                calls += 3;
            }
    printf("abi_validate_check: %lld calls, %d failures\n", calls, failures);
    return failures == 0 ? 0 : 1;
}
