// Host-side check of the C ABI under AddressSanitizer and UBSan (built
// host-only by tests/test_sanitizers.py; no GPU is touched). Every call below
// fails an argument check before anything is enqueued, so the pointers are
// fake 16-byte-aligned addresses; the workspace queries run on ordinary and
// extreme shapes, where a signed overflow in the size arithmetic would be
// reported by UBSan.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "ssd.h"

static int failures = 0;
#define EXPECT(call, want)                                                                      \
    do {                                                                                        \
        const int got_ = (int)(call);                                                           \
        if (got_ != (int)(want)) {                                                              \
            fprintf(stderr, "line %d: %s -> %d, expected %d\n", __LINE__, #call, got_, (int)(want)); \
            ++failures;                                                                         \
        }                                                                                       \
    } while (0)

int main() {
    void *P = reinterpret_cast<void *>(0x10000);
    float *F = reinterpret_cast<float *>(0x10000);
    void *MIS = reinterpret_cast<void *>(0x10004);
    void *WS = reinterpret_cast<void *>(0x100000);
    const size_t BIG = (size_t)1 << 40, NONE = (size_t)-1;

    for (int s = -1; s <= 8; ++s) {
        const char *str = ssd_status_string(s);
        if (!str || !str[0]) ++failures;
    }
    // workspace queries: ordinary, empty, invalid and extreme shapes
    const int64_t huge[] = {0, 1, 2, 4096, (int64_t)1 << 31, (int64_t)1 << 40, INT64_MAX, -1, INT64_MIN};
    for (int64_t b : huge)
        for (int64_t t : huge) {
            (void)ssd_chunk_scan_fwd_workspace_bytes(b, t, 64, 64, 128, 1, 256, SSD_BF16);
            (void)ssd_chunk_scan_varlen_workspace_bytes(b, t, 64, 64, 128, 1, 256, SSD_BF16);
            (void)ssd_chunk_scan_bwd_workspace_bytes(b, t, 64, 64, 128, 1, 256, SSD_BF16);
            for (int64_t h : huge) {
                (void)ssd_chunk_scan_fwd_workspace_bytes(b, t, h, 64, 128, 1, 256, SSD_F32);
                (void)ssd_chunk_scan_bwd_workspace_bytes(b, t, h, 32, 32, 1, 64, SSD_F32);
            }
        }
    EXPECT(ssd_chunk_scan_fwd_workspace_bytes(4, 2048, 64, 64, 128, 3, 256, SSD_BF16) == NONE, 1);
    EXPECT(ssd_chunk_scan_fwd_workspace_bytes(0, 2048, 64, 64, 128, 1, 256, SSD_BF16), 0);

    // forward family: NULL, shape, support, alignment and workspace checks
    EXPECT(ssd_chunk_scan_fwd(nullptr, P, F, P, P, F, 256, P, F, 4, 2048, 64, 64, 128, 1, SSD_BF16, WS, BIG, nullptr), SSD_ERR_NULL);
    EXPECT(ssd_chunk_scan_fwd(P, P, F, P, P, F, 256, P, F, -1, 2048, 64, 64, 128, 1, SSD_BF16, WS, BIG, nullptr), SSD_ERR_SHAPE);
    EXPECT(ssd_chunk_scan_fwd(P, P, F, P, P, F, 100, P, F, 4, 2048, 64, 64, 128, 1, SSD_BF16, WS, BIG, nullptr), SSD_ERR_UNSUPPORTED);
    EXPECT(ssd_chunk_scan_fwd(P, P, F, P, P, F, 256, P, F, 4, INT64_MAX, 64, 64, 128, 1, SSD_BF16, WS, BIG, nullptr), SSD_ERR_UNSUPPORTED);
    EXPECT(ssd_chunk_scan_fwd(P, P, F, P, P, F, 256, P, F, INT64_MAX, 2048, 64, 64, 128, 1, SSD_BF16, WS, BIG, nullptr), SSD_ERR_UNSUPPORTED);
    EXPECT(ssd_chunk_scan_fwd(MIS, P, F, P, P, F, 256, P, F, 4, 2048, 64, 64, 128, 1, SSD_BF16, WS, BIG, nullptr), SSD_ERR_ALIGN);
    EXPECT(ssd_chunk_scan_fwd(P, P, F, P, P, F, 256, P, F, 4, 2048, 64, 64, 128, 1, SSD_BF16, nullptr, 0, nullptr), SSD_ERR_WORKSPACE);
    EXPECT(ssd_chunk_scan_fwd(P, P, F, P, P, F, 256, P, F, 4, 2048, 64, 64, 128, 1, SSD_BF16, WS, 16, nullptr), SSD_ERR_WORKSPACE);
    EXPECT(ssd_chunk_scan_fwd(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 256, nullptr, nullptr, 0, 2048, 64, 64, 128, 1, SSD_BF16, nullptr, 0, nullptr), SSD_OK);
    EXPECT(ssd_chunk_scan_prepare(nullptr, F, P, P, 256, 4, 2048, 64, 64, 128, 1, SSD_BF16, WS, BIG, nullptr), SSD_ERR_NULL);
    EXPECT(ssd_chunk_scan_prepare(P, F, P, P, 256, 4, 2048, 64, 64, 128, 1, SSD_BF16, WS, 16, nullptr), SSD_ERR_WORKSPACE);
    EXPECT(ssd_chunk_scan_walk(P, P, P, F, reinterpret_cast<float *>(MIS), 256, P, F, 4, 2048, 64, 64, 128, 1, SSD_BF16, WS, BIG, nullptr), SSD_ERR_ALIGN);
    EXPECT(ssd_chunk_scan_walk(P, P, P, nullptr, nullptr, 256, P, F, 4, 2048, 64, 64, 128, 1, SSD_BF16, WS, BIG, nullptr), SSD_ERR_NULL);
    EXPECT(ssd_chunk_scan_fwd_gated(P, P, F, 3, F, P, P, F, nullptr, 256, P, F, 4, 2048, 64, 64, 128, 1, SSD_BF16, WS, BIG, nullptr), SSD_ERR_UNSUPPORTED);
    EXPECT(ssd_chunk_scan_fwd_fused(P, nullptr, F, P, nullptr, 0, F, P, P, F, nullptr, 256, P, F, 4, 2048, 64, 64, 128, 1, SSD_BF16, WS, BIG, nullptr), SSD_ERR_NULL);
    EXPECT(ssd_chunk_scan_fwd_fused(P, reinterpret_cast<float *>(MIS), nullptr, P, nullptr, 0, F, P, P, F, nullptr, 256, P, F, 4, 2048, 64, 64, 128, 1, SSD_BF16, WS, BIG, nullptr), SSD_ERR_ALIGN);
    EXPECT(ssd_chunk_scan_fwd_noalloc(P, P, F, P, P, F, 256, P, F, 8, 16384, 64, 64, 256, 8, SSD_BF16, nullptr), SSD_ERR_TOO_LARGE);
    EXPECT(ssd_chunk_scan_fwd_noalloc(nullptr, P, F, P, P, F, 256, P, F, 4, 2048, 64, 64, 128, 1, SSD_BF16, nullptr), SSD_ERR_NULL);
    EXPECT(ssd_chunk_scan_fwd_noalloc(P, P, F, P, P, F, 256, P, F, INT64_MAX, INT64_MAX, 64, 64, 128, 1, SSD_BF16, nullptr), SSD_ERR_UNSUPPORTED);
    // variable-length batches
    const int32_t *CU = reinterpret_cast<const int32_t *>(0x10000);
    EXPECT(ssd_chunk_scan_fwd_varlen(P, P, F, P, P, F, 256, nullptr, 3, 100, 200, nullptr, P, F, 64, 64, 128, 1, SSD_BF16, WS, BIG, nullptr), SSD_ERR_NULL);
    EXPECT(ssd_chunk_scan_fwd_varlen(P, P, F, P, P, F, 256, CU, 3, 100, -5, nullptr, P, F, 64, 64, 128, 1, SSD_BF16, WS, BIG, nullptr), SSD_ERR_SHAPE);
    EXPECT(ssd_chunk_scan_fwd_varlen(P, P, F, P, P, F, 256, CU, 3, 100, INT64_MAX, nullptr, P, F, 64, 64, 128, 1, SSD_BF16, WS, BIG, nullptr), SSD_ERR_SHAPE);
    // decode step
    EXPECT(ssd_step(nullptr, P, P, F, P, P, F, P, 256, 64, 64, 128, 1, SSD_BF16, nullptr), SSD_ERR_NULL);
    EXPECT(ssd_step(F, P, P, F, P, P, F, P, 256, 64, 64, 100, 1, SSD_BF16, nullptr), SSD_ERR_UNSUPPORTED);
    EXPECT(ssd_step(F, P, P, F, P, P, F, P, INT64_MAX, 64, 64, 128, 1, SSD_BF16, nullptr), SSD_ERR_UNSUPPORTED);
    EXPECT(ssd_step_gated(F, P, P, F, 7, F, P, P, F, nullptr, P, 256, 64, 64, 128, 1, SSD_BF16, nullptr), SSD_ERR_UNSUPPORTED);
    // backward
    EXPECT(ssd_chunk_scan_bwd(P, P, F, P, P, F, 256, nullptr, P, nullptr, P, P, F, P, P, F, nullptr, 4, 2048, 64, 128, 128, 1, SSD_BF16, WS, BIG, nullptr), SSD_ERR_UNSUPPORTED);
    EXPECT(ssd_chunk_scan_bwd(P, P, F, P, P, F, 256, nullptr, P, nullptr, P, P, nullptr, P, P, F, nullptr, 4, 2048, 64, 64, 128, 1, SSD_BF16, WS, BIG, nullptr), SSD_ERR_NULL);
    EXPECT(ssd_chunk_scan_bwd(P, P, F, P, P, F, 256, nullptr, P, nullptr, P, P, F, P, P, F, nullptr, 4, 2048, 64, 64, 128, 1, SSD_BF16, WS, 16, nullptr), SSD_ERR_WORKSPACE);
    EXPECT(ssd_chunk_scan_bwd(P, P, F, P, P, F, 256, nullptr, P, nullptr, P, P, F, P, P, F, nullptr, INT64_MAX, 2048, 64, 64, 128, 1, SSD_BF16, WS, BIG, nullptr), SSD_ERR_UNSUPPORTED);

    if (failures) {
        fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    printf("abi checks passed\n");
    return 0;
}
