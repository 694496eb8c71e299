// Sanitizer driver for the host side of libgdn: argument validation of every
// entry point, the workspace-size queries over a grid of shapes, and the
// carving of the prefill workspace into its regions.  Built with
// AddressSanitizer and UndefinedBehaviorSanitizer on the host code only (the
// kernels are not compiled: every call made here is rejected before any HIP
// call, and none touches a GPU), by tests/test_sanitizers.py.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../include/gdn.h"
#include "../../linear_attention_sequence_gdn_amd/csrc/gdn_prefill.h"

static int failures = 0;
#define EXPECT(e, want)                                                                    \
    do {                                                                                   \
        int got_ = (e);                                                                    \
        if (got_ != (want)) {                                                              \
            fprintf(stderr, "line %d: %s returned %d, expected %d\n", __LINE__, #e, got_, (want)); \
            ++failures;                                                                    \
        }                                                                                  \
    } while (0)

int main()
{
    // never dereferenced: validation rejects every call below first
    void *F = reinterpret_cast<void *>(uintptr_t(0x10000));
    const uint16_t *u = static_cast<const uint16_t *>(F);
    uint16_t *uo = static_cast<uint16_t *>(F);
    const float *f = static_cast<const float *>(F);
    float *fo = static_cast<float *>(F);
    const int32_t *cu = static_cast<const int32_t *>(F);

    for (int s = -2; s < 8; ++s)
        if (!gdn_status_string(s)) ++failures;

    // workspace queries over a grid of shapes (and the unsupported ones)
    const int Ts[] = {0, 1, 63, 64, 65, 511, 8192, 262144};
    const int Hs[][2] = {{1, 1}, {2, 6}, {16, 48}, {4, 32}, {3, 7}};
    for (int T : Ts)
        for (auto &h : Hs)
            for (int B = 0; B < 3; ++B) {
                (void)gdn_prefill_workspace_size(B, T, h[0], h[1], 128, 128);
                (void)gdn_prefill_varlen_workspace_size(B + 1, T, h[0], h[1], 128, 128);
                (void)gdn_prefill_backward_workspace_size(B, T, h[0], h[1], 128, 128);
                (void)gdn_prefill_backward_varlen_workspace_size(B + 1, T, h[0], h[1], 128, 128);
            }
    EXPECT((int)gdn_prefill_workspace_size(1, 64, 16, 48, 64, 128), 0);
    EXPECT((int)gdn_prefill_workspace_size(-1, 64, 16, 48, 128, 128), 0);

    // the backward's window plan (host-only): a sweep of workspace sizes from
    // nothing to the one-pass size, including the native-context length whose
    // plan search walks thousands of window counts
    {
        const int wTs[] = {1, 64, 333, 8192, 262144};
        for (int T : wTs)
            for (auto &h : Hs) {
                if (h[1] % h[0]) continue;
                const size_t one = gdn_prefill_backward_workspace_size(1, T, h[0], h[1], 128, 128);
                for (int k = 0; k <= 16; ++k) {
                    int tw = -1;
                    const int rc = gdn_prefill_backward_windows(1, T, h[0], h[1], 128, 128, one / 16 * k, &tw);
                    if (rc == GDN_OK && (tw <= 0 || tw > T || (tw < T && tw % 64))) ++failures;
                    if (rc != GDN_OK && rc != GDN_ERR_WORKSPACE_TOO_SMALL) ++failures;
                }
                int tw = -1;
                EXPECT(gdn_prefill_backward_windows(2, T, h[0], h[1], 128, 128, 2 * one, &tw), GDN_OK);
                if (tw != T) ++failures;
            }
        int tw = 0;
        EXPECT(gdn_prefill_backward_windows(1, 64, 2, 6, 128, 128, 1 << 30, nullptr), GDN_ERR_INVALID_ARGUMENT);
        EXPECT(gdn_prefill_backward_windows(1, 64, 3, 7, 128, 128, 1 << 30, &tw), GDN_ERR_UNSUPPORTED);
        EXPECT(gdn_prefill_backward_windows(-1, 64, 2, 6, 128, 128, 1 << 30, &tw), GDN_ERR_INVALID_ARGUMENT);
    }

    // the carved regions lie inside the workspace and do not overlap: each is
    // written in full inside an allocation of exactly the queried size
    const int carve[][4] = {{1, 1, 1, 1}, {3, 2, 2, 6}, {130, 4, 2, 8}, {129, 1, 16, 48}};
    for (auto &c : carve) {
        const int max_chunks = c[0], N = c[1], Hqk = c[2], Hv = c[3];
        const size_t need = gdn::prefill_workspace_bytes(max_chunks, N, Hqk, Hv);
        uint8_t *base = static_cast<uint8_t *>(malloc(need));
        const gdn::Workspace ws = gdn::carve_workspace(base, max_chunks, N, Hqk, Hv);
        const int segs = gdn::max_segments(max_chunks, N, gdn::choose_seg_chunks(max_chunks, N, Hv));
        memset(ws.chunk_info, 1, sizeof(int4) * max_chunks);
        memset(ws.seq_info, 2, sizeof(int4) * N);
        memset(ws.qfrag, 3, gdn::kQFragBytes * max_chunks * Hqk);
        memset(ws.kfrag, 4, gdn::kKFragBytes * max_chunks * Hqk);
        memset(ws.hrec, 5, gdn::kRecBytes * max_chunks * Hv);
        memset(ws.seg_info, 6, sizeof(int4) * segs);
        memset(ws.seg_order, 6, sizeof(int) * segs);
        memset(ws.seq_seg, 7, sizeof(int4) * N);
        memset(ws.bstate, 8, sizeof(float) * gdn::kStateFloats * segs * Hv);
        memset(ws.seg_done, 9, sizeof(int) * N * Hv);
        free(base);
    }

    // argument validation: each call fails before any HIP call
    EXPECT(gdn_prefill(nullptr, u, u, f, f, u, nullptr, nullptr, nullptr, fo, uo, 1, 64, 2, 6, 128, 128, 0.1f,
                       1.f, F, 1 << 30, nullptr), GDN_ERR_INVALID_ARGUMENT);
    EXPECT(gdn_prefill(u, u, u, f, f, u, nullptr, nullptr, nullptr, fo, uo, 1, 64, 2, 6, 64, 128, 0.1f, 1.f, F,
                       1 << 30, nullptr), GDN_ERR_UNSUPPORTED);
    EXPECT(gdn_prefill(u, u, u, f, f, u, nullptr, nullptr, nullptr, fo, uo, 1, 64, 2, 6, 128, 128, 0.1f, 1.f, F,
                       10, nullptr), GDN_ERR_WORKSPACE_TOO_SMALL);
    EXPECT(gdn_prefill(u, u, u, f, f, u, nullptr, nullptr, nullptr, fo, uo, 1, 64, 2, 6, 128, 128, 0.1f, 1.f,
                       static_cast<uint8_t *>(F) + 8, 1 << 30, nullptr), GDN_ERR_INVALID_ARGUMENT);
    EXPECT(gdn_prefill(u, u, u, f, f, u, nullptr, nullptr, nullptr, fo, uo, 70000, 70000, 2, 6, 128, 128, 0.1f,
                       1.f, F, 1 << 30, nullptr), GDN_ERR_UNSUPPORTED);
    EXPECT(gdn_prefill_varlen(u, u, u, f, f, u, nullptr, nullptr, nullptr, fo, uo, nullptr, 2, 100, 2, 6, 128,
                              128, 0.1f, 1.f, F, 1 << 30, nullptr), GDN_ERR_INVALID_ARGUMENT);
    EXPECT(gdn_prefill_varlen(u, u, u, f, f, u, nullptr, nullptr, nullptr, fo, uo, cu, -1, 100, 2, 6, 128, 128,
                              0.1f, 1.f, F, 1 << 30, nullptr), GDN_ERR_INVALID_ARGUMENT);
    // a batch whose first 64-token window alone exceeds the array (longer
    // calls with smaller batches run in windows)
    EXPECT(gdn_prefill_noalloc(u, u, u, f, f, u, nullptr, nullptr, nullptr, fo, uo, 64, 16384, 16, 48, 128, 128,
                               0.1f, 1.f, nullptr), GDN_ERR_WORKSPACE_TOO_SMALL);
    EXPECT(gdn_prefill_noalloc(nullptr, u, u, f, f, u, nullptr, nullptr, nullptr, fo, uo, 1, 64, 2, 6, 128, 128,
                               0.1f, 1.f, nullptr), GDN_ERR_INVALID_ARGUMENT);
    EXPECT(gdn_prefill_varlen_slots(u, u, u, f, f, u, nullptr, nullptr, nullptr, fo, uo, cu, nullptr, 4, 2, 100, 2,
                                    6, 128, 128, 0.1f, 1.f, F, 1 << 30, nullptr), GDN_ERR_INVALID_ARGUMENT);
    EXPECT(gdn_prefill_varlen_slots(u, u, u, f, f, u, nullptr, nullptr, nullptr, fo, uo, cu, cu, -1, 2, 100, 2, 6,
                                    128, 128, 0.1f, 1.f, F, 1 << 30, nullptr), GDN_ERR_INVALID_ARGUMENT);
    EXPECT(gdn_decode_step(nullptr, u, u, f, f, u, uo, f, fo, uo, 2, 2, 6, 128, 128, 0.1f, 1.f, nullptr),
           GDN_ERR_INVALID_ARGUMENT);
    EXPECT(gdn_decode_multi(u, u, u, f, f, u, uo, f, fo, uo, nullptr, 0, 2, 5, 2, 6, 128, 128, 0.1f, 1.f,
                            nullptr), GDN_ERR_UNSUPPORTED);
    EXPECT(gdn_decode_multi(u, u, u, f, f, u, uo, f, fo, uo, cu, -1, 2, 2, 2, 6, 128, 128, 0.1f, 1.f, nullptr),
           GDN_ERR_INVALID_ARGUMENT);
    EXPECT(gdn_prefill_backward(u, u, u, f, f, u, nullptr, nullptr, nullptr, nullptr, fo, fo, fo, fo, fo, fo,
                                nullptr, nullptr, 1, 64, 2, 6, 128, 128, 0.1f, 1.f, F, 1 << 30, nullptr),
           GDN_ERR_INVALID_ARGUMENT);
    EXPECT(gdn_prefill_backward_varlen(u, u, u, f, f, u, nullptr, nullptr, u, nullptr, fo, fo, fo, fo, fo, fo,
                                       nullptr, nullptr, cu, 2, 100, 2, 6, 128, 128, 0.1f, 1.f, F, 10, nullptr),
           GDN_ERR_WORKSPACE_TOO_SMALL);
    if (failures) {
        fprintf(stderr, "%d failures\n", failures);
        return 1;
    }
    puts("abi sanitizer run ok");
    return 0;
}
