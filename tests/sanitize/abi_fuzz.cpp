// Host-only driver for the C ABI's validation and planning code, built with
// AddressSanitizer and UndefinedBehaviorSanitizer on the host side only.
//
// Every entry point is called with sizes drawn from edge values (negative,
// zero, small, tile and chunk boundaries, 2^31, 2^32, 2^62, INT64_MAX) and
// from random ranges.  Each call passes one output pointer misaligned, so a
// call that accepts its sizes stops at the alignment check: no call reaches
// the HIP runtime, and none may return SSM_OK or SSM_ERR_HIP.  The sanitizers
// report any signed overflow, bad shift or out-of-bounds access the size
// arithmetic makes on the way.  The planner queries are called with the same
// sizes and checked for basic consistency.
//
// Pointers are fake addresses inside a static buffer and are never
// dereferenced by validation.  Exit status 0: no finding.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "ssm.h"

namespace {

alignas(256) char g_buf[1024];
void* const kOk = g_buf;            // 256-byte aligned
void* const kMis = g_buf + 2;       // misaligned for every rule
float* const kOkF = reinterpret_cast<float*>(g_buf + 256);

const int64_t kEdge[] = {INT64_MIN, INT64_MIN + 1, -(int64_t(1) << 40), -1, 0, 1, 2, 3, 7, 15,
                         16, 17, 31, 32, 33, 48, 63, 64, 65, 96, 127, 128, 129, 255, 256, 257,
                         511, 512, 1000, 2048, 4096, 65535, 65536, 131072, int64_t(1) << 20,
                         (int64_t(1) << 31) - 1, int64_t(1) << 31, int64_t(1) << 32,
                         int64_t(1) << 40, int64_t(1) << 50, int64_t(1) << 62, INT64_MAX - 1,
                         INT64_MAX};
constexpr int kNumEdge = sizeof(kEdge) / sizeof(kEdge[0]);

uint64_t g_state = 0x9E3779B97F4A7C15ull;
uint64_t next() {                   // splitmix64
    uint64_t z = (g_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

int64_t draw() {
    switch (next() % 4) {
        case 0: case 1: return kEdge[next() % kNumEdge];
        case 2: return (int64_t)(next() % 5000);
        default: return (int64_t)(next() >> (next() % 64));
    }
}

int g_failures = 0;
void expect_rejected(const char* name, int rc, int64_t a, int64_t b, int64_t c, int64_t d) {
    if (rc == SSM_OK || rc == SSM_ERR_HIP || rc < 0 || rc > SSM_ERR_HIP) {
        fprintf(stderr, "%s(%lld, %lld, %lld, %lld): unexpected status %d\n", name, (long long)a,
                (long long)b, (long long)c, (long long)d, rc);
        ++g_failures;
    }
}

}  // namespace

int main(int argc, char** argv) {
    const long iters = argc > 1 ? atol(argv[1]) : 200000;
    for (int s = -3; s < 12; ++s)
        if (!ssm_status_string(s)) { fprintf(stderr, "status string %d is NULL\n", s); return 1; }
    for (long it = 0; it < iters; ++it) {
        const int64_t B = draw(), L = draw(), D = draw(), N = draw();
        const int dtype = (int)(next() % 4) - 1;
        const unsigned flags = (unsigned)(next() % 5);
        // planner queries: pure functions of the sizes
        const size_t ws = ssm_selective_scan_workspace_bytes(B, L, D, N, dtype);
        const int segs = ssm_selective_scan_segments(B, L, D, N);
        const int lanes = ssm_selective_scan_lanes(B, L, D, N);
        if (segs < 0 || segs > 256 || (lanes != 0 && lanes != 1) || (lanes && segs == 0) ||
            (segs > 1 && ws == 0 && dtype >= 0 && dtype <= 1)) {
            fprintf(stderr, "plan(%lld, %lld, %lld, %lld): segments %d lanes %d workspace %zu\n",
                    (long long)B, (long long)L, (long long)D, (long long)N, segs, lanes, ws);
            ++g_failures;
        }
        (void)ssm_selective_scan_bwd_workspace_bytes(B, L, D, N, dtype);
        (void)ssm_selective_scan_bwd_ckpt_workspace_bytes(B, L, D, N, dtype);
        (void)ssm_selective_scan_ckpt_bytes(B, L, D, N, dtype);
        void* wsp = (next() & 1) ? kOk : nullptr;
        const size_t wsb = (next() & 1) ? ws : (size_t)next();
        // forward scan family: y misaligned
        expect_rejected("fwd", ssm_selective_scan_fwd(kOk, kOk, kOkF, kOk, kOk, kOkF, nullptr, kOkF,
                                                      flags, kOkF, kMis, kOkF, B, L, D, N, dtype,
                                                      wsp, wsb, nullptr), B, L, D, N);
        expect_rejected("fwd_noalloc", ssm_selective_scan_fwd_noalloc(
                            kOk, kOk, kOkF, kOk, kOk, nullptr, kOk, nullptr, flags, nullptr,
                            kMis, nullptr, B, L, D, N, dtype, nullptr), B, L, D, N);
        expect_rejected("fwd_varlen", ssm_selective_scan_fwd_varlen(
                            kOk, kOk, kOkF, kOk, kOk, nullptr, nullptr, nullptr, flags, nullptr,
                            kMis, kOkF, reinterpret_cast<const int32_t*>(kOk), B, L, D, N, dtype,
                            wsp, wsb, nullptr), B, L, D, N);
        void* ev[4] = {nullptr, nullptr, nullptr, nullptr};
        expect_rejected("fwd_timed", ssm_selective_scan_fwd_timed(
                            kOk, kOk, kOkF, kOk, kOk, nullptr, nullptr, nullptr, flags, nullptr,
                            kMis, nullptr, B, L, D, N, dtype, wsp, wsb, nullptr, ev), B, L, D, N);
        const int64_t K = draw();
        expect_rejected("conv_fwd", ssm_selective_scan_conv_fwd(
                            kOk, kOkF, kOkF, nullptr, kOkF, K, kOk, kOk, kOkF, kOk, kOk, nullptr,
                            nullptr, nullptr, flags, nullptr, kMis, nullptr, B, L, D, N, dtype,
                            wsp, wsb, nullptr), B, L, D, K);
        expect_rejected("bwd", ssm_selective_scan_bwd(
                            kOk, kOk, kOkF, kOk, kOk, nullptr, nullptr, nullptr, flags, nullptr,
                            kOk, nullptr, kMis, kOk, kOkF, kOkF, kOkF, nullptr, nullptr, nullptr,
                            nullptr, B, L, D, N, dtype, wsp, wsb, nullptr), B, L, D, N);
        expect_rejected("bwd_varlen", ssm_selective_scan_bwd_varlen(
                            kOk, kOk, kOkF, kOk, kOk, nullptr, nullptr, nullptr, flags, nullptr,
                            kOk, nullptr, kMis, kOk, kOkF, kOkF, kOkF, nullptr, nullptr, nullptr,
                            nullptr, reinterpret_cast<const int32_t*>(kOk), B, L, D, N, dtype,
                            wsp, wsb, nullptr), B, L, D, N);
        expect_rejected("fwd_ckpt", ssm_selective_scan_fwd_ckpt(
                            kOk, kOk, kOkF, kOk, kOk, nullptr, nullptr, nullptr, flags, nullptr,
                            kMis, nullptr, reinterpret_cast<float*>(kOk), B, L, D, N, dtype, wsp,
                            wsb, nullptr), B, L, D, N);
        expect_rejected("bwd_ckpt", ssm_selective_scan_bwd_ckpt(
                            kOk, kOk, kOkF, kOk, kOk, nullptr, nullptr, nullptr, flags, nullptr,
                            reinterpret_cast<const float*>(kOk), kOk, nullptr, kMis, kOk, kOkF,
                            kOkF, kOkF, nullptr, nullptr, nullptr, nullptr, B, L, D, N, dtype, wsp,
                            wsb, nullptr), B, L, D, N);
        expect_rejected("state_update", ssm_selective_state_update(
                            kOkF, kOk, kOk, kOkF, kOk, kOk, nullptr, nullptr, nullptr, flags,
                            kMis, B, D, N, dtype, nullptr), B, D, N, 0);
        expect_rejected("conv1d", ssm_causal_conv1d_silu(
                            kOk, kOkF, nullptr, nullptr, 1, kMis, nullptr, B, L, D, K, dtype,
                            nullptr), B, L, D, K);
        // SSD: six sizes plus the chunk
        const int64_t H = draw(), P = draw(), G = (next() & 1) ? draw() : 1 + (int64_t)(next() % 4);
        const int64_t chunk = (next() & 1) ? draw() : (int64_t)64 << (next() % 3);
        (void)ssm_ssd_chunk_workspace_bytes(B, L, H, P, G, N, chunk, dtype);
        expect_rejected("ssd", ssm_ssd_chunk_fwd(kOk, kOk, kOkF, kOk, kOk, nullptr, nullptr,
                                                 nullptr, flags & 1u, nullptr, kMis, nullptr, B,
                                                 L, H, P, G, N, chunk, dtype, nullptr, 0, nullptr),
                        B, L, H, P);
        expect_rejected("ssd_varlen", ssm_ssd_chunk_fwd_varlen(
                            kOk, kOk, kOkF, kOk, kOk, nullptr, nullptr, nullptr, flags & 1u,
                            nullptr, kMis, nullptr, reinterpret_cast<const int32_t*>(kOk), B, L,
                            H, P, G, N, chunk, dtype, nullptr, 0, nullptr), B, L, H, P);
    }
    if (g_failures) {
        fprintf(stderr, "%d unexpected results\n", g_failures);
        return 1;
    }
    printf("abi_fuzz: %ld iterations, no finding\n", iters);
    return 0;
}
