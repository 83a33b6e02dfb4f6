// C ABI of the library: argument validation (host only, before any HIP
// call), planning, and dispatch to the kernel launchers.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "ssm.h"
#include "ssm_internal.h"

namespace {

constexpr int64_t kMaxElems = int64_t(1) << 60;   // keeps every byte offset in int64

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int64_t esize(int dtype) { return dtype == SSM_BF16 ? 2 : 4; }

// a*b*c without int64 overflow; -1 if it would exceed kMaxElems
int64_t mul3(int64_t a, int64_t b, int64_t c) {
    if (a < 0 || b < 0 || c < 0) return -1;
    if (a == 0 || b == 0 || c == 0) return 0;
    if (a > kMaxElems / b) return -1;
    const int64_t ab = a * b;
    if (ab > kMaxElems / c) return -1;
    return ab * c;
}

int s6_fwd_impl(const void* u, const void* delta, const float* A, const void* Bm, const void* Cm,
                const float* Dskip, const void* z, const float* delta_bias, unsigned flags,
                const float* h0, void* y, float* h_last, const int32_t* seq_lens,
                int64_t B, int64_t L, int64_t D, int64_t N, int dtype,
                void* workspace, size_t workspace_bytes, void* stream, void* const* events,
                bool static_scratch = false, float* ckpt = nullptr);

int s6_bwd_impl(const void* u, const void* delta, const float* A, const void* Bm, const void* Cm,
                const float* Dskip, const void* z, const float* delta_bias, unsigned flags,
                const float* h0, const void* dy, const float* dh_last, void* du, void* ddelta,
                float* dA, float* dB, float* dC, float* dDskip, void* dz, float* ddelta_bias,
                float* dh0, const float* ckpt, const int32_t* seq_lens, int64_t B, int64_t L,
                int64_t D, int64_t N, int dtype, void* workspace, size_t workspace_bytes,
                void* stream);

int ssd_fwd_impl(const void* X, const void* delta, const float* A, const void* Bm, const void* Cm,
                 const float* Dskip, const void* z, const float* delta_bias, unsigned flags,
                 const float* h0, void* Y, float* h_last, const int32_t* seq_lens, int64_t B,
                 int64_t L, int64_t H, int64_t P, int64_t G, int64_t N, int64_t chunk, int dtype,
                 void* workspace, size_t workspace_bytes, void* stream);

int s6_check_sizes(int64_t B, int64_t L, int64_t D, int64_t N, int dtype) {
    if (dtype != SSM_F32 && dtype != SSM_BF16) return SSM_ERR_BAD_DTYPE;
    if (B < 1 || D < 1 || N < 1 || L < 0) return SSM_ERR_BAD_SHAPE;
    if (mul3(B, L, D) < 0 || mul3(B, L, N) < 0 || mul3(B, D, N) < 0) return SSM_ERR_BAD_SHAPE;
    if (mul3(B, L, D) > kMaxElems / esize(dtype)) return SSM_ERR_BAD_SHAPE;
    if (N > 64) return SSM_ERR_UNSUPPORTED;
    if (B > 65535) return SSM_ERR_UNSUPPORTED;                 // grid y
    // state copies (L = 0) and conv-state copies run B*D*N (or B*D*3) threads
    if ((B * D * N * 4 + 255) / 256 > 0x7fffffffLL) return SSM_ERR_UNSUPPORTED;
    if ((D + 63) / 64 > 0x7fffffffLL) return SSM_ERR_UNSUPPORTED;
    if (((L + 63) / 64) * D * 4 > (int64_t)0xFFFFFFFF) return SSM_ERR_UNSUPPORTED;  // 32-bit segment offsets
    return SSM_OK;
}

int ssd_check_sizes(int64_t B, int64_t L, int64_t H, int64_t P, int64_t G, int64_t N,
                    int64_t chunk, int dtype) {
    if (dtype != SSM_F32 && dtype != SSM_BF16) return SSM_ERR_BAD_DTYPE;
    if (B < 1 || H < 1 || P < 1 || G < 1 || N < 1 || L < 0 || chunk < 1) return SSM_ERR_BAD_SHAPE;
    if (H % G != 0) return SSM_ERR_BAD_SHAPE;
    // bound the products B*H*P and B*G*N first, then every tensor's element count
    if (mul3(B, H, P) < 0 || mul3(B, G, N) < 0) return SSM_ERR_BAD_SHAPE;
    if (mul3(B, L, H) < 0 || mul3(B * H, L, P) < 0 || mul3(B * G, L, N) < 0) return SSM_ERR_BAD_SHAPE;
    if (mul3(B * H, P, N) < 0) return SSM_ERR_BAD_SHAPE;          // h0, h_last
    if (mul3(B * H, L, P) > kMaxElems / esize(dtype)) return SSM_ERR_BAD_SHAPE;
    if (dtype != SSM_BF16 || P % 32 != 0 || N % 32 != 0 || N > 128) return SSM_ERR_UNSUPPORTED;
    if (chunk != 64 && chunk != 128 && chunk != 256) return SSM_ERR_UNSUPPORTED;
    // one workgroup per (b, h, slice of 64 head-dim rows, or 32 when P is not a multiple of 64)
    const int64_t slices = P % 64 == 0 ? P / 64 : P / 32;
    if (B * H > 0x7fffffffLL / slices) return SSM_ERR_UNSUPPORTED;
    // one batch row of X (and of B/C) is addressed with 32-bit byte offsets,
    // including the reads past a ragged last chunk and the prefetch of the
    // chunk after the last (up to two chunks of 256 past L)
    if (H * P * 2 > (int64_t)0xFFFFFFFF / (L + 512) || G * N * 2 > (int64_t)0xFFFFFFFF / (L + 512))
        return SSM_ERR_UNSUPPORTED;
    return SSM_OK;
}

int s6_bwd_check_sizes(int64_t B, int64_t L, int64_t D, int64_t N, int dtype) {
    int rc = s6_check_sizes(B, L, D, N, dtype);
    if (rc != SSM_OK) return rc;
    if (N > 16) return SSM_ERR_UNSUPPORTED;
    const int64_t G = (D + 15) / 16;
    if (G > 0x7fffffffLL || 2 * B * L * N + D * N + D > (int64_t)0x7fffffff * 256)
        return SSM_ERR_UNSUPPORTED;
    if (G * B > 0xffffffffLL) return SSM_ERR_UNSUPPORTED;   // workgroup ids are 32-bit
    if (mul3(2 * G, B * L, N) < 0) return SSM_ERR_BAD_SHAPE;
    if ((L + 16) * N * esize(dtype) >= (int64_t)0x80000000LL) return SSM_ERR_UNSUPPORTED;  // B/C row offsets
    if ((L + 16) * D * esize(dtype) >= (int64_t)0x80000000LL) return SSM_ERR_UNSUPPORTED;  // activation row offsets
    return SSM_OK;
}

}  // namespace

extern "C" {

int ssm_abi_version(void) { return SSM_ABI_VERSION; }

const char* ssm_status_string(int status) {
    switch (status) {
        case SSM_OK: return "ok";
        case SSM_ERR_NULL_ARG: return "a required pointer argument is NULL";
        case SSM_ERR_BAD_SHAPE: return "invalid or overflowing tensor size";
        case SSM_ERR_BAD_DTYPE: return "dtype is not SSM_F32 or SSM_BF16";
        case SSM_ERR_UNSUPPORTED: return "request outside the sizes/dtypes the kernels implement";
        case SSM_ERR_MISALIGNED: return "pointer violates the alignment rule (16 B tensors, 4 B fp32 vectors)";
        case SSM_ERR_WORKSPACE: return "workspace is NULL or smaller than the query returned";
        case SSM_ERR_HIP: return "a HIP call or kernel launch failed";
        default: return "unknown status";
    }
}

int ssm_selective_scan_segments(int64_t B, int64_t L, int64_t D, int64_t N) {
    if (s6_check_sizes(B, L, D, N, SSM_F32) != SSM_OK) return 0;
    const ssm::S6Plan pl = ssm::plan_s6(B, L, D, N);
    return pl.lanes ? pl.S_lanes : pl.S;
}

int ssm_selective_scan_lanes(int64_t B, int64_t L, int64_t D, int64_t N) {
    if (s6_check_sizes(B, L, D, N, SSM_F32) != SSM_OK) return 0;
    return ssm::plan_s6(B, L, D, N).lanes ? 1 : 0;
}

size_t ssm_selective_scan_workspace_bytes(int64_t B, int64_t L, int64_t D, int64_t N,
                                          int dtype) {
    if (s6_check_sizes(B, L, D, N, dtype) != SSM_OK) return 0;
    return ssm::plan_s6(B, L, D, N).workspace_bytes;
}

int ssm_selective_scan_fwd(const void* u, const void* delta, const float* A,
                           const void* Bm, const void* Cm, const float* Dskip,
                           const void* z, const float* delta_bias, unsigned flags,
                           const float* h0, void* y, float* h_last,
                           int64_t B, int64_t L, int64_t D, int64_t N, int dtype,
                           void* workspace, size_t workspace_bytes, void* stream) {
    return ssm_selective_scan_fwd_timed(u, delta, A, Bm, Cm, Dskip, z, delta_bias, flags, h0, y,
                                        h_last, B, L, D, N, dtype, workspace, workspace_bytes,
                                        stream, nullptr);
}

int ssm_selective_scan_fwd_varlen(const void* u, const void* delta, const float* A,
                                  const void* Bm, const void* Cm, const float* Dskip,
                                  const void* z, const float* delta_bias, unsigned flags,
                                  const float* h0, void* y, float* h_last,
                                  const int32_t* seq_lens, int64_t B, int64_t L, int64_t D,
                                  int64_t N, int dtype, void* workspace, size_t workspace_bytes,
                                  void* stream) {
    if (!seq_lens) return SSM_ERR_NULL_ARG;
    if (!aligned(seq_lens, 4)) return SSM_ERR_MISALIGNED;
    return s6_fwd_impl(u, delta, A, Bm, Cm, Dskip, z, delta_bias, flags, h0, y, h_last, seq_lens,
                       B, L, D, N, dtype, workspace, workspace_bytes, stream, nullptr);
}

int ssm_selective_scan_fwd_noalloc(const void* u, const void* delta, const float* A,
                                   const void* Bm, const void* Cm, const float* Dskip,
                                   const void* z, const float* delta_bias, unsigned flags,
                                   const float* h0, void* y, float* h_last,
                                   int64_t B, int64_t L, int64_t D, int64_t N, int dtype,
                                   void* stream) {
    return s6_fwd_impl(u, delta, A, Bm, Cm, Dskip, z, delta_bias, flags, h0, y, h_last, nullptr,
                       B, L, D, N, dtype, nullptr, 0, stream, nullptr, true);
}

int ssm_selective_scan_fwd_timed(const void* u, const void* delta, const float* A,
                                 const void* Bm, const void* Cm, const float* Dskip,
                                 const void* z, const float* delta_bias, unsigned flags,
                                 const float* h0, void* y, float* h_last,
                                 int64_t B, int64_t L, int64_t D, int64_t N, int dtype,
                                 void* workspace, size_t workspace_bytes, void* stream,
                                 void* const* events) {
    return s6_fwd_impl(u, delta, A, Bm, Cm, Dskip, z, delta_bias, flags, h0, y, h_last, nullptr,
                       B, L, D, N, dtype, workspace, workspace_bytes, stream, events);
}

size_t ssm_selective_scan_ckpt_bytes(int64_t B, int64_t L, int64_t D, int64_t N, int dtype) {
    if (s6_bwd_check_sizes(B, L, D, N, dtype) != SSM_OK) return 0;
    return (size_t)(B * D * ((L + 15) / 16) * N) * sizeof(float);
}

int ssm_selective_scan_fwd_ckpt(const void* u, const void* delta, const float* A,
                                const void* Bm, const void* Cm, const float* Dskip,
                                const void* z, const float* delta_bias, unsigned flags,
                                const float* h0, void* y, float* h_last, float* ckpt,
                                int64_t B, int64_t L, int64_t D, int64_t N, int dtype,
                                void* workspace, size_t workspace_bytes, void* stream) {
    // the sizes and flags the backward takes
    const int rc = s6_bwd_check_sizes(B, L, D, N, dtype);
    if (rc != SSM_OK) return rc;
    if (flags & ~(unsigned)SSM_FLAG_DELTA_SOFTPLUS) return SSM_ERR_UNSUPPORTED;
    if (L > 0 && !ckpt) return SSM_ERR_NULL_ARG;
    if (ckpt && !aligned(ckpt, 16)) return SSM_ERR_MISALIGNED;
    return s6_fwd_impl(u, delta, A, Bm, Cm, Dskip, z, delta_bias, flags, h0, y, h_last, nullptr,
                       B, L, D, N, dtype, workspace, workspace_bytes, stream, nullptr, false,
                       L > 0 ? ckpt : nullptr);
}

}  // extern "C"

namespace {

int s6_fwd_impl(const void* u, const void* delta, const float* A, const void* Bm, const void* Cm,
                const float* Dskip, const void* z, const float* delta_bias, unsigned flags,
                const float* h0, void* y, float* h_last, const int32_t* seq_lens,
                int64_t B, int64_t L, int64_t D, int64_t N, int dtype,
                void* workspace, size_t workspace_bytes, void* stream, void* const* events,
                bool static_scratch, float* ckpt) {
    int rc = s6_check_sizes(B, L, D, N, dtype);
    if (rc != SSM_OK) return rc;
    if (flags & ~(unsigned)(SSM_FLAG_DELTA_SOFTPLUS | SSM_FLAG_ZOH)) return SSM_ERR_UNSUPPORTED;
    if (!A) return SSM_ERR_NULL_ARG;
    if (L > 0 && (!u || !delta || !Bm || !Cm || !y)) return SSM_ERR_NULL_ARG;
    const void* big[] = {u, delta, Bm, Cm, z, y};
    for (const void* p : big)
        if (p && !aligned(p, 16)) return SSM_ERR_MISALIGNED;
    const void* vec[] = {A, Dskip, delta_bias, h0, h_last};
    for (const void* p : vec)
        if (p && !aligned(p, 4)) return SSM_ERR_MISALIGNED;
    const ssm::S6Plan plan = ssm::plan_s6(B, L, D, N);
    if (static_scratch) {
        // validation is complete once the plan fits the static scratch; only
        // then is the HIP runtime asked for this device's copy of it
        if (plan.workspace_bytes > ssm::kNoAllocScratchBytes) return SSM_ERR_WORKSPACE;
        workspace = nullptr;
        if (plan.workspace_bytes > 0 && ssm::noalloc_scratch(&workspace) != hipSuccess)
            return SSM_ERR_HIP;
    } else if (plan.workspace_bytes > 0) {
        if (!workspace || workspace_bytes < plan.workspace_bytes) return SSM_ERR_WORKSPACE;
        if (!aligned(workspace, 16)) return SSM_ERR_MISALIGNED;
    }
    ssm::S6Args a{};
    a.u = u; a.delta = delta; a.A = A; a.Bm = Bm; a.Cm = Cm; a.Dskip = Dskip; a.z = z;
    a.delta_bias = delta_bias; a.h0 = h0; a.y = y; a.h_last = h_last;
    a.B = B; a.L = L; a.D = D; a.N = N;
    a.lanes = plan.lanes && !(flags & SSM_FLAG_ZOH);
    a.S = a.lanes ? plan.S_lanes : plan.S;
    a.seg_len = a.lanes ? plan.seg_len_lanes : plan.seg_len;
    a.flags = flags; a.bf16 = dtype == SSM_BF16;
    a.events = reinterpret_cast<hipEvent_t const*>(events);
    a.seq_lens = seq_lens;
    ssm::s6_carve(a, workspace);
    // checkpoints for the backward: written by the state-per-lane scan itself
    // where it runs (segments after the first completed by the fix-up; its
    // per-channel run of checkpoints addressed with 32-bit offsets), else by
    // the backward's forward sweep afterwards
    const int64_t nck = (L + ssm::plan::kBwdTile - 1) / ssm::plan::kBwdTile;
    const bool fused = ckpt && a.lanes && ssm::plan::kLanesChans * nck * 64 < (int64_t)1 << 31;
    a.ckpt = fused ? ckpt : nullptr;
    a.ckpt_blocks = nck;
    hipError_t e = ssm::launch_s6(a, static_cast<hipStream_t>(stream));
    if (e == hipSuccess && ckpt && !fused && L > 0) {
        ssm::S6BwdArgs c{};
        c.u = u; c.delta = delta; c.A = A; c.Bm = Bm; c.delta_bias = delta_bias; c.h0 = h0;
        c.B = B; c.L = L; c.D = D; c.N = N; c.flags = flags; c.bf16 = dtype == SSM_BF16;
        c.ckpt = ckpt;
        e = ssm::launch_s6_bwd_ckpt(c, static_cast<hipStream_t>(stream));
    }
    return e == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

}  // namespace

extern "C" {

int ssm_selective_scan_conv_fwd(const void* x, const float* conv_weight, const float* conv_bias,
                                const float* conv_state_in, float* conv_state_out, int64_t K,
                                void* u_out, const void* delta, const float* A, const void* Bm,
                                const void* Cm, const float* Dskip, const void* z,
                                const float* delta_bias, unsigned flags, const float* h0, void* y,
                                float* h_last, int64_t B, int64_t L, int64_t D, int64_t N,
                                int dtype, void* workspace, size_t workspace_bytes, void* stream) {
    int rc = s6_check_sizes(B, L, D, N, dtype);
    if (rc != SSM_OK) return rc;
    if (flags & ~(unsigned)SSM_FLAG_DELTA_SOFTPLUS) return SSM_ERR_UNSUPPORTED;
    if (N != 16) return SSM_ERR_UNSUPPORTED;
    if (K < 1) return SSM_ERR_BAD_SHAPE;
    if (K > 4) return SSM_ERR_UNSUPPORTED;
    if (!A || !conv_weight) return SSM_ERR_NULL_ARG;
    if (L > 0 && (!x || !delta || !Bm || !Cm || !y)) return SSM_ERR_NULL_ARG;
    const void* big[] = {x, delta, Bm, Cm, z, y, u_out};
    for (const void* p : big)
        if (p && !aligned(p, 16)) return SSM_ERR_MISALIGNED;
    const void* vec[] = {A, Dskip, delta_bias, h0, h_last, conv_weight, conv_bias, conv_state_in,
                         conv_state_out};
    for (const void* p : vec)
        if (p && !aligned(p, 4)) return SSM_ERR_MISALIGNED;
    const ssm::S6Plan plan = ssm::plan_s6(B, L, D, N);
    if (plan.workspace_bytes > 0) {
        if (!workspace || workspace_bytes < plan.workspace_bytes) return SSM_ERR_WORKSPACE;
        if (!aligned(workspace, 16)) return SSM_ERR_MISALIGNED;
    }
    ssm::S6Args a{};
    a.u = x; a.delta = delta; a.A = A; a.Bm = Bm; a.Cm = Cm; a.Dskip = Dskip; a.z = z;
    a.delta_bias = delta_bias; a.h0 = h0; a.y = y; a.h_last = h_last;
    a.B = B; a.L = L; a.D = D; a.N = N;
    a.lanes = plan.lanes;
    a.S = a.lanes ? plan.S_lanes : plan.S;
    a.seg_len = a.lanes ? plan.seg_len_lanes : plan.seg_len;
    a.flags = flags; a.bf16 = dtype == SSM_BF16;
    a.conv_w = conv_weight; a.conv_b = conv_bias; a.conv_state_in = conv_state_in;
    a.conv_state_out = conv_state_out; a.u_out = u_out; a.conv_K = K;
    ssm::s6_carve(a, workspace);
    const hipError_t e = ssm::launch_s6(a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

size_t ssm_ssd_chunk_workspace_bytes(int64_t B, int64_t L, int64_t H, int64_t P,
                                     int64_t G, int64_t N, int64_t chunk, int dtype) {
    (void)ssd_check_sizes(B, L, H, P, G, N, chunk, dtype);
    return 0;   // the chunk kernel carries its state on chip
}

int ssm_ssd_chunk_fwd(const void* X, const void* delta, const float* A,
                      const void* Bm, const void* Cm, const float* Dskip,
                      const void* z, const float* delta_bias, unsigned flags,
                      const float* h0, void* Y, float* h_last,
                      int64_t B, int64_t L, int64_t H, int64_t P, int64_t G,
                      int64_t N, int64_t chunk, int dtype,
                      void* workspace, size_t workspace_bytes, void* stream) {
    return ssd_fwd_impl(X, delta, A, Bm, Cm, Dskip, z, delta_bias, flags, h0, Y, h_last, nullptr,
                        B, L, H, P, G, N, chunk, dtype, workspace, workspace_bytes, stream);
}

int ssm_ssd_chunk_fwd_varlen(const void* X, const void* delta, const float* A,
                             const void* Bm, const void* Cm, const float* Dskip,
                             const void* z, const float* delta_bias, unsigned flags,
                             const float* h0, void* Y, float* h_last, const int32_t* seq_lens,
                             int64_t B, int64_t L, int64_t H, int64_t P, int64_t G,
                             int64_t N, int64_t chunk, int dtype,
                             void* workspace, size_t workspace_bytes, void* stream) {
    if (!seq_lens) return SSM_ERR_NULL_ARG;
    if (!aligned(seq_lens, 4)) return SSM_ERR_MISALIGNED;
    return ssd_fwd_impl(X, delta, A, Bm, Cm, Dskip, z, delta_bias, flags, h0, Y, h_last, seq_lens,
                        B, L, H, P, G, N, chunk, dtype, workspace, workspace_bytes, stream);
}

int ssm_selective_state_update(float* state, const void* u, const void* delta, const float* A,
                               const void* Bm, const void* Cm, const float* Dskip,
                               const void* z, const float* delta_bias, unsigned flags, void* y,
                               int64_t B, int64_t D, int64_t N, int dtype, void* stream) {
    if (dtype != SSM_F32 && dtype != SSM_BF16) return SSM_ERR_BAD_DTYPE;
    if (B < 1 || D < 1 || N < 1) return SSM_ERR_BAD_SHAPE;
    if (mul3(B, D, N) < 0 || mul3(B, D, N) > kMaxElems / 4) return SSM_ERR_BAD_SHAPE;
    if (N > 64) return SSM_ERR_UNSUPPORTED;
    if ((B * D * N + 255) / 256 > 0x7fffffffLL) return SSM_ERR_UNSUPPORTED;   // grid x
    if (flags & ~(unsigned)(SSM_FLAG_DELTA_SOFTPLUS | SSM_FLAG_ZOH)) return SSM_ERR_UNSUPPORTED;
    if (!state || !u || !delta || !A || !Bm || !Cm || !y) return SSM_ERR_NULL_ARG;
    const void* big[] = {state, A, u, delta, Bm, Cm, z, y};
    for (const void* p : big)
        if (p && !aligned(p, 16)) return SSM_ERR_MISALIGNED;
    const void* vec[] = {Dskip, delta_bias};
    for (const void* p : vec)
        if (p && !aligned(p, 4)) return SSM_ERR_MISALIGNED;
    ssm::StepArgs a{};
    a.state = state; a.u = u; a.delta = delta; a.A = A; a.Bm = Bm; a.Cm = Cm; a.Dskip = Dskip;
    a.z = z; a.delta_bias = delta_bias; a.y = y;
    a.B = B; a.D = D; a.N = N; a.flags = flags; a.bf16 = dtype == SSM_BF16;
    const hipError_t e = ssm::launch_s6_step(a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

size_t ssm_selective_scan_bwd_workspace_bytes(int64_t B, int64_t L, int64_t D, int64_t N,
                                              int dtype) {
    if (s6_bwd_check_sizes(B, L, D, N, dtype) != SSM_OK) return 0;
    return ssm::s6_bwd_workspace_bytes(B, L, D, N, true);
}

int ssm_selective_scan_bwd(const void* u, const void* delta, const float* A, const void* Bm,
                           const void* Cm, const float* Dskip, const void* z,
                           const float* delta_bias, unsigned flags, const float* h0,
                           const void* dy, const float* dh_last, void* du, void* ddelta,
                           float* dA, float* dB, float* dC, float* dDskip, void* dz,
                           float* ddelta_bias, float* dh0, int64_t B, int64_t L, int64_t D,
                           int64_t N, int dtype, void* workspace, size_t workspace_bytes,
                           void* stream) {
    return s6_bwd_impl(u, delta, A, Bm, Cm, Dskip, z, delta_bias, flags, h0, dy, dh_last, du,
                       ddelta, dA, dB, dC, dDskip, dz, ddelta_bias, dh0, nullptr, nullptr, B, L,
                       D, N, dtype, workspace, workspace_bytes, stream);
}

int ssm_selective_scan_bwd_varlen(const void* u, const void* delta, const float* A,
                                  const void* Bm, const void* Cm, const float* Dskip,
                                  const void* z, const float* delta_bias, unsigned flags,
                                  const float* h0, const void* dy, const float* dh_last, void* du,
                                  void* ddelta, float* dA, float* dB, float* dC, float* dDskip,
                                  void* dz, float* ddelta_bias, float* dh0,
                                  const int32_t* seq_lens, int64_t B, int64_t L, int64_t D,
                                  int64_t N, int dtype, void* workspace, size_t workspace_bytes,
                                  void* stream) {
    if (!seq_lens) return SSM_ERR_NULL_ARG;
    if (!aligned(seq_lens, 4)) return SSM_ERR_MISALIGNED;
    return s6_bwd_impl(u, delta, A, Bm, Cm, Dskip, z, delta_bias, flags, h0, dy, dh_last, du,
                       ddelta, dA, dB, dC, dDskip, dz, ddelta_bias, dh0, nullptr, seq_lens, B, L,
                       D, N, dtype, workspace, workspace_bytes, stream);
}

int ssm_selective_scan_bwd_segments(int64_t B, int64_t L, int64_t D, int64_t N) {
    if (s6_bwd_check_sizes(B, L, D, N, SSM_F32) != SSM_OK) return 0;
    return ssm::plan_s6_bwd(B, L, D, N).S;
}

size_t ssm_selective_scan_bwd_ckpt_workspace_bytes(int64_t B, int64_t L, int64_t D, int64_t N,
                                                   int dtype) {
    if (s6_bwd_check_sizes(B, L, D, N, dtype) != SSM_OK) return 0;
    return ssm::s6_bwd_workspace_bytes(B, L, D, N, false);
}

int ssm_selective_scan_bwd_ckpt(const void* u, const void* delta, const float* A, const void* Bm,
                                const void* Cm, const float* Dskip, const void* z,
                                const float* delta_bias, unsigned flags, const float* h0,
                                const float* ckpt, const void* dy, const float* dh_last,
                                void* du, void* ddelta, float* dA, float* dB, float* dC,
                                float* dDskip, void* dz, float* ddelta_bias, float* dh0,
                                int64_t B, int64_t L, int64_t D, int64_t N, int dtype,
                                void* workspace, size_t workspace_bytes, void* stream) {
    if (L > 0 && !ckpt) return SSM_ERR_NULL_ARG;
    if (ckpt && !aligned(ckpt, 16)) return SSM_ERR_MISALIGNED;
    return s6_bwd_impl(u, delta, A, Bm, Cm, Dskip, z, delta_bias, flags, h0, dy, dh_last, du,
                       ddelta, dA, dB, dC, dDskip, dz, ddelta_bias, dh0, L > 0 ? ckpt : nullptr,
                       nullptr, B, L, D, N, dtype, workspace, workspace_bytes, stream);
}

int ssm_causal_conv1d_silu(const void* x, const float* weight, const float* bias,
                           const float* state_in, int silu, void* u, float* state_out,
                           int64_t B, int64_t L, int64_t D, int64_t K, int dtype, void* stream) {
    if (dtype != SSM_F32 && dtype != SSM_BF16) return SSM_ERR_BAD_DTYPE;
    if (B < 1 || D < 1 || L < 0 || K < 1) return SSM_ERR_BAD_SHAPE;
    if (mul3(B, L, D) < 0 || mul3(B, L, D) > kMaxElems / esize(dtype)) return SSM_ERR_BAD_SHAPE;
    if (K > 4) return SSM_ERR_UNSUPPORTED;
    if (mul3(B, D, K) < 0) return SSM_ERR_BAD_SHAPE;                // states [B, D, K-1]
    if ((B * D * K + 255) / 256 > 0x7fffffffLL) return SSM_ERR_UNSUPPORTED;   // state-pass grid
    const int64_t tiles = mul3(B, D, (L + 31) / 32);
    if (tiles < 0 || tiles / 256 > 0x7fffffffLL) return SSM_ERR_UNSUPPORTED;  // grid x
    if (!weight) return SSM_ERR_NULL_ARG;
    if (L > 0 && (!x || !u)) return SSM_ERR_NULL_ARG;
    const void* big[] = {x, u};
    for (const void* p : big)
        if (p && !aligned(p, 16)) return SSM_ERR_MISALIGNED;
    const void* vec[] = {weight, bias, state_in, state_out};
    for (const void* p : vec)
        if (p && !aligned(p, 4)) return SSM_ERR_MISALIGNED;
    ssm::ConvArgs a{};
    a.x = x; a.weight = weight; a.bias = bias; a.state_in = state_in; a.u = u;
    a.state_out = state_out; a.B = B; a.L = L; a.D = D; a.K = K; a.silu = silu != 0;
    a.bf16 = dtype == SSM_BF16;
    const hipError_t e = ssm::launch_conv1d(a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

}  // extern "C"

namespace {

int s6_bwd_impl(const void* u, const void* delta, const float* A, const void* Bm, const void* Cm,
                const float* Dskip, const void* z, const float* delta_bias, unsigned flags,
                const float* h0, const void* dy, const float* dh_last, void* du, void* ddelta,
                float* dA, float* dB, float* dC, float* dDskip, void* dz, float* ddelta_bias,
                float* dh0, const float* ckpt, const int32_t* seq_lens, int64_t B, int64_t L,
                int64_t D, int64_t N, int dtype, void* workspace, size_t workspace_bytes,
                void* stream) {
    int rc = s6_bwd_check_sizes(B, L, D, N, dtype);
    if (rc != SSM_OK) return rc;
    if (flags & ~(unsigned)SSM_FLAG_DELTA_SOFTPLUS) return SSM_ERR_UNSUPPORTED;
    if (!A || !dA) return SSM_ERR_NULL_ARG;
    if (L > 0 && (!u || !delta || !Bm || !Cm || !dy || !du || !ddelta || !dB || !dC))
        return SSM_ERR_NULL_ARG;
    if (L > 0 && z && !dz) return SSM_ERR_NULL_ARG;
    const void* big[] = {u, delta, Bm, Cm, z, dy, du, ddelta, dB, dC, dz};
    for (const void* p : big)
        if (p && !aligned(p, 16)) return SSM_ERR_MISALIGNED;
    const void* vec[] = {A, Dskip, delta_bias, h0, dh_last, dA, dDskip, ddelta_bias, dh0};
    for (const void* p : vec)
        if (p && !aligned(p, 4)) return SSM_ERR_MISALIGNED;
    const bool own = ckpt == nullptr;
    const size_t need = ssm::s6_bwd_workspace_bytes(B, L, D, N, own);
    if (!workspace || workspace_bytes < need) return SSM_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return SSM_ERR_MISALIGNED;
    ssm::S6BwdArgs a{};
    a.u = u; a.delta = delta; a.A = A; a.Bm = Bm; a.Cm = Cm; a.Dskip = Dskip;
    a.z = L > 0 ? z : nullptr; a.delta_bias = delta_bias; a.h0 = h0; a.dy = dy;
    a.dh_last = dh_last; a.du = du; a.ddelta = ddelta; a.dA = dA; a.dB = dB; a.dC = dC;
    a.dDskip = dDskip; a.dz = dz; a.ddelta_bias = ddelta_bias; a.dh0 = dh0;
    a.B = B; a.L = L; a.D = D; a.N = N; a.flags = flags; a.bf16 = dtype == SSM_BF16;
    a.own_ckpt = own;
    a.ckpt = const_cast<float*>(ckpt);
    a.seq_lens = seq_lens;
    const ssm::S6BwdPlan plan = ssm::plan_s6_bwd(B, L, D, N);
    a.S = plan.S;
    a.seg_tiles = plan.seg_tiles;
    ssm::s6_bwd_carve(a, workspace);
    const hipError_t e = ssm::launch_s6_bwd(a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

int ssd_fwd_impl(const void* X, const void* delta, const float* A, const void* Bm, const void* Cm,
                 const float* Dskip, const void* z, const float* delta_bias, unsigned flags,
                 const float* h0, void* Y, float* h_last, const int32_t* seq_lens, int64_t B,
                 int64_t L, int64_t H, int64_t P, int64_t G, int64_t N, int64_t chunk, int dtype,
                 void* workspace, size_t workspace_bytes, void* stream) {
    (void)workspace;
    (void)workspace_bytes;
    int rc = ssd_check_sizes(B, L, H, P, G, N, chunk, dtype);
    if (rc != SSM_OK) return rc;
    if (flags & ~(unsigned)SSM_FLAG_DELTA_SOFTPLUS) return SSM_ERR_UNSUPPORTED;
    if (!A) return SSM_ERR_NULL_ARG;
    if (L > 0 && (!X || !delta || !Bm || !Cm || !Y)) return SSM_ERR_NULL_ARG;
    const void* big[] = {X, delta, Bm, Cm, z, Y};
    for (const void* p : big)
        if (p && !aligned(p, 16)) return SSM_ERR_MISALIGNED;
    const void* vec[] = {A, Dskip, delta_bias, h0, h_last};
    for (const void* p : vec)
        if (p && !aligned(p, 4)) return SSM_ERR_MISALIGNED;
    ssm::SSDArgs a{};
    a.X = X; a.delta = delta; a.A = A; a.Bm = Bm; a.Cm = Cm; a.Dskip = Dskip; a.z = z;
    a.delta_bias = delta_bias; a.h0 = h0; a.Y = Y; a.h_last = h_last;
    a.B = B; a.L = L; a.H = H; a.P = P; a.G = G; a.N = N; a.chunk = chunk; a.flags = flags;
    a.seq_lens = seq_lens;
    const hipError_t e = ssm::launch_ssd(a, static_cast<hipStream_t>(stream));
    if (e == hipErrorNotSupported) return SSM_ERR_UNSUPPORTED;
    return e == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

}  // namespace
