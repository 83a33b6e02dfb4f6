// Internal declarations shared by the C-ABI layer and the kernel launchers.
// Not part of the public interface (include/ssm.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ssm.h"

namespace ssm {

// One S6 call, fully validated, with the segment plan resolved.
struct S6Args {
    const void* u;
    const void* delta;
    const float* A;
    const void* Bm;
    const void* Cm;
    const float* Dskip;
    const void* z;
    const float* delta_bias;
    const float* h0;
    void* y;
    float* h_last;
    // workspace: per (b, d, segment, n) decay and offset, fp32 each
    float* seg_a;
    float* seg_b;
    int64_t B, L, D, N;
    int64_t seg_len;   // tokens per segment (last one may be shorter)
    int S;             // number of segments along L (1 = no carry)
    unsigned flags;
    int bf16;          // storage dtype of activations: 1 = bf16, 0 = fp32
    hipEvent_t const* events;   // NULL, or 4 events recorded at the phase boundaries
    // causal conv1d + SiLU fused in front of the scan (u then holds its input x)
    const float* conv_w;        // [D, conv_K] or NULL (no convolution)
    const float* conv_b;        // [D] or NULL
    const float* conv_state_in; // [B, D, conv_K - 1] or NULL
    float* conv_state_out;      // [B, D, conv_K - 1] or NULL
    void* u_out;                // [B, L, D] or NULL: the convolution's output u
    int64_t conv_K;
    const int32_t* seq_lens;    // [B] tokens per batch row (device), or NULL: all L
    bool lanes;                 // state-per-lane kernel (unsplit) for N = 16 without ZOH
};

struct S6Plan {
    int S;                  // segments of the split path
    int64_t seg_len;
    size_t workspace_bytes; // of the split path (also required when lanes is set)
    bool lanes;             // an N = 16 call without ZOH takes the state-per-lane kernel
};

// Deterministic in the sizes (plus the SSM_S6_SEGMENTS / SSM_S6_LANES overrides).
S6Plan plan_s6(int64_t B, int64_t L, int64_t D, int64_t N);

hipError_t launch_s6(const S6Args& a, hipStream_t stream);

struct SSDArgs {
    const void* X;
    const void* delta;
    const float* A;
    const void* Bm;
    const void* Cm;
    const float* Dskip;
    const void* z;
    const float* delta_bias;
    const float* h0;
    void* Y;
    float* h_last;
    int64_t B, L, H, P, G, N, chunk;
    unsigned flags;
};

hipError_t launch_ssd(const SSDArgs& a, hipStream_t stream);

// One decode step of the selective scan against a resident state.
struct StepArgs {
    float* state;          // [B, D, N] fp32, read and written in place
    const void* u;         // [B, D]
    const void* delta;     // [B, D]
    const float* A;        // [D, N]
    const void* Bm;        // [B, N]
    const void* Cm;        // [B, N]
    const float* Dskip;
    const void* z;
    const float* delta_bias;
    void* y;               // [B, D]
    int64_t B, D, N;
    unsigned flags;
    int bf16;
};

hipError_t launch_s6_step(const StepArgs& a, hipStream_t stream);

// Backward pass of the selective scan (states recomputed, not stored).
struct S6BwdArgs {
    const void* u;
    const void* delta;
    const float* A;
    const void* Bm;
    const void* Cm;
    const float* Dskip;
    const void* z;
    const float* delta_bias;
    const float* h0;
    const void* dy;
    const float* dh_last;
    void* du;
    void* ddelta;
    float* dA;
    float* dB;
    float* dC;
    float* dDskip;
    void* dz;
    float* ddelta_bias;
    float* dh0;
    int64_t B, L, D, N;
    unsigned flags;
    int bf16;
    // workspace, carved by s6_bwd_carve
    float* ckpt;       // [B, D, ceil(L/16), N] state before each 16-token tile
    float* part_bc;    // [2][ceil(D/16)][B, L, N] per-channel-group dB, dC
    float* part_dA;    // [B, D, N]
    float* part_dD;    // [B, D]
    float* part_db;    // [B, D]
};

size_t s6_bwd_workspace_bytes(int64_t B, int64_t L, int64_t D, int64_t N);
void s6_bwd_carve(S6BwdArgs& a, void* workspace);
hipError_t launch_s6_bwd(const S6BwdArgs& a, hipStream_t stream);

// Causal depthwise conv1d (+ SiLU) over tokens.
struct ConvArgs {
    const void* x;            // [B, L, D]
    const float* weight;      // [D, K]
    const float* bias;        // [D] or NULL
    const float* state_in;    // [B, D, K-1] or NULL
    void* u;                  // [B, L, D]
    float* state_out;         // [B, D, K-1] or NULL
    int64_t B, L, D, K;
    int silu;
    int bf16;
};

hipError_t launch_conv1d(const ConvArgs& a, hipStream_t stream);

}  // namespace ssm
