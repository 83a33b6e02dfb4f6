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
    // state-per-lane segments: per (segment, chunk, b, d) the sum of dt over
    // the segment up to the end of that chunk of plan::kFixChunk tokens
    float* seg_cum;
    int64_t fix_chunks;   // chunks per segment
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
    bool lanes;                 // state-per-lane kernel for N = 16 without ZOH
    // the state entering every 16-token tile, [B, D, ckpt_blocks, 16] fp32,
    // written by the one-pass state-per-lane scan (NULL: not written)
    float* ckpt;
    int64_t ckpt_blocks;        // ceil(L / 16)
};

struct S6Plan {
    int S;                  // segments of the split path (ZOH calls, or lanes off)
    int64_t seg_len;
    int S_lanes;            // segments of the state-per-lane path
    int64_t seg_len_lanes;
    size_t workspace_bytes; // pairs of either path
    bool lanes;             // an N = 16 call without ZOH takes the state-per-lane kernel
};

// Deterministic in the sizes (plus the SSM_S6_SEGMENTS / SSM_S6_LANES overrides).
// Host code only (s6_plan.cpp): no HIP call.
S6Plan plan_s6(int64_t B, int64_t L, int64_t D, int64_t N);

// Points a call's segment buffers (pairs, and on the state-per-lane path the
// dt checkpoints) into its workspace, after a.S, a.seg_len and a.lanes are set.
void s6_carve(S6Args& a, void* ws);

// Tiling the planners share with the kernels (the kernel sources assert that
// their own constants agree).
namespace plan {
constexpr int kWave = 64;                 // lanes per wavefront
constexpr int64_t kMaxSegments = 256;     // sequence segments per call at most
constexpr int kLanesSpan = 128;           // state-per-lane segments: whole multiples of this
constexpr int kLanesChans = 16;           // state-per-lane kernel: channels per workgroup
constexpr int kFixChunk = 1024;           // state-per-lane fix-up: tokens per workgroup
constexpr int kBwdTile = 16;              // backward: tokens per state checkpoint
constexpr int kBwdChans = 48;             // backward: channels per adjoint-sweep workgroup
constexpr int kBwdSuper = 8;              // backward: tiles per super-tile of the checkpoint sweep
constexpr int kBwdMaxSegments = 64;       // backward: sequence segments at most
// SIMDs the S6 planner balances wavefronts over: MI355X has 256 CUs of four
// SIMDs.  A constant, so that the plan (and the workspace size it implies) is
// a pure function of the sizes and no HIP call is needed before validation.
constexpr int64_t kSimds = 4 * 256;
}  // namespace plan

hipError_t launch_s6(const S6Args& a, hipStream_t stream);

// Size of the static device scratch of ssm_selective_scan_fwd_noalloc.
constexpr size_t kNoAllocScratchBytes = SSM_NOALLOC_SCRATCH_BYTES;
// Device address of the current device's copy of that scratch (looked up once
// per device with hipGetSymbolAddress, then cached).
hipError_t noalloc_scratch(void** out);

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
    const int32_t* seq_lens;    // [B] tokens per batch row (device), or NULL: all L
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
    const int32_t* seq_lens;   // [B] tokens per batch row (device), or NULL: all L
    // the state before each 16-token tile, [B, D, ceil(L/16), N]: carved
    // from the workspace and written by the call's own forward sweep, or
    // given by the caller (own_ckpt false: the sweep is skipped)
    float* ckpt;
    bool own_ckpt;
    // sequence segments (S = 1: none): segment s holds the 16-token tiles
    // [s * seg_tiles, (s + 1) * seg_tiles), all scanned in parallel from the
    // state and adjoint that the carry pass folds from the segment pairs
    int S;
    int64_t seg_tiles;
    float* seg_dsum;   // [S, B, D]    sum of the steps over the segment
    float* seg_fend;   // [S, B, D, N] state at the segment's end, from zero at its start
    float* seg_radj;   // [S, B, D, N] a_t m_t after its first token, from zero at its end
    float* seg_hin;    // [S, B, D, N] state entering the segment
    float* seg_qin;    // [S, B, D, N] a m entering the segment from its right (dh_last for the last)
    // workspace, carved by s6_bwd_carve
    float* part_bc;    // [2][ceil(D/16)][B, L, N] per-channel-group dB, dC
    float* part_dA;    // [S, B, D, N]
    float* part_dD;    // [S, B, D]
    float* part_db;    // [S, B, D]
};

// Sequence segments of a backward call: a pure function of the sizes (and
// the SSM_BWD_SEGMENTS override), like the forward's plan.
struct S6BwdPlan {
    int S;
    int64_t seg_tiles;
};
S6BwdPlan plan_s6_bwd(int64_t B, int64_t L, int64_t D, int64_t N);

// Workspace of a backward call: the partial sums, the segment buffers, then
// (own_ckpt) the checkpoints.
size_t s6_bwd_workspace_bytes(int64_t B, int64_t L, int64_t D, int64_t N, bool own_ckpt);
void s6_bwd_carve(S6BwdArgs& a, void* workspace);
hipError_t launch_s6_bwd(const S6BwdArgs& a, hipStream_t stream);
// The backward's forward sweep alone: fills a.ckpt (reads u, delta, A, Bm,
// delta_bias, h0, flags and the sizes).
hipError_t launch_s6_bwd_ckpt(const S6BwdArgs& a, hipStream_t stream);

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
