// Host-side planning of the library's calls: the S6 segment plan (which
// kernel, how many sequence segments, the workspace they need) and the layout
// of the backward call's workspace.  Plain host code: pure functions of the
// sizes (and two environment overrides), no HIP call, so the C-ABI layer can
// run them while validating its arguments.
#include <stdint.h>
#include <stdlib.h>

#include "ssm_internal.h"

namespace ssm {

using namespace plan;

S6Plan plan_s6(int64_t B, int64_t L, int64_t D, int64_t N) {
    S6Plan pl{};
    pl.S = 1;
    pl.seg_len = L > 0 ? L : 1;
    pl.S_lanes = 1;
    pl.seg_len_lanes = pl.seg_len;
    if (L <= 0) return pl;
    const char* env_seg = getenv("SSM_S6_SEGMENTS");
    const int64_t forced = (env_seg && atoi(env_seg) > 0) ? atoi(env_seg) : 0;
    // State-per-lane kernel: N = 16, D a multiple of 16 and a batch row's
    // activations (plus two super-tiles) within 32-bit buffer offsets at 4
    // bytes per element.  SSM_S6_LANES=0 turns it off.  It runs B*D/4
    // wavefronts per segment: unsplit with at least two per SIMD, else cut
    // into the fewest segments (whole 128-token multiples) that give six per
    // SIMD; the segments after the first are fixed up afterwards.  (Six is
    // more than fit at once, five by registers, but the scan's gain from the
    // extra wavefronts outweighs the tail and the longer fix-up: at B=1
    // L=131072 D=2048 fp32, 12 segments ran 1.25-1.27 ms, 8 segments
    // (four per SIMD, one round) 1.27-1.30 ms, 16 segments 1.33 ms.)
    {
        const bool shape_ok = N == 16 && D % kLanesChans == 0 &&
                              (L + 2 * kLanesSpan) * D * 4 <= (int64_t)0xFFFFFFFF;
        pl.lanes = shape_ok;
        const char* env = getenv("SSM_S6_LANES");
        if (env && env[0] == '0') pl.lanes = false;
        const int64_t waves = B * D / 4;
        int64_t S = waves >= 2 * kSimds ? 1 : (6 * kSimds + waves - 1) / (waves > 0 ? waves : 1);
        if (forced) S = forced;
        int64_t maxS = (L + kLanesSpan - 1) / kLanesSpan;
        if (maxS > kMaxSegments) maxS = kMaxSegments;
        if (S > maxS) S = maxS;
        if (S < 1) S = 1;
        int64_t seg_len = (L + S - 1) / S;
        seg_len = (seg_len + kLanesSpan - 1) / kLanesSpan * kLanesSpan;
        pl.S_lanes = (int)((L + seg_len - 1) / seg_len);
        pl.seg_len_lanes = seg_len;
        // the fix-up runs one 256-thread workgroup per (16 channels, batch
        // row, later segment, chunk), the groups padded to four per row: a
        // one-dimensional grid of fewer than 2^24 workgroups (else the split
        // path takes the call)
        if (pl.lanes && pl.S_lanes > 1) {
            const int64_t K = (seg_len + kFixChunk - 1) / kFixChunk;
            const int64_t rows = (D / kLanesChans + 3) / 4 * 4;
            if (rows * B * (pl.S_lanes - 1) * K >= ((int64_t)1 << 24)) pl.lanes = false;
        }
    }
    // Split path (one lane per channel; ZOH calls, other N, or the
    // state-per-lane kernel turned off).  With at least one wavefront per SIMD
    // the sequence is not split; otherwise the segment count is the smallest
    // that gives every SIMD at least three wavefronts and all SIMDs the same
    // number (a whole multiple of the SIMD count), else the one nearest three
    // per SIMD.
    const int64_t waves = B * ((D + kWave - 1) / kWave);
    const int64_t simds = kSimds;
    const int64_t min_seg = 32;
    int64_t maxS = (L + min_seg - 1) / min_seg;
    if (maxS > kMaxSegments) maxS = kMaxSegments;
    int64_t S = waves >= simds ? 1 : 0;
    for (int64_t c = 1; c <= maxS && S == 0; ++c)
        if (waves * c >= 3 * simds && (waves * c) % simds == 0) S = c;
    if (S == 0) S = (3 * simds + waves - 1) / waves;
    if (forced) S = forced;
    if (S > maxS) S = maxS;
    if (S < 1) S = 1;
    int64_t seg_len = (L + S - 1) / S;
    // the kernels address one segment through 32-bit buffer offsets
    while (seg_len * D * 4 > (int64_t)0xFFFFFFFF && S < kMaxSegments) {
        ++S;
        seg_len = (L + S - 1) / S;
    }
    S = (L + seg_len - 1) / seg_len;   // no empty trailing segment
    pl.S = (int)S;
    pl.seg_len = seg_len;
    // one workspace serves both paths (the size query has no flags, and ZOH
    // calls take the split path): (decay, offset) pairs per segment, and on
    // the state-per-lane path a dt checkpoint per fix-up chunk
    size_t split = 0, lanes = 0;
    if (pl.S > 1) split = (size_t)2 * (size_t)(B * D * pl.S * N) * sizeof(float);
    if (pl.lanes && pl.S_lanes > 1) {
        const int64_t K = (pl.seg_len_lanes + kFixChunk - 1) / kFixChunk;
        lanes = ((size_t)2 * (size_t)(B * D * pl.S_lanes * N) + (size_t)(pl.S_lanes * K * B * D)) *
                sizeof(float);
    }
    pl.workspace_bytes = split > lanes ? split : lanes;
    return pl;
}

void s6_carve(S6Args& a, void* ws) {
    a.seg_a = a.seg_b = a.seg_cum = nullptr;
    a.fix_chunks = 0;
    if (a.S <= 1) return;
    a.seg_a = static_cast<float*>(ws);
    a.seg_b = a.seg_a + a.B * a.D * (int64_t)a.S * a.N;
    if (a.lanes) {
        a.seg_cum = a.seg_b + a.B * a.D * (int64_t)a.S * a.N;
        a.fix_chunks = (a.seg_len + kFixChunk - 1) / kFixChunk;
    }
}

}  // namespace ssm
