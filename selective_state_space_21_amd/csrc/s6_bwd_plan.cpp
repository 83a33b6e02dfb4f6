// Host-side planning of the backward call: its sequence segments and the
// layout of its workspace.  Plain host code: pure functions of the sizes (and
// the SSM_BWD_SEGMENTS override), no HIP call, so the C-ABI layer can run them
// while validating its arguments.
#include <stdint.h>
#include <stdlib.h>

#include "ssm_internal.h"

namespace ssm {

using namespace plan;

S6BwdPlan plan_s6_bwd(int64_t B, int64_t L, int64_t D, int64_t N) {
    (void)N;
    S6BwdPlan pl{1, 0};
    const int64_t nblk = (L + kBwdTile - 1) / kBwdTile;
    pl.seg_tiles = nblk;
    if (nblk == 0) return pl;
    // Both sweeps walk the sequence tile by tile, one workgroup per channel
    // group and batch row (the adjoint sweep's take a CU each).  With fewer
    // than 128 of those the sequence is cut into segments of at least 1024
    // tokens: as many as keep the adjoint-sweep workgroups within four rounds
    // of one per CU (256 CUs), rounded down, since a fifth round with a few
    // workgroups costs a whole workgroup's time.  (At B = 1, L = 131072,
    // D = 2048, fp32, 43 channel groups: 23 segments, 989 workgroups,
    // 7.33 ms; 24 segments, 1032 workgroups, 7.98 ms; 22 7.58; 21 7.84;
    // earlier: 5 segments 9.28 ms, 8 10.0, 11 7.73, 16 7.80, 32 7.65.)
    const int64_t wgs = B * ((D + kBwdChans - 1) / kBwdChans);
    int64_t S = 1;
    if (wgs < 128) {
        S = 1024 / wgs;
        if (S > nblk / 64) S = nblk / 64;
    }
    const char* env = getenv("SSM_BWD_SEGMENTS");
    if (env && atoi(env) > 0) S = atoi(env);
    if (S > kBwdMaxSegments) S = kBwdMaxSegments;
    if (S > nblk) S = nblk;
    if (S < 1) S = 1;
    // whole super-tiles of the checkpoint sweep per segment
    int64_t seg = (nblk + S - 1) / S;
    seg = (seg + kBwdSuper - 1) / kBwdSuper * kBwdSuper;
    pl.S = (int)((nblk + seg - 1) / seg);
    pl.seg_tiles = pl.S > 1 ? seg : nblk;
    return pl;
}

namespace {
int64_t al256(int64_t bytes) { return (bytes + 255) / 256 * 256; }

// byte sizes of the workspace regions, in carve order
struct BwdRegions {
    int64_t part_bc, part_dA, part_dD, part_db, dsum, fend, radj, hin, qin, ckpt;
};

BwdRegions bwd_regions(int64_t B, int64_t L, int64_t D, int64_t N, int S) {
    const int64_t nblk = (L + kBwdTile - 1) / kBwdTile;
    const int64_t G = (D + kBwdChans - 1) / kBwdChans;
    const int64_t seg = S > 1 ? S : 0;
    BwdRegions r;
    r.part_bc = al256(2 * G * B * L * N * 4);
    r.part_dA = al256(S * B * D * N * 4);
    r.part_dD = al256(S * B * D * 4);
    r.part_db = r.part_dD;
    r.dsum = al256(seg * B * D * 4);
    r.fend = r.radj = r.hin = r.qin = al256(seg * B * D * N * 4);
    r.ckpt = al256(B * D * nblk * N * 4);
    return r;
}
}  // namespace

size_t s6_bwd_workspace_bytes(int64_t B, int64_t L, int64_t D, int64_t N, bool own_ckpt) {
    const BwdRegions r = bwd_regions(B, L, D, N, plan_s6_bwd(B, L, D, N).S);
    return (size_t)(r.part_bc + r.part_dA + r.part_dD + r.part_db + r.dsum + r.fend + r.radj +
                    r.hin + r.qin + (own_ckpt ? r.ckpt : 0));
}

void s6_bwd_carve(S6BwdArgs& a, void* ws) {
    const BwdRegions r = bwd_regions(a.B, a.L, a.D, a.N, a.S);
    char* p = static_cast<char*>(ws);
    auto take = [&](int64_t bytes) {
        float* f = reinterpret_cast<float*>(p);
        p += bytes;
        return f;
    };
    a.part_bc = take(r.part_bc);
    a.part_dA = take(r.part_dA);
    a.part_dD = take(r.part_dD);
    a.part_db = take(r.part_db);
    a.seg_dsum = take(r.dsum);
    a.seg_fend = take(r.fend);
    a.seg_radj = take(r.radj);
    a.seg_hin = take(r.hin);
    a.seg_qin = take(r.qin);
    if (a.own_ckpt) a.ckpt = take(r.ckpt);
}

}  // namespace ssm
