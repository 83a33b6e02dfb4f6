// Backward pass of the selective scan with recomputation.
//
// The states are not stored by the forward pass; they are regenerated from
// the saved inputs (the backward pass of the fused kernel in the
// Transformer-math "Selective state space" article, "Why the fused kernel is
// the real contribution", and the recompute idea of section 3 of the
// temporalbook "Selective State-Space Models (Mamba)" chapter).
//
// Forward, per (b, d, n) (include/ssm.h):
//   dt_t = softplus(x_t), x_t = delta_t + bias;  a_t = exp(dt_t A);
//   h_t  = a_t h_{t-1} + dt_t u_t B_t;  r_t = sum_n C_t h_t + D u_t;  y_t = r_t silu(z_t)
// Reverse-mode, with g_t = dy_t silu(z_t) and the adjoint m_t = dL/dh_t:
//   m_t   = g_t C_t + a_{t+1} m_{t+1}          (a_L m_L := dh_last)
//   dC_t += g_t h_t,  dB_t += m_t dt_t u_t     (summed over the channels d)
//   ddt_t = sum_n m_t (h_{t-1} A a_t + B_t u_t);  ddelta_t = ddt_t sigma(x_t)
//   du_t  = g_t D + dt_t sum_n m_t B_t;  dz_t = dy_t r_t silu'(z_t)
//   dA   += m_t h_{t-1} dt_t a_t;  dD += g_t u_t;  dbias += ddelta_t;  dh0 = a_0 m_0
//
// Mapping: a workgroup of 8 wavefronts covers 32 channels of one batch row;
// each 16-lane row of a wavefront is one channel and lane n holds state n
// (N <= 16), so a lane carries one state and one adjoint.  Per-channel,
// per-token scalars (dt, u, g, ...) of a 16-token tile are computed by lane j
// for token j and broadcast along the row with DPP.
//   1. s6_bwd_ckpt: forward sweep storing the state before every tile.
//   2. s6_bwd_main: tiles in reverse; each tile recomputes its 16 states
//      from the checkpoint into registers, then runs the adjoint backwards.
//      Sums over n are row all-reduces (4 DPP adds); dB and dC are summed
//      over the wavefront's 4 rows (xor swizzles) and the workgroup's 8
//      wavefronts (LDS), giving one partial per (channel group, b, t, n).
//   3. s6_bwd_reduce: sums the channel-group partials of dB and dC and the
//      batch partials of dA, D and bias.  No atomics: results are
//      deterministic.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "device_math.h"
#include "lane_ops.h"
#include "ssm_internal.h"

namespace ssm {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kChans = 4 * kWaves;     // channels per workgroup
constexpr int kTile = 16;              // tokens per tile = per checkpoint

struct LaneId {
    int w, l, row, n;
    int64_t b, d, dc;      // dc: d clamped into range for addressing
    bool chan_ok, ok;      // channel exists; channel and state exist
};

__device__ __forceinline__ LaneId lane_id(const S6BwdArgs& p) {
    LaneId id;
    const int tid = threadIdx.x;
    id.w = tid / 64;
    id.l = tid % 64;
    id.row = id.l / 16;
    id.n = id.l % 16;
    id.b = blockIdx.y;
    id.d = (int64_t)blockIdx.x * kChans + 4 * id.w + id.row;
    id.chan_ok = id.d < p.D;
    id.dc = id.chan_ok ? id.d : p.D - 1;
    id.ok = id.chan_ok && id.n < p.N;
    return id;
}

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
        0, __builtin_bit_cast(int, x), CTRL, 0xf, 0xf, true));
}

// sum over the 16 lanes of each row, result in every lane of the row
__device__ __forceinline__ float row_sum(float v) {
    v += dpp_mov<0xB1>(v);    // quad_perm [1,0,3,2]
    v += dpp_mov<0x4E>(v);    // quad_perm [2,3,0,1]: every lane of a quad holds its sum
    v += dpp_mov<0x124>(v);   // row_ror 4: quads q and q+1
    v += dpp_mov<0x128>(v);   // row_ror 8: all four quads
    return v;
}

__device__ __forceinline__ float sigmoid_f(float x) {
    return fast_rcp(1.0f + fast_exp2(-x * kLog2e));
}

// Per-channel scalars of token t0 + j, computed by lane j of the row.
template <typename T, bool HAS_Z, bool SOFTPLUS, bool FULL>
struct TileScalars {
    float dt, dtu, u, g, sig, z, dy;

    __device__ __forceinline__ void load(const S6BwdArgs& p, const LaneId& id, int64_t t0,
                                         float bias) {
        const int64_t t = t0 + id.n;
        const bool in = id.chan_ok && t < p.L;
        const int64_t i = (id.b * p.L + (in ? t : 0)) * p.D + id.dc;
        const float x = Elem<T>::load(static_cast<const T*>(p.delta), i) + bias;
        u = in ? Elem<T>::load(static_cast<const T*>(p.u), i) : 0.0f;
        dt = in ? (SOFTPLUS ? softplus_f(x) : x) : 0.0f;
        dtu = dt * u;
        if constexpr (FULL) {
            sig = SOFTPLUS ? sigmoid_f(x) : 1.0f;
            dy = in ? Elem<T>::load(static_cast<const T*>(p.dy), i) : 0.0f;
            if constexpr (HAS_Z) {
                z = Elem<T>::load(static_cast<const T*>(p.z), i);
                g = dy * silu_f(z);
            } else {
                z = 0.0f;
                g = dy;
            }
        }
    }
};

// B or C [B, L, N] of tokens t0 .. t0 + 15 for this lane's state n, through a
// buffer resource over batch row b: reads past the row (tokens t >= L, and
// lanes n >= N, pointed past the end) return zero.
template <typename T>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t bc_rsrc(const S6BwdArgs& p, int64_t b,
                                                          const void* src) {
    return make_rsrc(static_cast<const T*>(src) + b * p.L * p.N, (uint32_t)(p.L * p.N * sizeof(T)));
}

template <typename T>
__device__ __forceinline__ void load_bc(const S6BwdArgs& p, const LaneId& id, int64_t t0,
                                        __amdgpu_buffer_rsrc_t r, float (&v)[kTile]) {
    const uint32_t vn = id.n < p.N ? (uint32_t)(id.n * sizeof(T)) : 0x80000000u;
    const uint32_t row = (uint32_t)(p.N * sizeof(T));
#pragma unroll
    for (int j = 0; j < kTile; ++j)
        v[j] = Buf<T>::load(r, vn + (uint32_t)(t0 + j) * row, 0);
}

template <typename T, bool SOFTPLUS>
__global__ __launch_bounds__(kThreads) void s6_bwd_ckpt(S6BwdArgs p) {
    const LaneId id = lane_id(p);
    const float a2 = id.ok ? p.A[id.dc * p.N + id.n] * kLog2e : 0.0f;
    const float bias = p.delta_bias ? p.delta_bias[id.dc] : 0.0f;
    const int64_t nblk = (p.L + kTile - 1) / kTile;
    float h = (id.ok && p.h0) ? p.h0[(id.b * p.D + id.d) * p.N + id.n] : 0.0f;
    const auto rB = bc_rsrc<T>(p, id.b, p.Bm);
    float* ck = p.ckpt + (id.b * p.D + id.dc) * nblk * p.N + id.n;
    for (int64_t k = 0; k < nblk; ++k) {
        if (id.ok) ck[k * p.N] = h;
        const int64_t t0 = k * kTile;
        TileScalars<T, false, SOFTPLUS, false> s;
        s.load(p, id, t0, bias);
        float bv[kTile];
        load_bc<T>(p, id, t0, rB, bv);
#pragma unroll
        for (int j = 0; j < kTile; ++j) {
            const float dA = fast_exp2(row_bcast(s.dt, j) * a2);
            h = fmaf(dA, h, bv[j] * row_bcast(s.dtu, j));
        }
    }
}

template <typename T, bool HAS_Z, bool SOFTPLUS>
__global__ __launch_bounds__(kThreads) void s6_bwd_main(S6BwdArgs p) {
    __shared__ float red[2][kWaves][kTile][16];     // [dB|dC][wave][token][n]
    const LaneId id = lane_id(p);
    const float an = id.ok ? p.A[id.dc * p.N + id.n] : 0.0f;
    const float a2 = an * kLog2e;
    const float bias = p.delta_bias ? p.delta_bias[id.dc] : 0.0f;
    const float dsk = p.Dskip ? p.Dskip[id.dc] : 0.0f;
    const int64_t nblk = (p.L + kTile - 1) / kTile;
    const float* ck = p.ckpt + (id.b * p.D + id.dc) * nblk * p.N + id.n;
    const int64_t G = (p.D + kChans - 1) / kChans;
    T* du_out = static_cast<T*>(p.du);
    T* dd_out = static_cast<T*>(p.ddelta);
    T* dz_out = static_cast<T*>(p.dz);

    const auto rB = bc_rsrc<T>(p, id.b, p.Bm);
    const auto rC = bc_rsrc<T>(p, id.b, p.Cm);
    float mu = (id.ok && p.dh_last) ? p.dh_last[(id.b * p.D + id.d) * p.N + id.n] : 0.0f;
    float dA_acc = 0.0f, dD_acc = 0.0f, db_acc = 0.0f;
    for (int64_t k = nblk - 1; k >= 0; --k) {
        const int64_t t0 = k * kTile;
        const float hprev0 = id.ok ? ck[k * p.N] : 0.0f;
        TileScalars<T, HAS_Z, SOFTPLUS, true> s;
        s.load(p, id, t0, bias);
        float bv[kTile], cv[kTile];
        load_bc<T>(p, id, t0, rB, bv);
        load_bc<T>(p, id, t0, rC, cv);
        // states of the tile, recomputed from its checkpoint
        float hs[kTile], da[kTile];
        {
            float h = hprev0;
#pragma unroll
            for (int j = 0; j < kTile; ++j) {
                da[j] = fast_exp2(row_bcast(s.dt, j) * a2);
                h = fmaf(da[j], h, bv[j] * row_bcast(s.dtu, j));
                hs[j] = h;
            }
        }
        // adjoint, token by token backwards; lane j keeps the row sums of token j
        float r_ddt = 0.0f, r_su = 0.0f, r_y = 0.0f;
        float pb[kTile], pc[kTile];
#pragma unroll
        for (int j = kTile - 1; j >= 0; --j) {
            const float gj = row_bcast(s.g, j);
            const float dtj = row_bcast(s.dt, j);
            const float m = fmaf(gj, cv[j], mu);
            const float hp = j > 0 ? hs[j - 1] : hprev0;
            pc[j] = gj * hs[j];
            pb[j] = m * row_bcast(s.dtu, j);
            const float vt = row_sum(m * fmaf(hp, an * da[j], bv[j] * row_bcast(s.u, j)));
            const float vu = row_sum(m * bv[j]);
            const float vy = row_sum(cv[j] * hs[j]);
            if (id.n == j) {
                r_ddt = vt;
                r_su = vu;
                r_y = vy;
            }
            dA_acc = fmaf(m * hp, dtj * da[j], dA_acc);
            mu = da[j] * m;
        }
        // per-channel results of token t0 + j in lane j
        {
            const int64_t t = t0 + id.n;
            if (id.chan_ok && t < p.L) {
                const int64_t i = (id.b * p.L + t) * p.D + id.d;
                const float r = r_y + dsk * s.u;
                if constexpr (HAS_Z) {
                    const float sz = sigmoid_f(s.z);
                    Elem<T>::store(dz_out, i, s.dy * r * (sz * fmaf(s.z, 1.0f - sz, 1.0f)));
                }
                Elem<T>::store(du_out, i, fmaf(s.g, dsk, s.dt * r_su));
                const float dd = r_ddt * s.sig;
                Elem<T>::store(dd_out, i, dd);
                db_acc += dd;
                dD_acc = fmaf(s.g, s.u, dD_acc);
            }
        }
        // dB, dC: rows 0-1 of the wavefront gather dB, rows 2-3 dC (xor 32), then
        // both rows of a pair hold the wavefront sum (xor 16)
#pragma unroll
        for (int j = 0; j < kTile; ++j) {
            const bool lowhalf = id.row < 2;
            const float keep = lowhalf ? pb[j] : pc[j];
            const float send = lowhalf ? pc[j] : pb[j];
            float v = keep + __shfl_xor(send, 32, 64);
            v += lane_xor<16>(v);
            pb[j] = v;
        }
        __syncthreads();                     // previous tile's partials consumed
        if (id.row == 0 || id.row == 2) {
            const int q = id.row / 2;
#pragma unroll
            for (int j = 0; j < kTile; ++j) red[q][id.w][j][id.n] = pb[j];
        }
        __syncthreads();
        {
            // thread -> (q, token, n); sum over the workgroup's wavefronts
            const int tid = threadIdx.x;
            const int q = tid / (kTile * 16), j = (tid / 16) % kTile, n = tid % 16;
            float v = 0.0f;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) v += red[q][w][j][n];
            const int64_t t = t0 + j;
            if (t < p.L && n < p.N)
                p.part_bc[(((int64_t)q * G + blockIdx.x) * p.B + id.b) * p.L * p.N + t * p.N + n] = v;
        }
    }
    if (id.ok) {
        p.part_dA[(id.b * p.D + id.d) * p.N + id.n] = dA_acc;
        if (p.dh0) p.dh0[(id.b * p.D + id.d) * p.N + id.n] = mu;
    }
    dD_acc = row_sum(dD_acc);
    db_acc = row_sum(db_acc);
    if (id.chan_ok && id.n == 0) {
        p.part_dD[id.b * p.D + id.d] = dD_acc;
        p.part_db[id.b * p.D + id.d] = db_acc;
    }
}

// dB, dC [B, L, N]: sums over the channel groups; dA [D, N], dD, dbias [D]:
// sums over the batch rows.  One thread per output element.
__global__ __launch_bounds__(256) void s6_bwd_reduce(S6BwdArgs p) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t G = (p.D + kChans - 1) / kChans;
    const int64_t nbc = p.B * p.L * p.N;
    if (i < 2 * nbc) {
        const int64_t q = i / nbc, e = i % nbc;
        float v = 0.0f;
        for (int64_t g = 0; g < G; ++g) v += p.part_bc[(q * G + g) * nbc + e];
        (q == 0 ? p.dB : p.dC)[e] = v;
        return;
    }
    const int64_t j = i - 2 * nbc;
    if (j < p.D * p.N) {
        float v = 0.0f;
        for (int64_t b = 0; b < p.B; ++b) v += p.part_dA[b * p.D * p.N + j];
        p.dA[j] = v;
        return;
    }
    const int64_t k = j - p.D * p.N;
    if (k < p.D) {
        float v = 0.0f, w = 0.0f;
        for (int64_t b = 0; b < p.B; ++b) {
            v += p.part_dD[b * p.D + k];
            w += p.part_db[b * p.D + k];
        }
        if (p.dDskip) p.dDskip[k] = v;
        if (p.ddelta_bias) p.ddelta_bias[k] = w;
    }
}

template <typename T>
hipError_t launch_t(const S6BwdArgs& a, hipStream_t stream) {
    const dim3 grid((unsigned)((a.D + kChans - 1) / kChans), (unsigned)a.B);
    const bool sp = (a.flags & SSM_FLAG_DELTA_SOFTPLUS) != 0;
    if (sp) s6_bwd_ckpt<T, true><<<grid, kThreads, 0, stream>>>(a);
    else s6_bwd_ckpt<T, false><<<grid, kThreads, 0, stream>>>(a);
    const bool hz = a.z != nullptr;
    if (hz && sp) s6_bwd_main<T, true, true><<<grid, kThreads, 0, stream>>>(a);
    else if (hz) s6_bwd_main<T, true, false><<<grid, kThreads, 0, stream>>>(a);
    else if (sp) s6_bwd_main<T, false, true><<<grid, kThreads, 0, stream>>>(a);
    else s6_bwd_main<T, false, false><<<grid, kThreads, 0, stream>>>(a);
    const int64_t total = 2 * a.B * a.L * a.N + a.D * a.N + a.D;
    s6_bwd_reduce<<<(unsigned)((total + 255) / 256), 256, 0, stream>>>(a);
    return hipGetLastError();
}

}  // namespace

size_t s6_bwd_workspace_bytes(int64_t B, int64_t L, int64_t D, int64_t N) {
    const int64_t nblk = (L + kTile - 1) / kTile;
    const int64_t G = (D + kChans - 1) / kChans;
    auto al = [](int64_t bytes) { return (bytes + 255) / 256 * 256; };
    return (size_t)(al(B * D * nblk * N * 4) + al(2 * G * B * L * N * 4) + al(B * D * N * 4) +
                    2 * al(B * D * 4));
}

void s6_bwd_carve(S6BwdArgs& a, void* ws) {
    const int64_t nblk = (a.L + kTile - 1) / kTile;
    const int64_t G = (a.D + kChans - 1) / kChans;
    auto al = [](int64_t bytes) { return (bytes + 255) / 256 * 256; };
    char* p = static_cast<char*>(ws);
    a.ckpt = reinterpret_cast<float*>(p);
    p += al(a.B * a.D * nblk * a.N * 4);
    a.part_bc = reinterpret_cast<float*>(p);
    p += al(2 * G * a.B * a.L * a.N * 4);
    a.part_dA = reinterpret_cast<float*>(p);
    p += al(a.B * a.D * a.N * 4);
    a.part_dD = reinterpret_cast<float*>(p);
    p += al(a.B * a.D * 4);
    a.part_db = reinterpret_cast<float*>(p);
}

hipError_t launch_s6_bwd(const S6BwdArgs& a, hipStream_t stream) {
    return a.bf16 ? launch_t<uint16_t>(a, stream) : launch_t<float>(a, stream);
}

}  // namespace ssm
