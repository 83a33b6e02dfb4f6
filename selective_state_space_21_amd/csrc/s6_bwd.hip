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
// Mapping: each 16-lane row of a wavefront is one channel of one batch row
// and lane n holds state n (N <= 16), so a lane carries one state and one
// adjoint.  Per-channel, per-token scalars (dt, u, g, ...) of a 16-token tile
// are computed by lane j for token j and broadcast along the row with DPP.
//   1. s6_bwd_ckpt (4 wavefronts, 16 channels per workgroup): forward sweep
//      storing the state before every tile.
//   2. s6_bwd_main (12 wavefronts, 48 channels per workgroup): tiles in
//      reverse; each tile recomputes its 16 states from the checkpoint into
//      registers, then runs the adjoint backwards.  Sums over n are row
//      reduce-scatters (DPP); each lane writes its dB and dC terms to LDS and
//      they are summed over the workgroup's 48 channels after the tile,
//      giving one partial per (48-channel group, b, t, n).
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

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kTile = 16;              // tokens per tile = per checkpoint
// Checkpoint sweep: 4 wavefronts, 16 channels per workgroup.
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kChans = 4 * kWaves;
// Adjoint sweep: 12 wavefronts (three per SIMD, its register budget), 48
// channels per workgroup, so dB and dC are summed over 48 channels before
// their partials leave the chip (one partial per 48 channels).
constexpr int kMainWaves = 12;
constexpr int kMainThreads = 64 * kMainWaves;
constexpr int kMainChans = 4 * kMainWaves;
static_assert(kTile == plan::kBwdTile && kMainChans == plan::kBwdChans,
              "the host workspace layout's tiling constants");

struct LaneId {
    int w, l, row, n;
    int64_t b, grp, d, dc; // grp: channel group; dc: d clamped into range for addressing
    int64_t len;           // tokens of batch row b: L, or its own length (variable-length batch)
    bool chan_ok, ok;      // channel exists; channel and state exist
};

template <int CH>
__device__ __forceinline__ LaneId lane_id(const S6BwdArgs& p) {
    LaneId id;
    const int tid = threadIdx.x;
    id.w = tid / 64;
    id.l = tid % 64;
    id.row = id.l / 16;
    id.n = id.l % 16;
    // Workgroups are dealt to the 8 XCDs round robin (i -> XCD i % 8).  The
    // id is renumbered to give each XCD a contiguous range of channel groups,
    // so groups that share 128-byte rows of u, delta, z and dy fetch them
    // into one L2.
    const uint32_t n = gridDim.x * gridDim.y, i = blockIdx.x + gridDim.x * blockIdx.y;
    const uint32_t x = i % 8, q = n / 8, r = n % 8;
    const uint32_t lid = x * q + min(x, r) + i / 8;
    id.b = lid / gridDim.x;
    id.grp = lid % gridDim.x;
    id.d = (int64_t)id.grp * CH + 4 * id.w + id.row;
    id.chan_ok = id.d < p.D;
    id.dc = id.chan_ok ? id.d : p.D - 1;
    id.ok = id.chan_ok && id.n < p.N;
    id.len = p.seq_lens ? min(max((int64_t)p.seq_lens[id.b], (int64_t)0), p.L) : p.L;
    return id;
}

// sum over the 16 lanes of each row, result in every lane of the row
__device__ __forceinline__ float row_sum(float v) {
    v += dpp_mov<0xB1>(v);    // quad_perm [1,0,3,2]
    v += dpp_mov<0x4E>(v);    // quad_perm [2,3,0,1]: every lane of a quad holds its sum
    v += dpp_mov<0x124>(v);   // row_ror 4: quads q and q+1
    v += dpp_mov<0x128>(v);   // row_ror 8: all four quads
    return v;
}

// acc + (lane K of the row's s) * x in one v_fmac_f32_dpp: the broadcast
// that row_bcast feeds to a multiply, for a fused multiply-add (which the
// compiler does not fold).  DPP reads its source two wait states after a VALU
// write at the earliest, so the statement opens with s_nop 1.
template <int K>
__device__ __forceinline__ float fmac_bcast_c(float acc, float s, float x) {
    asm("s_nop 1\n\tv_fmac_f32_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf"
        : "+v"(acc) : "v"(s), "v"(x), "n"(K));
    return acc;
}
// k must fold to a constant after unrolling.
__device__ __forceinline__ float fmac_bcast(float acc, float s, float x, int k) {
    switch (k) {
        case 0: return fmac_bcast_c<0>(acc, s, x);   case 1: return fmac_bcast_c<1>(acc, s, x);
        case 2: return fmac_bcast_c<2>(acc, s, x);   case 3: return fmac_bcast_c<3>(acc, s, x);
        case 4: return fmac_bcast_c<4>(acc, s, x);   case 5: return fmac_bcast_c<5>(acc, s, x);
        case 6: return fmac_bcast_c<6>(acc, s, x);   case 7: return fmac_bcast_c<7>(acc, s, x);
        case 8: return fmac_bcast_c<8>(acc, s, x);   case 9: return fmac_bcast_c<9>(acc, s, x);
        case 10: return fmac_bcast_c<10>(acc, s, x); case 11: return fmac_bcast_c<11>(acc, s, x);
        case 12: return fmac_bcast_c<12>(acc, s, x); case 13: return fmac_bcast_c<13>(acc, s, x);
        case 14: return fmac_bcast_c<14>(acc, s, x); default: return fmac_bcast_c<15>(acc, s, x);
    }
}

__device__ __forceinline__ float sigmoid_f(float x) {
    return fast_rcp(1.0f + fast_exp2(-x * kLog2e));
}

// Per-channel inputs of token t0 + j, loaded by lane j of the row (raw, so
// that they can be fetched a tile ahead).  Buffer resources over batch row b
// make every load unconditional: tokens past the row's length read as zero
// (so no padding of a variable-length batch is ever read), and no branch (and
// no wait at its join) separates a prefetch from the work it overlaps.
struct RowRsrc {
    __amdgpu_buffer_rsrc_t delta, u, z, dy;
};

template <typename T>
__device__ __forceinline__ RowRsrc row_rsrc(const S6BwdArgs& p, int64_t b, int64_t len) {
    const uint32_t bytes = (uint32_t)(len * p.D * sizeof(T));
    const int64_t off = b * p.L * p.D;
    RowRsrc r;
    r.delta = make_rsrc(static_cast<const T*>(p.delta) + off, bytes);
    r.u = make_rsrc(static_cast<const T*>(p.u) + off, bytes);
    r.z = make_rsrc(p.z ? static_cast<const T*>(p.z) + off : static_cast<const T*>(p.u) + off, bytes);
    r.dy = make_rsrc(p.dy ? static_cast<const T*>(p.dy) + off : static_cast<const T*>(p.u) + off, bytes);
    return r;
}

// Loaded storage bits, widened to fp32 only where they are used: a
// conversion next to the load would make the compiler wait for the load
// there, in the iteration that issues the prefetch.
template <typename T> struct Bits;
template <> struct Bits<float> {
    static __device__ __forceinline__ uint32_t load(__amdgpu_buffer_rsrc_t r, uint32_t off) {
        return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
    }
    static __device__ __forceinline__ float f32(uint32_t v) { return __uint_as_float(v); }
};
template <> struct Bits<uint16_t> {
    static __device__ __forceinline__ uint32_t load(__amdgpu_buffer_rsrc_t r, uint32_t off) {
        return __builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0);
    }
    static __device__ __forceinline__ float f32(uint32_t v) { return __uint_as_float(v << 16); }
};

template <typename T, bool HAS_Z, bool FULL>
struct TileRaw {
    uint32_t delta, u, z, dy;
    __device__ __forceinline__ void load(const S6BwdArgs& p, const LaneId& id, const RowRsrc& r,
                                         int64_t t0) {
        const uint32_t off = (uint32_t)(((t0 + id.n) * p.D + id.dc) * sizeof(T));
        delta = Bits<T>::load(r.delta, off);
        u = Bits<T>::load(r.u, off);
        if constexpr (FULL) {
            dy = Bits<T>::load(r.dy, off);
            z = HAS_Z ? Bits<T>::load(r.z, off) : 0u;
        }
    }
};

template <bool HAS_Z, bool SOFTPLUS, bool FULL>
struct TileScalars {
    float dt, dtu, u, g, sig, z, dy;

    template <typename T, typename R>
    __device__ __forceinline__ void from(const R& r, const S6BwdArgs& p, const LaneId& id,
                                         int64_t t0, float bias) {
        const bool in = id.chan_ok && t0 + id.n < id.len;
        const float x = Bits<T>::f32(r.delta) + bias;
        u = in ? Bits<T>::f32(r.u) : 0.0f;
        dt = in ? (SOFTPLUS ? softplus_f(x) : x) : 0.0f;
        dtu = dt * u;
        if constexpr (FULL) {
            sig = SOFTPLUS ? sigmoid_f(x) : 1.0f;
            dy = in ? Bits<T>::f32(r.dy) : 0.0f;
            z = Bits<T>::f32(r.z);
            g = HAS_Z ? dy * silu_f(z) : dy;
        }
    }
};

// Activations of the workgroup's 16 channels, loaded cooperatively as 16-byte
// pieces of each token's channel run (32 bytes in bf16, 64 in fp32) and
// staged in LDS as [tensor][channel][token].  A lane loading its own 2-byte
// element touches 16 cache lines per load instruction; a piece covers 8 (or
// 4) channels of one token.  Used when D * sizeof(T) is a multiple of 16, so
// that every piece is aligned; tokens outside [0, L) read as zero.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <typename T>
struct Run {
    static constexpr int kPerToken = kChans * (int)sizeof(T) / 16;   // pieces per token
    static constexpr int kVals = 16 / (int)sizeof(T);                 // elements per piece
};

template <typename T>
__device__ __forceinline__ uint32_t piece_off(const S6BwdArgs& p, int64_t grp, int64_t t, int pc) {
    return (t < 0 || t >= p.L) ? 0xFFFFFFF0u
                               : (uint32_t)((t * p.D + grp * kChans) * (int64_t)sizeof(T) + 16 * pc);
}

// Four consecutive channels of one token (8 bytes in bf16, 16 in fp32), for a
// workgroup of CH channels.
template <typename T, int CH>
__device__ __forceinline__ uint32_t quad_off(const S6BwdArgs& p, int64_t grp, int64_t t, int q) {
    return (t < 0 || t >= p.L) ? 0xFFFFFFF0u
                               : (uint32_t)((t * p.D + grp * CH + 4 * q) * (int64_t)sizeof(T));
}
template <typename T> struct Quad;
template <> struct Quad<uint16_t> {
    typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
    u32x2 v = {0u, 0u};
    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, uint32_t off) {
        v = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0));
    }
    __device__ __forceinline__ uint16_t elem(int q) const {
        return (uint16_t)(v[q >> 1] >> (16 * (q & 1)));
    }
};
template <> struct Quad<float> {
    u32x4 v = {0u, 0u, 0u, 0u};
    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, uint32_t off) {
        v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
    }
    __device__ __forceinline__ float elem(int q) const { return __uint_as_float(v[q]); }
};

template <typename T> __device__ __forceinline__ uint32_t elem_bits(T v);
template <> __device__ __forceinline__ uint32_t elem_bits<uint16_t>(uint16_t v) { return v; }
template <> __device__ __forceinline__ uint32_t elem_bits<float>(float v) { return __float_as_uint(v); }

// B or C [B, L, N] of a tile is shared by every channel of the workgroup:
// thread (j, n) = (tid / 16, tid % 16) loads element (t0 + j, n) through a
// buffer resource over the len tokens of batch row b (tokens past them and
// n >= N read as zero), and the tile is staged in LDS as [token][n].
template <typename T>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t bc_rsrc(const S6BwdArgs& p, int64_t b,
                                                          int64_t len, const void* src) {
    return make_rsrc(static_cast<const T*>(src) + b * p.L * p.N, (uint32_t)(len * p.N * sizeof(T)));
}

// LDS tile of B or C stored per state n as 16 consecutive tokens, rows padded
// to 20 floats: the transposed store by thread (j, n) is conflict-free and
// lane n reads its 16 tokens as four 16-byte loads.
constexpr int kPitch = kTile + 4;

__device__ __forceinline__ void tile_row(const float* tile, int n, float (&v)[kTile]) {
#pragma unroll
    for (int q = 0; q < kTile / 4; ++q) {
        const float4 x = *reinterpret_cast<const float4*>(tile + n * kPitch + 4 * q);
        v[4 * q] = x.x; v[4 * q + 1] = x.y; v[4 * q + 2] = x.z; v[4 * q + 3] = x.w;
    }
}

// Threads past the tile's 256 elements load nothing (an offset past the
// resource reads zero without a memory access).
template <typename T>
__device__ __forceinline__ uint32_t load_bc_bits(const S6BwdArgs& p, int64_t t0,
                                                 __amdgpu_buffer_rsrc_t r) {
    const int j = threadIdx.x / 16, n = threadIdx.x % 16;
    const uint32_t off = (n < p.N && j < kTile) ? (uint32_t)(((t0 + j) * p.N + n) * sizeof(T))
                                                 : 0x80000000u;
    return Bits<T>::load(r, off);
}

// The same element for the super-tile fetch of the checkpoint sweep.  States
// n >= N read zero through an offset with bit 31 set (past the resource,
// which spans less than 2 GiB), formed without a select: of eight selects the
// compiler built branches whose joins waited for every outstanding load (the
// rest of the prefetch included) before the next offset was written.
template <typename T>
__device__ __forceinline__ uint32_t load_bc_bits_ahead(const S6BwdArgs& p, int64_t t0,
                                                       __amdgpu_buffer_rsrc_t r) {
    const int j = threadIdx.x / 16, n = threadIdx.x % 16;
    const uint32_t o = (((uint32_t)t0 + (uint32_t)j) * (uint32_t)p.N + (uint32_t)n) * (uint32_t)sizeof(T);
    const uint32_t past = ((uint32_t)((int)p.N - 1 - n) >> 31) << 31;   // n >= N
    return Bits<T>::load(r, o | past);
}

// Inputs of kSuper consecutive tiles, fetched together so that one memory
// round trip covers 128 tokens of the sequential sweep.
constexpr int kSuper = 8;

template <typename T, bool VEC>
struct SuperRaw {
    // VEC: this lane's pieces of the super-tile (wave w: tensor w / 2, tokens
    // 64 (w % 2) .. +63); otherwise its own element of every tile
    u32x4 a[VEC ? Run<T>::kPerToken : 1];
    uint32_t delta[VEC ? 1 : kSuper], u[VEC ? 1 : kSuper], b[kSuper];
    __device__ __forceinline__ void load(const S6BwdArgs& p, const LaneId& id, const RowRsrc& rr,
                                         int64_t t0, __amdgpu_buffer_rsrc_t rB) {
        if constexpr (VEC) {
            constexpr int kPT = Run<T>::kPerToken;
            const int wu = __builtin_amdgcn_readfirstlane(id.w);
            const __amdgpu_buffer_rsrc_t rs = (wu >> 1) == 0 ? rr.delta : rr.u;
#pragma unroll
            for (int i = 0; i < kPT; ++i) {
                const int idx = id.l + 64 * i;
                const int64_t t = t0 + 64 * (wu & 1) + idx / kPT;
                a[i] = __builtin_amdgcn_raw_buffer_load_b128(
                    rs, (int)piece_off<T>(p, id.grp, t, idx % kPT), 0, 0);
            }
        }
#pragma unroll
        for (int i = 0; i < kSuper; ++i) {
            if constexpr (!VEC) {
                TileRaw<T, false, false> r;
                r.load(p, id, rr, t0 + i * kTile);
                delta[i] = r.delta;
                u[i] = r.u;
            }
            b[i] = load_bc_bits_ahead<T>(p, t0 + i * kTile, rB);
        }
    }
};

// PAIR: the segment's forward pair instead of checkpoints: its state at the
// end from a zero state at its start (the carry pass folds these into every
// segment's incoming state).  Otherwise the segment is scanned from its
// incoming state (h0 for the first) and the state before each tile stored.
template <typename T, bool SOFTPLUS, bool VEC, bool PAIR>
__global__ __launch_bounds__(kThreads) void s6_bwd_ckpt(S6BwdArgs p) {
    static_assert(kThreads == kTile * 16, "one tile element per thread");
    static_assert(kSuper == plan::kBwdSuper, "the planner's segment rounding");
    constexpr int kSpan = kSuper * kTile;
    __shared__ __attribute__((aligned(16))) float bt[kSuper][16 * kPitch];
    __shared__ __attribute__((aligned(16))) T actc[VEC ? 2 : 1][kChans][kSpan + 8];
    const LaneId id = lane_id<kChans>(p);
    const int cl = 4 * id.w + id.row;                    // channel in the workgroup
    const float a2 = id.ok ? p.A[id.dc * p.N + id.n] * kLog2e : 0.0f;
    const float bias = p.delta_bias ? p.delta_bias[id.dc] : 0.0f;
    const int64_t nblk = (p.L + kTile - 1) / kTile;
    // segment s: tiles [k0, k1)
    const int seg = (int)blockIdx.z;
    const int64_t k0 = (int64_t)seg * p.seg_tiles;
    const int64_t k1 = k0 + p.seg_tiles < nblk ? k0 + p.seg_tiles : nblk;
    const int64_t nsup = k1 > k0 ? (k1 - k0 + kSuper - 1) / kSuper : 0;
    const int64_t chain = (((int64_t)seg * p.B + id.b) * p.D + id.dc) * p.N + id.n;
    float h = 0.0f;
    if (!PAIR && id.ok) {
        if (seg == 0) h = p.h0 ? p.h0[(id.b * p.D + id.d) * p.N + id.n] : 0.0f;
        else h = p.seg_hin[chain];
    }
    const auto rB = bc_rsrc<T>(p, id.b, id.len, p.Bm);
    float* ck = p.ckpt + (id.b * p.D + id.dc) * nblk * p.N + id.n;
    const RowRsrc rr = row_rsrc<T>(p, id.b, id.len);
    SuperRaw<T, VEC> nxt;
    if (nsup > 0) nxt.load(p, id, rr, k0 * kTile, rB);
    for (int64_t sg = 0; sg < nsup; ++sg) {
        const SuperRaw<T, VEC> cur = nxt;
        lds_barrier();                    // previous super-tile's LDS reads done
#pragma unroll
        for (int i = 0; i < kSuper; ++i)
            bt[i][(threadIdx.x % 16) * kPitch + threadIdx.x / 16] = Bits<T>::f32(cur.b[i]);
        if constexpr (VEC) {
            constexpr int kPT = Run<T>::kPerToken, kVals = Run<T>::kVals;
            const int wu = id.w;
#pragma unroll
            for (int i = 0; i < kPT; ++i) {
                const int idx = id.l + 64 * i;
                const int j = 64 * (wu & 1) + idx / kPT, pc = idx % kPT;
                const T* e = reinterpret_cast<const T*>(&cur.a[i]);
#pragma unroll
                for (int q = 0; q < kVals; ++q) actc[wu >> 1][kVals * pc + q][j] = e[q];
            }
        }
        lds_barrier();
        // travels meanwhile; issued unconditionally (past the end it reads
        // zeros) so that no branch join makes the compiler wait for it here
        nxt.load(p, id, rr, k0 * kTile + (sg + 1) * kSpan, rB);
#pragma unroll
        for (int i = 0; i < kSuper; ++i) {
            const int64_t k = k0 + sg * kSuper + i;
            if (k >= k1) break;
            if (!PAIR && id.ok) ck[k * p.N] = h;
            TileRaw<T, false, false> r;
            if constexpr (VEC) {
                r.delta = elem_bits<T>(actc[0][cl][kTile * i + id.n]);
                r.u = elem_bits<T>(actc[1][cl][kTile * i + id.n]);
            } else {
                r.delta = cur.delta[i];
                r.u = cur.u[i];
            }
            TileScalars<false, SOFTPLUS, false> s;
            s.template from<T>(r, p, id, k * kTile, bias);
            float bv[kTile], dA[kTile];
            tile_row(bt[i], id.n, bv);
            // all decay factors and input terms first, then the dependent chain
#pragma unroll
            for (int j = 0; j < kTile; ++j) {
                dA[j] = fast_exp2(row_bcast(s.dt, j) * a2);
                bv[j] *= row_bcast(s.dtu, j);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int j = 0; j < kTile; ++j) h = fmaf(dA[j], h, bv[j]);
        }
    }
    if (PAIR && id.ok) p.seg_fend[chain] = h;
}

// MODE kWhole: one segment, from dh_last.  kSegment: segment blockIdx.z of
// several, from its carried adjoint.  kPairs: the segment's adjoint pair
// only: the adjoint recurrence run back through the segment from zero at its
// end, without the states or any gradient (the carry pass folds these into
// every segment's incoming adjoint), plus the segment's sum of steps.  (The
// whole-sequence kernel is compiled apart: with the segment bounds and
// buffers at run time its tile loop measured 3% slower.)
enum { kWhole = 0, kSegment = 1, kPairs = 2 };

template <typename T, bool HAS_Z, bool SOFTPLUS, bool VEC, int MODE>
__global__ __launch_bounds__(kMainThreads) __attribute__((amdgpu_waves_per_eu(3)))
void s6_bwd_main(S6BwdArgs p) {
    constexpr bool PAIRS = MODE == kPairs;
    constexpr int kWaves = kMainWaves, kThreads = kMainThreads, kChans = kMainChans;
    // dB and dC terms of the tile per channel, [dB|dC][token][state][channel]:
    // each lane writes its own two terms per token, and the sums over the
    // workgroup's 48 channels are taken after the tile as 16-byte reads.  A
    // channel run holds kRedPitch floats, so the 64 lanes of one write (4
    // channels x 16 states; runs 52 floats apart) hit 64 distinct banks.
    constexpr int kRedPitch = kChans + 4;
    static_assert(kRedPitch % 4 == 0, "16-byte reads of a channel run");
    __shared__ __attribute__((aligned(16))) float red[2][kTile][16][kRedPitch];
    // du, ddelta, dz of the tile as stored ([output][token][channel]): written
    // per lane, then stored as 16-byte rows pieces, so that one store covers
    // a run of the workgroup's channels instead of one 2-byte element
    constexpr int kOut = HAS_Z ? 3 : 2;
    __shared__ __attribute__((aligned(16))) T outst[kOut][kTile][kChans];
    __shared__ __attribute__((aligned(16))) float bct[2][16 * kPitch];   // B, C: [n][token]
    // VEC: delta, u, dy (, z) of the tile as [tensor][channel][token].  Each
    // tensor's tile is 16 tokens x 12 runs of 4 channels, loaded by three
    // wavefronts: wave w loads tensor w / 3, lane l the run (64 (w % 3) + l)
    // % 12 of token (64 (w % 3) + l) / 12
    constexpr int kNT = HAS_Z ? 4 : 3;
    constexpr int kQuads = kChans / 4;                   // 4-channel runs per token
    static_assert(kTile * kQuads == 3 * 64, "three wavefronts per tensor");
    __shared__ __attribute__((aligned(16))) T actst[VEC ? kNT : 1][kChans][kTile + 8];
    const LaneId id = lane_id<kChans>(p);
    const int cl = 4 * id.w + id.row;                    // channel in the workgroup
    const float an = id.ok ? p.A[id.dc * p.N + id.n] : 0.0f;
    const float a2 = an * kLog2e;
    const float bias = p.delta_bias ? p.delta_bias[id.dc] : 0.0f;
    const float dsk = p.Dskip ? p.Dskip[id.dc] : 0.0f;
    const int64_t nblk = (p.L + kTile - 1) / kTile;
    // segment s: tiles [k0, k1), walked from k1 - 1 down
    const int seg = MODE == kWhole ? 0 : (int)blockIdx.z;
    const int64_t k0 = MODE == kWhole ? 0 : (int64_t)seg * p.seg_tiles;
    const int64_t k1 = MODE == kWhole ? nblk : (k0 + p.seg_tiles < nblk ? k0 + p.seg_tiles : nblk);
    // this lane's (segment, b, d, n) chain in the segment buffers, formed
    // where used (kept live across the tile loop it slowed the loop by 3%)
    auto chain = [&]() { return (((int64_t)seg * p.B + id.b) * p.D + id.dc) * p.N + id.n; };
    // n clamped: lanes past N read a valid (ignored) checkpoint
    const float* ck = p.ckpt + (id.b * p.D + id.dc) * nblk * p.N + (id.n < p.N ? id.n : 0);
    const int64_t G = (p.D + kChans - 1) / kChans;
    const RowRsrc rr = row_rsrc<T>(p, id.b, id.len);
    T* du_out = static_cast<T*>(p.du);
    T* dd_out = static_cast<T*>(p.ddelta);
    T* dz_out = static_cast<T*>(p.dz);
    const auto rB = bc_rsrc<T>(p, id.b, id.len, p.Bm);
    const auto rC = bc_rsrc<T>(p, id.b, id.len, p.Cm);

    // a_{t+1} m_{t+1} entering the segment's last token: dh_last for one
    // segment, the carried value for several, zero for the pair
    float mu = 0.0f;
    if constexpr (MODE == kWhole) mu = (id.ok && p.dh_last) ? p.dh_last[(id.b * p.D + id.d) * p.N + id.n] : 0.0f;
    if constexpr (MODE == kSegment) mu = id.ok ? p.seg_qin[chain()] : 0.0f;
    float dA_acc = 0.0f, dD_acc = 0.0f, db_acc = 0.0f, dt_sum = 0.0f;
    TileRaw<T, HAS_Z, true> raw;
    uint32_t bpre = 0, cpre = 0;
    float hck = 0.0f;
    const int wu = __builtin_amdgcn_readfirstlane(id.w);
    const int wt = wu / 3;                               // tensor this wavefront loads
    const __amdgpu_buffer_rsrc_t rs_act = wt == 0 ? rr.delta : wt == 1 ? rr.u : wt == 2 ? rr.dy : rr.z;
    const bool act_lane = wt < kNT;
    const int qi = 64 * (wu % 3) + id.l;                 // run index within the tensor's tile
    const int aq = qi % kQuads, at = qi / kQuads;        // channel run, token
    Quad<T> apre;
    // every lane loads (a wavefront without a tensor at an offset past the
    // resource), so no branch separates the prefetch from the work it overlaps
    auto load_act = [&](int64_t t0) {
        const int64_t t = act_lane ? t0 + at : -1;
        apre.load(rs_act, quad_off<T, kChans>(p, id.grp, t, aq));
    };
    if (k1 > k0) {
        if constexpr (VEC) load_act((k1 - 1) * kTile);
        else raw.load(p, id, rr, (k1 - 1) * kTile);
        bpre = load_bc_bits<T>(p, (k1 - 1) * kTile, rB);
        cpre = load_bc_bits<T>(p, (k1 - 1) * kTile, rC);
        if constexpr (!PAIRS) hck = ck[(k1 - 1) * p.N];
    }
    for (int64_t k = k1 - 1; k >= k0; --k) {
        const int64_t t0 = k * kTile;
        const float hprev0 = id.ok ? hck : 0.0f;
        TileScalars<HAS_Z, SOFTPLUS, true> s;
        if constexpr (!VEC) s.template from<T>(raw, p, id, t0, bias);
        // No barrier before the staging: the previous tile read bct and actst
        // only before its last barrier, and what follows that barrier (the
        // output stores and the dB/dC sums) reads outst and red, which this
        // tile writes only after the barrier below.
        if (threadIdx.x < kTile * 16) {
            bct[0][(threadIdx.x % 16) * kPitch + threadIdx.x / 16] = Bits<T>::f32(bpre);
            bct[1][(threadIdx.x % 16) * kPitch + threadIdx.x / 16] = Bits<T>::f32(cpre);
        }
        if constexpr (VEC) {
            if (act_lane) {
#pragma unroll
                for (int q = 0; q < 4; ++q) actst[wt][4 * aq + q][at] = apre.elem(q);
            }
        }
        lds_barrier();
        if constexpr (VEC) {
            raw.delta = elem_bits<T>(actst[0][cl][id.n]);
            raw.u = elem_bits<T>(actst[1][cl][id.n]);
            raw.dy = elem_bits<T>(actst[2][cl][id.n]);
            raw.z = HAS_Z ? elem_bits<T>(actst[kNT - 1][cl][id.n]) : 0u;
            s.template from<T>(raw, p, id, t0, bias);
        }
        // The previous tile's inputs travel during this one.  The loads are
        // unconditional (for k = 0 the buffer loads fall before the row and
        // read zeros, the checkpoint load repeats tile 0): a branch around
        // them would join the loaded and the old values, and the compiler
        // waits for the loads at that join, in the tile that issues them.
        if constexpr (VEC) load_act(t0 - kTile);
        else raw.load(p, id, rr, t0 - kTile);
        bpre = load_bc_bits<T>(p, t0 - kTile, rB);
        cpre = load_bc_bits<T>(p, t0 - kTile, rC);
        if constexpr (PAIRS) {
            // the adjoint alone: m_t = g_t C_t + mu, mu = a_t m_t
            float cv[kTile];
            tile_row(bct[1], id.n, cv);
#pragma unroll
            for (int j = kTile - 1; j >= 0; --j) {
                const float m = fmac_bcast(mu, s.g, cv[j], j);
                mu = fast_exp2(row_bcast(s.dt, j) * a2) * m;
            }
            dt_sum += s.dt;
            lds_barrier();                  // this tile's reads of bct and actst done
            continue;
        }
        hck = ck[(k > 0 ? k - 1 : 0) * p.N];
        // states of the tile, recomputed from its checkpoint
        float hs[kTile], da[kTile];
        {
            float bv[kTile];
            tile_row(bct[0], id.n, bv);
#pragma unroll
            for (int j = 0; j < kTile; ++j) {
                da[j] = fast_exp2(row_bcast(s.dt, j) * a2);
                bv[j] *= row_bcast(s.dtu, j);
            }
            __builtin_amdgcn_sched_barrier(0);
            float h = hprev0;
#pragma unroll
            for (int j = 0; j < kTile; ++j) {
                h = fmaf(da[j], h, bv[j]);
                hs[j] = h;
            }
        }
        // The reverse loop re-reads B and C from LDS and re-broadcasts the
        // per-token scalars instead of keeping the recompute's copies alive:
        // empty asm statements (no instruction) make the values opaque to
        // common-subexpression elimination across the two loops.
        asm volatile("" ::: "memory");
        asm volatile("" : "+v"(s.dt), "+v"(s.dtu), "+v"(s.u), "+v"(s.g));
        // adjoint, token by token backwards.  Per-lane terms of the sums over n
        // (pt: the A part of ddt, pu: sum m B, py: readout) are reduced after the loop; the
        // dB and dC terms of each token go to LDS as they are formed
        float pt[kTile], pu[kTile], py[kTile];
        float bv[kTile], cv[kTile];
        tile_row(bct[0], id.n, bv);
        tile_row(bct[1], id.n, cv);
#pragma unroll
        for (int j = kTile - 1; j >= 0; --j) {
            const float bj = bv[j], cj = cv[j];
            const float m = fmac_bcast(mu, s.g, cj, j);          // mu + g_t C_t
            const float hp = j > 0 ? hs[j - 1] : hprev0;
            const float pc = hs[j] * row_bcast(s.g, j);
            const float pb = m * row_bcast(s.dtu, j);
            // m_t h_{t-1} a_t serves both ddt (times A) and dA (times dt)
            const float ya = m * hp * da[j];
            pu[j] = m * bj;
            pt[j] = ya * an;       // ddt = sum_n ya A + u sum_n m B, the latter added below
            py[j] = cj * hs[j];
            dA_acc = fmac_bcast(dA_acc, s.dt, ya, j);
            mu = da[j] * m;
            red[0][j][id.n][cl] = pb;
            red[1][j][id.n][cl] = pc;
        }
        const float r_su = row_reduce_scatter16(pu, id.n);
        const float r_ddt = fmaf(s.u, r_su, row_reduce_scatter16(pt, id.n));
        const float r_y = row_reduce_scatter16(py, id.n);
        // per-channel results of token t0 + j in lane j, staged in LDS
        {
            const int64_t t = t0 + id.n;
            const float r = r_y + dsk * s.u;
            // past a row's end in a variable-length batch every term is zero
            // except the carried adjoint's m h a A: its step has no gradient
            const float dd = t < id.len ? r_ddt * s.sig : 0.0f;
            Elem<T>::store(&outst[0][id.n][0], cl, fmaf(s.g, dsk, s.dt * r_su));
            Elem<T>::store(&outst[1][id.n][0], cl, dd);
            if constexpr (HAS_Z) {
                const float sz = sigmoid_f(s.z);
                Elem<T>::store(&outst[2][id.n][0], cl, s.dy * r * (sz * fmaf(s.z, 1.0f - sz, 1.0f)));
            }
            if (id.chan_ok && t < id.len) {
                db_acc += dd;
                dD_acc = fmaf(s.g, s.u, dD_acc);
            }
        }
        lds_barrier();
        {
            // the staged rows: thread -> (output, token, 16-byte piece)
            constexpr int kPieces = kChans * (int)sizeof(T) / 16;
            const int64_t d0 = id.grp * kChans;
            const bool vec = d0 + kChans <= p.D && (p.D * (int64_t)sizeof(T)) % 16 == 0;
            // the last wavefronts (no dB/dC sums below) take the stores first
            const int st = (int)((threadIdx.x + kThreads - 2 * kTile * 16) % kThreads);
            for (int e = st; e < kOut * kTile * kPieces; e += kThreads) {
                const int o = e / (kTile * kPieces), j = (e / kPieces) % kTile, pc = e % kPieces;
                const int64_t t = t0 + j;
                if (t >= p.L) continue;
                constexpr int kPer = 16 / (int)sizeof(T);           // elements per piece
                T* dst = (o == 0 ? du_out : o == 1 ? dd_out : dz_out) + (id.b * p.L + t) * p.D + d0 + pc * kPer;
                const T* src = &outst[o][j][pc * kPer];
                if (vec) {
                    *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
                } else {
                    for (int c = 0; c < kPer; ++c)
                        if (d0 + pc * kPer + c < p.D) dst[c] = src[c];
                }
            }
            // thread -> (q, token, n) for 512 of them; sum over the 48 channels
            // (four running sums over 4-channel runs, then added pairwise)
            for (int e = threadIdx.x; e < 2 * kTile * 16; e += kThreads) {
                const int q = e / (kTile * 16), j = (e / 16) % kTile, n = e % 16;
                f32x4 acc = *reinterpret_cast<const f32x4*>(&red[q][j][n][0]);
#pragma unroll
                for (int c4 = 1; c4 < kChans / 4; ++c4)
                    acc += *reinterpret_cast<const f32x4*>(&red[q][j][n][4 * c4]);
                const float v = (acc[0] + acc[1]) + (acc[2] + acc[3]);
                const int64_t t = t0 + j;
                if (t < p.L && n < p.N)
                    p.part_bc[(((int64_t)q * G + id.grp) * p.B + id.b) * p.L * p.N + t * p.N + n] = v;
            }
        }
    }
    const int64_t bd = ((int64_t)seg * p.B + id.b) * p.D + id.d;   // (segment, b, d)
    if constexpr (PAIRS) {
        dt_sum = row_sum(dt_sum);
        if (id.ok) p.seg_radj[chain()] = mu;
        if (id.chan_ok && id.n == 0) p.seg_dsum[bd] = dt_sum;
        return;
    }
    if (id.ok) {
        p.part_dA[chain()] = dA_acc;
        if (p.dh0 && seg == 0) p.dh0[(id.b * p.D + id.d) * p.N + id.n] = mu;
    }
    dD_acc = row_sum(dD_acc);
    db_acc = row_sum(db_acc);
    if (id.chan_ok && id.n == 0) {
        p.part_dD[bd] = dD_acc;
        p.part_db[bd] = db_acc;
    }
}

// The segment pairs folded into every segment's incoming state (left to
// right, from h0) and incoming adjoint (right to left, from dh_last): one
// thread per (b, d, n) chain.  Over segment s both the state and the adjoint
// decay by exp2(A log2(e) sum of the segment's steps).
__global__ __launch_bounds__(256) void s6_bwd_carry(S6BwdArgs p) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t chains = p.B * p.D * p.N;
    if (i >= chains) return;
    const int64_t bd = i / p.N, d = bd % p.D, n = i % p.N;
    const float a2 = p.A[d * p.N + n] * kLog2e;
    const int64_t nbd = p.B * p.D;
    if (p.own_ckpt) {
        float h = p.h0 ? p.h0[i] : 0.0f;
        for (int s = 0; s < p.S; ++s) {
            p.seg_hin[s * chains + i] = h;
            h = fmaf(fast_exp2(a2 * p.seg_dsum[s * nbd + bd]), h, p.seg_fend[s * chains + i]);
        }
    }
    float q = p.dh_last ? p.dh_last[i] : 0.0f;
    for (int s = p.S - 1; s >= 0; --s) {
        p.seg_qin[s * chains + i] = q;
        q = fmaf(fast_exp2(a2 * p.seg_dsum[s * nbd + bd]), q, p.seg_radj[s * chains + i]);
    }
}

// dB, dC [B, L, N]: sums over the channel groups; dA [D, N], dD, dbias [D]:
// sums over the segments and batch rows.  One thread per output element.
__global__ __launch_bounds__(256) void s6_bwd_reduce(S6BwdArgs p) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t G = (p.D + kMainChans - 1) / kMainChans;
    const int64_t nbc = p.B * p.L * p.N;
    if (i < 2 * nbc) {
        const int64_t q = i / nbc, e = i % nbc;
        // eight partials in flight at a time, added in group order
        float v = 0.0f;
        int64_t g = 0;
        for (; g + 8 <= G; g += 8) {
            float t[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) t[k] = p.part_bc[(q * G + g + k) * nbc + e];
#pragma unroll
            for (int k = 0; k < 8; ++k) v += t[k];
        }
        for (; g < G; ++g) v += p.part_bc[(q * G + g) * nbc + e];
        (q == 0 ? p.dB : p.dC)[e] = v;
        return;
    }
    const int64_t j = i - 2 * nbc;
    if (j < p.D * p.N) {
        float v = 0.0f;
        int64_t b = 0;
        const int64_t rows = (int64_t)p.S * p.B;     // (segment, batch row) partials
        for (; b + 8 <= rows; b += 8) {
            float t[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) t[k] = p.part_dA[(b + k) * p.D * p.N + j];
#pragma unroll
            for (int k = 0; k < 8; ++k) v += t[k];
        }
        for (; b < rows; ++b) v += p.part_dA[b * p.D * p.N + j];
        p.dA[j] = v;
        return;
    }
    const int64_t k = j - p.D * p.N;
    if (k < p.D) {
        float v = 0.0f, w = 0.0f;
        for (int64_t b = 0; b < (int64_t)p.S * p.B; ++b) {
            v += p.part_dD[b * p.D + k];
            w += p.part_db[b * p.D + k];
        }
        if (p.dDskip) p.dDskip[k] = v;
        if (p.ddelta_bias) p.ddelta_bias[k] = w;
    }
}

template <typename T, bool VEC, bool PAIR>
void launch_ckpt_sweep(const S6BwdArgs& a, hipStream_t stream) {
    const dim3 grid((unsigned)((a.D + kChans - 1) / kChans), (unsigned)a.B, (unsigned)a.S);
    if (a.flags & SSM_FLAG_DELTA_SOFTPLUS) s6_bwd_ckpt<T, true, VEC, PAIR><<<grid, kThreads, 0, stream>>>(a);
    else s6_bwd_ckpt<T, false, VEC, PAIR><<<grid, kThreads, 0, stream>>>(a);
}

template <typename T, bool VEC, int MODE>
void launch_main(const S6BwdArgs& a, hipStream_t stream) {
    const bool sp = (a.flags & SSM_FLAG_DELTA_SOFTPLUS) != 0;
    const dim3 mgrid((unsigned)((a.D + kMainChans - 1) / kMainChans), (unsigned)a.B, (unsigned)a.S);
    const bool hz = a.z != nullptr;
    if (hz && sp) s6_bwd_main<T, true, true, VEC, MODE><<<mgrid, kMainThreads, 0, stream>>>(a);
    else if (hz) s6_bwd_main<T, true, false, VEC, MODE><<<mgrid, kMainThreads, 0, stream>>>(a);
    else if (sp) s6_bwd_main<T, false, true, VEC, MODE><<<mgrid, kMainThreads, 0, stream>>>(a);
    else s6_bwd_main<T, false, false, VEC, MODE><<<mgrid, kMainThreads, 0, stream>>>(a);
}

template <typename T, bool VEC>
void launch_sweeps(const S6BwdArgs& a, hipStream_t stream) {
    if (a.S > 1) {
        // the segments' adjoint pairs and step sums, their forward pairs, and
        // the carry of both into every segment's incoming state and adjoint
        launch_main<T, VEC, kPairs>(a, stream);
        if (a.own_ckpt) launch_ckpt_sweep<T, VEC, true>(a, stream);
        const int64_t chains = a.B * a.D * a.N;
        s6_bwd_carry<<<(unsigned)((chains + 255) / 256), 256, 0, stream>>>(a);
    }
    if (a.own_ckpt) launch_ckpt_sweep<T, VEC, false>(a, stream);
    if (a.S > 1) launch_main<T, VEC, kSegment>(a, stream);
    else launch_main<T, VEC, kWhole>(a, stream);
}

template <typename T>
hipError_t launch_t(const S6BwdArgs& a, hipStream_t stream) {
    // 16-byte activation pieces need every token's channel run 16-byte aligned
    if ((a.D * (int64_t)sizeof(T)) % 16 == 0) launch_sweeps<T, true>(a, stream);
    else launch_sweeps<T, false>(a, stream);
    const int64_t total = 2 * a.B * a.L * a.N + a.D * a.N + a.D;
    s6_bwd_reduce<<<(unsigned)((total + 255) / 256), 256, 0, stream>>>(a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_s6_bwd(const S6BwdArgs& a, hipStream_t stream) {
    return a.bf16 ? launch_t<uint16_t>(a, stream) : launch_t<float>(a, stream);
}

hipError_t launch_s6_bwd_ckpt(const S6BwdArgs& args, hipStream_t stream) {
    // one segment: the whole sequence from h0
    S6BwdArgs a = args;
    a.S = 1;
    a.seg_tiles = (a.L + kTile - 1) / kTile;
    if (a.bf16) {
        if ((a.D * 2) % 16 == 0) launch_ckpt_sweep<uint16_t, true, false>(a, stream);
        else launch_ckpt_sweep<uint16_t, false, false>(a, stream);
    } else {
        if ((a.D * 4) % 16 == 0) launch_ckpt_sweep<float, true, false>(a, stream);
        else launch_ckpt_sweep<float, false, false>(a, stream);
    }
    return hipGetLastError();
}

}  // namespace ssm
