// S6 selective-scan forward for gfx950.
//
// Operation (per batch row b, channel d, state index n; see include/ssm.h):
//   dt = softplus(delta + bias);  h[n] = exp(dt*A[d,n]) h[n] + dt*B_t[n]*u;
//   y = sum_n C_t[n] h[n] + D[d] u;  y *= silu(z)
// following the per-token discretisation of the Transformer-math "Selective
// state space" article ("Discretization becomes a per-token operation") and
// the fused-kernel idea of section 3 of the temporalbook Mamba chapter: the
// [B, L, D, N] expansion lives only in registers, HBM sees u/delta/z/B/C once
// and y once.
//
// Mapping: one lane owns one (b, d) channel and keeps all N states in VGPRs;
// a wavefront covers 64 consecutive channels of one batch row, so B_t and C_t
// are the same for every lane and every activation access is a contiguous
// 64-element row.  A is pre-scaled by log2(e) so each discretisation is one
// multiply and one v_exp_f32.
//
// Two kernel bodies:
//   s6_fast    -- N = 16, first-order input term.  Activations are prefetched
//                 twelve tokens ahead (the gate four) through buffer loads
//                 with a uniform row offset, kept as stored bits until their
//                 token comes up.  The B/C rows of the next 16 tokens are
//                 loaded one token per lane (lanes 0..15 of each 16-lane
//                 row); the reduce broadcasts B from there with DPP row
//                 broadcasts folded into the multiplies, the scan stages B and
//                 C in LDS and reads each token's rows as broadcasts.  No
//                 scalar load waits inside the token loop.
//   s6_generic -- any N <= 64 and the ZOH variant: plain token loop with
//                 wavefront-uniform scalar loads of B/C.
//
// Long sequences: the token axis is cut into S segments, each scanned on its
// own and its end state handed to the next (the chunked prefill of the
// Transformer-math article, section "What it costs at inference, and on a
// CPU").  Three launches:
//   1. s6_segment_reduce: each segment but the last reduces to the affine pair
//      (decay = exp(A * sum dt), offset = its end state from h = 0);
//   2. s6_carry_scan:    folds those pairs in segment order with the
//      composition (a1,b1) then (a2,b2) = (a2 a1, a2 b1 + b2) (section 3 of
//      the temporalbook chapter), one lane per (b, d, n) and 64 of them per
//      wavefront, giving each segment's incoming state;
//   3. s6_segment_scan:  every segment reruns from its incoming state, writes
//      y, and the last one writes h_last.
// With S = 1 only launch 3 runs.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <stdlib.h>

#include <mutex>

#include <type_traits>

#include "device_math.h"
#include "lane_ops.h"
#include "ssm_internal.h"

namespace ssm {
namespace {

constexpr int kWave = 64;
// s6_fast workgroups hold four independent wavefronts (256 channels): the
// dispatcher then places one on each SIMD of a CU, where single-wavefront
// workgroups were seen to pile up unevenly on the SIMDs.
constexpr int kFastBlock = 4 * kWave;
constexpr int64_t kMaxSegments = 256;    // segments per sequence (each >= 32 tokens)

// Row t of B (or C) for batch row b: NM floats, zero past N (zero-padded
// states keep h = 0 and add exact zeros to y).
template <typename T, int NM, bool FULL>
__device__ __forceinline__ void load_bc_row(const T* base, int64_t row, int N,
                                            float (&out)[NM]) {
    if constexpr (FULL && sizeof(T) == 2 && (NM % 2) == 0) {
        // two bf16 per dword: dword-wide uniform loads, split on the scalar unit
        const uint32_t* p = reinterpret_cast<const uint32_t*>(base + row * NM);
#pragma unroll
        for (int k = 0; k < NM / 2; ++k) {
            const uint32_t w = p[k];
            out[2 * k] = __uint_as_float(w << 16);
            out[2 * k + 1] = __uint_as_float(w & 0xffff0000u);
        }
    } else if constexpr (FULL) {
#pragma unroll
        for (int n = 0; n < NM; ++n) out[n] = Elem<T>::load(base, row * NM + n);
    } else {
#pragma unroll
        for (int n = 0; n < NM; ++n)
            out[n] = (n < N) ? Elem<T>::load(base, row * (int64_t)N + n) : 0.0f;
    }
}

// Exact zero-order hold: dB = (exp(dt*A) - 1) / A * B = dt*B * expm1(x)/x,
// x = dt*A (the ZOH formula of the Transformer-math article's discretisation
// section); expm1 keeps small x accurate.
// Tokens of batch row b: the row's length when lengths are given (clamped to
// [0, L]), else L.  Rows shorter than L leave their later positions of y
// untouched and end (h_last) at their own last token.
__device__ __forceinline__ int64_t row_len(const S6Args& p, int64_t b) {
    if (!p.seq_lens) return p.L;
    const int64_t n = p.seq_lens[b];
    return n < 0 ? 0 : (n > p.L ? p.L : n);
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Raw (storage-format) B or C row of one token: NM values, as 16-byte loads.
template <typename T, int NM>
struct RawRow {
    static constexpr int kWords = NM * (int)sizeof(T) / 16;   // 16-byte pieces
    u32x4 w[kWords > 0 ? kWords : 1];
};

template <typename T, int NM>
__device__ __forceinline__ void load_raw_row(RawRow<T, NM>& r, __amdgpu_buffer_rsrc_t rs,
                                             uint32_t voff, uint32_t soff) {
#pragma unroll
    for (int k = 0; k < RawRow<T, NM>::kWords; ++k)
        r.w[k] = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)(voff + 16 * k), (int)soff, 0);
}

template <typename T, int NM>
__device__ __forceinline__ void unpack_row(const RawRow<T, NM>& r, float (&out)[NM]) {
#pragma unroll
    for (int k = 0; k < RawRow<T, NM>::kWords; ++k) {
        const uint32_t v[4] = {r.w[k].x, r.w[k].y, r.w[k].z, r.w[k].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            if constexpr (sizeof(T) == 2) {
                out[8 * k + 2 * q] = __uint_as_float(v[q] << 16);
                out[8 * k + 2 * q + 1] = __uint_as_float(v[q] & 0xffff0000u);
            } else {
                out[4 * k + q] = __uint_as_float(v[q]);
            }
        }
    }
}

// ------------------------------------------------------------------ fast path
// Per-token inputs of U consecutive tokens as loaded (storage bits): they are
// widened to fp32 only where they are used, so that a load still in flight
// stalls nothing until its own token comes up.
template <int U>
struct TokBlock {
    uint32_t u[U], d[U];
};
template <int U>
struct GateBlock {
    uint32_t z[U];
};

template <typename T>
__device__ __forceinline__ uint32_t load_bits(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                              uint32_t soff) {
    if constexpr (sizeof(T) == 2)
        return __builtin_amdgcn_raw_buffer_load_b16(r, (int)voff, (int)soff, 0);
    else
        return __builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, (int)soff, 0);
}

template <typename T>
__device__ __forceinline__ float widen(uint32_t bits) {
    if constexpr (sizeof(T) == 2) return __uint_as_float(bits << 16);
    else return __uint_as_float(bits);
}

// One pass over segment s of the 64 channels of this wavefront, N = 16.
//   SCAN = false: reduce the segment to (decay, end state from zero);
//   SCAN = true : scan from the incoming state, write y (and h_last).
// RAGGED: D is not a multiple of 64 and the last wavefront of a row has
// inactive lanes, whose stores are skipped; otherwise every lane stores
// unconditionally and the token loop has no divergent branch.
// The tensors come in as __restrict__ arguments so that the compiler knows
// the y stores cannot alias the inputs.
template <typename T, bool SCAN, bool HAS_Z, bool RAGGED, bool SOFTPLUS, bool CONV>
__global__ __launch_bounds__(kFastBlock) __attribute__((amdgpu_waves_per_eu(3)))
void s6_fast(S6Args p, const T* __restrict__ u_, const T* __restrict__ delta_,
             const T* __restrict__ z_, const T* __restrict__ Bm_, const T* __restrict__ Cm_,
             T* __restrict__ y_) {
    constexpr int NS = 16;      // states per channel
    constexpr int U = 4;        // tokens per prefetch block
    constexpr int G = 16;       // tokens per B/C tile group (one per lane of a row)
    constexpr uint32_t E = sizeof(T);
    // a wavefront whose channels all lie past D has nothing to do
    const int64_t wave0 = (int64_t)blockIdx.x * kFastBlock +
                          kWave * (int64_t)__builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    if (wave0 >= p.D) return;
    const int64_t d = (int64_t)blockIdx.x * kFastBlock + threadIdx.x;
    const int64_t b = blockIdx.y;
    const int s = blockIdx.z;
    const bool active = d < p.D;
    const uint32_t col = (uint32_t)(active ? d : p.D - 1);
    const int64_t D = p.D;
    const int64_t t0 = (int64_t)s * p.seg_len;
    const int64_t Lb = row_len(p, b);                      // this row's tokens
    const int64_t t1 = t0 + p.seg_len < Lb ? t0 + p.seg_len : Lb;
    const int nt = t1 > t0 ? (int)(t1 - t0) : 0;           // segment fits 32-bit offsets
    const int64_t row0 = (b * p.L + t0) * D;
    const uint32_t seg_bytes = (uint32_t)nt * (uint32_t)D * E;
    const uint32_t row_bytes = (uint32_t)D * E;
    const uint32_t voff = col * E;
    const auto ru = make_rsrc(u_ + row0, seg_bytes);
    const auto rd = make_rsrc(delta_ + row0, seg_bytes);
    const auto rz = make_rsrc(HAS_Z ? z_ + row0 : nullptr, HAS_Z ? seg_bytes : 0u);
    const auto ry = make_rsrc(SCAN ? y_ + row0 : nullptr, SCAN ? seg_bytes : 0u);
    const uint32_t bc_row = NS * E;
    const auto rB = make_rsrc(Bm_ + (b * p.L + t0) * NS, (uint32_t)nt * bc_row);
    const auto rC = make_rsrc(SCAN ? Cm_ + (b * p.L + t0) * NS : nullptr,
                              SCAN ? (uint32_t)nt * bc_row : 0u);
    const float bias = p.delta_bias ? p.delta_bias[col] : 0.0f;
    const float dsk = (SCAN && p.Dskip) ? p.Dskip[col] : 0.0f;
    const uint32_t lane16 = threadIdx.x & 15u;

    float A2[NS], h[NS];
    const int64_t hb = (b * D + col) * NS;
    const int64_t sb = (int64_t)s * (p.B * D * NS) + hb;    // segment-major pairs
#pragma unroll
    for (int n = 0; n < NS; ++n) {
        A2[n] = p.A[(int64_t)col * NS + n] * kLog2e;
        float h_in = 0.0f;
        if (SCAN) {
            if (p.S > 1) h_in = p.seg_b[sb + n];
            else if (p.h0) h_in = p.h0[hb + n];
        }
        h[n] = h_in;
    }
    float dt_sum = 0.0f;

    // Causal conv1d + SiLU in front of the scan (CONV): u_ holds its input x.
    // Four taps (a width K < 4 is padded with leading zero weights); the
    // window holds x_{t-3}, x_{t-2}, x_{t-1}, starting from the tokens before
    // the segment, the carried state, or zeros.
    float cw[4] = {0.0f, 0.0f, 0.0f, 0.0f}, cb = 0.0f, xw[3] = {0.0f, 0.0f, 0.0f};
    if constexpr (CONV) {
        const int K = (int)p.conv_K;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int kk = k - (4 - K);
            cw[k] = kk >= 0 ? p.conv_w[(int64_t)col * K + kk] : 0.0f;
        }
        cb = p.conv_b ? p.conv_b[col] : 0.0f;
        // a segment past the row's end starts (and ends) at the row's last inputs
        const int64_t ts = t0 < Lb ? t0 : Lb;
#pragma unroll
        for (int i = 0; i < 3; ++i) {
            const int64_t tt = ts - 3 + i;
            const int slot = (int)tt + K - 1;           // index into the carried state
            if (tt >= 0)
                xw[i] = Elem<T>::load(u_, (b * p.L + tt) * D + col);
            else if (p.conv_state_in && slot >= 0)
                xw[i] = p.conv_state_in[(b * D + col) * (K - 1) + slot];
        }
    }
    const auto ruo = make_rsrc((CONV && SCAN && p.u_out) ? static_cast<T*>(p.u_out) + row0 : nullptr,
                               (CONV && SCAN && p.u_out) ? seg_bytes : 0u);
    auto input_u = [&](float xt) -> float {
        if constexpr (CONV) {
            const float sc = fmaf(cw[3], xt, fmaf(cw[2], xw[2], fmaf(cw[1], xw[1], fmaf(cw[0], xw[0], cb))));
            xw[0] = xw[1];
            xw[1] = xw[2];
            xw[2] = xt;
            return silu_f(sc);
        } else {
            return xt;
        }
    };

    // B/C tiles: fp32 rows of the current 16-token group, raw rows of the next.
    float btile[SCAN ? 1 : NS];
    RawRow<T, NS> rawB, rawC;
    // The scan keeps the B and C rows of the current 16-token group in LDS,
    // one 1 KiB slice each per wavefront ([token][state], fp32): every lane
    // reads the rows of the token at hand with the same address (a
    // broadcast), so neither the input term nor the readout needs a
    // cross-lane move, and no registers hold the group's rows.  Only this
    // wavefront touches its slices, and its LDS accesses are performed in
    // program order, so no barrier is needed.  The reduce keeps B in
    // registers and broadcasts it with DPP, folded into the multiply.
    __shared__ float4 cshare[SCAN ? (kFastBlock / kWave) * G * (NS / 4) : 1];
    float4* const cslice = cshare + (SCAN ? (threadIdx.x / kWave) * G * (NS / 4) : 0);
    __shared__ float4 bshare[SCAN ? (kFastBlock / kWave) * G * (NS / 4) : 1];
    float4* const bslice = bshare + (SCAN ? (threadIdx.x / kWave) * G * (NS / 4) : 0);
    const bool c_writer = (threadIdx.x & (kWave - 1)) < (uint32_t)G;
    auto load_tiles = [&](int jb) {
        const uint32_t off = (uint32_t)min(jb + (int)lane16, nt - 1) * bc_row;
        load_raw_row<T, NS>(rawB, rB, off, 0);
        if constexpr (SCAN) load_raw_row<T, NS>(rawC, rC, off, 0);
    };
    auto unpack_tiles = [&]() {
        if constexpr (!SCAN) unpack_row<T, NS>(rawB, btile);
        if constexpr (SCAN) {
            float c[NS], bb[NS];
            unpack_row<T, NS>(rawC, c);
            unpack_row<T, NS>(rawB, bb);
            if (c_writer) {
#pragma unroll
                for (int k = 0; k < NS / 4; ++k) {
                    cslice[lane16 * (NS / 4) + k] = make_float4(c[4 * k], c[4 * k + 1], c[4 * k + 2], c[4 * k + 3]);
                    bslice[lane16 * (NS / 4) + k] = make_float4(bb[4 * k], bb[4 * k + 1], bb[4 * k + 2], bb[4 * k + 3]);
                }
            }
        }
    };
    auto load_block = [&](TokBlock<U>& k, int jb) {
#pragma unroll
        for (int j = 0; j < U; ++j) {
            const uint32_t soff = (uint32_t)min(jb + j, nt - 1) * row_bytes;
            k.u[j] = load_bits<T>(ru, voff, soff);
            k.d[j] = load_bits<T>(rd, voff, soff);
        }
    };
    // the gate is needed last in a token and is requested one block ahead
    auto load_gate = [&](GateBlock<U>& g, int jb) {
        if constexpr (HAS_Z) {
#pragma unroll
            for (int j = 0; j < U; ++j)
                g.z[j] = load_bits<T>(rz, voff, (uint32_t)min(jb + j, nt - 1) * row_bytes);
        }
    };
    // q: which quarter of the tile group (lanes 4q .. 4q+3) holds these tokens
    // The step sizes of a block's tokens are formed first, as independent
    // chains, then the state updates run token by token.
    auto run_block = [&](const TokBlock<U>& k, const GateBlock<U>& g, int jb, auto guard, int q) {
        constexpr bool kGuard = decltype(guard)::value;
        float dtv[U], utv[U], dtu[U];
#pragma unroll
        for (int j = 0; j < U; ++j) {
            if constexpr (kGuard) {
                if (jb + j >= nt) break;
            }
            const float x = widen<T>(k.d[j]) + bias;
            if constexpr (SOFTPLUS) dtv[j] = softplus_f(x); else dtv[j] = x;
            utv[j] = input_u(widen<T>(k.u[j]));
            dtu[j] = dtv[j] * utv[j];
            if constexpr (!SCAN) dt_sum += dtv[j];
        }
#pragma unroll
        for (int j = 0; j < U; ++j) {
            const int r = jb + j;
            if constexpr (kGuard) {
                if (r >= nt) break;
            }
            const float dt = dtv[j];
            if constexpr (SCAN) {
                const float ut = utv[j];
                if constexpr (CONV) {
                    if (p.u_out && (!RAGGED || active)) Buf<T>::store(ruo, voff, (uint32_t)r * row_bytes, ut);
                }
                float ct[NS], bt[NS];
#pragma unroll
                for (int k = 0; k < NS / 4; ++k) {
                    const float4 v = cslice[(4 * q + j) * (NS / 4) + k];
                    ct[4 * k] = v.x; ct[4 * k + 1] = v.y; ct[4 * k + 2] = v.z; ct[4 * k + 3] = v.w;
                    const float4 w = bslice[(4 * q + j) * (NS / 4) + k];
                    bt[4 * k] = w.x; bt[4 * k + 1] = w.y; bt[4 * k + 2] = w.z; bt[4 * k + 3] = w.w;
                }
                float acc = 0.0f;
#pragma unroll
                for (int n = 0; n < NS; ++n) {
                    const float dA = fast_exp2(dt * A2[n]);
                    h[n] = fmaf(dA, h[n], bt[n] * dtu[j]);
                    acc = fmaf(ct[n], h[n], acc);
                }
                acc = fmaf(dsk, ut, acc);
                if constexpr (HAS_Z) acc *= silu_f(widen<T>(g.z[j]));
                if (!RAGGED || active) Buf<T>::store(ry, voff, (uint32_t)r * row_bytes, acc);
            } else {
#pragma unroll
                for (int n = 0; n < NS; ++n) {
                    const float dA = fast_exp2(dt * A2[n]);
                    h[n] = fmaf(dA, h[n], row_bcast(btile[n], 4 * q + j) * dtu[j]);
                }
            }
        }
    };

    using Full = std::false_type;
    using Tail = std::true_type;
    // Four rotating blocks: the block three ahead (12 tokens) is requested
    // before a block is run, the B/C rows one 16-token group ahead.
    TokBlock<U> k0, k1, k2, k3;
    GateBlock<U> g0, g1;
    int jb = 0;
    load_tiles(0);
    load_block(k0, 0);
    load_block(k1, 4);
    load_block(k2, 8);
    load_gate(g0, 0);
    unpack_tiles();
    // The scheduling fences keep each refill after the last use of the
    // registers it refills, so that no loop-carried copy of a value still in
    // flight (and no wait for it) is needed at the back edge.
    // Written as a bottom-tested loop: the exit then sits at the latch and
    // the loop-carried registers need no renaming copies.
    const int groups = nt / G;
    if (groups > 0) do {
        load_tiles(jb + G);
        load_block(k3, jb + 12);
        load_gate(g1, jb + 4);
        run_block(k0, g0, jb, Full{}, 0);
        __builtin_amdgcn_sched_barrier(0);
        load_block(k0, jb + 16);
        load_gate(g0, jb + 8);
        run_block(k1, g1, jb + 4, Full{}, 1);
        __builtin_amdgcn_sched_barrier(0);
        load_block(k1, jb + 20);
        load_gate(g1, jb + 12);
        run_block(k2, g0, jb + 8, Full{}, 2);
        __builtin_amdgcn_sched_barrier(0);
        load_block(k2, jb + 24);
        load_gate(g0, jb + 16);
        run_block(k3, g1, jb + 12, Full{}, 3);
        __builtin_amdgcn_sched_barrier(0);
        unpack_tiles();
        jb += G;
    } while (jb < groups * G);
    if (jb < nt) {                       // fewer than 16 tokens left
        load_gate(g1, jb + 4);
        run_block(k0, g0, jb, Tail{}, 0);
        if (jb + 4 < nt) {
            load_gate(g0, jb + 8);
            run_block(k1, g1, jb + 4, Tail{}, 1);
            if (jb + 8 < nt) {
                load_gate(g1, jb + 12);
                run_block(k2, g0, jb + 8, Tail{}, 2);
                if (jb + 12 < nt) {
                    load_block(k3, jb + 12);
                    run_block(k3, g1, jb + 12, Tail{}, 3);
                }
            }
        }
    }

    if constexpr (SCAN) {
        if (p.h_last && active && s == p.S - 1) {
#pragma unroll
            for (int n = 0; n < NS; ++n) p.h_last[hb + n] = h[n];
        }
        if constexpr (CONV) {
            // the last K-1 inputs of the sequence, oldest first
            if (p.conv_state_out && active && s == p.S - 1) {
                const int K = (int)p.conv_K;
                for (int i = 0; i < K - 1; ++i)
                    p.conv_state_out[(b * D + col) * (K - 1) + i] = xw[4 - K + i];
            }
        }
    } else if (active) {
#pragma unroll
        for (int n = 0; n < NS; ++n) {
            p.seg_a[sb + n] = fast_exp2(A2[n] * dt_sum);
            p.seg_b[sb + n] = h[n];
        }
    }
}

// -------------------------------------------------------- state-per-lane path
// N = 16, first-order input term, D a multiple of 16.
// One lane per (channel, state): each 16-lane row of a wavefront is one
// channel and lane n holds its state n, so a workgroup of four wavefronts
// covers 16 channels of one batch row.  With B*D/4 wavefronts the chip is
// filled without splitting the sequence, so every decay factor is computed
// once (the split path computes it in the segment reduce and again in the
// segment scan) and there is no carry launch.
//
// The sequence is walked in super-tiles of 128 tokens.  Per super-tile the
// workgroup loads u, delta, z (the 16 channels' 32-byte run of each token)
// and the B and C rows as 16-byte pieces, one of each per thread, and stages
// them in LDS: the activations as loaded ([token][channel], 16-byte writes),
// B and C as fp32 [tile][state][token].  A lane loading its own 2-byte element instead
// touches 16 cache lines per instruction, which ran 1.7x slower.
// Per 16-token tile, lane j of a row forms the per-channel scalars of token j
// (step size, dt*u, skip, gate); the decay exp(dt*A) and input term dt*u*B of
// each token reach the row through DPP row broadcasts folded into the
// multiplies.  All 16 decay factors of a tile are formed before the state
// chain h <- a*h + b runs through them.  The readout terms C*h of the tile are
// summed over the row by a reduce-scatter that leaves token j's y in lane j,
// which adds skip and gate and stages y in LDS; y leaves as 16-byte pieces of
// the workgroup's channel run when the next super-tile starts.
// The next super-tile's pieces are loaded while this one is computed.
// CONV: the causal conv1d + SiLU runs in front (u_ holds its input x): lane j
// convolves token j's window x_{t-3..t} from the staged row; the three inputs
// before a super-tile come from the previous one (or the carried conv state),
// kept in fp32 in a double-buffered LDS halo.
namespace lanes {
constexpr int kTile = 16;                 // tokens per tile (one per lane of a row)
constexpr int kSpan = 128;                // segments are whole multiples of this many tokens
constexpr int kChans = 16;                // channels per workgroup
constexpr int kPitch = kTile + 4;         // staged B/C row of one state (floats)
// Tiles per super-tile: 64-token super-tiles keep the LDS of a workgroup small
// enough for four to share a CU.
constexpr int kSuper = 4;
// Readout of y: bf16 one-pass calls fold the row's 16 partial products with
// one DPP exchange and finish through LDS (fewer VALU instructions, measured
// faster there); the others reduce entirely with DPP (row_reduce_scatter16).
template <typename T, bool SEG>
constexpr bool lds_readout() { return sizeof(T) == 2 && !SEG; }
// Readout buffer of one wavefront: after the first halving exchange each lane
// holds 8 partial sums (token k + 8 * (lane / 8), states lane % 8 and + 8);
// the 8 lanes that share a token write them next to each other and the
// token's lane reads them back.  Token k + 8h, partial j sits at 16k + 8h + j
// (the 16 lanes' writes of one k hit 16 banks); rows sit 16 banks apart.
constexpr int kRedRow = 8 * kTile + 16;   // floats per row (channel)

template <typename T> __device__ __forceinline__ uint32_t elem_bits(T v);
template <> __device__ __forceinline__ uint32_t elem_bits<uint16_t>(uint16_t v) { return v; }
template <> __device__ __forceinline__ uint32_t elem_bits<float>(float v) { return __float_as_uint(v); }

// One super-tile's inputs as loaded: 16-byte pieces, kPer per thread and
// tensor (kPieces in all; with fewer than 256 some threads load none).
template <typename T, bool HAS_Z, int SPAN>
struct Pieces {
    static constexpr int kPerToken = kChans * (int)sizeof(T) / 16;   // channels' run of a token
    static constexpr int kPieces = SPAN * kPerToken;
    static constexpr int kPer = (kPieces + 255) / 256;
    u32x4 u[kPer], d[kPer], z[HAS_Z ? kPer : 1], b[kPer], c[kPer];
};
}  // namespace lanes

static_assert(lanes::kSpan % (lanes::kTile * lanes::kSuper) == 0, "segments are whole super-tiles");
static_assert(kWave == plan::kWave && kMaxSegments == plan::kMaxSegments &&
                  lanes::kSpan == plan::kLanesSpan && lanes::kChans == plan::kLanesChans,
              "the host planner's tiling constants");
static_assert(plan::kFixChunk % (lanes::kTile * lanes::kSuper) == 0,
              "fix-up chunks are whole super-tiles of the segmented scan");

template <typename T, bool HAS_Z, bool SOFTPLUS, bool CONV, bool SEG, bool CKPT = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4)))
void s6_lanes(S6Args p, const T* __restrict__ u_, const T* __restrict__ delta_,
              const T* __restrict__ z_, const T* __restrict__ Bm_, const T* __restrict__ Cm_,
              T* __restrict__ y_) {
    using namespace lanes;
    constexpr int kSpan = kTile * kSuper;                 // tokens per super-tile
    constexpr bool kLdsReadout = lds_readout<T, SEG>();
    using Raw = Pieces<T, HAS_Z, kSpan>;
    constexpr uint32_t E = sizeof(T);
    constexpr int kPerToken = Raw::kPerToken, kPer = Raw::kPer;
    constexpr int kVals = 16 / (int)E;                  // elements per piece
    constexpr int kActPitch = kChans + 8;   // [tensor][token][channel], 48-byte token rows
    __shared__ __attribute__((aligned(16))) float bct[2][kSuper][16 * kPitch];
    __shared__ __attribute__((aligned(16))) T act[HAS_Z ? 3 : 2][kSpan][kActPitch];
    __shared__ __attribute__((aligned(16))) T yst[kSpan][kChans];
    __shared__ __attribute__((aligned(16))) float red[kLdsReadout ? 4 : 1][kLdsReadout ? 4 * kRedRow : 1];
    // CONV: inputs x_{t0-3 .. t0-1} before the super-tile (fp32), by parity;
    // the convolution's output u when the caller asks for it
    __shared__ float xh[CONV ? 2 : 1][kChans][4];
    __shared__ __attribute__((aligned(16))) T ust[CONV ? kSpan : 1][kChans];
    const int tid = threadIdx.x;
    const int w = tid >> 6, row = (tid >> 4) & 3, n = tid & 15;
    // Workgroups are dealt to the 8 XCDs round robin (i -> XCD i % 8); the id
    // is renumbered so each XCD runs a contiguous range of channel groups, and
    // the four groups that share a 128-byte activation row share one L2.
    const uint32_t groups = gridDim.x, total = gridDim.x * gridDim.y;
    const uint32_t bi = blockIdx.x + gridDim.x * blockIdx.y;
    const uint32_t xcd = bi % 8, per = total / 8, extra = total % 8;
    const uint32_t lid = xcd * per + min(xcd, extra) + bi / 8;
    const int64_t b = lid / groups;
    const int64_t grp = lid % groups;
    const int chan = 4 * w + row;
    const int64_t D = p.D;
    const int64_t d = grp * kChans + chan;
    const int64_t Lb = row_len(p, b);
    // segment s of the row (one segment: the whole row): tokens [t0, t1)
    const int s = (int)blockIdx.z;
    const int64_t t0 = (int64_t)s * p.seg_len;
    const int64_t t1 = t0 + p.seg_len < Lb ? t0 + p.seg_len : Lb;
    const float a2 = p.A[d * 16 + n] * kLog2e;
    const float bias = p.delta_bias ? p.delta_bias[d] : 0.0f;
    const float dsk = p.Dskip ? p.Dskip[d] : 0.0f;
    // the first segment starts from h0, the others from zero (their incoming
    // state is added to y afterwards, by the fix-up pass)
    float h = (s == 0 && p.h0) ? p.h0[(b * D + d) * 16 + n] : 0.0f;
    float dt_sum = 0.0f;                  // segments: this lane's share of the segment's sum of dt
    // CKPT (no convolution): the state entering every 16-token tile for the
    // backward pass, one 4-byte store per lane and tile, through a buffer
    // resource over the workgroup's 16 channels; a tile past the row's end
    // stores at an offset past the resource, which is dropped.  A segment
    // after the first stores its states from zero, which the fix-up completes.
    static_assert(!CKPT || !CONV, "checkpoints are written by the scan without the convolution");
    const int64_t nck = CKPT ? p.ckpt_blocks : 0;
    const auto rck = make_rsrc(CKPT ? p.ckpt + (b * D + grp * kChans) * nck * 16 : nullptr,
                               CKPT ? (uint32_t)(kChans * nck * 64) : 0u);
    const uint32_t ck_lane = CKPT ? (uint32_t)((chan * nck * 16 + n) * 4) : 0u;
    // buffer resources over this row's tokens: loads past the row's end read
    // zero, stores there are dropped (the planner keeps offsets in 32 bits)
    const int64_t rowoff = b * p.L * D;
    const uint32_t act_bytes = (uint32_t)(Lb * D * E);
    const auto ru = make_rsrc(u_ + rowoff, act_bytes);
    const auto rd = make_rsrc(delta_ + rowoff, act_bytes);
    const auto rz = make_rsrc(HAS_Z ? z_ + rowoff : nullptr, HAS_Z ? act_bytes : 0u);
    const auto ry = make_rsrc(y_ + rowoff, act_bytes);
    const uint32_t bc_bytes = (uint32_t)(Lb * 16 * E);
    const auto rB = make_rsrc(Bm_ + b * p.L * 16, bc_bytes);
    const auto rC = make_rsrc(Cm_ + b * p.L * 16, bc_bytes);
    const uint32_t row_bytes = (uint32_t)(D * E);
    const uint32_t grp_bytes = (uint32_t)(grp * kChans * E);
    // CONV: four taps (a width K < 4 padded with leading zero weights)
    float cw[4] = {0.0f, 0.0f, 0.0f, 0.0f}, cb = 0.0f;
    const bool want_u = CONV && p.u_out != nullptr;
    const auto ruo = make_rsrc(want_u ? static_cast<T*>(p.u_out) + rowoff : nullptr,
                               want_u ? act_bytes : 0u);
    if constexpr (CONV) {
        const int K = (int)p.conv_K;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int kk = k - (4 - K);
            cw[k] = kk >= 0 ? p.conv_w[d * K + kk] : 0.0f;
        }
        cb = p.conv_b ? p.conv_b[d] : 0.0f;
        if (tid < 3 * kChans) {
            // the inputs before the segment's first token: inside the row the
            // previous tokens; before token 0 the carried state (its last K-1
            // slots are x_{-K+1 .. -1}) or zeros
            const int ch = tid / 3, i = tid % 3, slot = i + K - 4;
            const int64_t tt = t0 - 3 + i;
            const int64_t dd = grp * kChans + ch;
            float v = 0.0f;
            if (tt >= 0 && tt < Lb) v = widen<T>(elem_bits<T>(u_[(b * p.L + tt) * D + dd]));
            else if (tt < 0 && p.conv_state_in && slot >= 0)
                v = p.conv_state_in[(b * D + dd) * (K - 1) + slot];
            xh[0][ch][i] = v;
        }
    }

    // thread -> (token idx / kPerToken, piece idx % kPerToken) of the super-tile
    auto load = [&](Raw& r, int64_t st0) {
        const uint32_t soff = (uint32_t)st0 * row_bytes;
        const uint32_t bsoff = (uint32_t)st0 * (16 * E);
#pragma unroll
        for (int k = 0; k < kPer; ++k) {
            const uint32_t idx = tid + 256 * k, t = idx / kPerToken, pc = idx % kPerToken;
            if (Raw::kPieces % 256 != 0 && idx >= (uint32_t)Raw::kPieces) break;
            const uint32_t voff = t * row_bytes + grp_bytes + 16 * pc;
            r.u[k] = __builtin_amdgcn_raw_buffer_load_b128(ru, (int)voff, (int)soff, 0);
            r.d[k] = __builtin_amdgcn_raw_buffer_load_b128(rd, (int)voff, (int)soff, 0);
            if constexpr (HAS_Z)
                r.z[k] = __builtin_amdgcn_raw_buffer_load_b128(rz, (int)voff, (int)soff, 0);
            const uint32_t bvoff = t * (16 * E) + 16 * pc;
            r.b[k] = __builtin_amdgcn_raw_buffer_load_b128(rB, (int)bvoff, (int)bsoff, 0);
            r.c[k] = __builtin_amdgcn_raw_buffer_load_b128(rC, (int)bvoff, (int)bsoff, 0);
        }
    };
    auto stage = [&](const Raw& r) {
#pragma unroll
        for (int k = 0; k < kPer; ++k) {
            const int idx = tid + 256 * k, t = idx / kPerToken, pc = idx % kPerToken;
            if (Raw::kPieces % 256 != 0 && idx >= Raw::kPieces) break;
            const T* vb = reinterpret_cast<const T*>(&r.b[k]);
            const T* vc = reinterpret_cast<const T*>(&r.c[k]);
            *reinterpret_cast<u32x4*>(&act[0][t][kVals * pc]) = r.u[k];
            *reinterpret_cast<u32x4*>(&act[1][t][kVals * pc]) = r.d[k];
            if constexpr (HAS_Z) *reinterpret_cast<u32x4*>(&act[2][t][kVals * pc]) = r.z[k];
#pragma unroll
            for (int e = 0; e < kVals; ++e) {
                const int ch = kVals * pc + e;           // state for B/C
                bct[0][t / kTile][ch * kPitch + t % kTile] = widen<T>(elem_bits<T>(vb[e]));
                bct[1][t / kTile][ch * kPitch + t % kTile] = widen<T>(elem_bits<T>(vc[e]));
            }
        }
    };
    auto store_y = [&](int64_t st0) {
#pragma unroll
        for (int k = 0; k < kPer; ++k) {
            const uint32_t idx = tid + 256 * k, t = idx / kPerToken, pc = idx % kPerToken;
            if (Raw::kPieces % 256 != 0 && idx >= (uint32_t)Raw::kPieces) break;
            const u32x4 v = *reinterpret_cast<const u32x4*>(
                reinterpret_cast<const char*>(&yst[t][0]) + 16 * pc);
            __builtin_amdgcn_raw_buffer_store_b128(v, ry, (int)(t * row_bytes + grp_bytes + 16 * pc),
                                                   (int)((uint32_t)st0 * row_bytes), 0);
            if (want_u) {
                const u32x4 w = *reinterpret_cast<const u32x4*>(
                    reinterpret_cast<const char*>(&ust[t][0]) + 16 * pc);
                __builtin_amdgcn_raw_buffer_store_b128(w, ruo, (int)(t * row_bytes + grp_bytes + 16 * pc),
                                                       (int)((uint32_t)st0 * row_bytes), 0);
            }
        }
    };

    // The 8 tiles of one super-tile (TAIL: the super-tile reaches past the
    // row's end, so tokens there are masked to dt = 0).
    auto tiles = [&](int64_t st0, int64_t sg, auto tail_tag) __attribute__((always_inline)) {
        constexpr bool kTail = decltype(tail_tag)::value;
#pragma unroll
        for (int i = 0; i < kSuper; ++i) {
            const int tl = kTile * i + n;   // this lane's token within the super-tile
            if constexpr (CKPT) {
                uint32_t off = ck_lane + (uint32_t)((st0 / kTile + i) * 64);
                if constexpr (kTail) off = st0 + kTile * i < t1 ? off : 0x80000000u;
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(h), rck, (int)off, 0, 0);
            }
            // past the row's end (TAIL) dt = 0 leaves h unchanged; the step is
            // masked rather than branched on, so no branch splits the
            // super-tile into one basic block per tile (which kept the
            // scheduler from overlapping a tile's exponentials with the
            // previous tile's chain)
            const float xr = widen<T>(elem_bits<T>(act[1][tl][chan])) + bias;
            float dt = SOFTPLUS ? softplus_f(xr) : xr;
            if constexpr (kTail) {
                const uint32_t keep = st0 + tl < t1 ? 0xffffffffu : 0u;
                dt = __uint_as_float(__float_as_uint(dt) & keep);
            }
            if constexpr (SEG) dt_sum += dt;
            float ut;
            if constexpr (CONV) {
                // window x_{t-3..t}: the staged row, before the super-tile the halo
                float xw[4];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const int m = tl - 3 + k;
                    if (i == 0 && k < 3) {
                        const float xa = widen<T>(elem_bits<T>(act[0][m < 0 ? 0 : m][chan]));
                        const float xb = xh[sg & 1][chan][m < 0 ? m + 3 : 0];
                        xw[k] = m < 0 ? xb : xa;
                    } else {
                        xw[k] = widen<T>(elem_bits<T>(act[0][m][chan]));
                    }
                }
                // the same product order as the split path's fused convolution
                const float sc = fmaf(cw[3], xw[3], fmaf(cw[2], xw[2], fmaf(cw[1], xw[1], fmaf(cw[0], xw[0], cb))));
                ut = silu_f(sc);
                if (want_u) {
                    if constexpr (sizeof(T) == 2) ust[tl][chan] = f32_to_bf16_bits(ut);
                    else ust[tl][chan] = ut;
                }
                // the next super-tile's halo: this one's last three inputs
                if (i == kSuper - 1 && n >= kTile - 3) xh[(sg + 1) & 1][chan][n - (kTile - 3)] = xw[3];
            } else {
                ut = widen<T>(elem_bits<T>(act[0][tl][chan]));
            }
            const float dtu = dt * ut;
            float bv[kTile], cv[kTile], dA[kTile], pr[kTile];
#pragma unroll
            for (int q = 0; q < kTile / 4; ++q) {
                const f32x4 x = *reinterpret_cast<const f32x4*>(&bct[0][i][n * kPitch + 4 * q]);
                const f32x4 c = *reinterpret_cast<const f32x4*>(&bct[1][i][n * kPitch + 4 * q]);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    bv[4 * q + r] = x[r];
                    cv[4 * q + r] = c[r];
                }
            }
#pragma unroll
            for (int j = 0; j < kTile; ++j) {
                dA[j] = fast_exp2(row_bcast(dt, j) * a2);
                bv[j] *= row_bcast(dtu, j);
            }
#pragma unroll
            for (int j = 0; j < kTile; ++j) {
                h = fmaf(dA[j], h, bv[j]);
                pr[j] = cv[j] * h;
            }
            float yv;
            if constexpr (kLdsReadout) {
                // fold the row's two halves of states with DPP, then the
                // remaining 8 partial sums of each token through this
                // wavefront's LDS buffer (LDS performs a wavefront's accesses
                // in order)
                float a8[8];
                // raised wave priority from the fold to the issue of the
                // reads: the wavefront gets its LDS round trip under way
                // ahead of the other wavefronts' vector work, which then
                // covers it (0.1254 -> 0.1224 ms at the Mamba-130M layer,
                // 0.3675 -> 0.361 ms at the 2.8B layer, three alternating runs)
                __builtin_amdgcn_s_setprio(1);
                row_fold_halves16(pr, a8);
                float* const rb = &red[w][row * kRedRow];
#pragma unroll
                for (int k = 0; k < 8; ++k) rb[16 * k + 8 * (n >> 3) + (n & 7)] = a8[k];
                wave_lds_fence();
                // token n's block: its first half read first for n % 8 < 4,
                // else its second, so the row's 16 first reads cover all 64
                // banks (the sum is the same: the half sums are added last)
                const int blk = 16 * (n & 7) + 8 * (n >> 3);
                const int sw = 4 * ((n >> 2) & 1);
                const f32x4 q0 = *reinterpret_cast<const f32x4*>(&rb[blk + sw]);
                const f32x4 q1 = *reinterpret_cast<const f32x4*>(&rb[blk + 4 - sw]);
                __builtin_amdgcn_s_setprio(0);
                yv = ((q0[0] + q0[1]) + (q0[2] + q0[3])) + ((q1[0] + q1[1]) + (q1[2] + q1[3]));
            } else {
                yv = row_reduce_scatter16(pr, n);
            }
            yv = fmaf(dsk, ut, yv);
            if constexpr (HAS_Z) yv *= silu_f(widen<T>(elem_bits<T>(act[2][tl][chan])));
            if constexpr (sizeof(T) == 2) yst[tl][chan] = f32_to_bf16_bits(yv);
            else yst[tl][chan] = yv;
        }
    };

    const int64_t nsup = t1 > t0 ? (t1 - t0 + kSpan - 1) / kSpan : 0;
    Raw nxt;
    if (nsup > 0) load(nxt, t0);
    for (int64_t sg = 0; sg < nsup; ++sg) {
        const Raw cur = nxt;
        const int64_t st0 = t0 + sg * kSpan;
        lds_barrier();                      // previous super-tile's LDS reads and y staging done
        // staged before the previous y leaves: the wait for this super-tile's
        // loads then does not also wait for those stores (~1-2% faster)
        stage(cur);
        if (sg > 0) store_y(st0 - kSpan);
        lds_barrier();
        load(nxt, st0 + kSpan);             // travels while this super-tile is computed
        if (st0 + kSpan <= t1) tiles(st0, sg, std::false_type{});
        else tiles(st0, sg, std::true_type{});
        if constexpr (SEG) {
            // where the fix-up's chunks start: the segment's sum of dt up to
            // the end of each whole chunk (the row's 16 shares added up)
            constexpr int64_t kSupChunk = plan::kFixChunk / kSpan;
            if (s > 0 && (sg + 1) % kSupChunk == 0) {
                float cum = dt_sum;
                cum += dpp_mov<0x128>(cum);            // row_ror:8
                cum += dpp_mov<0x124>(cum);            // row_ror:4
                cum += dpp_mov<0x122>(cum);            // row_ror:2
                cum += dpp_mov<0x121>(cum);            // row_ror:1
                if (n == 0)
                    p.seg_cum[(((int64_t)s * p.fix_chunks + (sg + 1) / kSupChunk - 1) * p.B + b) * D + d] = cum;
            }
        }
    }
    lds_barrier();
    if (nsup > 0) store_y(t0 + (nsup - 1) * kSpan);
    if (!SEG) {
        if (p.h_last) p.h_last[(b * D + d) * 16 + n] = h;
    } else {
        // the segment as an affine map of its incoming state: decay
        // exp(A * sum dt) (the row's sum over its 16 lanes) and the end state
        // from the segment's own start
        float tot = dt_sum;
        tot += dpp_mov<0x128>(tot);            // row_ror:8
        tot += dpp_mov<0x124>(tot);            // row_ror:4
        tot += dpp_mov<0x122>(tot);            // row_ror:2
        tot += dpp_mov<0x121>(tot);            // row_ror:1
        const int64_t pi = (int64_t)s * (p.B * D * 16) + (b * D + d) * 16 + n;   // segment-major
        p.seg_a[pi] = fast_exp2(a2 * tot);
        p.seg_b[pi] = h;
    }
    if constexpr (CONV) {
        // the last K-1 inputs of the row, oldest first (from the carried state
        // when the row is shorter than that)
        const int K = (int)p.conv_K;
        if (p.conv_state_out && s == p.S - 1 && tid < (K - 1) * kChans) {
            const int ch = tid / (K - 1), i = tid % (K - 1);
            const int64_t dd = grp * kChans + ch;
            const int64_t t = Lb - (K - 1) + i;
            float v = 0.0f;
            if (t >= 0) v = widen<T>(elem_bits<T>(u_[(b * p.L + t) * D + dd]));
            else if (p.conv_state_in) v = p.conv_state_in[(b * D + dd) * (K - 1) + (t + K - 1)];
            p.conv_state_out[(b * D + dd) * (K - 1) + i] = v;
        }
    }
}

// --------------------------------------------------------------- generic path
// Any N <= NM (states past N are zero-padded: A = 0, B = C = 0 keeps them at 0
// and adds exact zeros to y) and the exact-ZOH input term.
template <typename T, int NM, bool ZOH, bool SCAN>
__global__ __launch_bounds__(kWave) void s6_generic(S6Args p) {
    const int64_t d = (int64_t)blockIdx.x * kWave + threadIdx.x;
    const int64_t b = blockIdx.y;
    const int s = blockIdx.z;
    const bool active = d < p.D;
    const int64_t dd = active ? d : p.D - 1;
    const int N = (int)p.N;
    const T* u = static_cast<const T*>(p.u);
    const T* delta = static_cast<const T*>(p.delta);
    const T* Bm = static_cast<const T*>(p.Bm);
    const T* Cm = static_cast<const T*>(p.Cm);
    const T* z = static_cast<const T*>(p.z);
    T* y = static_cast<T*>(p.y);
    const float bias = p.delta_bias ? p.delta_bias[dd] : 0.0f;
    const float dsk = (SCAN && p.Dskip) ? p.Dskip[dd] : 0.0f;
    const bool softplus = (p.flags & SSM_FLAG_DELTA_SOFTPLUS) != 0;

    float A1[NM], A2[NM], h[NM];
    const int64_t hb = (b * p.D + dd) * (int64_t)N;
    const int64_t sb = (int64_t)s * (p.B * p.D * N) + hb;  // segment-major pairs
#pragma unroll
    for (int n = 0; n < NM; ++n) {
        const float a = n < N ? p.A[dd * N + n] : 0.0f;
        A1[n] = a;
        A2[n] = a * kLog2e;
        float h_in = 0.0f;
        if (SCAN && n < N) {
            if (p.S > 1) h_in = p.seg_b[sb + n];
            else if (p.h0) h_in = p.h0[hb + n];
        }
        h[n] = h_in;
    }
    const int64_t t0 = (int64_t)s * p.seg_len;
    const int64_t Lb = row_len(p, b);
    const int64_t t1 = t0 + p.seg_len < Lb ? t0 + p.seg_len : Lb;
    float dt_sum = 0.0f;
    for (int64_t t = t0; t < t1; ++t) {
        const int64_t i = (b * p.L + t) * p.D + dd;
        const float x = Elem<T>::load(delta, i) + bias;
        const float dt = softplus ? softplus_f(x) : x;
        const float ut = Elem<T>::load(u, i);
        const float dtu = dt * ut;
        float bt[NM];
        load_bc_row<T, NM, false>(Bm, b * p.L + t, N, bt);
        if constexpr (SCAN) {
            float ct[NM];
            load_bc_row<T, NM, false>(Cm, b * p.L + t, N, ct);
            float acc = 0.0f;
#pragma unroll
            for (int n = 0; n < NM; ++n) {
                const float dA = fast_exp2(dt * A2[n]);
                const float w = dtu * bt[n] * (ZOH ? zoh_factor(dt * A1[n]) : 1.0f);
                h[n] = fmaf(dA, h[n], w);
                acc = fmaf(ct[n], h[n], acc);
            }
            acc = fmaf(dsk, ut, acc);
            if (z) acc *= silu_f(Elem<T>::load(z, i));
            if (active) Elem<T>::store(y, i, acc);
        } else {
            dt_sum += dt;
#pragma unroll
            for (int n = 0; n < NM; ++n) {
                const float dA = fast_exp2(dt * A2[n]);
                const float w = dtu * bt[n] * (ZOH ? zoh_factor(dt * A1[n]) : 1.0f);
                h[n] = fmaf(dA, h[n], w);
            }
        }
    }
    if constexpr (SCAN) {
        if (p.h_last && active && s == p.S - 1) {
#pragma unroll
            for (int n = 0; n < NM; ++n)
                if (n < N) p.h_last[hb + n] = h[n];
        }
    } else if (active) {
#pragma unroll
        for (int n = 0; n < NM; ++n) {
            if (n < N) {
                p.seg_a[sb + n] = fast_exp2(A2[n] * dt_sum);
                p.seg_b[sb + n] = h[n];
            }
        }
    }
}

// Carry over segments.  The pairs are stored segment-major, pair s of chain
// i = (b*D + d)*N + n at s*B*D*N + i, so that for one segment a wavefront
// reads 64 consecutive chains.  Each lane folds the pairs of its chain in
// order, h <- a_s h + b_s starting from h0, and overwrites b_s with the state
// entering segment s (the composition (a1,b1) then (a2,b2) = (a2 a1,
// a2 b1 + b2) of section 3 of the temporalbook chapter, applied to h0).  With
// at most 64 segments the fold is short; the pairs of up to eight segments are
// loaded before any is used or overwritten.
__global__ __launch_bounds__(256) void s6_carry_scan(const float* __restrict__ seg_a,
                                                     float* __restrict__ seg_b,
                                                     const float* __restrict__ h0,
                                                     int64_t chains, int S) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= chains) return;
    float h = h0 ? h0[i] : 0.0f;
    constexpr int kBatch = 8;
    for (int s0 = 0; s0 < S - 1; s0 += kBatch) {
        float a[kBatch], c[kBatch];
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
            const bool in = s0 + k < S - 1;
            a[k] = in ? seg_a[(int64_t)(s0 + k) * chains + i] : 1.0f;
            c[k] = in ? seg_b[(int64_t)(s0 + k) * chains + i] : 0.0f;
        }
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
            if (s0 + k < S - 1) seg_b[(int64_t)(s0 + k) * chains + i] = h;
            h = fmaf(a[k], h, c[k]);
        }
    }
    seg_b[(int64_t)(S - 1) * chains + i] = h;      // entering the last segment
}

// Carry of the segmented state-per-lane path.  Segment 0 ran from h0, so its
// offset is the true state after it; every later segment ran from zero and is
// the affine map h -> decay * h + offset of its incoming state.  Each lane
// folds one (b, d, n) chain in segment order, overwrites each later offset
// with the state entering that segment (the composition of the temporalbook
// chapter's section 3), and writes the state after the last segment to
// h_last.
__global__ __launch_bounds__(256) void s6_carry_lanes(const float* __restrict__ seg_a,
                                                      float* __restrict__ seg_b,
                                                      float* __restrict__ h_last,
                                                      int64_t chains, int S) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= chains) return;
    float h = seg_b[i];
    constexpr int kBatch = 8;
    for (int s0 = 1; s0 < S; s0 += kBatch) {
        float a[kBatch], c[kBatch];
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
            const bool in = s0 + k < S;
            a[k] = in ? seg_a[(int64_t)(s0 + k) * chains + i] : 1.0f;
            c[k] = in ? seg_b[(int64_t)(s0 + k) * chains + i] : 0.0f;
        }
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
            if (s0 + k < S) seg_b[(int64_t)(s0 + k) * chains + i] = h;
            h = fmaf(a[k], h, c[k]);
        }
    }
    if (h_last) h_last[i] = h;
}

// Fix-up of the segmented state-per-lane path: segment s >= 1
// was scanned from a zero state, so its y lacks the part of the incoming state
// h_in that survives to each token, which is exp(A * cum_t) * h_in with cum_t
// the sum of dt over the segment up to and including t (each token multiplies
// the state by exp(dt * A)).  So
//   y_t += silu(z_t) * sum_n C_t[n] * exp(A[d,n] * cum_t) * h_in[n].
// The correction of a token needs only cum_t, so the tokens are independent
// given a running sum of dt: the segment is cut into chunks of kFixChunk
// tokens, one workgroup each, which start from the sum up to the chunk's
// start that the scan stored (seg_cum) and extend it over the chunk.  With
// softplus every dt >= 0, so cum never decreases within a chunk; once
// exp(A * cum) is exactly 0 in fp32 for every state of every channel of the
// workgroup (A <= 0), every later correction of the chunk is exactly zero and
// the walk stops there (a chunk that starts there returns before loading
// anything); a state whose decay is already 0 is skipped before that.
// Without softplus every chunk runs to its end.
// Workgroup: 16 channels (D a multiple of 16); it walks its chunk in blocks of
// 64 tokens.  Each block's delta, z, y and C rows are loaded as 16-byte
// pieces of the group's 16-channel run (one memory round trip per block),
// staged in LDS and read per (channel, token): lane j of 16-lane row c handles
// token 16k + j of the block for channel c.  The new y leaves through LDS as
// 16-byte pieces again.
namespace fixup {
constexpr int kBlock = 64;                 // tokens per block
constexpr int kPad = 4;                    // LDS row padding (floats)
}  // namespace fixup
static_assert(plan::kFixChunk % fixup::kBlock == 0, "fix-up chunks are whole blocks");

template <typename T, bool HAS_Z, bool SOFTPLUS, bool CKPT>
__global__ __launch_bounds__(256) void s6_fixup(S6Args p, const T* __restrict__ delta_,
                                                const T* __restrict__ z_,
                                                const T* __restrict__ Cm_, T* __restrict__ y_) {
    using namespace fixup;
    constexpr int kChans = lanes::kChans;
    constexpr uint32_t E = sizeof(T);
    constexpr int kPerTok = kChans * (int)E / 16;     // 16-byte pieces per token (2 bf16, 4 fp32)
    constexpr int kPieces = kBlock * kPerTok;         // per tensor and block
    constexpr int kPer = (kPieces + 255) / 256;       // per thread
    static_assert(kPieces % 256 == 0 || kPer == 1, "whole pieces per thread");
    constexpr int kVals = 16 / (int)E;
    constexpr int kW = kChans + kPad;
    constexpr uint32_t kLine = 128 / (kChans * E);    // channel groups per 128-byte row (2 fp32, 4 bf16)
    __shared__ __attribute__((aligned(16))) float sd[kBlock][kW];    // dt (raw), then y
    __shared__ __attribute__((aligned(16))) float sz[HAS_Z ? kBlock : 1][kW];
    __shared__ __attribute__((aligned(16))) float sy[kBlock][kW];
    __shared__ __attribute__((aligned(16))) float sc[kBlock][kW];    // C rows [token][state]
    __shared__ int sdone[3][4];         // exit votes per wavefront: by block parity, and at the start
    const int tid = threadIdx.x;
    const int j = tid & 15;                      // token within a 16-token tile
    const int c = tid >> 4;                      // channel within the group
    // One workgroup per (channel group, batch row, segment >= 1, chunk), in
    // the order: group within its 128-byte row fastest, then chunk, segment,
    // batch row, row of groups.  Workgroups are dealt to the 8 XCDs round
    // robin (i -> XCD i % 8): the id is renumbered so each XCD runs a
    // contiguous range of that order, so the groups that share 128-byte rows
    // of delta, y and z run side by side on one XCD and share its L2, and the
    // chunks of a segment (the first ones carry the work, later ones stop at
    // once) are spread evenly.
    const uint32_t total = gridDim.x;
    const uint32_t bi = blockIdx.x;
    const uint32_t xcd = bi % 8, per = total / 8, extra = total % 8;
    uint32_t q = xcd * per + min(xcd, extra) + bi / 8;
    const uint32_t r = q % kLine;
    q /= kLine;
    const int64_t k = q % (uint32_t)p.fix_chunks;
    q /= (uint32_t)p.fix_chunks;
    const int s = (int)(q % (uint32_t)(p.S - 1)) + 1;
    q /= (uint32_t)(p.S - 1);
    const int64_t b = q % (uint32_t)p.B;
    const int64_t grp = (int64_t)(q / (uint32_t)p.B) * kLine + r;
    const int64_t D = p.D;
    if (grp * kChans >= D) return;
    const int64_t d = grp * kChans + c;
    const int64_t Lb = row_len(p, b);
    const int64_t s0 = (int64_t)s * p.seg_len;
    const int64_t s1 = s0 + p.seg_len < Lb ? s0 + p.seg_len : Lb;
    const int64_t t0 = s0 + k * plan::kFixChunk;
    const int64_t t1 = t0 + plan::kFixChunk < s1 ? t0 + plan::kFixChunk : s1;
    if (t0 >= t1) return;
    float a2[16];
    float gmax[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};   // per group of four states
#pragma unroll
    for (int n = 0; n < 16; ++n) {
        a2[n] = p.A[d * 16 + n] * kLog2e;
        gmax[n / 4] = fmaxf(gmax[n / 4], a2[n]);
    }
    const float a2max = fmaxf(fmaxf(gmax[0], gmax[1]), fmaxf(gmax[2], gmax[3]));
    // cum at the last token before the chunk
    float carry = k == 0 ? 0.0f : p.seg_cum[(((int64_t)s * p.fix_chunks + k - 1) * p.B + b) * D + d];
    // every wavefront's vote through LDS; the barriers wait for LDS only (a
    // workgroup barrier with a memory fence would also wait for the y stores
    // and the next block's loads)
    auto all_spent = [&](int slot) {
        const bool spent = __all(fast_exp2(a2max * carry) == 0.0f);
        if ((tid & 63) == 0) sdone[slot][tid >> 6] = spent;
        lds_barrier();
        return sdone[slot][0] && sdone[slot][1] && sdone[slot][2] && sdone[slot][3];
    };
    if constexpr (SOFTPLUS) {
        if (all_spent(2)) return;
    }
    float hin[16];
    const int64_t hb = (int64_t)s * (p.B * D * 16) + (b * D + d) * 16;
#pragma unroll
    for (int n = 0; n < 16; ++n) hin[n] = p.seg_b[hb + n];
    // CKPT: lane j of a channel completes state j of the checkpoint of every
    // tile (stored from zero by the scan): + exp2(A log2(e) cum) h_in, with
    // cum the segment's sum of dt before the tile
    const float a2_ck = CKPT ? p.A[d * 16 + j] * kLog2e : 0.0f;
    const float hin_ck = CKPT ? p.seg_b[hb + j] : 0.0f;
    float* const ck_row = CKPT ? p.ckpt + (b * D + d) * p.ckpt_blocks * 16 + j : nullptr;
    const float bias = p.delta_bias ? p.delta_bias[d] : 0.0f;
    // buffer resources over the row's tokens (32-bit offsets as in the scan)
    const int64_t rowoff = b * p.L * D;
    const uint32_t act_bytes = (uint32_t)(Lb * D * E);
    const auto rd = make_rsrc(delta_ + rowoff, act_bytes);
    const auto rz = make_rsrc(HAS_Z ? z_ + rowoff : nullptr, HAS_Z ? act_bytes : 0u);
    const auto ry = make_rsrc(y_ + rowoff, act_bytes);
    const auto rC = make_rsrc(Cm_ + b * p.L * 16, (uint32_t)(Lb * 16 * E));
    const uint32_t row_bytes = (uint32_t)(D * E);
    const uint32_t grp_bytes = (uint32_t)(grp * kChans * E);
    // pieces of this thread: tid + 256 i (threads >= kPieces idle in the staging)
    const int pc = tid % kPerTok;
    const bool loader = tid < kPieces;
    auto ptok = [&](int i) { return (tid + 256 * i) / kPerTok; };
    auto widen4 = [&](const u32x4& v, float* out) __attribute__((always_inline)) {
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            if constexpr (E == 2) {
                out[2 * q] = __uint_as_float(w[q] << 16);
                out[2 * q + 1] = __uint_as_float(w[q] & 0xffff0000u);
            } else {
                out[q] = __uint_as_float(w[q]);
            }
        }
    };
    uint32_t live = 0xf;                         // groups of four states still contributing
    // one 16-byte piece of each tensor per loader thread, a block ahead: the
    // next block's loads are issued before this block's y stores, so the
    // wait for them (loads and stores complete in order) waits for no store
    u32x4 nd[kPer], ny[kPer], nz[HAS_Z ? kPer : 1], nc[kPer];
    auto load_block = [&](int64_t tb) {
        if (loader) {
            const uint32_t soff = (uint32_t)tb * row_bytes;
#pragma unroll
            for (int i = 0; i < kPer; ++i) {
                const uint32_t pt = (uint32_t)ptok(i);
                const uint32_t voff = pt * row_bytes + grp_bytes + 16 * pc;
                nd[i] = __builtin_amdgcn_raw_buffer_load_b128(rd, (int)voff, (int)soff, 0);
                ny[i] = __builtin_amdgcn_raw_buffer_load_b128(ry, (int)voff, (int)soff, 0);
                if constexpr (HAS_Z) nz[i] = __builtin_amdgcn_raw_buffer_load_b128(rz, (int)voff, (int)soff, 0);
                nc[i] = __builtin_amdgcn_raw_buffer_load_b128(
                    rC, (int)(pt * 16 * E + 16 * pc), (int)((uint32_t)tb * 16 * E), 0);
            }
        }
    };
    load_block(t0);
    for (int64_t tt = t0; tt < t1; tt += kBlock) {
        // stage the block
        if (loader) {
#pragma unroll
            for (int i = 0; i < kPer; ++i) {
                const int pt = ptok(i);
                float f[kVals];
                widen4(nd[i], f);
#pragma unroll
                for (int e = 0; e < kVals; ++e) sd[pt][kVals * pc + e] = f[e];
                widen4(ny[i], f);
#pragma unroll
                for (int e = 0; e < kVals; ++e) sy[pt][kVals * pc + e] = f[e];
                if constexpr (HAS_Z) {
                    widen4(nz[i], f);
#pragma unroll
                    for (int e = 0; e < kVals; ++e) sz[pt][kVals * pc + e] = f[e];
                }
                widen4(nc[i], f);
#pragma unroll
                for (int e = 0; e < kVals; ++e) sc[pt][kVals * pc + e] = f[e];
            }
        }
        // the next block of the chunk travels while this one is computed
        // (past the row's end the loads read zero; tokens past the chunk's
        // end in its last block are read and not used)
        if (tt + kBlock < t1) load_block(tt + kBlock);
        lds_barrier();
        if constexpr (SOFTPLUS) {
            // a group is spent once the decay of its slowest state is exactly
            // 0 (exp2 is monotone, so the others' are too) in every channel
            uint32_t m = 0;
#pragma unroll
            for (int g = 0; g < 4; ++g)
                if (__any(fast_exp2(gmax[g] * carry) != 0.0f)) m |= 1u << g;
            live &= __builtin_amdgcn_readfirstlane(m);
        }
        constexpr int kT = kBlock / 16;
        float cum[kT], corr[kT];
#pragma unroll
        for (int i = 0; i < kT; ++i) {
            const int tl = 16 * i + j;
            const bool in = tt + tl < t1;
            float x = in ? step_dt(sd[tl][c], bias, SOFTPLUS ? SSM_FLAG_DELTA_SOFTPLUS : 0u) : 0.0f;
            // inclusive prefix sum of dt over the 16 tokens of the row (DPP
            // row shifts; lanes shifted in from outside the row read 0)
            x += dpp_shr<1>(x);
            x += dpp_shr<2>(x);
            x += dpp_shr<4>(x);
            x += dpp_shr<8>(x);
            if constexpr (CKPT) {
                // carry: the sum before the tile; a term exactly 0 changes nothing
                const float add = fast_exp2(a2_ck * carry) * hin_ck;
                if (tt + 16 * i < t1 && add != 0.0f) {
                    float* const e = ck_row + ((tt + 16 * i) / 16) * 16;
                    *e += add;
                }
            }
            cum[i] = x + carry;
            carry = row_bcast_c<15>(cum[i]);
            corr[i] = 0.0f;
        }
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            if (live & (1u << g)) {
#pragma unroll
                for (int i = 0; i < kT; ++i) {
                    const f32x4 cq = *reinterpret_cast<const f32x4*>(&sc[16 * i + j][4 * g]);
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        corr[i] = fmaf(cq[r], fast_exp2(a2[4 * g + r] * cum[i]) * hin[4 * g + r], corr[i]);
                }
            }
        }
#pragma unroll
        for (int i = 0; i < kT; ++i) {
            const int tl = 16 * i + j;
            float g = 1.0f;
            if constexpr (HAS_Z) g = silu_f(sz[tl][c]);
            sy[tl][c] = fmaf(corr[i], g, sy[tl][c]);
        }
        lds_barrier();
        // the block's y back as 16-byte pieces, none past the chunk's end
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int pt = ptok(i);
            if (loader && tt + pt < t1) {
                float f[kVals];
#pragma unroll
                for (int e = 0; e < kVals; ++e) f[e] = sy[pt][kVals * pc + e];
                u32x4 v;
                if constexpr (E == 2) {
                    uint32_t w[4];
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        w[q] = (uint32_t)f32_to_bf16_bits(f[2 * q]) | ((uint32_t)f32_to_bf16_bits(f[2 * q + 1]) << 16);
                    v = u32x4{w[0], w[1], w[2], w[3]};
                } else {
                    v = u32x4{__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
                              __float_as_uint(f[3])};
                }
                __builtin_amdgcn_raw_buffer_store_b128(v, ry, (int)((uint32_t)pt * row_bytes + grp_bytes + 16 * pc),
                                                       (int)((uint32_t)tt * row_bytes), 0);
            }
        }
        // the next block's staging waits for these reads
        if constexpr (SOFTPLUS) {
            // exact stop: exp(A * cum) is 0 for every state from here to the
            // chunk's end
            if (all_spent((int)(((tt - t0) / kBlock) & 1))) break;
        } else {
            lds_barrier();
        }
    }
}

// h_last = h0 (or zeros) for an empty sequence.
__global__ void s6_copy_state(const float* h0, float* h_last, int64_t count) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < count) h_last[i] = h0 ? h0[i] : 0.0f;
}

void mark(const S6Args& a, int i, hipStream_t stream) {
    if (a.events) (void)hipEventRecord(a.events[i], stream);
}

// launch errors surface through the caller's hipGetLastError
void launch_carry(const S6Args& a, hipStream_t stream) {
    const int64_t chains = a.B * a.D * a.N;
    hipLaunchKernelGGL(s6_carry_scan, dim3((unsigned)((chains + 255) / 256)), dim3(256), 0,
                       stream, a.seg_a, a.seg_b, a.h0, chains, (int)a.S);
}

// The carry of the state-per-lane segments and the fix-up of segments 1..
// (marks the two phase boundaries in between).
template <typename T, bool SP>
void launch_carry_fixup(const S6Args& a, hipStream_t stream) {
    const int64_t chains = a.B * a.D * 16;
    hipLaunchKernelGGL(s6_carry_lanes, dim3((unsigned)((chains + 255) / 256)), dim3(256), 0,
                       stream, a.seg_a, a.seg_b, a.h_last, chains, (int)a.S);
    mark(a, 2, stream);
    // one workgroup per (channel group, batch row, segment after the first,
    // chunk), the groups padded to whole 128-byte rows (the planner keeps the
    // count within 32 bits)
    const int64_t line = 128 / (lanes::kChans * (int64_t)sizeof(T));
    const int64_t rows = (a.D / lanes::kChans + line - 1) / line;
    const dim3 fgrid((unsigned)(rows * line * a.B * (a.S - 1) * a.fix_chunks));
    const T* Dl = static_cast<const T*>(a.delta);
    const T* Z = static_cast<const T*>(a.z);
    const T* Cp = static_cast<const T*>(a.Cm);
    T* Y = static_cast<T*>(a.y);
    if (a.ckpt) {
        if (a.z)
            hipLaunchKernelGGL((s6_fixup<T, true, SP, true>), fgrid, dim3(256), 0, stream, a, Dl, Z, Cp, Y);
        else
            hipLaunchKernelGGL((s6_fixup<T, false, SP, true>), fgrid, dim3(256), 0, stream, a, Dl, Z, Cp, Y);
    } else {
        if (a.z)
            hipLaunchKernelGGL((s6_fixup<T, true, SP, false>), fgrid, dim3(256), 0, stream, a, Dl, Z, Cp, Y);
        else
            hipLaunchKernelGGL((s6_fixup<T, false, SP, false>), fgrid, dim3(256), 0, stream, a, Dl, Z, Cp, Y);
    }
    mark(a, 3, stream);
}

template <typename T, bool SP, bool CV>
hipError_t launch_fast_sp(const S6Args& a, hipStream_t stream) {
    const T* U = static_cast<const T*>(a.u);
    const T* Dl = static_cast<const T*>(a.delta);
    const T* Z = static_cast<const T*>(a.z);
    const T* Bp = static_cast<const T*>(a.Bm);
    const T* Cp = static_cast<const T*>(a.Cm);
    T* Y = static_cast<T*>(a.y);
    const unsigned dblocks = (unsigned)((a.D + kFastBlock - 1) / kFastBlock);
    const dim3 block(kFastBlock);
    mark(a, 0, stream);
    if (a.S > 1)
        hipLaunchKernelGGL((s6_fast<T, false, false, false, SP, CV>),
                           dim3(dblocks, (unsigned)a.B, (unsigned)(a.S - 1)), block, 0, stream,
                           a, U, Dl, Z, Bp, Cp, (T*)nullptr);
    mark(a, 1, stream);
    if (a.S > 1) launch_carry(a, stream);
    mark(a, 2, stream);
    const dim3 grid(dblocks, (unsigned)a.B, (unsigned)a.S);
    const bool ragged = (a.D % kWave) != 0;
    if (a.z) {
        if (ragged)
            hipLaunchKernelGGL((s6_fast<T, true, true, true, SP, CV>), grid, block, 0, stream, a, U,
                               Dl, Z, Bp, Cp, Y);
        else
            hipLaunchKernelGGL((s6_fast<T, true, true, false, SP, CV>), grid, block, 0, stream, a, U,
                               Dl, Z, Bp, Cp, Y);
    } else {
        if (ragged)
            hipLaunchKernelGGL((s6_fast<T, true, false, true, SP, CV>), grid, block, 0, stream, a, U,
                               Dl, Z, Bp, Cp, Y);
        else
            hipLaunchKernelGGL((s6_fast<T, true, false, false, SP, CV>), grid, block, 0, stream, a, U,
                               Dl, Z, Bp, Cp, Y);
    }
    mark(a, 3, stream);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_lanes(const S6Args& a, hipStream_t stream) {
    const bool sp = (a.flags & SSM_FLAG_DELTA_SOFTPLUS) != 0;
    const T* U = static_cast<const T*>(a.u);
    const T* Dl = static_cast<const T*>(a.delta);
    const T* Z = static_cast<const T*>(a.z);
    const T* Bp = static_cast<const T*>(a.Bm);
    const T* Cp = static_cast<const T*>(a.Cm);
    T* Y = static_cast<T*>(a.y);
    const unsigned groups = (unsigned)(a.D / lanes::kChans);
    const dim3 grid(groups, (unsigned)a.B, (unsigned)a.S), block(256);
    mark(a, 0, stream);
    const bool cv = a.conv_w != nullptr;
    // one pass: 128-token super-tiles (3 workgroups per CU by LDS);
    // segments: 64-token super-tiles (half the LDS, 4 wavefronts per SIMD)
#define SSM_LANES(Z_, SP_, CV_)                                                                   \
    do {                                                                                          \
        if (!(CV_) && a.ckpt && a.S == 1)                                                         \
            hipLaunchKernelGGL((s6_lanes<T, Z_, SP_, false, false, true>), grid, block, 0,        \
                               stream, a, U, Dl, Z, Bp, Cp, Y);                                   \
        else if (!(CV_) && a.ckpt)                                                                \
            hipLaunchKernelGGL((s6_lanes<T, Z_, SP_, false, true, true>), grid, block, 0,         \
                               stream, a, U, Dl, Z, Bp, Cp, Y);                                   \
        else if (a.S > 1)                                                                         \
            hipLaunchKernelGGL((s6_lanes<T, Z_, SP_, CV_, true>), grid, block, 0,                 \
                               stream, a, U, Dl, Z, Bp, Cp, Y);                                   \
        else                                                                                      \
            hipLaunchKernelGGL((s6_lanes<T, Z_, SP_, CV_, false>), grid, block, 0,                \
                               stream, a, U, Dl, Z, Bp, Cp, Y);                                   \
    } while (0)
    if (cv) {
        if (a.z) { if (sp) SSM_LANES(true, true, true); else SSM_LANES(true, false, true); }
        else { if (sp) SSM_LANES(false, true, true); else SSM_LANES(false, false, true); }
    } else {
        if (a.z) { if (sp) SSM_LANES(true, true, false); else SSM_LANES(true, false, false); }
        else { if (sp) SSM_LANES(false, true, false); else SSM_LANES(false, false, false); }
    }
#undef SSM_LANES
    mark(a, 1, stream);
    if (a.S > 1) {
        if (sp) launch_carry_fixup<T, true>(a, stream);
        else launch_carry_fixup<T, false>(a, stream);
    } else {
        mark(a, 2, stream);
        mark(a, 3, stream);
    }
    return hipGetLastError();
}

template <typename T>
hipError_t launch_fast(const S6Args& a, hipStream_t stream) {
    if (a.lanes) return launch_lanes<T>(a, stream);
    const bool sp = (a.flags & SSM_FLAG_DELTA_SOFTPLUS) != 0;
    if (a.conv_w)
        return sp ? launch_fast_sp<T, true, true>(a, stream) : launch_fast_sp<T, false, true>(a, stream);
    return sp ? launch_fast_sp<T, true, false>(a, stream) : launch_fast_sp<T, false, false>(a, stream);
}

template <typename T, int NM, bool ZOH>
hipError_t launch_generic(const S6Args& a, hipStream_t stream) {
    const unsigned dblocks = (unsigned)((a.D + kWave - 1) / kWave);
    mark(a, 0, stream);
    if (a.S > 1)
        hipLaunchKernelGGL((s6_generic<T, NM, ZOH, false>),
                           dim3(dblocks, (unsigned)a.B, (unsigned)(a.S - 1)), dim3(kWave), 0,
                           stream, a);
    mark(a, 1, stream);
    if (a.S > 1) launch_carry(a, stream);
    mark(a, 2, stream);
    hipLaunchKernelGGL((s6_generic<T, NM, ZOH, true>), dim3(dblocks, (unsigned)a.B, (unsigned)a.S),
                       dim3(kWave), 0, stream, a);
    mark(a, 3, stream);
    return hipGetLastError();
}

template <typename T, bool ZOH>
hipError_t launch_n(const S6Args& a, hipStream_t stream) {
    const int64_t N = a.N;
    if (N <= 4) return launch_generic<T, 4, ZOH>(a, stream);
    if (N <= 8) return launch_generic<T, 8, ZOH>(a, stream);
    if (N <= 16) return launch_generic<T, 16, ZOH>(a, stream);
    if (N <= 32) return launch_generic<T, 32, ZOH>(a, stream);
    return launch_generic<T, 64, ZOH>(a, stream);
}

}  // namespace

hipError_t launch_s6(const S6Args& a, hipStream_t stream) {
    if (a.L == 0) {
        for (int i = 0; i < 3; ++i) mark(a, i, stream);
        if (a.h_last) {
            const int64_t count = a.B * a.D * a.N;
            hipLaunchKernelGGL(s6_copy_state, dim3((unsigned)((count + 255) / 256)), dim3(256),
                               0, stream, a.h0, a.h_last, count);
        }
        const int64_t ccount = a.B * a.D * (a.conv_K - 1);
        if (a.conv_w && a.conv_state_out && ccount > 0)
            hipLaunchKernelGGL(s6_copy_state, dim3((unsigned)((ccount + 255) / 256)), dim3(256),
                               0, stream, a.conv_state_in, a.conv_state_out, ccount);
        mark(a, 3, stream);
        return hipGetLastError();
    }
    const bool zoh = (a.flags & SSM_FLAG_ZOH) != 0;
    if (a.N == 16 && !zoh) return a.bf16 ? launch_fast<uint16_t>(a, stream) : launch_fast<float>(a, stream);
    if (a.bf16) return zoh ? launch_n<uint16_t, true>(a, stream) : launch_n<uint16_t, false>(a, stream);
    return zoh ? launch_n<float, true>(a, stream) : launch_n<float, false>(a, stream);
}

// ------------------------------------------------- static scratch (no allocation)
// Device scratch for callers that cannot allocate: the split path's segment
// pairs live here instead of in a caller workspace.  One copy per GPU, held
// until the process ends; every call on a GPU shares it, so calls that overlap
// on one GPU (different streams, or host threads) race.  Nothing in it has to
// start at zero: the segment pass writes every pair before the carry reads it.
static __device__ __align__(256) float scratch[kNoAllocScratchBytes / sizeof(float)];

namespace {
constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t noalloc_scratch(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (!scratch_ptr[dev]) {
        // the array's name is a host-side stand-in: its device address (this
        // device's copy) comes from the runtime, once per device
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        scratch_ptr[dev] = p;
    }
    *out = scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace ssm
