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
// are wavefront-uniform (scalar loads, SGPR operands) and every activation
// access is a contiguous 64-element row.  A is pre-scaled by log2(e) so each
// discretisation is one multiply and one v_exp_f32.
//
// Long sequences: the token axis is cut into S segments ("scan within a
// block, carry the block's state forward", Transformer-math article, "What it
// costs at inference").  Three launches:
//   1. s6_segment_reduce: each segment but the last reduces to the affine pair
//      (decay = exp(A * sum dt), offset = its end state from h = 0);
//   2. s6_carry_scan:    a wavefront-level inclusive scan of those pairs with
//      the composition (a1,b1) then (a2,b2) = (a2 a1, a2 b1 + b2) (section 3
//      of the temporalbook chapter), one lane per segment, giving each
//      segment's incoming state;
//   3. s6_segment_scan:  every segment reruns from its incoming state, writes
//      y, and the last one writes h_last.
// With S = 1 only launch 3 runs.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <stdlib.h>

#include "device_math.h"
#include "ssm_internal.h"

namespace ssm {
namespace {

constexpr int kWave = 64;

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
__device__ __forceinline__ float zoh_factor(float x) {
    return x != 0.0f ? expm1f(x) / x : 1.0f;
}

__device__ __forceinline__ float step_dt(float raw, float bias, unsigned flags) {
    const float x = raw + bias;
    return (flags & SSM_FLAG_DELTA_SOFTPLUS) ? softplus_f(x) : x;
}

// Segment reduce: for segment s < S-1 of channel (b, d), the pair
// (prod_t exp(dt_t A), end state from zero).
template <typename T, int NM, bool FULL, bool ZOH>
__global__ __launch_bounds__(kWave) void s6_segment_reduce(S6Args p) {
    const int64_t d = (int64_t)blockIdx.x * kWave + threadIdx.x;
    const int64_t b = blockIdx.y;
    const int s = blockIdx.z;
    const bool active = d < p.D;
    const int64_t dd = active ? d : p.D - 1;
    const int N = (int)p.N;
    const T* u = static_cast<const T*>(p.u);
    const T* delta = static_cast<const T*>(p.delta);
    const T* Bm = static_cast<const T*>(p.Bm);
    const float bias = p.delta_bias ? p.delta_bias[dd] : 0.0f;

    float A1[NM], A2[NM], h[NM];
#pragma unroll
    for (int n = 0; n < NM; ++n) {
        const float a = (FULL || n < N) ? p.A[dd * N + n] : 0.0f;
        A1[n] = a;
        A2[n] = a * kLog2e;
        h[n] = 0.0f;
    }
    const int64_t t0 = (int64_t)s * p.seg_len;
    const int64_t t1 = t0 + p.seg_len < p.L ? t0 + p.seg_len : p.L;
    float dt_sum = 0.0f;
    for (int64_t t = t0; t < t1; ++t) {
        const int64_t i = (b * p.L + t) * p.D + dd;
        const float dt = step_dt(Elem<T>::load(delta, i), bias, p.flags);
        const float ut = Elem<T>::load(u, i);
        float bt[NM];
        load_bc_row<T, NM, FULL>(Bm, b * p.L + t, N, bt);
        const float dtu = dt * ut;
        dt_sum += dt;
#pragma unroll
        for (int n = 0; n < NM; ++n) {
            const float dA = fast_exp2(dt * A2[n]);
            const float w = dtu * bt[n] * (ZOH ? zoh_factor(dt * A1[n]) : 1.0f);
            h[n] = fmaf(dA, h[n], w);
        }
    }
    if (active) {
        const int64_t o = ((b * p.D + dd) * p.S + s) * (int64_t)N;
#pragma unroll
        for (int n = 0; n < NM; ++n) {
            if (FULL || n < N) {
                p.seg_a[o + n] = fast_exp2(A2[n] * dt_sum);
                p.seg_b[o + n] = h[n];
            }
        }
    }
}

// Wavefront-level scan over segments.  Lane j of a group of SP lanes (SP a
// power of two >= S) holds segment j of one (b, d, n); after log2(SP) steps
// of __shfl_up it holds the inclusive composition of segments 0..j.  The
// incoming state of segment j is the exclusive one applied to h0; it
// overwrites seg_b (each lane reads its pair before any lane writes).
__global__ __launch_bounds__(256) void s6_carry_scan(S6Args p, int SP) {
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int j = (int)(gid % SP);
    const int64_t bdn = gid / SP;
    const int64_t total = p.B * p.D * p.N;
    const bool valid = bdn < total;
    const int64_t bd = valid ? bdn / p.N : 0;
    const int n = valid ? (int)(bdn % p.N) : 0;
    const int64_t o = (bd * p.S + j) * p.N + n;
    float a = 1.0f, c = 0.0f;                     // identity map
    if (valid && j < p.S - 1) {
        a = p.seg_a[o];
        c = p.seg_b[o];
    }
    for (int off = 1; off < SP; off <<= 1) {
        const float ap = __shfl_up(a, off, SP);
        const float cp = __shfl_up(c, off, SP);
        if (j >= off) {                           // earlier segments first, then ours
            c = fmaf(a, cp, c);
            a = a * ap;
        }
    }
    const float h0 = (valid && p.h0) ? p.h0[bd * p.N + n] : 0.0f;
    float ae = __shfl_up(a, 1, SP);
    float ce = __shfl_up(c, 1, SP);
    if (j == 0) { ae = 1.0f; ce = 0.0f; }
    if (valid && j < p.S) p.seg_b[o] = fmaf(ae, h0, ce);
}

// Segment scan with readout: start from the incoming state, write y.
template <typename T, int NM, bool FULL, bool ZOH>
__global__ __launch_bounds__(kWave) void s6_segment_scan(S6Args p) {
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
    const float dsk = p.Dskip ? p.Dskip[dd] : 0.0f;

    float A1[NM], A2[NM], h[NM];
    const int64_t hb = (b * p.D + dd) * (int64_t)N;
#pragma unroll
    for (int n = 0; n < NM; ++n) {
        const float a = (FULL || n < N) ? p.A[dd * N + n] : 0.0f;
        A1[n] = a;
        A2[n] = a * kLog2e;
        float h_in = 0.0f;
        if (FULL || n < N) {
            if (p.S > 1)
                h_in = p.seg_b[((b * p.D + dd) * p.S + s) * (int64_t)N + n];
            else if (p.h0)
                h_in = p.h0[hb + n];
        }
        h[n] = h_in;
    }
    const int64_t t0 = (int64_t)s * p.seg_len;
    const int64_t t1 = t0 + p.seg_len < p.L ? t0 + p.seg_len : p.L;
    for (int64_t t = t0; t < t1; ++t) {
        const int64_t i = (b * p.L + t) * p.D + dd;
        const float dt = step_dt(Elem<T>::load(delta, i), bias, p.flags);
        const float ut = Elem<T>::load(u, i);
        float bt[NM], ct[NM];
        load_bc_row<T, NM, FULL>(Bm, b * p.L + t, N, bt);
        load_bc_row<T, NM, FULL>(Cm, b * p.L + t, N, ct);
        const float dtu = dt * ut;
        float acc = 0.0f;
#pragma unroll
        for (int n = 0; n < NM; ++n) {
            const float dA = fast_exp2(dt * A2[n]);
            const float w = dtu * bt[n] * (ZOH ? zoh_factor(dt * A1[n]) : 1.0f);
            h[n] = fmaf(dA, h[n], w);
            acc = fmaf(ct[n], h[n], acc);
        }
        acc = fmaf(dsk, ut, acc);
        if (p.z) acc *= silu_f(Elem<T>::load(z, i));
        if (active) Elem<T>::store(y, i, acc);
    }
    if (p.h_last && active && s == p.S - 1) {
#pragma unroll
        for (int n = 0; n < NM; ++n)
            if (FULL || n < N) p.h_last[hb + n] = h[n];
    }
}

// h_last = h0 (or zeros) for an empty sequence.
__global__ void s6_copy_state(const float* h0, float* h_last, int64_t count) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < count) h_last[i] = h0 ? h0[i] : 0.0f;
}

template <typename T, int NM, bool FULL, bool ZOH>
hipError_t launch_typed(const S6Args& a, hipStream_t stream) {
    const dim3 block(kWave);
    const unsigned dblocks = (unsigned)((a.D + kWave - 1) / kWave);
    if (a.S > 1) {
        hipLaunchKernelGGL((s6_segment_reduce<T, NM, FULL, ZOH>),
                           dim3(dblocks, (unsigned)a.B, (unsigned)(a.S - 1)), block, 0,
                           stream, a);
        int SP = 1;
        while (SP < a.S) SP <<= 1;
        const int64_t threads = a.B * a.D * a.N * SP;
        hipLaunchKernelGGL(s6_carry_scan, dim3((unsigned)((threads + 255) / 256)),
                           dim3(256), 0, stream, a, SP);
    }
    hipLaunchKernelGGL((s6_segment_scan<T, NM, FULL, ZOH>),
                       dim3(dblocks, (unsigned)a.B, (unsigned)a.S), block, 0, stream, a);
    return hipGetLastError();
}

template <typename T, bool ZOH>
hipError_t launch_n(const S6Args& a, hipStream_t stream) {
    const int64_t N = a.N;
    if (N <= 4) return N == 4 ? launch_typed<T, 4, true, ZOH>(a, stream) : launch_typed<T, 4, false, ZOH>(a, stream);
    if (N <= 8) return N == 8 ? launch_typed<T, 8, true, ZOH>(a, stream) : launch_typed<T, 8, false, ZOH>(a, stream);
    if (N <= 16) return N == 16 ? launch_typed<T, 16, true, ZOH>(a, stream) : launch_typed<T, 16, false, ZOH>(a, stream);
    if (N <= 32) return N == 32 ? launch_typed<T, 32, true, ZOH>(a, stream) : launch_typed<T, 32, false, ZOH>(a, stream);
    return N == 64 ? launch_typed<T, 64, true, ZOH>(a, stream) : launch_typed<T, 64, false, ZOH>(a, stream);
}

}  // namespace

S6Plan plan_s6(int64_t B, int64_t L, int64_t D, int64_t N) {
    S6Plan pl{1, L > 0 ? L : 1, 0};
    if (L <= 0) return pl;
    // Enough wavefronts to give every SIMD of the 256 CUs about two.
    const int64_t waves = B * ((D + kWave - 1) / kWave);
    int64_t target = 2048;
    int64_t S = (target + waves - 1) / waves;
    const char* env = getenv("SSM_S6_SEGMENTS");
    if (env && atoi(env) > 0) S = atoi(env);
    const int64_t min_seg = 32;
    int64_t maxS = (L + min_seg - 1) / min_seg;
    if (S > maxS) S = maxS;
    if (S > 64) S = 64;
    if (S < 1) S = 1;
    const int64_t seg_len = (L + S - 1) / S;
    S = (L + seg_len - 1) / seg_len;   // no empty trailing segment
    pl.S = (int)S;
    pl.seg_len = seg_len;
    if (S > 1) pl.workspace_bytes = (size_t)2 * (size_t)(B * D * S * N) * sizeof(float);
    return pl;
}

hipError_t launch_s6(const S6Args& a, hipStream_t stream) {
    if (a.L == 0) {
        if (a.h_last) {
            const int64_t count = a.B * a.D * a.N;
            hipLaunchKernelGGL(s6_copy_state, dim3((unsigned)((count + 255) / 256)), dim3(256),
                               0, stream, a.h0, a.h_last, count);
        }
        return hipGetLastError();
    }
    const bool zoh = (a.flags & SSM_FLAG_ZOH) != 0;
    if (a.bf16) return zoh ? launch_n<uint16_t, true>(a, stream) : launch_n<uint16_t, false>(a, stream);
    return zoh ? launch_n<float, true>(a, stream) : launch_n<float, false>(a, stream);
}

}  // namespace ssm
