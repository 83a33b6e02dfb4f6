// Short causal depthwise convolution over tokens followed by SiLU: the
// branch of the Mamba block that produces the scan input u (temporalbook
// "Selective State-Space Models (Mamba)", section 4; width d_conv = 4 in the
// block constructor of section 5).  Per (b, channel d):
//   s_t = bias[d] + sum_{k<K} w[d,k] x_{t-(K-1)+k},   u_t = s_t sigmoid(s_t)
// with x at negative times taken from the carried state (the previous call's
// last K-1 inputs) or zero.
//
// The layout is [B, L, D] with channels contiguous, so a thread owns VEC
// consecutive channels (4 bytes of bf16, 16 of fp32) and streams a run of kRun tokens,
// keeping the last K-1 inputs in registers: x is read once (plus a K-1 token
// halo per run) and u written once -- the kernel is bound by those bytes.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "device_math.h"
#include "ssm_internal.h"

namespace ssm {
namespace {

constexpr int kBlock = 256;
constexpr int kRun = 32;       // tokens per thread
constexpr int kTokensInFlight = 16;   // loads in flight per thread (4-byte vectors)

// x and u are streamed once: nontemporal accesses (48.0 -> 42.5 us at
// B=8 L=2048 D=1536 bf16, against 30 us for a plain device copy of x).  In
// bf16 a thread owns two channels (4-byte accesses): four times the threads
// of one 16-byte vector each, so more loads are in flight per SIMD (with 8
// tokens in flight: 42.6 -> 34.4 us; four channels 36.8 us, one 59 us).
// Loads are held as loaded and widened at use, which leaves the registers
// for 16 tokens in flight per thread: 34.4 -> 25.9 us, 3.88 TB/s (32 tokens
// in flight: the same; 64-token runs: 26.4 us; 8 bf16 channels per thread
// with 16 in flight: 43.4 us).
typedef float f32x4 __attribute__((ext_vector_type(4)));

// VEC channels of one token: loaded as RAW (the stored bits), widened to fp32
// by unpack; store narrows VEC fp32 values back to the element type.
template <typename T, int VEC> struct Vec;
template <> struct Vec<uint16_t, 2> {
    using Raw = uint32_t;
    static __device__ __forceinline__ Raw load(const uint16_t* p) {
        return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
    }
    static __device__ __forceinline__ void unpack(const Raw& r, float (&v)[2]) {
        v[0] = __uint_as_float(r << 16); v[1] = __uint_as_float(r & 0xffff0000u);
    }
    static __device__ __forceinline__ void store(uint16_t* p, const float (&v)[2]) {
        const uint32_t a = (uint32_t)f32_to_bf16_bits(v[0]) | ((uint32_t)f32_to_bf16_bits(v[1]) << 16);
        __builtin_nontemporal_store(a, reinterpret_cast<uint32_t*>(p));
    }
};
template <> struct Vec<float, 4> {
    using Raw = f32x4;
    static __device__ __forceinline__ Raw load(const float* p) {
        return __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
    }
    static __device__ __forceinline__ void unpack(const Raw& r, float (&v)[4]) {
        v[0] = r.x; v[1] = r.y; v[2] = r.z; v[3] = r.w;
    }
    static __device__ __forceinline__ void store(float* p, const float (&v)[4]) {
        __builtin_nontemporal_store((f32x4){v[0], v[1], v[2], v[3]}, reinterpret_cast<f32x4*>(p));
    }
};
template <typename T> struct Vec<T, 1> {
    using Raw = float;
    static __device__ __forceinline__ Raw load(const T* p) { return Elem<T>::load(p, 0); }
    static __device__ __forceinline__ void unpack(const Raw& r, float (&v)[1]) { v[0] = r; }
    static __device__ __forceinline__ void store(T* p, const float (&v)[1]) { Elem<T>::store(p, 0, v[0]); }
};

// one thread per (channel vector, b, run), channel vectors fastest
template <typename T, int VEC, int K, bool SILU>
__global__ __launch_bounds__(kBlock) void conv1d_silu_kernel(ConvArgs p) {
    using V = Vec<T, VEC>;
    // 16 tokens in flight for 4-byte vectors; 16-byte vectors keep 8 (16 of
    // them would halve the wavefronts per SIMD)
    constexpr int kUnroll = VEC * (int)sizeof(T) == 16 ? 8 : kTokensInFlight;
    const int64_t groups = (p.D + VEC - 1) / VEC;
    const int64_t nrun = (p.L + kRun - 1) / kRun;
    const int64_t gi = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (gi >= groups * p.B * nrun) return;
    const int64_t d0 = (gi % groups) * VEC;
    const int64_t br = gi / groups;
    const int64_t b = br / nrun, run = br % nrun;
    const int64_t t0 = run * kRun;
    const T* x = static_cast<const T*>(p.x) + b * p.L * p.D + d0;
    T* u = static_cast<T*>(p.u) + b * p.L * p.D + d0;

    float w[VEC][K], bias[VEC];
#pragma unroll
    for (int c = 0; c < VEC; ++c) {
#pragma unroll
        for (int k = 0; k < K; ++k) w[c][k] = p.weight[(d0 + c) * K + k];
        bias[c] = p.bias ? p.bias[d0 + c] : 0.0f;
    }
    // window[i] = x_{t-(K-1)+i} for the next output t; i = K-1 is filled per token
    float win[K][VEC];
#pragma unroll
    for (int i = 0; i < K - 1; ++i) {
        const int64_t t = t0 - (K - 1) + i;
        if (t >= 0) {
            V::unpack(V::load(x + t * p.D), win[i]);
        } else {
#pragma unroll
            for (int c = 0; c < VEC; ++c)
                win[i][c] = p.state_in ? p.state_in[((b * p.D) + d0 + c) * (K - 1) + (t + K - 1)] : 0.0f;
        }
    }
    const int64_t tend = t0 + kRun < p.L ? t0 + kRun : p.L;
    for (int64_t tb = t0; tb < tend; tb += kUnroll) {
        typename V::Raw xs[kUnroll];
#pragma unroll
        for (int j = 0; j < kUnroll; ++j)
            if (tb + j < tend) xs[j] = V::load(x + (tb + j) * p.D);
#pragma unroll
        for (int j = 0; j < kUnroll; ++j) {
            if (tb + j >= tend) break;
            V::unpack(xs[j], win[K - 1]);
            float o[VEC];
#pragma unroll
            for (int c = 0; c < VEC; ++c) {
                float s = bias[c];
#pragma unroll
                for (int k = 0; k < K; ++k) s = fmaf(w[c][k], win[k][c], s);
                o[c] = SILU ? silu_f(s) : s;
            }
            V::store(u + (tb + j) * p.D, o);
#pragma unroll
            for (int i = 0; i < K - 1; ++i)
#pragma unroll
                for (int c = 0; c < VEC; ++c) win[i][c] = win[i + 1][c];
        }
    }
    // the last run leaves the final K-1 inputs in the window
    if (p.state_out && run == nrun - 1) {
#pragma unroll
        for (int i = 0; i < K - 1; ++i)
#pragma unroll
            for (int c = 0; c < VEC; ++c)
                p.state_out[((b * p.D) + d0 + c) * (K - 1) + i] = win[i][c];
    }
}

template <typename T, int VEC, int K>
hipError_t launch_k(const ConvArgs& a, hipStream_t stream) {
    const int64_t groups = (a.D + VEC - 1) / VEC;
    const int64_t nrun = (a.L + kRun - 1) / kRun;
    const unsigned grid = (unsigned)((groups * a.B * nrun + kBlock - 1) / kBlock);
    if (a.silu) conv1d_silu_kernel<T, VEC, K, true><<<grid, kBlock, 0, stream>>>(a);
    else conv1d_silu_kernel<T, VEC, K, false><<<grid, kBlock, 0, stream>>>(a);
    return hipGetLastError();
}

template <typename T, int VEC>
hipError_t launch_v(const ConvArgs& a, hipStream_t stream) {
    switch (a.K) {
        case 1: return launch_k<T, VEC, 1>(a, stream);
        case 2: return launch_k<T, VEC, 2>(a, stream);
        case 3: return launch_k<T, VEC, 3>(a, stream);
        default: return launch_k<T, VEC, 4>(a, stream);
    }
}

// no tokens: the carried state passes through unchanged (zeros without one)
__global__ __launch_bounds__(kBlock) void conv_state_pass(ConvArgs p) {
    const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (i < p.B * p.D * (p.K - 1)) p.state_out[i] = p.state_in ? p.state_in[i] : 0.0f;
}

}  // namespace

hipError_t launch_conv1d(const ConvArgs& a, hipStream_t stream) {
    if (a.L == 0) {
        const int64_t n = a.B * a.D * (a.K - 1);
        if (a.state_out && n > 0)
            conv_state_pass<<<(unsigned)((n + kBlock - 1) / kBlock), kBlock, 0, stream>>>(a);
        return hipGetLastError();
    }
    if (a.bf16) {
        if (a.D % 2 == 0) return launch_v<uint16_t, 2>(a, stream);
        return launch_v<uint16_t, 1>(a, stream);
    }
    if (a.D % 4 == 0) return launch_v<float, 4>(a, stream);
    return launch_v<float, 1>(a, stream);
}

}  // namespace ssm
