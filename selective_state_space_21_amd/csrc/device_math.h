// Small device helpers for gfx950: storage conversions and the scalar
// nonlinearities of the selective scan, built on the hardware exp2/log2/rcp.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssm {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// bf16 <-> fp32.  Widening is exact (bf16 is the top half of an fp32);
// narrowing rounds to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}

template <typename T> struct Elem;
template <> struct Elem<float> {
    using storage = float;
    static __device__ __forceinline__ float load(const storage* p, int64_t i) { return p[i]; }
    static __device__ __forceinline__ void store(storage* p, int64_t i, float v) { p[i] = v; }
};
template <> struct Elem<uint16_t> {   // bf16 held as raw bits
    using storage = uint16_t;
    static __device__ __forceinline__ float load(const storage* p, int64_t i) {
        return bf16_bits_to_f32(p[i]);
    }
    static __device__ __forceinline__ void store(storage* p, int64_t i, float v) {
        p[i] = f32_to_bf16_bits(v);
    }
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// log(1 + e^x) = max(x, 0) + log1p(e^-|x|), with the accurate library
// log1p so that small steps keep full relative precision.
__device__ __forceinline__ float softplus_f(float x) {
    return fmaxf(x, 0.0f) + log1pf(fast_exp2(-fabsf(x) * kLog2e));
}

// z * sigma(z).  For z < -88 the exponential is +inf and the result -0.
__device__ __forceinline__ float silu_f(float z) {
    return z * fast_rcp(1.0f + fast_exp2(-z * kLog2e));
}

}  // namespace ssm
