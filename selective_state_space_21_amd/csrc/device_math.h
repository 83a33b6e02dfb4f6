// Small device helpers for gfx950: storage conversions and the scalar
// nonlinearities of the selective scan, built on the hardware exp2/log2/rcp.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ssm.h"

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

// log1p(e) for e in [0, 1]: with w = 1 + e rounded to fp32, the rounding
// error c = e - (w - 1) is exact (Fast2Sum), and log1p(e) = log(w) + c / w to
// first order in c.  The correction is taken as c rather than c / w: |c| is at
// most half an ulp of w, so the difference, c e / w, stays below 2^-25 e,
// about a quarter ulp of the result (which is at least e / 2).  v_log_f32
// gives log2(w) to about one ulp, so the result keeps full relative precision
// even for tiny e (then w = 1, c = e).
__device__ __forceinline__ float log1p_unit(float e) {
    const float w = 1.0f + e;
    const float c = e - (w - 1.0f);
    return fmaf(fast_log2(w), kLn2, c);
}

// log(1 + e^x) = max(x, 0) + log1p(e^-|x|).
__device__ __forceinline__ float softplus_f(float x) {
    return fmaxf(x, 0.0f) + log1p_unit(fast_exp2(-fabsf(x) * kLog2e));
}

// z * sigma(z).  For z < -88 the exponential is +inf and the result -0.
__device__ __forceinline__ float silu_f(float z) {
    return z * fast_rcp(1.0f + fast_exp2(-z * kLog2e));
}

// (e^x - 1) / x, the exact zero-order-hold input factor for x = dt * A;
// its limit 1 at x = 0.
__device__ __forceinline__ float zoh_factor(float x) {
    return x != 0.0f ? expm1f(x) / x : 1.0f;
}

// The step size of one token: softplus(raw + bias) when the flag is set.
__device__ __forceinline__ float step_dt(float raw, float bias, unsigned flags) {
    const float x = raw + bias;
    return (flags & SSM_FLAG_DELTA_SOFTPLUS) ? softplus_f(x) : x;
}

// Buffer resources (gfx9 V#): loads through a resource take a per-lane byte
// offset in a VGPR and a uniform byte offset in an SGPR, so a token-row access
// costs no vector address arithmetic; accesses past num_records read as zero
// and stores there are dropped.
constexpr int kBufferConfig = 0x00020000;   // raw, untyped buffer (gfx9 family)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             kBufferConfig);
}

template <typename T> struct Buf;
template <> struct Buf<float> {
    static __device__ __forceinline__ float load(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                                 uint32_t soff) {
        return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, (int)soff, 0));
    }
    static __device__ __forceinline__ void store(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                                 uint32_t soff, float v) {
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, (int)voff, (int)soff, 0);
    }
};
template <> struct Buf<uint16_t> {
    static __device__ __forceinline__ float load(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                                 uint32_t soff) {
        return bf16_bits_to_f32(__builtin_amdgcn_raw_buffer_load_b16(r, (int)voff, (int)soff, 0));
    }
    static __device__ __forceinline__ void store(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                                 uint32_t soff, float v) {
        __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16_bits(v), r, (int)voff, (int)soff, 0);
    }
};

}  // namespace ssm
