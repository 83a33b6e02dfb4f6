// Single-token state update of the selective scan (decode).
//
// Autoregressive generation runs the plain recurrence one token at a time
// against a resident state of D x N numbers per sequence; there is nothing to
// scan (Transformer-math "Selective state space" article, section "What it
// costs at inference, and on a CPU").  Per (b, d):
//   dt = softplus(x_dt + bias);  h[n] = exp(dt A[d,n]) h[n] + dt B[b,n] u;
//   y  = sum_n C[b,n] h[n] + D u;  y *= silu(z)
// The state is read and written once; the call is bound by those bytes.
//
// Mapping: for N in {4, 8, 16, 32, 64} a channel is handled by GL = N / 4
// consecutive lanes, each holding one float4 of the state, of A, B and C, so
// every state access is a contiguous 16-byte piece and a wavefront covers
// 64 / GL channels; the readout sum over n closes with log2(GL) xor-shuffles.
// Other N <= 64 use one lane per channel.  The per-state arithmetic is that
// of the scan kernels (dA = exp2(dt * A log2 e), input term B * dt u, then
// skip, then gate); the readout sum is associated per 4 states and then
// pairwise across the channel's lanes.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "device_math.h"
#include "ssm_internal.h"

namespace ssm {
namespace {

constexpr int kBlock = 256;
typedef float f32x4 __attribute__((ext_vector_type(4)));

// load 4 consecutive storage elements as fp32
template <typename T> struct Quad;
template <> struct Quad<float> {
    static __device__ __forceinline__ float4 load(const float* p) {
        return *reinterpret_cast<const float4*>(p);
    }
};
template <> struct Quad<uint16_t> {
    static __device__ __forceinline__ float4 load(const uint16_t* p) {
        const uint2 v = *reinterpret_cast<const uint2*>(p);
        return make_float4(__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xffff0000u),
                           __uint_as_float(v.y << 16), __uint_as_float(v.y & 0xffff0000u));
    }
};

// Items (channel, group of 4 states) per thread: all their loads are issued
// before any of them is computed, so a thread keeps kItems 16-byte state
// loads in flight; item r of a thread is r grid strides past its first, so
// each load instruction of a wavefront still covers contiguous bytes.
constexpr int kItems = 4;

template <typename T, int GL, bool ZOH>
__global__ __launch_bounds__(kBlock) void s6_step_vec(StepArgs p) {
    constexpr int N = 4 * GL;
    const int64_t nitems = p.B * p.D * GL;
    const int64_t stride = (int64_t)gridDim.x * kBlock;
    const int64_t first = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    const T* xs = static_cast<const T*>(p.u);
    const T* dts = static_cast<const T*>(p.delta);
    const T* zs = static_cast<const T*>(p.z);

    struct Item {
        int64_t ch;                 // flattened (b, d); an in-range address for idle items
        int q;                      // which 4 states
        bool valid;
        f32x4 h;
        float4 a, bv, cv;
        float u, dtr, bias, zval, dskv;
    } it[kItems];
#pragma unroll
    for (int r = 0; r < kItems; ++r) {
        const int64_t item = first + r * stride;
        it[r].valid = item < nitems;
        const int64_t ic = it[r].valid ? item : 0;
        it[r].ch = ic / GL;
        it[r].q = (int)(ic % GL);
        const int64_t b = it[r].ch / p.D, d = it[r].ch % p.D;
        it[r].u = Elem<T>::load(xs, it[r].ch);
        it[r].dtr = Elem<T>::load(dts, it[r].ch);
        it[r].bias = p.delta_bias ? p.delta_bias[d] : 0.0f;
        // the gate and skip are loaded with everything else, not after the sum
        it[r].zval = zs ? Elem<T>::load(zs, it[r].ch) : 0.0f;
        it[r].dskv = p.Dskip ? p.Dskip[d] : 0.0f;
        // The state is touched once per call: nontemporal accesses keep it
        // from displacing other data in the caches (18.4 -> 16.3 us for 64
        // sequences of a D=5120, N=16 layer; 15.3 us with the gate and skip
        // loads hoisted).
        it[r].h = __builtin_nontemporal_load(
            reinterpret_cast<const f32x4*>(p.state + it[r].ch * N + 4 * it[r].q));
        it[r].a = *reinterpret_cast<const float4*>(p.A + d * N + 4 * it[r].q);
        it[r].bv = Quad<T>::load(static_cast<const T*>(p.Bm) + b * N + 4 * it[r].q);
        it[r].cv = Quad<T>::load(static_cast<const T*>(p.Cm) + b * N + 4 * it[r].q);
    }
#pragma unroll
    for (int r = 0; r < kItems; ++r) {
        const float dt = step_dt(it[r].dtr, it[r].bias, p.flags);
        const float dtu = dt * it[r].u;
        const float av[4] = {it[r].a.x, it[r].a.y, it[r].a.z, it[r].a.w};
        const float bb[4] = {it[r].bv.x, it[r].bv.y, it[r].bv.z, it[r].bv.w};
        const float cc[4] = {it[r].cv.x, it[r].cv.y, it[r].cv.z, it[r].cv.w};
        float hh[4] = {it[r].h.x, it[r].h.y, it[r].h.z, it[r].h.w};
        float acc = 0.0f;
#pragma unroll
        for (int n = 0; n < 4; ++n) {
            const float dA = fast_exp2(dt * (av[n] * kLog2e));
            const float w = ZOH ? dtu * bb[n] * zoh_factor(dt * av[n]) : bb[n] * dtu;
            hh[n] = fmaf(dA, hh[n], w);
            acc = fmaf(cc[n], hh[n], acc);
        }
        // the partial sums of a channel's GL lanes, combined pairwise (every
        // lane takes part, idle items included)
#pragma unroll
        for (int off = 1; off < GL; off <<= 1) acc += __shfl_xor(acc, off, 64);
        if (!it[r].valid) continue;
        __builtin_nontemporal_store((f32x4){hh[0], hh[1], hh[2], hh[3]},
                                    reinterpret_cast<f32x4*>(p.state + it[r].ch * N + 4 * it[r].q));
        if (it[r].q == 0) {
            acc = fmaf(it[r].dskv, it[r].u, acc);
            if (zs) acc *= silu_f(it[r].zval);
            Elem<T>::store(static_cast<T*>(p.y), it[r].ch, acc);
        }
    }
}

template <typename T, bool ZOH>
__global__ __launch_bounds__(kBlock) void s6_step_any(StepArgs p) {
    const int64_t ch = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (ch >= p.B * p.D) return;
    const int64_t b = ch / p.D, d = ch % p.D;
    const int N = (int)p.N;
    const T* xs = static_cast<const T*>(p.u);
    const T* zs = static_cast<const T*>(p.z);
    const float u = Elem<T>::load(xs, ch);
    const float dt = step_dt(Elem<T>::load(static_cast<const T*>(p.delta), ch),
                             p.delta_bias ? p.delta_bias[d] : 0.0f, p.flags);
    const float dtu = dt * u;
    const T* Bm = static_cast<const T*>(p.Bm) + b * N;
    const T* Cm = static_cast<const T*>(p.Cm) + b * N;
    float* st = p.state + ch * N;
    float acc = 0.0f;
    for (int n = 0; n < N; ++n) {
        const float an = p.A[d * N + n];
        const float bn = Elem<T>::load(Bm, n);
        const float dA = fast_exp2(dt * (an * kLog2e));
        const float w = ZOH ? dtu * bn * zoh_factor(dt * an) : bn * dtu;
        const float hn = fmaf(dA, __builtin_nontemporal_load(st + n), w);
        __builtin_nontemporal_store(hn, st + n);
        acc = fmaf(Elem<T>::load(Cm, n), hn, acc);
    }
    if (p.Dskip) acc = fmaf(p.Dskip[d], u, acc);
    if (zs) acc *= silu_f(Elem<T>::load(zs, ch));
    Elem<T>::store(static_cast<T*>(p.y), ch, acc);
}

template <typename T, bool ZOH>
hipError_t launch_t(const StepArgs& a, hipStream_t stream) {
    const int64_t chans = a.B * a.D;
    auto blocks = [](int64_t lanes) { return (unsigned)((lanes + kBlock - 1) / kBlock); };
    // kItems items per thread on the vector path
    auto vblocks = [](int64_t items) {
        return (unsigned)((items + (int64_t)kBlock * kItems - 1) / ((int64_t)kBlock * kItems));
    };
    switch (a.N) {
        case 4: s6_step_vec<T, 1, ZOH><<<vblocks(chans), kBlock, 0, stream>>>(a); break;
        case 8: s6_step_vec<T, 2, ZOH><<<vblocks(chans * 2), kBlock, 0, stream>>>(a); break;
        case 16: s6_step_vec<T, 4, ZOH><<<vblocks(chans * 4), kBlock, 0, stream>>>(a); break;
        case 32: s6_step_vec<T, 8, ZOH><<<vblocks(chans * 8), kBlock, 0, stream>>>(a); break;
        case 64: s6_step_vec<T, 16, ZOH><<<vblocks(chans * 16), kBlock, 0, stream>>>(a); break;
        default: s6_step_any<T, ZOH><<<blocks(chans), kBlock, 0, stream>>>(a); break;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_s6_step(const StepArgs& a, hipStream_t stream) {
    const bool zoh = (a.flags & SSM_FLAG_ZOH) != 0;
    if (a.bf16) return zoh ? launch_t<uint16_t, true>(a, stream) : launch_t<uint16_t, false>(a, stream);
    return zoh ? launch_t<float, true>(a, stream) : launch_t<float, false>(a, stream);
}

}  // namespace ssm
