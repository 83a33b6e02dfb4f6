// Issue-rate probes for gfx950 behind the compute-bound view of the selective
// scan: fp32 FMA issue, v_exp_f32 issue, the per-state-element update of the
// selective scan (decay exponential, input term, state FMA, readout FMA; the
// discretised recurrence of "12. Selective State Space", section on
// discretisation) with and without the exponential, at 1..8 wavefronts per
// SIMD, and a streaming copy for the HBM side.
//
//   python -m selective_state_space_21_amd.microbench
//
// Every kernel writes one float per lane to a buffer sized for the largest
// grid launched (8192 blocks x 64 lanes); the copy kernel is grid-strided
// over two equal buffers.
#include <hip/hip_runtime.h>
#include <stdio.h>

#define CK(x)                                                                        \
    do {                                                                             \
        hipError_t err_ = (x);                                                       \
        if (err_ != hipSuccess) {                                                    \
            printf("HIP error %s at line %d\n", hipGetErrorString(err_), __LINE__);  \
            return 1;                                                                \
        }                                                                            \
    } while (0)

namespace {

constexpr int kMaxBlocks = 8192;   // 8 waves per SIMD on 256 CUs x 4 SIMDs

__global__ void fma_rate(float* out, int iters) {
    float a[8];
    const float m = 0.999f + threadIdx.x * 1e-7f, c = 1e-3f;
    for (int k = 0; k < 8; ++k) a[k] = threadIdx.x + k;
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int k = 0; k < 8; ++k) a[k] = fmaf(a[k], m, c);
    }
    float s = 0.0f;
    for (int k = 0; k < 8; ++k) s += a[k];
    out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

__global__ void exp_rate(float* out, int iters) {
    float a[8];
    const float m = -0.01f - threadIdx.x * 1e-7f;
    for (int k = 0; k < 8; ++k) a[k] = 0.5f + k * 0.01f;
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int k = 0; k < 8; ++k) a[k] = __builtin_amdgcn_exp2f(a[k] * m);
    }
    float s = 0.0f;
    for (int k = 0; k < 8; ++k) s += a[k];
    out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// one lane = one channel with NS states in registers
template <int NS, bool EXP>
__global__ void state_update_rate(float* out, int iters, const float* bc) {
    float a2[NS], h[NS], bv[NS], cv[NS];
    for (int n = 0; n < NS; ++n) {
        a2[n] = -(n + 1) * 1.4427f;
        h[n] = 0.0f;
        bv[n] = bc[n];
        cv[n] = bc[NS + n];
    }
    float dt = 0.05f + threadIdx.x * 1e-6f, dtu = 0.01f, acc = 0.0f;
#pragma unroll 2
    for (int i = 0; i < iters; ++i) {
        dt = fmaf(dt, 0.99999f, 1e-7f);
        dtu = fmaf(dtu, -0.9999f, 1e-5f);
        float y = 0.0f;
#pragma unroll
        for (int n = 0; n < NS; ++n) {
            const float x = dt * a2[n];
            const float e = EXP ? __builtin_amdgcn_exp2f(x) : (x + 1.0f);
            h[n] = fmaf(e, h[n], dtu * bv[n]);
            y = fmaf(cv[n], h[n], y);
        }
        acc += y;
    }
    out[blockIdx.x * blockDim.x + threadIdx.x] = acc + h[0];
}

__global__ void copy_rate(const float4* __restrict__ in, float4* __restrict__ out, size_t n) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) out[i] = in[i];
}

}  // namespace

int main() {
    float* out;
    float* bc;
    CK(hipMalloc(&out, (size_t)kMaxBlocks * 64 * sizeof(float)));
    CK(hipMalloc(&bc, 64 * sizeof(float)));
    float hb[64];
    for (int i = 0; i < 64; ++i) hb[i] = 0.5f + 0.01f * i;
    CK(hipMemcpy(bc, hb, sizeof(hb), hipMemcpyHostToDevice));
    hipEvent_t t0, t1;
    CK(hipEventCreate(&t0));
    CK(hipEventCreate(&t1));
    hipDeviceProp_t prop;
    CK(hipGetDeviceProperties(&prop, 0));
    printf("device %s, %d CUs, clock %d MHz\n", prop.gcnArchName, prop.multiProcessorCount,
           prop.clockRate / 1000);
    const int iters = 4096;
    float ms;
    for (int w : {1, 2, 4, 8}) {
        const int blocks = prop.multiProcessorCount * 4 * w;   // 64-lane blocks: w waves per SIMD
        if (blocks > kMaxBlocks) return 1;
        fma_rate<<<blocks, 64>>>(out, 16);
        CK(hipDeviceSynchronize());
        const double lane_ops = (double)blocks * 64 * iters * 8;
        CK(hipEventRecord(t0));
        fma_rate<<<blocks, 64>>>(out, iters);
        CK(hipEventRecord(t1));
        CK(hipEventSynchronize(t1));
        CK(hipEventElapsedTime(&ms, t0, t1));
        printf("waves/SIMD %d  fp32 FMA            %6.2f T lane-instr/s\n", w, lane_ops / ms / 1e9);
        CK(hipEventRecord(t0));
        exp_rate<<<blocks, 64>>>(out, iters);
        CK(hipEventRecord(t1));
        CK(hipEventSynchronize(t1));
        CK(hipEventElapsedTime(&ms, t0, t1));
        printf("waves/SIMD %d  v_exp_f32 (+1 mul)  %6.2f T exp/s\n", w, lane_ops / ms / 1e9);
        const double elems = (double)blocks * 64 * (iters / 4) * 16;
        CK(hipEventRecord(t0));
        state_update_rate<16, true><<<blocks, 64>>>(out, iters / 4, bc);
        CK(hipEventRecord(t1));
        CK(hipEventSynchronize(t1));
        CK(hipEventElapsedTime(&ms, t0, t1));
        printf("waves/SIMD %d  state update, exp   %6.2f T elem/s\n", w, elems / ms / 1e9);
        CK(hipEventRecord(t0));
        state_update_rate<16, false><<<blocks, 64>>>(out, iters / 4, bc);
        CK(hipEventRecord(t1));
        CK(hipEventSynchronize(t1));
        CK(hipEventElapsedTime(&ms, t0, t1));
        printf("waves/SIMD %d  state update, no exp%6.2f T elem/s\n", w, elems / ms / 1e9);
    }
    const size_t bytes = (size_t)1 << 30, n = bytes / 16;
    float4 *a, *b;
    CK(hipMalloc(&a, bytes));
    CK(hipMalloc(&b, bytes));
    CK(hipMemset(a, 0, bytes));
    CK(hipMemset(b, 0, bytes));
    for (int blocks : {2048, 8192, 32768}) {
        for (int r = 0; r < 2; ++r) {
            CK(hipEventRecord(t0));
            copy_rate<<<blocks, 256>>>(a, b, n);
            CK(hipEventRecord(t1));
            CK(hipEventSynchronize(t1));
            CK(hipEventElapsedTime(&ms, t0, t1));
            if (r == 1) printf("copy 1 GiB, %5d blocks        %6.0f GB/s (read + write)\n", blocks,
                               2.0 * bytes / ms / 1e6);
        }
    }
    CK(hipFree(a));
    CK(hipFree(b));
    CK(hipFree(out));
    CK(hipFree(bc));
    return 0;
}
