// SSD (Mamba-2 scalar-decay) chunked forward for gfx950.
//
// Per (batch b, head h), with scalar decay a_t = exp(dt_t * A_h), the state
// S (P x N) evolves as S_t = a_t S_{t-1} + dt_t X_t B_t^T and Y_t = S_t C_t
// (plus skip and gate).  Section 3 of "Mamba & Mamba-2 Architecture" gives
// the same map as a masked product Y = (M o (C B^T)) X with the
// 1-semiseparable M[t,s] = prod_{k=s+1..t} a_k; the kernel uses that form
// inside a chunk of Q tokens and the carried state across chunks:
//   Y_off[t]  = exp(cum_t) * C_t S_prev^T                 (MFMA, K = N)
//   Y_diag[t] = sum_{s<=t} (C_t . B_s) exp(cum_t - cum_s) dt_s X_s   (MFMA, K = N then K = Q)
//   S_new     = exp(cum_Q) S_prev + sum_s exp(cum_Q - cum_s) dt_s X_s B_s^T (MFMA, K = Q)
// with cum the in-chunk inclusive sum of dt * A_h (kept in log2 units).
//
// One workgroup of four wavefronts owns one (b, h) for the whole sequence and
// walks its chunks in order, so the P x N state never leaves the chip: it
// sits in fp32 MFMA accumulators (each wavefront owns N/4 columns of it) and
// a bf16 copy in LDS feeds the next chunk's Y_off.  Per chunk the B rows and
// the transposed X (plain and decay-weighted) are staged in LDS; each
// wavefront keeps the C rows of its Q/4 output rows in registers, which serve
// as the A operand of C S^T and, with the same lane layout, as the B operand
// of B C^T.  Matrix products use v_mfma_f32_16x16x32_bf16 (bf16 operands,
// fp32 accumulation); masks, decays, skip and gate are fp32.
//
// Operand lane layout of v_mfma_f32_16x16x32_bf16 (lane l, g = l / 16,
// c = l % 16): A holds row c, k = 8g..8g+7; B holds k = 8g..8g+7 of column c;
// the result holds rows 4g..4g+3 of column c.  Any permutation of k applied
// to both operands gives the same product; the masked-score tiles use that
// to feed the result layout of one product straight into the next.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "device_math.h"
#include "ssm_internal.h"

namespace ssm {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kP = 64;          // head dimension
constexpr int kThreads = 256;   // four wavefronts

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ __bf16 bf(float x) { return static_cast<__bf16>(x); }
__device__ __forceinline__ float f32(__bf16 x) { return static_cast<float>(x); }

template <int Q, int N>
struct SsdLds {
    static constexpr int kBStride = N + 8;       // bf16 elements per B row (16 B pad)
    static constexpr int kXStride = Q + 8;       // bf16 elements per X^T row
    static constexpr int kHStride = N + 8;       // bf16 elements per state row
    alignas(16) float dt[Q];                      // step per token
    alignas(16) float cum[Q];                     // inclusive sum of dt*A*log2(e)
    alignas(16) float part[kThreads / 64];        // per-wavefront scan totals
    alignas(16) __bf16 B[Q * kBStride];           // B rows of the chunk
    alignas(16) __bf16 Xt[kP * kXStride];         // X^T
    alignas(16) __bf16 XWt[kP * kXStride];        // X^T scaled by exp(cum_Q - cum_s) dt_s
    alignas(16) __bf16 H[kP * kHStride];          // state (bf16) for the next Y_off
};

template <int Q, int N, bool HAS_Z>
__global__ __launch_bounds__(kThreads) void ssd_chunk_kernel(SSDArgs p) {
    constexpr int RW = Q / 4;        // output rows per wavefront
    constexpr int TT = RW / 16;      // 16-row tiles per wavefront
    constexpr int KN = N / 32;       // k-steps over N
    constexpr int NW = N / 4;        // state columns per wavefront
    constexpr int NT = NW / 16;      // 16-column state tiles per wavefront
    constexpr int KQ = Q / 32;       // k-steps over the chunk
    using Lds = SsdLds<Q, N>;
    __shared__ Lds sm;

    const int tid = threadIdx.x;
    const int w = tid / 64;
    const int l = tid % 64;
    const int g = l / 16;
    const int c = l % 16;
    const int64_t bh = blockIdx.x;
    const int64_t b = bh / p.H;
    const int64_t h = bh % p.H;
    const int64_t grp = h / (p.H / p.G);
    const int64_t L = p.L;
    const int64_t H = p.H;
    const int64_t G = p.G;

    const uint16_t* X = static_cast<const uint16_t*>(p.X);
    const uint16_t* Dl = static_cast<const uint16_t*>(p.delta);
    const uint16_t* Bg = static_cast<const uint16_t*>(p.Bm);
    const uint16_t* Cg = static_cast<const uint16_t*>(p.Cm);
    const uint16_t* Zg = static_cast<const uint16_t*>(p.z);
    uint16_t* Y = static_cast<uint16_t*>(p.Y);

    const float A2 = p.A[h] * kLog2e;
    const float bias = p.delta_bias ? p.delta_bias[h] : 0.0f;
    const float dsk = p.Dskip ? p.Dskip[h] : 0.0f;
    const bool softplus = (p.flags & SSM_FLAG_DELTA_SOFTPLUS) != 0;

    // ---- state: fp32 accumulators hacc[j][nt] = S[p = 16j + 4g + r][n = (NT*w + nt)*16 + c]
    f32x4 hacc[4][NT];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int pp = 16 * j + 4 * g + r;
                const int nn = (NT * w + nt) * 16 + c;
                hacc[j][nt][r] = p.h0 ? p.h0[(bh * kP + pp) * N + nn] : 0.0f;
            }
        }
    // bf16 copy of the whole state in LDS
    for (int i = tid; i < kP * N; i += kThreads) {
        const int pp = i / N, nn = i % N;
        sm.H[pp * Lds::kHStride + nn] = bf(p.h0 ? p.h0[(bh * kP + pp) * N + nn] : 0.0f);
    }

    const int64_t nchunks = (L + Q - 1) / Q;
    for (int64_t ch = 0; ch < nchunks; ++ch) {
        const int64_t tc = ch * Q;                       // first token of the chunk
        __syncthreads();                                 // previous chunk done with LDS
        // ---- 1. steps and in-chunk cumulative decay (log2 units)
        {
            float a2 = 0.0f, dtv = 0.0f;
            if (tid < Q) {
                const int64_t t = tc + tid;
                if (t < L) {
                    const float x = bf16_bits_to_f32(Dl[(b * L + t) * H + h]) + bias;
                    dtv = softplus ? softplus_f(x) : x;
                    a2 = dtv * A2;
                }
            }
            // inclusive scan within the wavefront, then across wavefronts
            float v = a2;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const float o = __shfl_up(v, off, 64);
                if (l >= off) v += o;
            }
            if (l == 63) sm.part[w] = v;
            __syncthreads();
            float base = 0.0f;
            for (int k = 0; k < w; ++k) base += sm.part[k];
            if (tid < Q) {
                sm.dt[tid] = dtv;
                sm.cum[tid] = base + v;
            }
        }
        __syncthreads();
        const float cumQ = sm.cum[Q - 1];
        // ---- 2. stage B rows, X^T and decay-weighted X^T
        {
            constexpr int kBVec = N / 8;                 // 16-byte pieces per B row
            for (int i = tid; i < Q * kBVec; i += kThreads) {
                const int s = i / kBVec, k8 = i % kBVec;
                const int64_t t = tc + s;
                uint4 v = make_uint4(0, 0, 0, 0);
                if (t < L)
                    v = *reinterpret_cast<const uint4*>(Bg + ((b * L + t) * G + grp) * N + 8 * k8);
                *reinterpret_cast<uint4*>(&sm.B[s * Lds::kBStride + 8 * k8]) = v;
            }
            constexpr int kXVec = kP / 8;
            for (int i = tid; i < Q * kXVec; i += kThreads) {
                const int s = i / kXVec, p8 = i % kXVec;
                const int64_t t = tc + s;
                uint4 v = make_uint4(0, 0, 0, 0);
                if (t < L)
                    v = *reinterpret_cast<const uint4*>(X + ((b * L + t) * H + h) * kP + 8 * p8);
                const float wgt = fast_exp2(cumQ - sm.cum[s]) * sm.dt[s];
                const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int pp = 8 * p8 + 2 * q;
                    const uint16_t lo = (uint16_t)(u[q] & 0xffffu), hi = (uint16_t)(u[q] >> 16);
                    sm.Xt[pp * Lds::kXStride + s] = __builtin_bit_cast(__bf16, lo);
                    sm.Xt[(pp + 1) * Lds::kXStride + s] = __builtin_bit_cast(__bf16, hi);
                    sm.XWt[pp * Lds::kXStride + s] = bf(bf16_bits_to_f32(lo) * wgt);
                    sm.XWt[(pp + 1) * Lds::kXStride + s] = bf(bf16_bits_to_f32(hi) * wgt);
                }
            }
        }
        // ---- 3. C rows of this wavefront's output tiles, A-operand layout
        bf16x8 cop[TT][KN];
#pragma unroll
        for (int i = 0; i < TT; ++i) {
            const int64_t t = tc + w * RW + 16 * i + c;
#pragma unroll
            for (int kk = 0; kk < KN; ++kk) {
                uint4 v = make_uint4(0, 0, 0, 0);
                if (t < L)
                    v = *reinterpret_cast<const uint4*>(Cg + ((b * L + t) * G + grp) * N + 32 * kk + 8 * g);
                cop[i][kk] = __builtin_bit_cast(bf16x8, v);
            }
        }
        __syncthreads();

        // ---- 4. Y_off = exp(cum_t) * C S^T, then Y_diag accumulated on top
        f32x4 yacc[TT][4];
#pragma unroll
        for (int i = 0; i < TT; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) yacc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int kk = 0; kk < KN; ++kk) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                // B operand: S^T[n = 32kk + 8g + e][p = 16j + c] = S[p][n] (bf16 row of the state)
                const bf16x8 hop = *reinterpret_cast<const bf16x8*>(
                    &sm.H[(16 * j + c) * Lds::kHStride + 32 * kk + 8 * g]);
#pragma unroll
                for (int i = 0; i < TT; ++i) yacc[i][j] = mfma(cop[i][kk], hop, yacc[i][j]);
            }
        }
#pragma unroll
        for (int i = 0; i < TT; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float e = fast_exp2(sm.cum[w * RW + 16 * i + 4 * g + r]);
#pragma unroll
                for (int j = 0; j < 4; ++j) yacc[i][j][r] *= e;
            }

#pragma unroll
        for (int i = 0; i < TT; ++i) {
            const int t0 = w * RW + 16 * i;              // first row of the tile (in chunk)
            const int tl = t0 + c;                       // this lane's row in the score tiles
            const float cum_t = sm.cum[tl];
            const int nsb = (t0 + 15) / 32 + 1;          // causal: s-blocks touching s <= t
            for (int sb = 0; sb < nsb; ++sb) {
                // scores S^T[s][t] = B_s . C_t for s in two 16-row halves of the block
                f32x4 st[2];
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    st[hh] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
                    const int s0 = 32 * sb + 16 * hh;
#pragma unroll
                    for (int kk = 0; kk < KN; ++kk) {
                        const bf16x8 bop = *reinterpret_cast<const bf16x8*>(
                            &sm.B[(s0 + c) * Lds::kBStride + 32 * kk + 8 * g]);
                        st[hh] = mfma(bop, cop[i][kk], st[hh]);
                    }
                }
                // mask and scale; k-slot e of this lane is s = 32sb + 16(e/4) + 4g + e%4
                bf16x8 mop;
#pragma unroll
                for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int s = 32 * sb + 16 * hh + 4 * g + r;
                        float m = 0.0f;
                        if (s <= tl) m = st[hh][r] * fast_exp2(cum_t - sm.cum[s]) * sm.dt[s];
                        mop[4 * hh + r] = bf(m);
                    }
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const __bf16* xr = &sm.Xt[(16 * j + c) * Lds::kXStride + 32 * sb + 4 * g];
                    const bf16x4 lo = *reinterpret_cast<const bf16x4*>(xr);
                    const bf16x4 hi = *reinterpret_cast<const bf16x4*>(xr + 16);
                    bf16x8 xop;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        xop[e] = lo[e];
                        xop[4 + e] = hi[e];
                    }
                    yacc[i][j] = mfma(mop, xop, yacc[i][j]);
                }
            }
        }

        // ---- 5. state update on this wavefront's columns
        const float decay = fast_exp2(cumQ);
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) hacc[j][nt] *= decay;
#pragma unroll
        for (int ks = 0; ks < KQ; ++ks) {
            bf16x8 bcol[NT];
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const int nn = (NT * w + nt) * 16 + c;
#pragma unroll
                for (int e = 0; e < 8; ++e) bcol[nt][e] = sm.B[(32 * ks + 8 * g + e) * Lds::kBStride + nn];
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const bf16x8 xw = *reinterpret_cast<const bf16x8*>(
                    &sm.XWt[(16 * j + c) * Lds::kXStride + 32 * ks + 8 * g]);
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) hacc[j][nt] = mfma(xw, bcol[nt], hacc[j][nt]);
            }
        }
        __syncthreads();                                 // all Y_off reads of sm.H done
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    sm.H[(16 * j + 4 * g + r) * Lds::kHStride + (NT * w + nt) * 16 + c] = bf(hacc[j][nt][r]);

        // ---- 6. skip, gate, store Y
#pragma unroll
        for (int i = 0; i < TT; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int tl = w * RW + 16 * i + 4 * g + r;
                const int64_t t = tc + tl;
                if (t >= L) continue;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int pp = 16 * j + c;
                    float yv = yacc[i][j][r] + dsk * f32(sm.Xt[pp * Lds::kXStride + tl]);
                    const int64_t o = ((b * L + t) * H + h) * kP + pp;
                    if constexpr (HAS_Z) yv *= silu_f(bf16_bits_to_f32(Zg[o]));
                    Y[o] = f32_to_bf16_bits(yv);
                }
            }
    }
    if (p.h_last) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int pp = 16 * j + 4 * g + r;
                    const int nn = (NT * w + nt) * 16 + c;
                    p.h_last[(bh * kP + pp) * N + nn] = hacc[j][nt][r];
                }
    }
}

template <int Q, int N>
hipError_t launch_qn(const SSDArgs& a, hipStream_t stream) {
    const dim3 grid((unsigned)(a.B * a.H));
    if (a.z)
        hipLaunchKernelGGL((ssd_chunk_kernel<Q, N, true>), grid, dim3(kThreads), 0, stream, a);
    else
        hipLaunchKernelGGL((ssd_chunk_kernel<Q, N, false>), grid, dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

template <int N>
hipError_t launch_n(const SSDArgs& a, hipStream_t stream) {
    switch (a.chunk) {
        case 64: return launch_qn<64, N>(a, stream);
        case 128: return launch_qn<128, N>(a, stream);
        case 256: return launch_qn<256, N>(a, stream);
        default: return hipErrorNotSupported;
    }
}

}  // namespace

hipError_t launch_ssd(const SSDArgs& a, hipStream_t stream) {
    if (a.P != kP) return hipErrorNotSupported;
    if (a.N == 128) return launch_n<128>(a, stream);
    if (a.N == 64) return launch_n<64>(a, stream);
    return hipErrorNotSupported;
}

}  // namespace ssm
