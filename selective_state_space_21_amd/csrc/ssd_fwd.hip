// SSD (Mamba-2 scalar-decay) chunked forward for gfx950.
//
// Per (batch b, head h), with scalar decay a_t = exp(dt_t * A_h), the state
// S (P x N) evolves as S_t = a_t S_{t-1} + dt_t X_t B_t^T and Y_t = S_t C_t
// (plus skip and gate).  Section 3 of "Mamba & Mamba-2 Architecture" gives
// the same map as a masked product Y = (M o (C B^T)) X with the
// 1-semiseparable M[t,s] = prod_{k=s+1..t} a_k; the kernel uses that form
// inside a chunk of Q tokens and the carried state across chunks.  With cum
// the in-chunk inclusive sum of dt * A_h (kept in log2 units), the kernel
// computes the transposed output tile Y^T (P x Q):
//   Y_off^T[p][t]  = exp(cum_t) * sum_n S[p][n] C[t][n]              (K = N)
//   Y_diag^T[p][t] = sum_s X[s][p] M^T[s][t],
//       M^T[s][t]  = (B_s . C_t) exp(cum_t - cum_s) dt_s for s <= t   (K = N, then K = Q)
//   S_new[p][n]    = exp(cum_Q) S[p][n] + sum_s X[s][p] w_s B[s][n],
//       w_s        = exp(cum_Q - cum_s) dt_s                         (K = Q)
//
// Work mapping: one workgroup of eight wavefronts owns one (b, h) -- or, for a
// head dimension P above 64, one slice of PT = 64 (or 32) head-dim rows of it
// -- for the whole sequence and walks its chunks in order, so its PT x N part
// of the state never leaves the chip: it sits in fp32 MFMA accumulators (each
// wavefront owns 16 state columns) with a bf16 copy in LDS for the next
// chunk's Y_off.  Slices of one head repeat the head's score products.  The next
// chunk's B, X, C and delta are fetched into registers while the current one
// is computed; barriers wait on LDS only, so those loads stay in flight.  Per
// chunk, B rows and X^T are staged in LDS and each wavefront keeps the C rows
// of its output columns in registers (the B operand of both S C^T and B C^T).
// The state update scales its B operand (8 consecutive tokens of one state
// column) by the tokens' weights w_s in registers, so no scaled copy of X^T
// is staged.
// Output tiles are paired first-with-last so every wavefront does the same
// share of the causal work.  Products use v_mfma_f32_16x16x32_bf16 (bf16
// operands, fp32 accumulation); masks, decays, skip and gate are fp32.
//
// Lane layout of v_mfma_f32_16x16x32_bf16 (lane l, g = l / 16, c = l % 16):
// A holds row c, k = 8g..8g+7; B holds k = 8g..8g+7 of column c; the result
// holds rows 4g..4g+3 of column c.  Applying one permutation of k to both
// operands leaves the product unchanged; the score tiles use that to pass a
// result straight on as the next product's B operand.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <type_traits>

#include "device_math.h"
#include "lane_ops.h"
#include "ssm_internal.h"

namespace ssm {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ __bf16 bf(float x) { return static_cast<__bf16>(x); }
__device__ __forceinline__ float f32(__bf16 x) { return static_cast<float>(x); }

// lds_barrier() (lane_ops.h) waits for this wavefront's LDS traffic only:
// global loads issued before it (the next chunk's prefetch) stay in flight.

template <int Q, int N, int PT>
struct SsdLds {
    static constexpr int kBStride = N + 16;      // bf16 per B row (32-byte pad: ~1% faster than 16)
    static constexpr int kXStride = Q + 8;       // bf16 per X^T row
    // X^T rows are swizzled by 32-token blocks: element (p, s) sits in column
    // s ^ 32 * ((p / 16) % KX).  The staging writes put eight rows 8 apart in
    // one instruction; unswizzled those rows start on two LDS banks only (a
    // 4-way conflict), swizzled they spread over four.  The product reads take
    // 32-token blocks of one row range, which the swizzle only renumbers.
    static constexpr int KX = Q / 32 < 4 ? Q / 32 : 4;
    static __device__ __forceinline__ int xcol(int p, int s) { return s ^ (32 * ((p / 16) % KX)); }
    static constexpr int kHStride = N + 8;       // bf16 per state row
    alignas(16) float dt[Q];                      // step per token
    alignas(16) float cum[Q];                     // inclusive sum of dt*A*log2(e)
    alignas(16) float fblk[Q];                    // exp(cum_{32 floor(s/32)} - cum_s) * dt_s
    alignas(16) float part[Q / 64];               // scan totals of the wavefronts holding tokens
    alignas(16) int wide[Q / 64];                 // per such wavefront: a 32-token block spans > 2^64
    alignas(16) __bf16 B[Q * kBStride];           // B rows of the chunk
    alignas(16) __bf16 Xt[PT * kXStride];         // X^T of the chunk (this workgroup's rows)
    alignas(16) float wst[Q];                     // exp(cum_Q - cum_s) dt_s: token s's weight in the final state
    alignas(16) __bf16 H[PT * kHStride];          // state (bf16) for Y_off
};

template <int Q, int N, int PT>
struct Tiles {
    static constexpr int T = Q / 16;                           // output column tiles
    static constexpr int TPW = T >= 2 * kWaves ? 2 : 1;        // tiles per wavefront
    static constexpr int NTILE = N / 16;                       // state column tiles
    static constexpr int KN = N / 32;
    static constexpr int KQ = Q / 32;
    static constexpr int JP = PT / 16;                         // head-dim row tiles
    static constexpr int BPIECES = Q * N / 8;                  // 16-B pieces of a chunk's B rows
    static constexpr int BPIECE = (BPIECES + kThreads - 1) / kThreads;   // per thread
    // state update: wavefront w owns state column tile w % NTILE and JW of
    // the JP head-dim row tiles (group w / NTILE); waves past NTILE * WPN idle
    static constexpr int WPN = (kWaves / NTILE < JP) ? kWaves / NTILE : JP;   // wavefronts per column tile
    static constexpr int JW = JP / WPN;
    static constexpr int XGROUP = (Q / 4) * (PT / 8);          // (4 tokens x 8 p) groups
    static constexpr int XPIECE = 4;                           // 16-B rows per group
    // B pieces fetched ahead of the output tiles; the rest after them.  At the
    // largest tile shape all of B is fetched after the tiles (it is mostly an
    // L2 hit, shared by the heads of a batch row): the tiles then have 16 more
    // registers, 338 -> 325 us at Q = 256, N = 128 (all early: 368)
    static constexpr int BEARLY = (Q == 256 && N == 128) ? 0 : BPIECE;
    // k-th output tile of wavefront w (-1: none); pairs first with last
    static __device__ __forceinline__ int tile(int w, int k) {
        if constexpr (T >= 2 * kWaves) return k == 0 ? w : T - 1 - w;
        else return w < T ? w : -1;
    }
};

// 4 tokens x 8 head-dim values (bf16 pairs xs[token][pair]) -> rows 8 p8 .. 8 p8 + 7
// of a transposed [p][s] tile, columns 4 sg .. 4 sg + 3: eight 8-byte writes
template <typename Lds>
__device__ __forceinline__ void stage_xt_rows(__bf16* xt, int sg, int p8, const uint32_t (&xs)[4][4]) {
    constexpr int XSTRIDE = Lds::kXStride;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        u32x2 even, odd;       // values 2m and 2m+1 of the group, tokens 0..3
        even.x = __builtin_amdgcn_perm(xs[1][m], xs[0][m], 0x05040100u);
        even.y = __builtin_amdgcn_perm(xs[3][m], xs[2][m], 0x05040100u);
        odd.x = __builtin_amdgcn_perm(xs[1][m], xs[0][m], 0x07060302u);
        odd.y = __builtin_amdgcn_perm(xs[3][m], xs[2][m], 0x07060302u);
        const int pp = 8 * p8 + 2 * m;                  // pp and pp + 1 share the swizzle
        const int col = Lds::xcol(pp, 4 * sg);
        *reinterpret_cast<u32x2*>(&xt[pp * XSTRIDE + col]) = even;
        *reinterpret_cast<u32x2*>(&xt[(pp + 1) * XSTRIDE + col]) = odd;
    }
}

// two bf16 (round to nearest even) in one dword, a in the low half
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    typedef float f2 __attribute__((ext_vector_type(2)));
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2){a, b}, b2));
}

// ds_read_b64_tr_b16: within each 16-lane group, lane 4q + m receives in
// element j the 16-bit word m of the 8 bytes addressed by lane 4j + q.
__device__ __forceinline__ bf16x4 lds_read_tr16(const __bf16* p) {
    typedef short s4 __attribute__((ext_vector_type(4)));
    const s4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s4*)(p));
    return __builtin_bit_cast(bf16x4, v);
}

template <int Q, int N, int PT, bool HAS_Z>
__global__ __launch_bounds__(kThreads) void ssd_chunk_kernel(SSDArgs p) {
    using TL = Tiles<Q, N, PT>;
    constexpr int TPW = TL::TPW, KN = TL::KN, KQ = TL::KQ, JP = TL::JP, JW = TL::JW;
    using Lds = SsdLds<Q, N, PT>;
    __shared__ Lds sm;
    auto stage_xt = [](__bf16* xt, int sg, int p8, const uint32_t (&xs)[4][4]) {
        stage_xt_rows<Lds>(xt, sg, p8, xs);
    };

    const int tid = threadIdx.x;
    const int w = tid / 64;
    const int l = tid % 64;
    const int g = l / 16;
    const int c = l % 16;
    // Workgroups are dealt to the 8 XCDs round robin (i -> XCD i % 8); renumber
    // them so that each XCD receives a contiguous range of (batch, head, slice)
    // triples.  Heads of one batch row share B and C, so those rows are then
    // fetched into about two of the eight L2 caches instead of all eight.
    const int64_t wg = [] {
        const uint32_t n = gridDim.x, i = blockIdx.x, x = i % 8, q = n / 8, r = n % 8;
        return (int64_t)(x * q + min(x, r) + i / 8);
    }();
    // A head of P > PT values is split over P / PT workgroups, each owning PT
    // consecutive rows of the state (rows of S evolve independently: the
    // decay is one scalar per head and the input term is an outer product).
    const int64_t P = p.P;
    const int64_t nslice = P / PT;
    const int64_t bh = wg / nslice;
    const int64_t pbase = (wg % nslice) * PT;     // first head-dim row of this workgroup
    const int64_t b = bh / p.H;
    const int64_t h = bh % p.H;
    const int64_t grp = h / (p.H / p.G);
    const int64_t L = p.L;
    // tokens of this batch row: all L, or its own length in a variable-length
    // batch (right-padded to L); the row's tensors keep their [L, ...] strides
    const int64_t Lr = p.seq_lens ? min(max((int64_t)p.seq_lens[b], (int64_t)0), L) : L;
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
    // this wavefront's state columns (-1: none) and first head-dim row tile
    const int ntile = w < TL::NTILE * TL::WPN ? (TL::WPN == 1 ? w : w % TL::NTILE) : -1;
    const int jbase = TL::WPN == 1 ? 0 : (w / TL::NTILE) * JW;

    // ---- state: hacc[jj] = S[p = pbase + 16 (jbase + jj) + 4g + r][n = 16 * ntile + c]
    f32x4 hacc[JW];
#pragma unroll
    for (int jj = 0; jj < JW; ++jj)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            hacc[jj][r] = (p.h0 && ntile >= 0)
                              ? p.h0[(bh * P + pbase + 16 * (jbase + jj) + 4 * g + r) * N + 16 * ntile + c]
                              : 0.0f;
    for (int i = tid; i < PT * N; i += kThreads) {
        const int pp = i / N, nn = i % N;
        sm.H[pp * Lds::kHStride + nn] = bf(p.h0 ? p.h0[(bh * P + pbase + pp) * N + nn] : 0.0f);
    }

    // ---- inputs through buffer resources over batch row b's Lr tokens: a
    // read past them (chunk tail, padding) returns zero, so no load is guarded
    static_assert(TL::XGROUP <= kThreads, "one X group per thread at most");
    const auto rX = make_rsrc(X + b * L * H * P, (uint32_t)(Lr * H * P * 2));
    const auto rB = make_rsrc(Bg + b * L * G * N, (uint32_t)(Lr * G * N * 2));
    const auto rC = make_rsrc(Cg + b * L * G * N, (uint32_t)(Lr * G * N * 2));
    const auto rD = make_rsrc(Dl + b * L * H, (uint32_t)(Lr * H * 2));
    uint32_t dbits = 0;                  // step of this thread's token, bf16 bits
    uint4 bpre[TL::BPIECE];
    uint4 xpre[TL::XPIECE];
    // B pieces [k0, k1), X and delta of chunk ch into registers
    auto prefetch_b = [&](int64_t ch, auto k0, auto k1) {
        const uint32_t tc = (uint32_t)(ch * Q);
#pragma unroll
        for (int k = decltype(k0)::value; k < decltype(k1)::value; ++k) {
            const uint32_t i = tid + k * kThreads;
            if (TL::BPIECES % kThreads != 0 && i >= (uint32_t)TL::BPIECES) break;
            const uint32_t s = i / (N / 8), k8 = i % (N / 8);
            bpre[k] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                rB, (int)((((tc + s) * (uint32_t)G + (uint32_t)grp) * N + 8 * k8) * 2), 0, 0));
        }
    };
    auto prefetch = [&](int64_t ch) {
        const uint32_t tc = (uint32_t)(ch * Q);
        // kept as loaded and widened where used: widening here would wait for
        // the load right after issuing it
        dbits = __builtin_amdgcn_raw_buffer_load_b16(
            rD, (int)(((tc + min(tid, Q - 1)) * (uint32_t)H + (uint32_t)h) * 2), 0, 0);
        prefetch_b(ch, std::integral_constant<int, 0>{}, std::integral_constant<int, TL::BEARLY>{});
        {
            // thread -> tokens 4*sg .. 4*sg+3, head-dim values 8*p8 .. 8*p8+7;
            // X is read once, so its loads are nontemporal (cache policy 2).
            // The Y stores stay cached: each 128-byte row of a token is
            // written in four 32-byte pieces, which the L2 merges; as
            // nontemporal stores they doubled the bytes written to HBM.
            const uint32_t sg = min(tid, TL::XGROUP - 1) / (PT / 8), p8 = tid % (PT / 8);
#pragma unroll
            for (int q = 0; q < 4; ++q)
                xpre[q] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                    rX, (int)((((tc + 4 * sg + q) * (uint32_t)H + (uint32_t)h) * (uint32_t)P
                               + (uint32_t)pbase + 8 * p8) * 2),
                    0, 2));
        }
    };
    // C rows of this wavefront's output columns, B-operand layout
    auto load_c = [&](int64_t ch, bf16x8 (&cop)[TPW][KN]) {
        const uint32_t tc = (uint32_t)(ch * Q);
#pragma unroll
        for (int k = 0; k < TPW; ++k) {
            const int ti = TL::tile(w, k);
            const uint32_t t = tc + 16 * (ti < 0 ? 0 : ti) + c;
#pragma unroll
            for (int kk = 0; kk < KN; ++kk)
                cop[k][kk] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
                    rC, (int)(((t * (uint32_t)G + (uint32_t)grp) * N + 32 * kk + 8 * g) * 2), 0, 0));
        }
    };

    const int64_t nchunks = (Lr + Q - 1) / Q;
    if (nchunks > 0) {
        prefetch(0);
        prefetch_b(0, std::integral_constant<int, TL::BEARLY>{},
                   std::integral_constant<int, TL::BPIECE>{});
    }
    for (int64_t ch = 0; ch < nchunks; ++ch) {
        const int64_t tc = ch * Q;
        lds_barrier();                                   // previous chunk done with LDS
        bf16x8 cop[TPW][KN];
        load_c(ch, cop);
        // ---- 1. steps and in-chunk cumulative decay (log2 units)
        float dtv = 0.0f, a2 = 0.0f;
        if (tid < Q && tc + tid < Lr) {             // past the end: no step, no decay
            const float x = bf16_bits_to_f32(dbits) + bias;
            dtv = softplus ? softplus_f(x) : x;
            a2 = dtv * A2;
        }
        float v = a2;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const float o = __shfl_up(v, off, 64);
            if (l >= off) v += o;
        }
        if (l == 63 && w < Q / 64) sm.part[w] = v;
        // ---- 2. stage B rows and X^T; C rows to the operand registers
#pragma unroll
        for (int k = 0; k < TL::BPIECE; ++k) {
            const int i = tid + k * kThreads;
            if (TL::BPIECES % kThreads != 0 && i >= TL::BPIECES) break;
            const int s = i / (N / 8), k8 = i % (N / 8);
            *reinterpret_cast<uint4*>(&sm.B[s * Lds::kBStride + 8 * k8]) = bpre[k];
        }
        if (tid < TL::XGROUP) {
            const int sg = tid / (PT / 8), p8 = tid % (PT / 8);
            uint32_t xs[4][4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                xs[q][0] = xpre[q].x; xs[q][1] = xpre[q].y; xs[q][2] = xpre[q].z; xs[q][3] = xpre[q].w;
            }
            stage_xt(sm.Xt, sg, p8, xs);
        }
        lds_barrier();
        {
            float base = 0.0f;
#pragma unroll
            for (int k = 0; k < Q / 64 - 1; ++k) base += k < w ? sm.part[k] : 0.0f;
            if (tid < Q) {
                sm.dt[tid] = dtv;
                sm.cum[tid] = base + v;
            }
        }
        lds_barrier();
        const float cumQ = sm.cum[Q - 1];
        bool far = false;
        if (tid < Q) {
            const float cs = sm.cum[tid], ds = sm.dt[tid];
            const float rel = sm.cum[tid & ~31] - cs;
            far = fabsf(rel) > 64.0f;
            sm.fblk[tid] = fast_exp2(rel) * ds;
        }
        if (tid < Q) sm.wst[tid] = fast_exp2(cumQ - sm.cum[tid]) * sm.dt[tid];
        far = __any(far);
        if (l == 0 && w < Q / 64) sm.wide[w] = far;
        lds_barrier();
        bool wide = false;
#pragma unroll
        for (int k = 0; k < Q / 64; ++k) wide |= sm.wide[k] != 0;

        // The C rows are waited for here, before the next chunk's inputs are
        // requested: loads complete in order, so a wait for them after the
        // prefetch (which the compiler otherwise places at the second tile)
        // would also wait for the whole prefetch.
#pragma unroll
        for (int k = 0; k < TPW; ++k)
#pragma unroll
            for (int kk = 0; kk < KN; ++kk) asm volatile("" : : "v"(cop[k][kk]));
        // next chunk's inputs travel while this one is computed (past the last
        // chunk the loads read zero: unconditional, so no copy at a branch
        // join waits for them)
        prefetch(ch + 1);

        // ---- 5. skip, gate, store of one output tile: lane writes rows
        // p = 16j + 4g .. +3 (of this workgroup's PT) of token t
        auto store_tile = [&](int ti, const f32x4 (&yacc)[JP]) __attribute__((always_inline)) {
            const int tl = 16 * ti + c;
            const int64_t t = tc + tl;
            if (t >= Lr) return;
#pragma unroll
            for (int j = 0; j < JP; ++j) {
                const int p0 = 16 * j + 4 * g;
                const int64_t o = ((b * L + t) * H + h) * P + pbase + p0;
                float yv[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) yv[r] = yacc[j][r];
                if (p.Dskip) {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        yv[r] += dsk * f32(sm.Xt[(p0 + r) * Lds::kXStride + Lds::xcol(p0 + r, tl)]);
                }
                if constexpr (HAS_Z) {
                    const u32x2 zz = *reinterpret_cast<const u32x2*>(Zg + o);
                    yv[0] *= silu_f(__uint_as_float(zz.x << 16));
                    yv[1] *= silu_f(__uint_as_float(zz.x & 0xffff0000u));
                    yv[2] *= silu_f(__uint_as_float(zz.y << 16));
                    yv[3] *= silu_f(__uint_as_float(zz.y & 0xffff0000u));
                }
                u32x2 out;
                out.x = (uint32_t)f32_to_bf16_bits(yv[0]) | ((uint32_t)f32_to_bf16_bits(yv[1]) << 16);
                out.y = (uint32_t)f32_to_bf16_bits(yv[2]) | ((uint32_t)f32_to_bf16_bits(yv[3]) << 16);
                *reinterpret_cast<u32x2*>(Y + o) = out;
            }
        };

        // ---- 3. output tiles Y^T[p][t]: yacc[j] rows p = 16j + 4g + r, column t = tile*16 + c
        // Mask and scale of the intra-chunk scores by exp(cum_t - cum_s) dt_s.
        // Factored as E_t * fblk[s] with E_t = exp(cum_t - cum_{32 sb}): one
        // exponential per lane and block instead of one per element.  fblk holds
        // up to one 32-token block's decay, so a chunk where that exceeds 2^64
        // takes the per-element form (a separately compiled copy of the loop).
        auto out_tiles = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int k = 0; k < TPW; ++k) {
            const int ti = TL::tile(w, k);
            if (ti < 0) continue;
            f32x4 yacc[JP];
#pragma unroll
            for (int j = 0; j < JP; ++j) yacc[j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            // Y_off^T = S C^T, scaled per column by exp(cum_t)
#pragma unroll
            for (int kk = 0; kk < KN; ++kk)
#pragma unroll
                for (int j = 0; j < JP; ++j) {
                    const bf16x8 hop = *reinterpret_cast<const bf16x8*>(
                        &sm.H[(16 * j + c) * Lds::kHStride + 32 * kk + 8 * g]);
                    yacc[j] = mfma(hop, cop[k][kk], yacc[j]);
                }
            const int tl = 16 * ti + c;                  // this lane's column (token in chunk)
            const float cum_t = sm.cum[tl];
            const float eoff = fast_exp2(cum_t);
#pragma unroll
            for (int j = 0; j < JP; ++j) yacc[j] *= eoff;
            auto diag_blocks = [&](auto wide_tag) __attribute__((always_inline)) {
            constexpr bool kWide = decltype(wide_tag)::value;
            // Y_diag^T over the causal s-blocks of 32 tokens
            const int nsb = (16 * ti + 15) / 32 + 1;
            for (int sb = 0; sb < nsb; ++sb) {
                // scores S^T[s][t] = B_s . C_t, two 16-row halves
                f32x4 st[2];
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    st[hh] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
                    const int s0 = 32 * sb + 16 * hh;
#pragma unroll
                    for (int kk = 0; kk < KN; ++kk) {
                        const bf16x8 bop = *reinterpret_cast<const bf16x8*>(
                            &sm.B[(s0 + c) * Lds::kBStride + 32 * kk + 8 * g]);
                        st[hh] = mfma(bop, cop[k][kk], st[hh]);
                    }
                }
                // k-slot e <-> s = 32sb + 16(e/4) + 4g + e%4
                const bool diag = 32 * sb + 31 > 16 * ti;    // block reaches the tile's first row
                f32x4 fac[2];
                if constexpr (!kWide) {
                    const float et = fast_exp2(cum_t - sm.cum[32 * sb]);
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh)
                        fac[hh] = *reinterpret_cast<const f32x4*>(&sm.fblk[32 * sb + 16 * hh + 4 * g]) * et;
                } else {
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh) {
                        const int sq = 32 * sb + 16 * hh + 4 * g;
                        const f32x4 cs = *reinterpret_cast<const f32x4*>(&sm.cum[sq]);
                        const f32x4 ds = *reinterpret_cast<const f32x4*>(&sm.dt[sq]);
#pragma unroll
                        for (int r = 0; r < 4; ++r) fac[hh][r] = fast_exp2(cum_t - cs[r]) * ds[r];
                    }
                }
                bf16x8 mop;
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const int sq = 32 * sb + 16 * hh + 4 * g;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        float m = st[hh][r] * fac[hh][r];
                        if (diag && sq + r > tl) m = 0.0f;
                        mop[4 * hh + r] = bf(m);
                    }
                }
#pragma unroll
                for (int j = 0; j < JP; ++j) {
                    const __bf16* xr = &sm.Xt[(16 * j + c) * Lds::kXStride + Lds::xcol(16 * j + c, 32 * sb + 4 * g)];
                    const bf16x4 lo = *reinterpret_cast<const bf16x4*>(xr);
                    const bf16x4 hi = *reinterpret_cast<const bf16x4*>(xr + 16);
                    const bf16x8 xop = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                    yacc[j] = mfma(xop, mop, yacc[j]);
                }
            }
            };
            if (wide) diag_blocks(std::true_type{});
            else diag_blocks(std::false_type{});
            store_tile(ti, yacc);
        }
        };
        // Both output tiles of the wavefront at once (two tiles per wavefront:
        // t0 = w and t1 = T - 1 - w).  The state rows of Y_off, and the B rows
        // and X^T blocks of the score blocks below t0's diagonal, are read from
        // LDS once for both tiles.
        auto make_mop = [&](const f32x4 (&st)[2], int sb, int ti, float cum_t, auto wide_tag)
            __attribute__((always_inline)) {
            constexpr bool kWide = decltype(wide_tag)::value;
            const int tl = 16 * ti + c;
            const bool diag = 32 * sb + 31 > 16 * ti;
            f32x4 fac[2];
            if constexpr (!kWide) {
                const float et = fast_exp2(cum_t - sm.cum[32 * sb]);
#pragma unroll
                for (int hh = 0; hh < 2; ++hh)
                    fac[hh] = *reinterpret_cast<const f32x4*>(&sm.fblk[32 * sb + 16 * hh + 4 * g]) * et;
            } else {
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const int sq = 32 * sb + 16 * hh + 4 * g;
                    const f32x4 cs = *reinterpret_cast<const f32x4*>(&sm.cum[sq]);
                    const f32x4 ds = *reinterpret_cast<const f32x4*>(&sm.dt[sq]);
#pragma unroll
                    for (int r = 0; r < 4; ++r) fac[hh][r] = fast_exp2(cum_t - cs[r]) * ds[r];
                }
            }
            bf16x8 mop;
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const int sq = 32 * sb + 16 * hh + 4 * g;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float m = st[hh][r] * fac[hh][r];
                    if (diag && sq + r > tl) m = 0.0f;
                    mop[4 * hh + r] = bf(m);
                }
            }
            return mop;
        };
        auto xop_at = [&](int j, int sb) __attribute__((always_inline)) {
            const __bf16* xr = &sm.Xt[(16 * j + c) * Lds::kXStride + Lds::xcol(16 * j + c, 32 * sb + 4 * g)];
            const bf16x4 lo = *reinterpret_cast<const bf16x4*>(xr);
            const bf16x4 hi = *reinterpret_cast<const bf16x4*>(xr + 16);
            return (bf16x8)__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        };
        auto out_pair = [&]() __attribute__((always_inline)) {
            const int t0 = w, t1 = TL::T - 1 - w;
            f32x4 y0[JP], y1[JP];
#pragma unroll
            for (int j = 0; j < JP; ++j) {
                y0[j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
                y1[j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            }
#pragma unroll
            for (int kk = 0; kk < KN; ++kk)
#pragma unroll
                for (int j = 0; j < JP; ++j) {
                    const bf16x8 hop = *reinterpret_cast<const bf16x8*>(
                        &sm.H[(16 * j + c) * Lds::kHStride + 32 * kk + 8 * g]);
                    y0[j] = mfma(hop, cop[0][kk], y0[j]);
                    y1[j] = mfma(hop, cop[1][kk], y1[j]);
                }
            const float cum0 = sm.cum[16 * t0 + c], cum1 = sm.cum[16 * t1 + c];
            const float e0 = fast_exp2(cum0), e1 = fast_exp2(cum1);
#pragma unroll
            for (int j = 0; j < JP; ++j) {
                y0[j] *= e0;
                y1[j] *= e1;
            }
            const int nsb0 = (16 * t0 + 15) / 32 + 1, nsb1 = (16 * t1 + 15) / 32 + 1;
            auto scores = [&](int sb, int k, f32x4 (&st)[2]) __attribute__((always_inline)) {
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    st[hh] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                    for (int kk = 0; kk < KN; ++kk) {
                        const bf16x8 bop = *reinterpret_cast<const bf16x8*>(
                            &sm.B[(32 * sb + 16 * hh + c) * Lds::kBStride + 32 * kk + 8 * g]);
                        st[hh] = mfma(bop, cop[k][kk], st[hh]);
                    }
                }
            };
            auto blocks = [&](auto wide_tag) __attribute__((always_inline)) {
                for (int sb = 0; sb < nsb0; ++sb) {
                    f32x4 s0[2], s1[2];
                    // Both matrix-product groups of the block run at a raised
                    // wave priority, the mask between them at the normal one:
                    // of the two wavefronts sharing a SIMD, the one that has
                    // reached its products issues them first while the other
                    // works on its mask, so the two drift out of step and the
                    // matrix core sees fewer gaps (0.3371 -> 0.3284 ms at the
                    // Mamba-2 shape, four alternating runs; raising it around
                    // the Y_off products, the second tile's blocks or the
                    // state update as well measured no better)
                    __builtin_amdgcn_s_setprio(1);
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh) {
                        s0[hh] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
                        s1[hh] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                        for (int kk = 0; kk < KN; ++kk) {
                            const bf16x8 bop = *reinterpret_cast<const bf16x8*>(
                                &sm.B[(32 * sb + 16 * hh + c) * Lds::kBStride + 32 * kk + 8 * g]);
                            s0[hh] = mfma(bop, cop[0][kk], s0[hh]);
                            s1[hh] = mfma(bop, cop[1][kk], s1[hh]);
                        }
                    }
                    __builtin_amdgcn_s_setprio(0);
                    const bf16x8 m0 = make_mop(s0, sb, t0, cum0, wide_tag);
                    const bf16x8 m1 = make_mop(s1, sb, t1, cum1, wide_tag);
                    __builtin_amdgcn_s_setprio(1);
#pragma unroll
                    for (int j = 0; j < JP; ++j) {
                        const bf16x8 xop = xop_at(j, sb);
                        y0[j] = mfma(xop, m0, y0[j]);
                        y1[j] = mfma(xop, m1, y1[j]);
                    }
                    __builtin_amdgcn_s_setprio(0);
                }
                store_tile(t0, y0);
                for (int sb = nsb0; sb < nsb1; ++sb) {
                    f32x4 s1[2];
                    scores(sb, 1, s1);
                    const bf16x8 m1 = make_mop(s1, sb, t1, cum1, wide_tag);
#pragma unroll
                    for (int j = 0; j < JP; ++j) y1[j] = mfma(xop_at(j, sb), m1, y1[j]);
                }
                store_tile(t1, y1);
            };
            if (wide) blocks(std::true_type{});
            else blocks(std::false_type{});
        };
        // measured at N = 128 (326 against 337 us); the paired form spills a
        // few registers there, which are reloaded only around the tile stores
        if constexpr (TPW == 2 && N == 128) out_pair();
        else out_tiles();
        if constexpr (TL::BEARLY < TL::BPIECE)
            prefetch_b(ch + 1, std::integral_constant<int, TL::BEARLY>{},
                       std::integral_constant<int, TL::BPIECE>{});

        // ---- 4. state update on this wavefront's 16 columns, JW row tiles
        if (ntile >= 0) {
            const float decay = fast_exp2(cumQ);
#pragma unroll
            for (int jj = 0; jj < JW; ++jj) hacc[jj] *= decay;
            // B operand B[s][n = 16 ntile + c] for 8 consecutive s through two
            // transposed reads; as supplier this lane addresses row 8g + c/4 (+4),
            // columns 16 ntile + 4 (c % 4) .. +3
            const __bf16* bsrc = &sm.B[(8 * g + c / 4) * Lds::kBStride + 16 * ntile + 4 * (c % 4)];
#pragma unroll
            for (int ks = 0; ks < KQ; ++ks) {
                const int s8 = 32 * ks + 8 * g;
                const bf16x4 lo = lds_read_tr16(bsrc + 32 * ks * Lds::kBStride);
                const bf16x4 hi = lds_read_tr16(bsrc + (32 * ks + 4) * Lds::kBStride);
                const bf16x8 braw = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                // the column scaled by w_s (rounded once to bf16, as the product
                // X^T (w o B) needs one of its operands scaled)
                const f32x4 w0 = *reinterpret_cast<const f32x4*>(&sm.wst[s8]);
                const f32x4 w1 = *reinterpret_cast<const f32x4*>(&sm.wst[s8 + 4]);
                bf16x8 bcol;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    bcol[e] = bf(f32(braw[e]) * w0[e]);
                    bcol[4 + e] = bf(f32(braw[4 + e]) * w1[e]);
                }
#pragma unroll
                for (int jj = 0; jj < JW; ++jj) {
                    const int j = jbase + jj;
                    const bf16x8 xa = *reinterpret_cast<const bf16x8*>(
                        &sm.Xt[(16 * j + c) * Lds::kXStride + Lds::xcol(16 * j + c, s8)]);
                    hacc[jj] = mfma(xa, bcol, hacc[jj]);
                }
            }
        }
        lds_barrier();                                   // all reads of the old state copy done
        if (ntile >= 0) {
#pragma unroll
            for (int jj = 0; jj < JW; ++jj)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    sm.H[(16 * (jbase + jj) + 4 * g + r) * Lds::kHStride + 16 * ntile + c] = bf(hacc[jj][r]);
        }

    }
    if (p.h_last && ntile >= 0) {
#pragma unroll
        for (int jj = 0; jj < JW; ++jj)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                p.h_last[(bh * P + pbase + 16 * (jbase + jj) + 4 * g + r) * N + 16 * ntile + c] =
                    hacc[jj][r];
    }
}

template <int Q, int N, int PT>
hipError_t launch_qnp(const SSDArgs& a, hipStream_t stream) {
    const dim3 grid((unsigned)(a.B * a.H * (a.P / PT)));
    if (a.z)
        hipLaunchKernelGGL((ssd_chunk_kernel<Q, N, PT, true>), grid, dim3(kThreads), 0, stream, a);
    else
        hipLaunchKernelGGL((ssd_chunk_kernel<Q, N, PT, false>), grid, dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

// P tile: 64 head-dim rows per workgroup where P allows, else 32
template <int Q, int N>
hipError_t launch_qn(const SSDArgs& a, hipStream_t stream) {
    if (a.P % 64 == 0) return launch_qnp<Q, N, 64>(a, stream);
    if (a.P % 32 == 0) return launch_qnp<Q, N, 32>(a, stream);
    return hipErrorNotSupported;
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
    switch (a.N) {
        case 32: return launch_n<32>(a, stream);
        case 64: return launch_n<64>(a, stream);
        case 96: return launch_n<96>(a, stream);
        case 128: return launch_n<128>(a, stream);
        default: return hipErrorNotSupported;
    }
}

}  // namespace ssm
