// Cross-lane helpers for 64-wide wavefronts on gfx950: DPP row broadcasts,
// row permutes and reduce-scatters, xor exchanges inside 32-lane halves
// (ds_swizzle, no memory access), and a workgroup barrier over LDS.
#pragma once

#include <hip/hip_runtime.h>

namespace ssm {

// Broadcast lane k of each 16-lane row to the whole row (DPP row_newbcast,
// gfx90a and later).  Used as an operand of a multiply, it folds into the
// instruction (v_mul_f32_dpp) at no cost.
template <int K>
__device__ __forceinline__ float row_bcast_c(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
        0, __builtin_bit_cast(int, v), 0x150 + K, 0xf, 0xf, true));
}
// k must fold to a constant after unrolling.
__device__ __forceinline__ float row_bcast(float v, int k) {
    switch (k) {
        case 0: return row_bcast_c<0>(v);   case 1: return row_bcast_c<1>(v);
        case 2: return row_bcast_c<2>(v);   case 3: return row_bcast_c<3>(v);
        case 4: return row_bcast_c<4>(v);   case 5: return row_bcast_c<5>(v);
        case 6: return row_bcast_c<6>(v);   case 7: return row_bcast_c<7>(v);
        case 8: return row_bcast_c<8>(v);   case 9: return row_bcast_c<9>(v);
        case 10: return row_bcast_c<10>(v); case 11: return row_bcast_c<11>(v);
        case 12: return row_bcast_c<12>(v); case 13: return row_bcast_c<13>(v);
        case 14: return row_bcast_c<14>(v); default: return row_bcast_c<15>(v);
    }
}

// Value of lane j - K of the same 16-lane row (DPP row_shr:K); lanes j < K
// read 0.
template <int K>
__device__ __forceinline__ float dpp_shr(float v) {
    static_assert(K > 0 && K < 16, "row shift");
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
        0, __builtin_bit_cast(int, v), 0x110 + K, 0xf, 0xf, true));
}

// Value of lane (lane ^ M) for M < 32 (ds_swizzle bit-mask mode: the xor
// mask in bits 10-14, and-mask 0x1f).
template <int M>
__device__ __forceinline__ float lane_xor(float v) {
    static_assert(M > 0 && M < 32, "xor inside a 32-lane half");
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v),
                                                                 0x1f | (M << 10)));
}

// Value of another lane of the same 16-lane row, chosen by a DPP control
// (quad_perm, row_ror, row_half_mirror, ...), every lane written.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
        0, __builtin_bit_cast(int, x), CTRL, 0xf, 0xf, true));
}

// The first halving exchange of row_reduce_scatter16 below, on its own: lane
// j < 8 ends with a[k] = v[k] + (v[k] of lane j + 8), the partial sum of token
// k; lane j >= 8 with a[k] = v[k + 8] + (v[k + 8] of lane j - 8), token k + 8.
// Two bank-masked DPP adds per result; the block opens with s_nop 1 because
// DPP reads its inputs two wait states after a VALU write at the earliest.
__device__ __forceinline__ void row_fold_halves16(const float (&v)[16], float (&a)[8]) {
    asm("s_nop 1\n\t"
        "v_add_f32_dpp %0, %8, %8 row_ror:8 row_mask:0xf bank_mask:0x3\n\t"
        "v_add_f32_dpp %0, %16, %16 row_ror:8 row_mask:0xf bank_mask:0xc\n\t"
        "v_add_f32_dpp %1, %9, %9 row_ror:8 row_mask:0xf bank_mask:0x3\n\t"
        "v_add_f32_dpp %1, %17, %17 row_ror:8 row_mask:0xf bank_mask:0xc\n\t"
        "v_add_f32_dpp %2, %10, %10 row_ror:8 row_mask:0xf bank_mask:0x3\n\t"
        "v_add_f32_dpp %2, %18, %18 row_ror:8 row_mask:0xf bank_mask:0xc\n\t"
        "v_add_f32_dpp %3, %11, %11 row_ror:8 row_mask:0xf bank_mask:0x3\n\t"
        "v_add_f32_dpp %3, %19, %19 row_ror:8 row_mask:0xf bank_mask:0xc\n\t"
        "v_add_f32_dpp %4, %12, %12 row_ror:8 row_mask:0xf bank_mask:0x3\n\t"
        "v_add_f32_dpp %4, %20, %20 row_ror:8 row_mask:0xf bank_mask:0xc\n\t"
        "v_add_f32_dpp %5, %13, %13 row_ror:8 row_mask:0xf bank_mask:0x3\n\t"
        "v_add_f32_dpp %5, %21, %21 row_ror:8 row_mask:0xf bank_mask:0xc\n\t"
        "v_add_f32_dpp %6, %14, %14 row_ror:8 row_mask:0xf bank_mask:0x3\n\t"
        "v_add_f32_dpp %6, %22, %22 row_ror:8 row_mask:0xf bank_mask:0xc\n\t"
        "v_add_f32_dpp %7, %15, %15 row_ror:8 row_mask:0xf bank_mask:0x3\n\t"
        "v_add_f32_dpp %7, %23, %23 row_ror:8 row_mask:0xf bank_mask:0xc"
        : "=&v"(a[0]), "=&v"(a[1]), "=&v"(a[2]), "=&v"(a[3]),
          "=&v"(a[4]), "=&v"(a[5]), "=&v"(a[6]), "=&v"(a[7])
        : "v"(v[0]), "v"(v[1]), "v"(v[2]), "v"(v[3]), "v"(v[4]), "v"(v[5]), "v"(v[6]), "v"(v[7]),
          "v"(v[8]), "v"(v[9]), "v"(v[10]), "v"(v[11]), "v"(v[12]), "v"(v[13]), "v"(v[14]),
          "v"(v[15]));
}

// Reduce-scatter over the 16 lanes of each row: v[i] is this lane's term for
// token i; the result in lane j is the row's sum over all lanes for token j.
// Four halving exchanges, each between lanes that differ in one bit of j:
// lane j keeps the half of its tokens whose index bit equals its own bit and
// adds the partner's copy of that half.  Partners: j ^ 8 (DPP row_ror:8),
// j ^ 7 (row_half_mirror, which flips bit 2 and keeps bit 3), j ^ 2 and j ^ 1
// (quad permutes).  In the first two exchanges the kept half is fixed per
// group of four lanes (a DPP "bank"), so each result is two bank-masked DPP
// adds (lanes of disabled banks are not written) instead of two selects and
// an add.  DPP reads a VGPR two wait states after a VALU write at the
// earliest: the blocks open with s_nop 1 for their inputs and the second ends
// with one for its outputs, which the compiler does not see being written.
__device__ __forceinline__ float row_reduce_scatter16(const float (&v)[16], int j) {
    float a[8], c[4], e[2];
    row_fold_halves16(v, a);
    asm("s_nop 1\n\t"
        "v_add_f32_dpp %0, %4, %4 row_half_mirror row_mask:0xf bank_mask:0x5\n\t"
        "v_add_f32_dpp %0, %8, %8 row_half_mirror row_mask:0xf bank_mask:0xa\n\t"
        "v_add_f32_dpp %1, %5, %5 row_half_mirror row_mask:0xf bank_mask:0x5\n\t"
        "v_add_f32_dpp %1, %9, %9 row_half_mirror row_mask:0xf bank_mask:0xa\n\t"
        "v_add_f32_dpp %2, %6, %6 row_half_mirror row_mask:0xf bank_mask:0x5\n\t"
        "v_add_f32_dpp %2, %10, %10 row_half_mirror row_mask:0xf bank_mask:0xa\n\t"
        "v_add_f32_dpp %3, %7, %7 row_half_mirror row_mask:0xf bank_mask:0x5\n\t"
        "v_add_f32_dpp %3, %11, %11 row_half_mirror row_mask:0xf bank_mask:0xa\n\t"
        "s_nop 1"
        : "=&v"(c[0]), "=&v"(c[1]), "=&v"(c[2]), "=&v"(c[3])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7]));
    const bool b1 = j & 2, b0 = j & 1;
#pragma unroll
    for (int i = 0; i < 2; ++i)
        e[i] = (b1 ? c[i + 2] : c[i]) + dpp_mov<0x4E>(b1 ? c[i] : c[i + 2]);   // quad xor 2
    return (b0 ? e[1] : e[0]) + dpp_mov<0xB1>(b0 ? e[0] : e[1]);               // quad xor 1
}

// Compiler-level ordering of one wavefront's LDS accesses at a point: LDS
// performs a wavefront's accesses in issue order, so lanes of the wavefront
// read what other lanes of it wrote before the fence with no wait.
__device__ __forceinline__ void wave_lds_fence() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Workgroup barrier that first waits for this wavefront's own LDS accesses.
// The compiler does not always put that wait before s_barrier (at a loop
// header it was omitted after the previous iteration's last LDS store), and
// without it another wavefront could read a location before the store landed.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

}  // namespace ssm
