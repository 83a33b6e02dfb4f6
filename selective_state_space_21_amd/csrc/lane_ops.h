// Cross-lane helpers for 64-wide wavefronts on gfx950: DPP row broadcasts
// and xor exchanges inside 32-lane halves (ds_swizzle, no memory access).
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

// Value of lane (lane ^ M) for M < 32 (ds_swizzle bit-mask mode: the xor
// mask in bits 10-14, and-mask 0x1f).
template <int M>
__device__ __forceinline__ float lane_xor(float v) {
    static_assert(M > 0 && M < 32, "xor inside a 32-lane half");
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v),
                                                                 0x1f | (M << 10)));
}

}  // namespace ssm
