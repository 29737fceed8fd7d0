// gfx950 matrix-core helpers shared by the MFMA kernels.
//
// v_mfma_f32_16x16x32_{bf16,f16}: D[16 x 16] += A[16 x 32] . B[32 x 16] in
// fp32.  Lane l = 16 q + c supplies A[c][8q .. 8q+7] and B[8q .. 8q+7][c]
// (eight 16-bit elements in one 16-byte register quad) and receives
// D[4q + r][c] for r = 0..3.
#pragma once

#include "pkv_device.h"

namespace pkv {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

template <int DT>
__device__ __forceinline__ f32x4_t mfma_16x16x32(const u32x4 a, const u32x4 b, f32x4_t c) {
    if constexpr (DT == kBF16)
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                       __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                      __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

}  // namespace pkv
