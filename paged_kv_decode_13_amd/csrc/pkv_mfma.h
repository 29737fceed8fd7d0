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

template <int DT>
__device__ __forceinline__ f32x4_t mfma_16x16x32(const u32x4 a, const u32x4 b, f32x4_t c) {
    if constexpr (DT == kBF16)
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                       __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                      __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

// Max / sum over the four lanes l, l ^ 16, l ^ 32, l ^ 48 (the four row
// groups of an MFMA column) with the gfx950 lane-swap instructions: each
// swap hands a lane its partner's value, so both steps stay on the VALU with
// no LDS round trip, and every lane of the four ends with the same result.
__device__ __forceinline__ float rowgroup_max(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float rowgroup_sum(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Two probabilities -> packed 16-bit pairs (hi, lo) with hi + lo = p to
// about 16 (bf16: hardware round-to-nearest-even both times) or 21 (fp16:
// hardware pack with round toward zero; the remainder carries the rest)
// significant bits.
template <int DT>
__device__ __forceinline__ void split_pack(float p0, float p1, uint32_t &hi, uint32_t &lo) {
    if constexpr (DT == kBF16) {
        typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
        const bf16x2_t h = {(__bf16)p0, (__bf16)p1};
        hi = __builtin_bit_cast(uint32_t, h);
        // both halves come from the packed pair (one shift, one mask); the
        // empty asm keeps the compiler from converting p0 a second time
        asm("" : "+v"(hi));
        const float r0 = p0 - __uint_as_float(hi << 16);
        const float r1 = p1 - __uint_as_float(hi & 0xffff0000u);
        const bf16x2_t l = {(__bf16)r0, (__bf16)r1};
        lo = __builtin_bit_cast(uint32_t, l);
    } else {
        const auto h = __builtin_amdgcn_cvt_pkrtz(p0, p1);
        hi = __builtin_bit_cast(uint32_t, h);
        const float r0 = p0 - (float)h[0];
        const float r1 = p1 - (float)h[1];
        lo = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(r0, r1));
    }
}

// max(a, b, c) in one instruction (the compiler emits two v_max_f32 for
// nested fmaxf).  Masked scores are -inf, never NaN.
__device__ __forceinline__ float max3f(float a, float b, float c) {
    float r;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}

__device__ __forceinline__ float max2f(float a, float b) {
    float r;
    asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}

// rowgroup_max for values that are never NaN (scores, masked ones -inf):
// no quieting of the swapped-in values.
__device__ __forceinline__ float rowgroup_max_nn(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = max2f(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return max2f(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// A register quad of 16-bit ones: the A operand that turns a value MFMA into
// a sum of its B operand over k.
template <int DT>
__device__ __forceinline__ u32x4 ones16() {
    constexpr uint32_t one = DT == kBF16 ? 0x3F803F80u : 0x3C003C00u;
    return u32x4{one, one, one, one};
}

// Two probabilities -> one packed 16-bit pair, each rounded to nearest even.
template <int DT>
__device__ __forceinline__ uint32_t pack_rne(float p0, float p1) {
    if constexpr (DT == kBF16) {
        typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
        const bf16x2_t h = {(__bf16)p0, (__bf16)p1};
        return __builtin_bit_cast(uint32_t, h);
    } else {
        typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
        const f16x2_t h = {(_Float16)p0, (_Float16)p1};
        return __builtin_bit_cast(uint32_t, h);
    }
}

}  // namespace pkv
