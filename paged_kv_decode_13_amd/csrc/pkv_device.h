// Device helpers shared by the gfx950 kernels: element conversion, 16-byte
// vector types and wavefront (DPP) reductions.  wave64 throughout.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

enum DType : int { kF32 = 0, kF16 = 1, kBF16 = 2 };

constexpr int kWave = 64;

// 16 bytes: the unit of every global load and store in these kernels.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int DT>
struct ElemTraits;
template <>
struct ElemTraits<kF32> {
    static constexpr int bytes = 4;
    static constexpr int per16 = 4;  // elements per 16-byte vector
};
template <>
struct ElemTraits<kF16> {
    static constexpr int bytes = 2;
    static constexpr int per16 = 8;
};
template <>
struct ElemTraits<kBF16> {
    static constexpr int bytes = 2;
    static constexpr int per16 = 8;
};

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float f16_lo(uint32_t w) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
}
__device__ __forceinline__ float f16_hi(uint32_t w) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

// Unpack one 16-byte vector into per16 floats.
template <int DT>
__device__ __forceinline__ void unpack16(const u32x4 v, float *f) {
    if constexpr (DT == kF32) {
        f[0] = __uint_as_float(v.x);
        f[1] = __uint_as_float(v.y);
        f[2] = __uint_as_float(v.z);
        f[3] = __uint_as_float(v.w);
    } else {
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if constexpr (DT == kBF16) {
                f[2 * i] = bf16_lo(w[i]);
                f[2 * i + 1] = bf16_hi(w[i]);
            } else {
                f[2 * i] = f16_lo(w[i]);
                f[2 * i + 1] = f16_hi(w[i]);
            }
        }
    }
}

// binary32 -> bfloat16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
    uint32_t u = __float_as_uint(x);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// binary32 -> binary16 bits (hardware conversion, round to nearest even).
__device__ __forceinline__ uint16_t f32_to_f16_bits(float x) {
    return __builtin_bit_cast(uint16_t, (_Float16)x);
}

template <int DT>
__device__ __forceinline__ uint16_t f32_to_bits16(float x) {
    if constexpr (DT == kBF16)
        return f32_to_bf16_bits(x);
    else
        return f32_to_f16_bits(x);
}

__device__ __forceinline__ u32x4 load16(const void *p) {
    return *reinterpret_cast<const u32x4 *>(p);
}

__device__ __forceinline__ void store16(void *p, u32x4 v) { *reinterpret_cast<u32x4 *>(p) = v; }

// Streaming 16-byte load: the KV history is read once per step, so it is
// marked non-temporal to keep it from displacing reused lines.
__device__ __forceinline__ u32x4 load16_stream(const void *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}

// 8 bytes: eight E4M3 elements of a quantised cache row.
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x2 load8_stream(const void *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(p));
}

// OCP E4M3 ("e4m3fn") <-> binary32 with the gfx950 conversion instructions.
// Four E4M3 bytes of a word -> four floats (exact).
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void e4m3x4_to_f32(uint32_t w, float *f) {
    const f32x2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
    const f32x2_t hi = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
    f[0] = lo[0];
    f[1] = lo[1];
    f[2] = hi[0];
    f[3] = hi[1];
}

// Largest finite E4M3 magnitude; quantised values saturate there.
constexpr float kE4M3Max = 448.f;

// Four floats -> four E4M3 bytes (round to nearest even after saturation to
// +-448; comparisons are false for NaN, which stays NaN).
__device__ __forceinline__ float sat_e4m3(float x) {
    return x > kE4M3Max ? kE4M3Max : (x < -kE4M3Max ? -kE4M3Max : x);
}
__device__ __forceinline__ uint32_t f32x4_to_e4m3(float a, float b, float c, float d) {
    uint32_t w = __builtin_amdgcn_cvt_pk_fp8_f32(sat_e4m3(a), sat_e4m3(b), 0u, false);
    return __builtin_amdgcn_cvt_pk_fp8_f32(sat_e4m3(c), sat_e4m3(d), w, true);
}

// ---------------------------------------------------------------------------
// DPP lane exchanges inside rows of 16 lanes.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <- lane 7-i within 8
constexpr int kDppMirror = 0x140;     // lane i <- lane 15-i within 16

// Sum over aligned groups of N lanes (N in {1,2,4,8,16,32,64}); every lane of
// a group receives the group's total.
template <int N>
__device__ __forceinline__ float group_sum(float v) {
    if constexpr (N >= 2) v += dpp<kDppXor1>(v);
    if constexpr (N >= 4) v += dpp<kDppXor2>(v);
    if constexpr (N >= 8) v += dpp<kDppHalfMirror>(v);
    if constexpr (N >= 16) v += dpp<kDppMirror>(v);
    if constexpr (N >= 32) v += __shfl_xor(v, 16);
    if constexpr (N >= 64) v += __shfl_xor(v, 32);
    return v;
}

template <int N>
__device__ __forceinline__ float group_max(float v) {
    if constexpr (N >= 2) v = fmaxf(v, dpp<kDppXor1>(v));
    if constexpr (N >= 4) v = fmaxf(v, dpp<kDppXor2>(v));
    if constexpr (N >= 8) v = fmaxf(v, dpp<kDppHalfMirror>(v));
    if constexpr (N >= 16) v = fmaxf(v, dpp<kDppMirror>(v));
    if constexpr (N >= 32) v = fmaxf(v, __shfl_xor(v, 16));
    if constexpr (N >= 64) v = fmaxf(v, __shfl_xor(v, 32));
    return v;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace pkv
