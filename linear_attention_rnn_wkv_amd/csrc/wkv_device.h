// wkv_device.h -- small device helpers shared by the WKV kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wkv {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.44269504088896340736f;

// e^x through the hardware base-2 exponential (v_exp_f32).  The product
// x*log2(e) is rounded once, so the relative error grows like |x| * 2^-24;
// callers only pass arguments whose results matter at |x| below ~20.
__device__ __forceinline__ float exp_fast(float x) {
    return __builtin_amdgcn_exp2f(x * kLog2e);
}

__device__ __forceinline__ float exp2_fast(float x) {
    return __builtin_amdgcn_exp2f(x);
}

// bf16 bits -> fp32 (exact)
__device__ __forceinline__ float bf16_lo(uint32_t packed) {
    return __uint_as_float(packed << 16);
}
__device__ __forceinline__ float bf16_hi(uint32_t packed) {
    return __uint_as_float(packed & 0xffff0000u);
}
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(((uint32_t)b) << 16);
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two fp32 -> two bf16 packed in one dword (lo in bits 0..15), round to
// nearest even: a single v_cvt_pk_bf16_f32 on gfx950.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const f32x2 f = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}

// fp32 rounded to bf16 and widened back (exact value of the rounded number).
__device__ __forceinline__ float round_bf16(float f) {
    return bf16_lo(pack_bf16x2(f, 0.0f));
}

}  // namespace wkv
