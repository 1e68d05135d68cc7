// Device-side helpers shared by the libpagedattn kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pagedattn.h"

namespace pa {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// 16-bit element types: storage is the raw 16-bit pattern.
struct F16 {
  using vec8 = f16x8;
  static __device__ __forceinline__ float to_f32(uint16_t u) {
    return (float)__builtin_bit_cast(_Float16, u);
  }
  static __device__ __forceinline__ uint16_t from_f32(float f) {
    return __builtin_bit_cast(uint16_t, (_Float16)f);  // round to nearest even
  }
  // two values rounded to nearest even, packed (low half = a)
  static __device__ __forceinline__ uint32_t pack2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, f16x2));
  }
  static __device__ __forceinline__ float lo_f32(uint32_t w) { return to_f32((uint16_t)w); }
  static __device__ __forceinline__ float hi_f32(uint32_t w) { return to_f32((uint16_t)(w >> 16)); }
  // acc + both halves of a packed pair, in one dot-product instruction
  static __device__ __forceinline__ float sum2(uint32_t w, float acc) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, w), f16x2{(_Float16)1.f, (_Float16)1.f},
                                  acc, false);
  }
  // acc + a.lo * b.lo + a.hi * b.hi of two packed pairs (products exact in fp32)
  static __device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float acc) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b), acc,
                                  false);
  }
  // four signed bytes -> four f16 (two packed words), exactly: with the sign
  // bit flipped a byte is c + 128 in [1, 255]; as the mantissa under 0x64 it
  // reads 1024 + c + 128, and subtracting 1152 leaves c (all values exact).
  static __device__ __forceinline__ u32x2 codes4(uint32_t c) {
    const uint32_t u = c ^ 0x80808080u;
    const f16x2 bias = {(_Float16)-1152.f, (_Float16)-1152.f};
    const uint32_t lo = __builtin_amdgcn_perm(0x64646464u, u, 0x04010400u);
    const uint32_t hi = __builtin_amdgcn_perm(0x64646464u, u, 0x04030402u);
    return u32x2{__builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, lo) + bias),
                 __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, hi) + bias)};
  }
  static __device__ __forceinline__ f32x4 mma(vec8 a, vec8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
};

struct BF16 {
  using vec8 = bf16x8;
  static __device__ __forceinline__ float to_f32(uint16_t u) {
    return __uint_as_float((uint32_t)u << 16);
  }
  static __device__ __forceinline__ uint16_t from_f32(float f) {
    return __builtin_bit_cast(uint16_t, (__bf16)f);  // round to nearest even
  }
  static __device__ __forceinline__ uint32_t pack2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
  }
  static __device__ __forceinline__ float lo_f32(uint32_t w) { return __uint_as_float(w << 16); }
  static __device__ __forceinline__ float hi_f32(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
  static __device__ __forceinline__ float sum2(uint32_t w, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w),
                                           __builtin_bit_cast(bf16x2, 0x3F803F80u), acc, false);
  }
  static __device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b),
                                           acc, false);
  }
  // four signed bytes -> four bf16, exactly (|c| <= 128 needs 8 significant bits)
  static __device__ __forceinline__ u32x2 codes4(uint32_t c) {
    return u32x2{pack2((float)(int8_t)c, (float)(int8_t)(c >> 8)),
                 pack2((float)(int8_t)(c >> 16), (float)(int8_t)(c >> 24))};
  }
  static __device__ __forceinline__ f32x4 mma(vec8 a, vec8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};

__device__ __forceinline__ u32x4 load16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

__device__ __forceinline__ void store16(void* p, u32x4 v) {
  *reinterpret_cast<u32x4*>(p) = v;
}

__device__ __forceinline__ float exp2_fast(float x) {
  return __builtin_amdgcn_exp2f(x);  // v_exp_f32; exp2(-inf) = 0
}

__host__ __device__ __forceinline__ int clampi(int v, int lo, int hi) {
  return v < lo ? lo : (v > hi ? hi : v);
}

// Wave-uniform value as a scalar (the compiler keeps it in an SGPR).
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

}  // namespace pa
