// Device-side helpers shared by the libpagedattn kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

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

// 8-bit codes of quantised caches (one fp32 scale per token and KV head; a
// cached value is value(code) * scale; a row x is stored with scale =
// max|x| / kMax and codes encode(x / scale), all in fp32).
// INT8: symmetric integers, encode = round to nearest even, clamped to
// [-127, 127].
struct I8Code {
  static constexpr float kMax = 127.f;
  static __device__ __forceinline__ uint32_t encode(float r) {
    return (uint32_t)(uint8_t)(int8_t)(int)fminf(fmaxf(rintf(r), -127.f), 127.f);
  }
  static __device__ __forceinline__ float value(uint32_t b) { return (float)(int8_t)(uint8_t)b; }
};

// FP8: the OCP E4M3 8-bit float (sign, 4 exponent bits with bias 7, 3
// mantissa bits; exponent field 0 holds the subnormals m * 2^-9; the largest
// finite magnitude is 448, and S.1111.111 is NaN).  encode rounds to the
// nearest E4M3 value, ties to an even mantissa, and saturates magnitudes of
// 448 and more (and NaN) to 448, so it never makes a NaN code.  value (of a
// code a write made) is exact.
struct Fp8Code {
  static constexpr float kMax = 448.f;
  static __device__ __forceinline__ uint32_t encode(float r) {
    const uint32_t u = __float_as_uint(r);
    const uint32_t sgn = (u >> 24) & 0x80u;
    const uint32_t a = u & 0x7FFFFFFFu;  // |r|
    if (!(__uint_as_float(a) < 448.f)) return sgn | 0x7Eu;
    if (a < 0x3C800000u)  // |r| < 2^-6: the subnormal grid, steps of 2^-9 (8 steps = 2^-6)
      return sgn | (uint32_t)rintf(__uint_as_float(a) * 512.f);
    // normal: 3 of the 23 mantissa bits, the 20 dropped ones rounded to
    // nearest even (a carry moves into the exponent); rebias 127 -> 7
    const uint32_t rounded = a + 0x7FFFFu + ((a >> 20) & 1u);
    return sgn | ((rounded >> 20) - (120u << 3));
  }
  // exact: the code's bits under an fp32 exponent bias of 127 read the value
  // times 2^-120 (subnormals included)
  static __device__ __forceinline__ float value(uint32_t b) {
    return __uint_as_float(((b & 0x80u) << 24) | ((b & 0x7Fu) << 20)) * 0x1p120f;
  }
};

// 16-bit element types: storage is the raw 16-bit pattern.  Code is the
// format of 8-bit caches read with queries of this type (INT8; Fp8Elem below
// for FP8), codes4 widens four of its codes to this type, exactly.
struct F16 {
  using vec8 = f16x8;
  using Code = I8Code;
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
  using Code = I8Code;
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

// The element type Base with FP8 (E4M3) cache codes.  codes4 is the gfx950
// conversion of two packed E4M3 codes (OCP format, scale 1: exact for every
// finite code; a NaN code gives NaN, so the kernels zero the codes of slots
// past a context, which no write has filled, before widening them).
template <typename Base>
struct Fp8Elem : Base {
  using Code = Fp8Code;
  static __device__ __forceinline__ u32x2 codes4(uint32_t c) {
    if constexpr (std::is_same<Base, F16>::value)
      return u32x2{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c, 1.f, false)),
                   __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c, 1.f, true))};
    else
      return u32x2{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c, 1.f, false)),
                   __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c, 1.f, true))};
  }
};

// Whether the 8-bit codes of element type Ty are FP8 (whose unwritten slots
// may hold NaN codes).
template <typename Ty>
constexpr bool kFp8Codes = std::is_same<typename Ty::Code, Fp8Code>::value;

// Byte mask of the codes of tokens first .. first + 3 (byte j: token first + j)
// that lie before end.
__device__ __forceinline__ uint32_t bytes_before(int first, int end) {
  uint32_t m = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) m |= first + j < end ? 0xFFu << (8 * j) : 0u;
  return m;
}

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
