// bf16 matrix-core helpers for gfx950 (wave64, v_mfma_f32_16x16x32_bf16).
//
// Operand layout of the 16x16x32 product, lane = l16 + 16 * q4:
//   A (16 x 32):  lane holds row l16, k-values 8*q4 .. 8*q4+7;
//   B (32 x 16):  lane holds column l16, k-values 8*q4 .. 8*q4+7;
//   C (16 x 16):  lane holds column l16, rows 4*q4 .. 4*q4+3.
// float32-faithful products split float32 operands into bf16 pieces:
//   split2: x ~ hi + lo (16 significant bits);
//   split3: x = p0 + p1 + p2 exactly for normal x.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma16x16x32(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ void split2(const float (&x)[8], bf16x8& hi, bf16x8& lo) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const __bf16 h = (__bf16)x[j];
    hi[j] = h;
    lo[j] = (__bf16)(x[j] - (float)h);
  }
}

// Each remainder is exact in float32 and the last has at most 8 significant bits.
__device__ __forceinline__ void split3(const float (&x)[8], bf16x8& p0, bf16x8& p1, bf16x8& p2) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const __bf16 a = (__bf16)x[j];
    const float r = x[j] - (float)a;
    const __bf16 b = (__bf16)r;
    p0[j] = a;
    p1[j] = b;
    p2[j] = (__bf16)(r - (float)b);
  }
}

// The same two splits converting pairs of values at a time (one packed
// round-to-nearest-even conversion per pair, as the scalar forms round).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ void split2_pk(const float (&x)[8], bf16x8& hi, bf16x8& lo) {
#pragma unroll
  for (int j = 0; j < 8; j += 2) {
    const f32x2_t v = {x[j], x[j + 1]};
    const bf16x2_t h = __builtin_convertvector(v, bf16x2_t);
    const bf16x2_t l = __builtin_convertvector(v - __builtin_convertvector(h, f32x2_t), bf16x2_t);
    hi[j] = h[0];
    hi[j + 1] = h[1];
    lo[j] = l[0];
    lo[j + 1] = l[1];
  }
}

__device__ __forceinline__ void split3_pk(const float (&x)[8], bf16x8& p0, bf16x8& p1, bf16x8& p2) {
#pragma unroll
  for (int j = 0; j < 8; j += 2) {
    const f32x2_t v = {x[j], x[j + 1]};
    const bf16x2_t a = __builtin_convertvector(v, bf16x2_t);
    const f32x2_t r = v - __builtin_convertvector(a, f32x2_t);
    const bf16x2_t b = __builtin_convertvector(r, bf16x2_t);
    const bf16x2_t c = __builtin_convertvector(r - __builtin_convertvector(b, f32x2_t), bf16x2_t);
    p0[j] = a[0];
    p0[j + 1] = a[1];
    p1[j] = b[0];
    p1[j + 1] = b[1];
    p2[j] = c[0];
    p2[j + 1] = c[1];
  }
}

__device__ __forceinline__ float comp(const float4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// (a, b) of every feature of the d = 64 lift in canonical order, a | b << 8.
struct PairTable64 {
  uint16_t ab[64 * 65 / 2];
  constexpr PairTable64() : ab{} {
    int f = 0;
    for (int a = 0; a < 64; ++a)
      for (int b = a; b < 64; ++b) ab[f++] = static_cast<uint16_t>(a | (b << 8));
  }
};

}  // namespace kla
