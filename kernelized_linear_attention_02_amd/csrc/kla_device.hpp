// Device helpers shared by the libkla kernels (gfx950, wave64).
//
// Feature lift (KATA page, §2.2): phi(x)_f = x_a * x_b * c_f with c_f = 1 on
// the diagonal (a == b) and sqrt(2) above it, f(a, b) = a*d - a*(a-1)/2 + (b-a).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kla {

constexpr float kSqrt2 = 1.41421356237309504880f;

__host__ __device__ constexpr int phi_dim(int d) { return d * (d + 1) / 2; }

// ---------------------------------------------------------------- bf16 <-> f32

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// Round to nearest, ties to even (inputs are finite).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

template <typename T> struct Elem;
template <> struct Elem<float> {
  static __device__ __forceinline__ float load(const float* p, size_t i) { return p[i]; }
  static __device__ __forceinline__ void store(float* p, size_t i, float x) { p[i] = x; }
};
template <> struct Elem<uint16_t> {
  static __device__ __forceinline__ float load(const uint16_t* p, size_t i) { return bf16_to_f32(p[i]); }
  static __device__ __forceinline__ void store(uint16_t* p, size_t i, float x) { p[i] = f32_to_bf16(x); }
};

// ---------------------------------------------------------------- feature table

// Packs (a, b) of feature f as a | (b << 8).
__device__ __forceinline__ uint16_t phi_pair(int f, int d) {
  int a = 0;
  int start = 0;
  while (a < d - 1 && start + (d - a) <= f) {
    start += d - a;
    ++a;
  }
  const int b = a + (f - start);
  return static_cast<uint16_t>(a | (b << 8));
}

// Fills tab[0..count) with the pairs of features first..first+count-1.
__device__ __forceinline__ void build_phi_table(uint16_t* tab, int first, int count, int d) {
  for (int i = threadIdx.x; i < count; i += blockDim.x) tab[i] = phi_pair(first + i, d);
}

__device__ __forceinline__ float phi_scale(uint16_t ab) {
  return ((ab & 0xFF) == (ab >> 8)) ? 1.0f : kSqrt2;
}

// phi_f(x) for x in LDS (or registers through a pointer).
__device__ __forceinline__ float phi_of(const float* x, uint16_t ab) {
  const int a = ab & 0xFF;
  const int b = ab >> 8;
  return x[a] * x[b] * phi_scale(ab);
}

// ---------------------------------------------------------------- reductions

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off, 64));
  return x;
}

// Sort key for top-k: scores are >= 0, so their float bits order them; the
// low word orders equal scores by ascending index.
__device__ __forceinline__ uint64_t topk_key(float score, uint32_t index) {
  return (static_cast<uint64_t>(__float_as_uint(score)) << 32) |
         static_cast<uint64_t>(0xFFFFFFFFu - index);
}
__device__ __forceinline__ uint32_t topk_index(uint64_t key) {
  return 0xFFFFFFFFu - static_cast<uint32_t>(key & 0xFFFFFFFFull);
}

// Bitonic sort of n (power of two, <= 4 * blockDim.x) keys in LDS, descending.
// Every thread of the block must call it.
__device__ __forceinline__ void bitonic_sort_desc(uint64_t* keys, int n) {
  // read once: after each barrier the compiler would load it again
  const int nt = blockDim.x;
  for (int k = 2; k <= n; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      __syncthreads();
      for (int i = threadIdx.x; i < n; i += nt) {
        const int p = i ^ j;
        if (p > i) {
          const uint64_t x = keys[i];
          const uint64_t y = keys[p];
          const bool desc_block = (i & k) == 0;
          // descending inside blocks with (i & k) == 0, ascending otherwise
          if (desc_block ? (x < y) : (x > y)) {
            keys[i] = y;
            keys[p] = x;
          }
        }
      }
    }
  }
  __syncthreads();
}

}  // namespace kla
