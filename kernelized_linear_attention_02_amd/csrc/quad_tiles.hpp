// LDS tile helpers of the quadratic-form kernels (forward and backward).
//
// A product whose contraction runs over tokens (P^T V, dS^T Q, dS K, ...)
// takes its A operand straight from the accumulator of the preceding score
// product: lane (l16, q4) holds the scores of tokens 4 q4 + i of two 16-token
// tiles. The B operand must list the same tokens in the same order, so token
// tiles are stored transposed ([dim][column]) with a column permutation that
// makes those eight tokens adjacent: one 16-byte read per lane.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kla {

// Within each group of 32 tokens, token 16 t + 4 g + i goes to column
// 8 g + 4 t + i.
__device__ __forceinline__ int vt_col(int tok) {
  const int r = tok & 15;
  return (tok & ~31) + 8 * (r >> 2) + 4 * ((tok >> 4) & 1) + (r & 3);
}

// The value of the neighbouring lane (lane ^ 1).
__device__ __forceinline__ uint32_t pair_swap(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, 0xB1, 0xF, 0xF, false);  // quad_perm [1,0,3,2]
}

// Stores dims d0 .. d0 + 7 (bf16, in u) of token `tok` into the transposed
// tile tr[dim * ts + column]. Tokens 2m and 2m + 1 must sit in adjacent lanes
// (lane ^ 1) with the same d0; they land in adjacent columns, so the two
// lanes trade half of their values and each writes four whole 32-bit words.
// Every lane of the pair must call it.
__device__ __forceinline__ void store_transposed8(uint16_t* tr, int ts, const uint4& u, int tok, int d0) {
  const int col = vt_col(tok) & ~1;
  const bool even = (tok & 1) == 0;
  // dims (2e, 2e + 1) of this token in word e of u
  const uint32_t x0 = pair_swap(even ? u.z : u.x);
  const uint32_t x1 = pair_swap(even ? u.w : u.y);
  // the even lane writes dims 0..3 of the group, the odd lane dims 4..7
  const uint32_t a0 = even ? u.x : x0, a1 = even ? u.y : x1;  // token 2m
  const uint32_t b0 = even ? x0 : u.z, b1 = even ? x1 : u.w;  // token 2m + 1
  const int d = d0 + (even ? 0 : 4);
  *reinterpret_cast<uint32_t*>(&tr[(size_t)d * ts + col]) = __builtin_amdgcn_perm(b0, a0, 0x05040100u);
  *reinterpret_cast<uint32_t*>(&tr[(size_t)(d + 1) * ts + col]) = __builtin_amdgcn_perm(b0, a0, 0x07060302u);
  *reinterpret_cast<uint32_t*>(&tr[(size_t)(d + 2) * ts + col]) = __builtin_amdgcn_perm(b1, a1, 0x05040100u);
  *reinterpret_cast<uint32_t*>(&tr[(size_t)(d + 3) * ts + col]) = __builtin_amdgcn_perm(b1, a1, 0x07060302u);
}

}  // namespace kla
