// Block-level self-recall-error scoring (LoLA page, section "O Mecanismo de
// Erro de Auto-Recuperação"): for up to 64 candidates (k_c, v_c),
//   pred_c = phi(k_c)^T H / (phi(k_c)^T s + eps)   (0 when that is 0),
//   score_c = ||pred_c - v_c||^2,
// all in float32. The block streams H through LDS in tiles of 32 feature
// rows; each candidate is served by 4 threads that own d_v/4 columns each.
#pragma once

#include "kla_device.hpp"

namespace kla {

template <int DQK, int DV>
struct SreShared {
  static constexpr int D = phi_dim(DQK);
  static constexpr int FT = 32;
  float kc[64][DQK + 1];
  float Ht[FT][DV];
  float st[FT];
  uint16_t tab[D];
};

// load_k(c, d) / load_v(c, d) give candidate c's key / value entries.
// Writes scores_n[c] for c in [cbase, min(cbase + 64, n_cand)).
template <int DQK, int DV, typename LK, typename LV>
__device__ __forceinline__ void sre_block(SreShared<DQK, DV>& sh, const float* __restrict__ Hn,
                                          const float* __restrict__ sn, int cbase, int n_cand,
                                          LK load_k, LV load_v, float* __restrict__ scores_n,
                                          float eps) {
  constexpr int D = phi_dim(DQK);
  constexpr int FT = SreShared<DQK, DV>::FT;
  constexpr int CPT = DV / 4;
  const int tid = threadIdx.x;
  const int cl = tid >> 2;
  const int qt = tid & 3;
  const int c = cbase + cl;
  const bool valid = c < n_cand;

  for (int i = tid; i < 64 * DQK; i += blockDim.x) {
    const int r = i / DQK, d = i % DQK;
    sh.kc[r][d] = (cbase + r < n_cand) ? load_k(cbase + r, d) : 0.0f;
  }
  build_phi_table(sh.tab, 0, D, DQK);

  float acc[CPT];
#pragma unroll
  for (int j = 0; j < CPT; ++j) acc[j] = 0.0f;
  float den = 0.0f;
#pragma unroll 1
  for (int f0 = 0; f0 < D; f0 += FT) {
    const int nf = min(FT, D - f0);
    __syncthreads();
    for (int i = threadIdx.x; i < FT * DV; i += blockDim.x) {
      const int r = i / DV, cc = i % DV;
      sh.Ht[r][cc] = r < nf ? Hn[(size_t)(f0 + r) * DV + cc] : 0.0f;
    }
    for (int i = threadIdx.x; i < FT; i += blockDim.x) sh.st[i] = i < nf ? sn[f0 + i] : 0.0f;
    __syncthreads();
#pragma unroll 4
    for (int r = 0; r < nf; ++r) {
      const float p = phi_of(sh.kc[cl], sh.tab[f0 + r]);
#pragma unroll
      for (int j = 0; j < CPT; ++j) acc[j] += p * sh.Ht[r][qt * CPT + j];
      den += p * sh.st[r];
    }
  }
  const float dt = den + eps;
  float err = 0.0f;
#pragma unroll
  for (int j = 0; j < CPT; ++j) {
    const float pred = dt != 0.0f ? acc[j] / dt : 0.0f;
    const float diff = pred - (valid ? load_v(c, qt * CPT + j) : 0.0f);
    err += diff * diff;
  }
  err += __shfl_xor(err, 1, 64);
  err += __shfl_xor(err, 2, 64);
  if (valid && qt == 0) scores_n[c] = err;
  __syncthreads();
}

}  // namespace kla
