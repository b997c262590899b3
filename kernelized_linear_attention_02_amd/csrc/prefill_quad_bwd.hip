// Backward of the quadratic-form prefill on the bf16 matrix cores (d_qk =
// d_v = 64, bf16 q, k, v).
//
// The forward (KATA page, §2.3, quadratic operating point, with the lift of
// §2.2: phi(q) . phi(k) = (q . k)^2) is, per head and query t,
//   s_ti = q_t . k_i,  w_ti = s_ti^2 (i <= t),  D_t = sum_i w_ti + eps,
//   o_t = sum_i w_ti v_i / D_t.
// For a loss with gradient g_t = dL/do_t the chain rule gives, with
// c_t = g_t . o_t = sum_i (w_ti / D_t) (g_t . v_i),
//   dv_i = sum_{t >= i} (w_ti / D_t) g_t,
//   ds_ti = 2 s_ti (g_t . v_i - c_t) / D_t,
//   dq_t = sum_{i <= t} ds_ti k_i,   dk_i = sum_{t >= i} ds_ti q_t.
// D_t comes from the forward; rows with D_t = 0 pass no gradient. ds is
// a difference scaled by s / D (= 1 / s for a lone token), so c_t is formed
// here from the same S and dP values that ds then uses, not from a stored
// output: any mismatch between the two would be amplified.
//
// Two kernels:
//   q    one work-group per head and pair of 64-query blocks, wave w owning
//        queries 16 w .. 16 w + 15. Pass 1 over the key blocks at or before
//        the query block: S^T = K Q_w^T and dP^T = V G_w^T on MFMA
//        16x16x32 bf16, c_t = sum_i P_ti dP_ti in float32 (stored for the
//        kv kernel). Pass 2: the same products, dS, and dQ += dS K;
//   kv   one work-group per head and pair of 64-key blocks (x, last - x),
//        wave w owning keys 16 w .. 16 w + 15. For every query block at or
//        after the key block (staged in LDS as rows and as transposed
//        tiles, double buffered) it forms S = Q K_w^T and dP = G V_w^T,
//        then P = S^2 / D and dS in float32, and adds P^T G into dV and
//        dS^T Q into dK.
// P and dS feed the second products straight from the accumulators (the
// tokens' k-slots in lane order, matched by the transposed tiles' column
// permutation). Products are bf16 x bf16 with float32 sums; P and dS enter
// the accumulating products as two bf16 pieces (hi + lo, 16 significant
// bits), since the large weights of the first keys (P near 1/(t+1)) would
// otherwise carry 2^-9 rounding into the sums.
#include <algorithm>

#include "kla_device.hpp"
#include "kla_internal.hpp"
#include "mfma_bf16.hpp"
#include "quad_tiles.hpp"

namespace kla {
namespace {

constexpr int kBD = 64;               // d_qk = d_v
constexpr int kBW = 4;                // waves per work-group
constexpr int kBT = 64 * kBW;         // threads
constexpr int kBB = 64;               // tokens per block
constexpr int kRS = kBD + 8;          // row stride (bf16) of token-row tiles
constexpr int kTS = kBB + 8;          // row stride (bf16) of transposed tiles
constexpr int kSD = kBD * kBB / kBT;  // dims per staging thread
constexpr int kSU = kSD / 8;          // 16-byte groups per staging thread

// Eight consecutive values as bf16 (rounded to nearest even from float32).
__device__ __forceinline__ uint4 load8(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ uint4 load8(const float* p) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  uint4 r;
  r.x = (uint32_t)f32_to_bf16(a.x) | ((uint32_t)f32_to_bf16(a.y) << 16);
  r.y = (uint32_t)f32_to_bf16(a.z) | ((uint32_t)f32_to_bf16(a.w) << 16);
  r.z = (uint32_t)f32_to_bf16(b.x) | ((uint32_t)f32_to_bf16(b.y) << 16);
  r.w = (uint32_t)f32_to_bf16(b.z) | ((uint32_t)f32_to_bf16(b.w) << 16);
  return r;
}

// One staging thread's share of a 64-token block: token tid % kBB, dims
// kSD g .. kSD g + kSD - 1 with g = tid / kBB; zero past the sequence.
struct RowLoad {
  uint4 x[kSU];
};
template <typename T>
__device__ __forceinline__ RowLoad load_rows(const T* __restrict__ base, size_t row0, int tok, int T_, int g) {
  RowLoad r;
#pragma unroll
  for (int j = 0; j < kSU; ++j) r.x[j] = make_uint4(0, 0, 0, 0);
  if (tok < T_) {
#pragma unroll
    for (int j = 0; j < kSU; ++j) r.x[j] = load8(base + (row0 + tok) * kBD + kSD * g + 8 * j);
  }
  return r;
}

__device__ __forceinline__ void stage_rows(uint16_t (*rows)[kRS], const RowLoad& r, int tok, int g) {
#pragma unroll
  for (int j = 0; j < kSU; ++j) *reinterpret_cast<uint4*>(&rows[tok][kSD * g + 8 * j]) = r.x[j];
}
__device__ __forceinline__ void stage_transposed(uint16_t (*tr)[kTS], const RowLoad& r, int tok, int g) {
#pragma unroll
  for (int j = 0; j < kSU; ++j) store_transposed8(&tr[0][0], kTS, r.x[j], tok, kSD * g + 8 * j);
}

// Row `tok` of a 64-row tile, dims 32 ks + 8 q4 .. + 7: an MFMA operand.
__device__ __forceinline__ bf16x8 frag(const uint16_t (*rows)[kRS], int tok, int ks, int q4) {
  return *reinterpret_cast<const bf16x8*>(&rows[tok][32 * ks + 8 * q4]);
}

// The same from global memory (zero past the sequence).
template <typename T>
__device__ __forceinline__ bf16x8 frag_global(const T* __restrict__ base, size_t row0, int tok, int T_, int ks,
                                              int q4) {
  uint4 u = make_uint4(0, 0, 0, 0);
  if (tok < T_) u = load8(base + (row0 + tok) * kBD + 32 * ks + 8 * q4);
  return __builtin_bit_cast(bf16x8, u);
}

// ---------------------------------------------------------------- dK, dV

struct KVLds {
  uint16_t q[2][kBB][kRS];    // query rows
  uint16_t qt[2][kBD][kTS];   // queries transposed (permuted columns)
  uint16_t g[2][kBB][kRS];    // dO rows
  uint16_t gt[2][kBD][kTS];   // dO transposed
  float c[2][kBB];
  float inv[2][kBB];
};

template <typename Tout>
__global__ __launch_bounds__(kBT, 2) void quad_bwd_kv_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const Tout* __restrict__ g, const float* __restrict__ cvec, const float* __restrict__ den,
    Tout* __restrict__ dk, Tout* __restrict__ dv, int T) {
  __shared__ __align__(16) KVLds sh;
  const int nb = (T + kBB - 1) / kBB;
  const int n = blockIdx.y;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l16 = lane & 15;
  const int q4 = lane >> 4;
  const size_t row0 = (size_t)n * T;
  const int stok = tid % kBB;  // staging role
  const int sgrp = tid / kBB;

  auto stage = [&](int buf, const RowLoad& rq, const RowLoad& rg, float c, float iv) {
    stage_rows(sh.q[buf], rq, stok, sgrp);
    stage_transposed(sh.qt[buf], rq, stok, sgrp);
    stage_rows(sh.g[buf], rg, stok, sgrp);
    stage_transposed(sh.gt[buf], rg, stok, sgrp);
    if (sgrp == 0) {
      sh.c[buf][stok] = c;
      sh.inv[buf][stok] = iv;
    }
  };

  // key blocks nb - 1 - x and x: every work-group does the same causal work
  for (int rep = 0; rep < 2; ++rep) {
    const int kb = rep == 0 ? nb - 1 - (int)blockIdx.x : (int)blockIdx.x;
    if (rep == 1 && kb >= nb - 1 - (int)blockIdx.x) break;
    const int kw0 = kb * kBB + 16 * w;  // this wave's first key
    const int key = kw0 + l16;          // the key this lane's score columns belong to

    // K_w and V_w as the B operands of S = Q K_w^T and dP = G V_w^T
    bf16x8 kf[2], vf[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      kf[ks] = frag_global(k, row0, key, T, ks, q4);
      vf[ks] = frag_global(v, row0, key, T, ks, q4);
    }
    f32x4 dka[4], dva[4];  // [dim tile]: lane holds keys kw0 + 4 q4 + i at dim 16 nt + l16
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) dka[nt] = dva[nt] = f32x4{0.f, 0.f, 0.f, 0.f};

    // query blocks kb .. nb - 1; block qb + 1 in registers while qb computes
    auto fetch = [&](int qb, RowLoad& rq, RowLoad& rg, float& c, float& iv) {
      const int t = qb * kBB + stok;
      rq = load_rows(q, row0, t, T, sgrp);
      rg = load_rows(g, row0, t, T, sgrp);
      c = 0.0f;
      iv = 0.0f;
      if (sgrp == 0 && t < T) {
        const float d = den[row0 + t];
        c = cvec[row0 + t];
        iv = d != 0.0f ? 1.0f / d : 0.0f;
      }
    };
    RowLoad rq, rg;
    float pc, piv;
    fetch(kb, rq, rg, pc, piv);
    stage(0, rq, rg, pc, piv);
    if (kb + 1 < nb) fetch(kb + 1, rq, rg, pc, piv);
    __syncthreads();

    for (int qb = kb; qb < nb; ++qb) {
      const int buf = (qb - kb) & 1;
      const int t0 = qb * kBB;
      // S and dP: query tiles mt (rows), this wave's 16 keys (columns)
      f32x4 sv[4], dp[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        f32x4 x = f32x4{0.f, 0.f, 0.f, 0.f}, y = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          x = mfma16x16x32(frag(sh.q[buf], 16 * mt + l16, ks, q4), kf[ks], x);
          y = mfma16x16x32(frag(sh.g[buf], 16 * mt + l16, ks, q4), vf[ks], y);
        }
        sv[mt] = x;
        dp[mt] = y;
      }
      // P = S^2 / D and dS = 2 S (dP - c) / D (zero where key > query); lane
      // (l16, q4) holds queries 16 mt + 4 q4 + i: k-slot 4 (mt & 1) + i of pair mt >> 1
      const bool diag = qb == kb;
      bf16x8 ph[2], pl[2], dh[2], dl[2];  // P and dS, each as hi + lo bf16 pieces
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        float p[8], ds[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int mt = 2 * ks + (j >> 2);
          const int i = j & 3;
          const int tl = 16 * mt + 4 * q4 + i;
          const float s = sv[mt][i];
          const float iv = sh.inv[buf][tl];
          p[j] = s * s * iv;
          ds[j] = 2.0f * s * (dp[mt][i] - sh.c[buf][tl]) * iv;
          if (diag && key > t0 + tl) p[j] = ds[j] = 0.0f;
        }
        split2(p, ph[ks], pl[ks]);
        split2(ds, dh[ks], dl[ks]);
      }
      // dV += P^T G and dK += dS^T Q over the block's 64 queries (two k-steps)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
          const bf16x8 bg = *reinterpret_cast<const bf16x8*>(&sh.gt[buf][16 * nt + l16][32 * ks + 8 * q4]);
          const bf16x8 bq = *reinterpret_cast<const bf16x8*>(&sh.qt[buf][16 * nt + l16][32 * ks + 8 * q4]);
          dva[nt] = mfma16x16x32(ph[ks], bg, dva[nt]);
          dva[nt] = mfma16x16x32(pl[ks], bg, dva[nt]);
          dka[nt] = mfma16x16x32(dh[ks], bq, dka[nt]);
          dka[nt] = mfma16x16x32(dl[ks], bq, dka[nt]);
        }
      }
      if (qb + 1 < nb) {
        stage(buf ^ 1, rq, rg, pc, piv);
        if (qb + 2 < nb) fetch(qb + 2, rq, rg, pc, piv);
      }
      __syncthreads();
    }

#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int kr = kw0 + 4 * q4 + i;
        if (kr < T) {
          Elem<Tout>::store(dk, (row0 + kr) * kBD + 16 * nt + l16, dka[nt][i]);
          Elem<Tout>::store(dv, (row0 + kr) * kBD + 16 * nt + l16, dva[nt][i]);
        }
      }
    }
  }  // rep
}

// ---------------------------------------------------------------- dQ

struct QLds {
  uint16_t k[2][kBB][kRS];    // key rows
  uint16_t kt[2][kBD][kTS];   // keys transposed (permuted columns)
  uint16_t v[2][kBB][kRS];    // value rows
};

template <typename Tout>
__global__ __launch_bounds__(kBT, 2) void quad_bwd_q_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const Tout* __restrict__ g, const float* __restrict__ den, float* __restrict__ cvec, Tout* __restrict__ dq,
    int T) {
  __shared__ __align__(16) QLds sh;
  const int nb = (T + kBB - 1) / kBB;
  const int n = blockIdx.y;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l16 = lane & 15;
  const int q4 = lane >> 4;
  const size_t row0 = (size_t)n * T;
  const int stok = tid % kBB;
  const int sgrp = tid / kBB;

  auto stage = [&](int buf, const RowLoad& rk, const RowLoad& rv) {
    stage_rows(sh.k[buf], rk, stok, sgrp);
    stage_transposed(sh.kt[buf], rk, stok, sgrp);
    stage_rows(sh.v[buf], rv, stok, sgrp);
  };
  auto fetch = [&](int kb, RowLoad& rk, RowLoad& rv) {
    rk = load_rows(k, row0, kb * kBB + stok, T, sgrp);
    rv = load_rows(v, row0, kb * kBB + stok, T, sgrp);
  };

  // query blocks nb - 1 - x and x
  for (int rep = 0; rep < 2; ++rep) {
    const int qb = rep == 0 ? nb - 1 - (int)blockIdx.x : (int)blockIdx.x;
    if (rep == 1 && qb >= nb - 1 - (int)blockIdx.x) break;
    const int qw0 = qb * kBB + 16 * w;  // this wave's first query
    const int qry = qw0 + l16;          // the query this lane's score columns belong to

    // Q_w and G_w as the B operands of S^T = K Q_w^T and dP^T = V G_w^T
    bf16x8 qf[2], gf[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      qf[ks] = frag_global(q, row0, qry, T, ks, q4);
      gf[ks] = frag_global(g, row0, qry, T, ks, q4);
    }
    float iq = 0.0f;
    if (qry < T) {
      const float d = den[row0 + qry];
      iq = d != 0.0f ? 1.0f / d : 0.0f;
    }
    float cq = 0.0f;  // c of query qry, after pass 1
    f32x4 dqa[4];     // [dim tile]: lane holds queries qw0 + 4 q4 + i at dim 16 nt + l16
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) dqa[nt] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int pass = 0; pass < 2; ++pass) {
      RowLoad rk, rv;
      fetch(0, rk, rv);
      stage(0, rk, rv);
      if (qb >= 1) fetch(1, rk, rv);
      __syncthreads();
      float cpart = 0.0f;
      for (int kb = 0; kb <= qb; ++kb) {
        const int buf = kb & 1;
        const int k0 = kb * kBB;
        // S^T and dP^T: key tiles kt (rows), this wave's 16 queries (columns)
        f32x4 st[4], dpt[4];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
          f32x4 x = f32x4{0.f, 0.f, 0.f, 0.f}, y = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            x = mfma16x16x32(frag(sh.k[buf], 16 * kt + l16, ks, q4), qf[ks], x);
            y = mfma16x16x32(frag(sh.v[buf], 16 * kt + l16, ks, q4), gf[ks], y);
          }
          st[kt] = x;
          dpt[kt] = y;
        }
        const bool diag = kb == qb;
        if (pass == 0) {
          // c: sum over this lane's keys 16 kt + 4 q4 + i of P dP
#pragma unroll
          for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float s = st[kt][i];
              float pd = s * s * iq * dpt[kt][i];
              if (diag && k0 + 16 * kt + 4 * q4 + i > qry) pd = 0.0f;
              cpart += pd;
            }
          }
        } else {
          // dS for keys 16 kt + 4 q4 + i: k-slot 4 (kt & 1) + i of pair kt >> 1
          bf16x8 dh[2], dl[2];  // dS as hi + lo bf16 pieces
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            float ds[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              const int kt = 2 * ks + (j >> 2);
              const int i = j & 3;
              const float s = st[kt][i];
              ds[j] = 2.0f * s * (dpt[kt][i] - cq) * iq;
              if (diag && k0 + 16 * kt + 4 * q4 + i > qry) ds[j] = 0.0f;
            }
            split2(ds, dh[ks], dl[ks]);
          }
          // dQ += dS K over the block's 64 keys (two k-steps)
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) {
              const bf16x8 bk = *reinterpret_cast<const bf16x8*>(&sh.kt[buf][16 * nt + l16][32 * ks + 8 * q4]);
              dqa[nt] = mfma16x16x32(dh[ks], bk, dqa[nt]);
              dqa[nt] = mfma16x16x32(dl[ks], bk, dqa[nt]);
            }
          }
        }
        if (kb + 1 <= qb) {
          stage(buf ^ 1, rk, rv);
          if (kb + 2 <= qb) fetch(kb + 2, rk, rv);
        }
        __syncthreads();
      }
      if (pass == 0) {
        // the four lane quarters of query qry hold disjoint keys
        cpart += __shfl_xor(cpart, 16, 64);
        cpart += __shfl_xor(cpart, 32, 64);
        cq = cpart;
        if (q4 == 0 && qry < T) cvec[row0 + qry] = cq;
      }
    }

#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int qr = qw0 + 4 * q4 + i;
        if (qr < T) Elem<Tout>::store(dq, (row0 + qr) * kBD + 16 * nt + l16, dqa[nt][i]);
      }
    }
  }  // rep
}

template <typename Tout>
hipError_t launch_bwd(const QuadBwdArgs& a, float* cvec, hipStream_t st) {
  const int nb = (a.T + kBB - 1) / kBB;
  const dim3 grid((nb + 1) / 2, a.N);
  // c comes out of the dQ kernel's first pass; the dK/dV kernel reads it
  hipLaunchKernelGGL(quad_bwd_q_kernel<Tout>, grid, dim3(kBT), 0, st, static_cast<const uint16_t*>(a.q),
                     static_cast<const uint16_t*>(a.k), static_cast<const uint16_t*>(a.v),
                     static_cast<const Tout*>(a.dout), a.den, cvec, static_cast<Tout*>(a.dq), a.T);
  hipLaunchKernelGGL(quad_bwd_kv_kernel<Tout>, grid, dim3(kBT), 0, st, static_cast<const uint16_t*>(a.q),
                     static_cast<const uint16_t*>(a.k), static_cast<const uint16_t*>(a.v),
                     static_cast<const Tout*>(a.dout), cvec, a.den, static_cast<Tout*>(a.dk),
                     static_cast<Tout*>(a.dv), a.T);
  return hipGetLastError();
}

}  // namespace

size_t prefill_quad_bwd_workspace(const QuadBwdArgs& a) { return align_up((size_t)a.N * a.T * sizeof(float)); }

hipError_t prefill_quad_bwd_launch(const QuadBwdArgs& a, void* ws, hipStream_t st) {
  if (a.T < 1) return hipErrorInvalidValue;
  float* cvec = static_cast<float*>(ws);
  prof_begin(st);
  const hipError_t e = a.out_bf16 ? launch_bwd<uint16_t>(a, cvec, st) : launch_bwd<float>(a, cvec, st);
  prof_end(st);
  return e;
}

}  // namespace kla
