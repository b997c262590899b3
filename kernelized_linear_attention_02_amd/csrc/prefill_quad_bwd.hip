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
// Kernels:
//   q    one work-group per head and pair of 128-query blocks, wave w owning
//        queries 32 w .. 32 w + 31 as two 16-query tiles, launched twice.
//        Pass 1 over the key blocks up to the block's last query: S^T = K Q_w^T and dP^T = V G_w^T on MFMA
//        16x16x32 bf16, c_t = sum_i P_ti dP_ti in float32 (stored for the
//        kv kernel). Pass 2: the same products, dS, and dQ += dS K;
//   kv   one work-group per head and pair of 128-key blocks (x, last - x),
//        wave w owning keys 32 w .. 32 w + 31 as two 16-key tiles (every
//        LDS fragment read then serves both). For every query block at or
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

constexpr int kKT = 2;                 // 16-key tiles per wave in the dK/dV kernel
constexpr int kKB = 16 * kKT * kBW;    // keys per dK/dV work-group

template <typename Tout>
__global__ __launch_bounds__(kBT, 2) void quad_bwd_kv_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const Tout* __restrict__ g, const float* __restrict__ cvec, const float* __restrict__ den,
    Tout* __restrict__ dk, Tout* __restrict__ dv, int T) {
  __shared__ __align__(16) KVLds sh;
  const int nkb = (T + kKB - 1) / kKB;  // key blocks
  const int nqb = (T + kBB - 1) / kBB;  // query blocks
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

  // key blocks nkb - 1 - x and x: every work-group does the same causal work
  for (int rep = 0; rep < 2; ++rep) {
    const int kb = rep == 0 ? nkb - 1 - (int)blockIdx.x : (int)blockIdx.x;
    if (rep == 1 && kb >= nkb - 1 - (int)blockIdx.x) break;
    const int kw0 = kb * kKB + 16 * kKT * w;  // this wave's first key; tile kk: keys kw0 + 16 kk + l16

    // K_w and V_w as the B operands of S = Q K_w^T and dP = G V_w^T
    bf16x8 kf[kKT][2], vf[kKT][2];
#pragma unroll
    for (int kk = 0; kk < kKT; ++kk)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        kf[kk][ks] = frag_global(k, row0, kw0 + 16 * kk + l16, T, ks, q4);
        vf[kk][ks] = frag_global(v, row0, kw0 + 16 * kk + l16, T, ks, q4);
      }
    // [key tile][dim tile]: lane holds keys kw0 + 16 kk + 4 q4 + i at dim 16 nt + l16
    f32x4 dka[kKT][4], dva[kKT][4];
#pragma unroll
    for (int kk = 0; kk < kKT; ++kk)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) dka[kk][nt] = dva[kk][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

    // query blocks from the one holding the key block's first key; block
    // qb + 1 in registers while qb computes
    const int qb0 = kb * kKB / kBB;
    RowLoad rq, rg;
    float pc, piv;
    fetch(qb0, rq, rg, pc, piv);
    stage(0, rq, rg, pc, piv);
    if (qb0 + 1 < nqb) fetch(qb0 + 1, rq, rg, pc, piv);
    __syncthreads();

    for (int qb = qb0; qb < nqb; ++qb) {
      const int buf = (qb - qb0) & 1;
      const int t0 = qb * kBB;
      const bool diag = t0 < (kb + 1) * kKB;  // the block reaches keys above some of its queries
      // S and dP: query tiles mt (rows), key tile kk (columns); each row
      // fragment read serves every key tile
      f32x4 sv[kKT][4], dp[kKT][4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        bf16x8 aq[2], ag[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          aq[ks] = frag(sh.q[buf], 16 * mt + l16, ks, q4);
          ag[ks] = frag(sh.g[buf], 16 * mt + l16, ks, q4);
        }
#pragma unroll
        for (int kk = 0; kk < kKT; ++kk) {
          f32x4 x = f32x4{0.f, 0.f, 0.f, 0.f}, y = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            x = mfma16x16x32(aq[ks], kf[kk][ks], x);
            y = mfma16x16x32(ag[ks], vf[kk][ks], y);
          }
          sv[kk][mt] = x;
          dp[kk][mt] = y;
        }
      }
      // P = S^2 / D and dS = 2 S (dP - c) / D (zero where key > query); lane
      // (l16, q4) holds queries 16 mt + 4 q4 + i: k-slot 4 (mt & 1) + i of pair mt >> 1
      bf16x8 ph[kKT][2], pl[kKT][2], dh[kKT][2], dl[kKT][2];  // hi + lo bf16 pieces
#pragma unroll
      for (int kk = 0; kk < kKT; ++kk) {
        const int key = kw0 + 16 * kk + l16;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          float p[8], ds[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int mt = 2 * ks + (j >> 2);
            const int i = j & 3;
            const int tl = 16 * mt + 4 * q4 + i;
            const float s = sv[kk][mt][i];
            const float iv = sh.inv[buf][tl];
            p[j] = s * s * iv;
            ds[j] = 2.0f * s * (dp[kk][mt][i] - sh.c[buf][tl]) * iv;
            if (diag && key > t0 + tl) p[j] = ds[j] = 0.0f;
          }
          split2(p, ph[kk][ks], pl[kk][ks]);
          split2(ds, dh[kk][ks], dl[kk][ks]);
        }
      }
      // dV += P^T G and dK += dS^T Q over the block's 64 queries (two k-steps);
      // each transposed fragment read serves every key tile
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
          const bf16x8 bg = *reinterpret_cast<const bf16x8*>(&sh.gt[buf][16 * nt + l16][32 * ks + 8 * q4]);
          const bf16x8 bq = *reinterpret_cast<const bf16x8*>(&sh.qt[buf][16 * nt + l16][32 * ks + 8 * q4]);
#pragma unroll
          for (int kk = 0; kk < kKT; ++kk) {
            dva[kk][nt] = mfma16x16x32(ph[kk][ks], bg, dva[kk][nt]);
            dva[kk][nt] = mfma16x16x32(pl[kk][ks], bg, dva[kk][nt]);
            dka[kk][nt] = mfma16x16x32(dh[kk][ks], bq, dka[kk][nt]);
            dka[kk][nt] = mfma16x16x32(dl[kk][ks], bq, dka[kk][nt]);
          }
        }
      }
      if (qb + 1 < nqb) {
        stage(buf ^ 1, rq, rg, pc, piv);
        if (qb + 2 < nqb) fetch(qb + 2, rq, rg, pc, piv);
      }
      __syncthreads();
    }

#pragma unroll
    for (int kk = 0; kk < kKT; ++kk)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int kr = kw0 + 16 * kk + 4 * q4 + i;
          if (kr < T) {
            Elem<Tout>::store(dk, (row0 + kr) * kBD + 16 * nt + l16, dka[kk][nt][i]);
            Elem<Tout>::store(dv, (row0 + kr) * kBD + 16 * nt + l16, dva[kk][nt][i]);
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

constexpr int kQT = 2;                 // 16-query tiles per wave in the dQ kernel
constexpr int kQB = 16 * kQT * kBW;    // queries per dQ work-group

// PASS 0 stores c for the block's queries; PASS 1 reads it back and forms dQ.
template <int PASS, typename Tout>
__global__ __launch_bounds__(kBT, 2) void quad_bwd_q_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const Tout* __restrict__ g, const float* __restrict__ den, float* __restrict__ cvec, Tout* __restrict__ dq,
    int T) {
  __shared__ __align__(16) QLds sh;
  const int nqb = (T + kQB - 1) / kQB;  // query blocks
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
    if (PASS == 1) stage_transposed(sh.kt[buf], rk, stok, sgrp);  // for dS K only
    stage_rows(sh.v[buf], rv, stok, sgrp);
  };
  auto fetch = [&](int kb, RowLoad& rk, RowLoad& rv) {
    rk = load_rows(k, row0, kb * kBB + stok, T, sgrp);
    rv = load_rows(v, row0, kb * kBB + stok, T, sgrp);
  };

  // query blocks nqb - 1 - x and x
  for (int rep = 0; rep < 2; ++rep) {
    const int qb = rep == 0 ? nqb - 1 - (int)blockIdx.x : (int)blockIdx.x;
    if (rep == 1 && qb >= nqb - 1 - (int)blockIdx.x) break;
    const int qw0 = qb * kQB + 16 * kQT * w;  // this wave's first query; tile tq: queries qw0 + 16 tq + l16
    const int last = min(T, (qb + 1) * kQB) - 1;  // the block's last query
    const int nkb = last / kBB + 1;               // key blocks with keys <= last

    // Q_w and G_w as the B operands of S^T = K Q_w^T and dP^T = V G_w^T
    bf16x8 qf[kQT][2], gf[kQT][2];
    float iq[kQT];
#pragma unroll
    for (int tq = 0; tq < kQT; ++tq) {
      const int qry = qw0 + 16 * tq + l16;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        qf[tq][ks] = frag_global(q, row0, qry, T, ks, q4);
        gf[tq][ks] = frag_global(g, row0, qry, T, ks, q4);
      }
      iq[tq] = 0.0f;
      if (qry < T) {
        const float d = den[row0 + qry];
        iq[tq] = d != 0.0f ? 1.0f / d : 0.0f;
      }
    }
    float cq[kQT] = {};  // c of the lane's queries (PASS 1)
    if (PASS == 1) {
#pragma unroll
      for (int tq = 0; tq < kQT; ++tq) {
        const int qry = qw0 + 16 * tq + l16;
        if (qry < T) cq[tq] = cvec[row0 + qry];
      }
    }
    f32x4 dqa[kQT][4];   // lane holds queries qw0 + 16 tq + 4 q4 + i at dim 16 nt + l16
#pragma unroll
    for (int tq = 0; tq < kQT; ++tq)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) dqa[tq][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

    {
      RowLoad rk, rv;
      fetch(0, rk, rv);
      stage(0, rk, rv);
      if (nkb > 1) fetch(1, rk, rv);
      __syncthreads();
      float cpart[kQT] = {};
      for (int kb = 0; kb < nkb; ++kb) {
        const int buf = kb & 1;
        const int k0 = kb * kBB;
        const bool diag = k0 + kBB - 1 > qw0;  // some key of the block is above a query of the wave
        // S^T and dP^T: key tiles kt (rows), query tile tq (columns); each row
        // fragment read serves every query tile
        f32x4 st[kQT][4], dpt[kQT][4];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
          bf16x8 ak[2], av[2];
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            ak[ks] = frag(sh.k[buf], 16 * kt + l16, ks, q4);
            av[ks] = frag(sh.v[buf], 16 * kt + l16, ks, q4);
          }
#pragma unroll
          for (int tq = 0; tq < kQT; ++tq) {
            f32x4 x = f32x4{0.f, 0.f, 0.f, 0.f}, y = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
              x = mfma16x16x32(ak[ks], qf[tq][ks], x);
              y = mfma16x16x32(av[ks], gf[tq][ks], y);
            }
            st[tq][kt] = x;
            dpt[tq][kt] = y;
          }
        }
        if (PASS == 0) {
          // c: sum over this lane's keys 16 kt + 4 q4 + i of P dP
#pragma unroll
          for (int tq = 0; tq < kQT; ++tq) {
            const int qry = qw0 + 16 * tq + l16;
#pragma unroll
            for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const float s = st[tq][kt][i];
                float pd = s * s * iq[tq] * dpt[tq][kt][i];
                if (diag && k0 + 16 * kt + 4 * q4 + i > qry) pd = 0.0f;
                cpart[tq] += pd;
              }
            }
          }
        } else {
          // per k-step: dS for keys 32 ks + 16 (j >> 2) + 4 q4 + (j & 3) as hi + lo
          // bf16 pieces (k-slot j), then dQ += dS K over those 32 keys; each
          // transposed fragment read serves every query tile
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            bf16x8 dh[kQT], dl[kQT];
#pragma unroll
            for (int tq = 0; tq < kQT; ++tq) {
              const int qry = qw0 + 16 * tq + l16;
              float ds[8];
#pragma unroll
              for (int j = 0; j < 8; ++j) {
                const int kt = 2 * ks + (j >> 2);
                const int i = j & 3;
                const float s = st[tq][kt][i];
                ds[j] = 2.0f * s * (dpt[tq][kt][i] - cq[tq]) * iq[tq];
                if (diag && k0 + 16 * kt + 4 * q4 + i > qry) ds[j] = 0.0f;
              }
              split2(ds, dh[tq], dl[tq]);
            }
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) {
              const bf16x8 bk = *reinterpret_cast<const bf16x8*>(&sh.kt[buf][16 * nt + l16][32 * ks + 8 * q4]);
#pragma unroll
              for (int tq = 0; tq < kQT; ++tq) {
                dqa[tq][nt] = mfma16x16x32(dh[tq], bk, dqa[tq][nt]);
                dqa[tq][nt] = mfma16x16x32(dl[tq], bk, dqa[tq][nt]);
              }
            }
          }
        }
        if (kb + 1 < nkb) {
          stage(buf ^ 1, rk, rv);
          if (kb + 2 < nkb) fetch(kb + 2, rk, rv);
        }
        __syncthreads();
      }
      if (PASS == 0) {
        // the four lane quarters of a query hold disjoint keys
#pragma unroll
        for (int tq = 0; tq < kQT; ++tq) {
          float c = cpart[tq];
          c += __shfl_xor(c, 16, 64);
          c += __shfl_xor(c, 32, 64);
          cq[tq] = c;
          const int qry = qw0 + 16 * tq + l16;
          if (q4 == 0 && qry < T) cvec[row0 + qry] = c;
        }
      }
    }

    if (PASS == 1) {
#pragma unroll
      for (int tq = 0; tq < kQT; ++tq)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int qr = qw0 + 16 * tq + 4 * q4 + i;
            if (qr < T) Elem<Tout>::store(dq, (row0 + qr) * kBD + 16 * nt + l16, dqa[tq][nt][i]);
          }
        }
    }
  }  // rep
}

template <typename Tout>
hipError_t launch_bwd(const QuadBwdArgs& a, float* cvec, hipStream_t st) {
  const int nqb = (a.T + kQB - 1) / kQB;
  const int nkb = (a.T + kKB - 1) / kKB;
  // c comes out of the dQ kernel's first pass; the second and the dK/dV kernel read it
  const dim3 qgrid((nqb + 1) / 2, a.N);
  hipLaunchKernelGGL((quad_bwd_q_kernel<0, Tout>), qgrid, dim3(kBT), 0, st, static_cast<const uint16_t*>(a.q),
                     static_cast<const uint16_t*>(a.k), static_cast<const uint16_t*>(a.v),
                     static_cast<const Tout*>(a.dout), a.den, cvec, static_cast<Tout*>(a.dq), a.T);
  hipLaunchKernelGGL((quad_bwd_q_kernel<1, Tout>), qgrid, dim3(kBT), 0, st, static_cast<const uint16_t*>(a.q),
                     static_cast<const uint16_t*>(a.k), static_cast<const uint16_t*>(a.v),
                     static_cast<const Tout*>(a.dout), a.den, cvec, static_cast<Tout*>(a.dq), a.T);
  hipLaunchKernelGGL(quad_bwd_kv_kernel<Tout>, dim3((nkb + 1) / 2, a.N), dim3(kBT), 0, st,
                     static_cast<const uint16_t*>(a.q),
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
