// LoLA's three memories, token by token (LoLA page, "Estratégia de
// Inferência": the token-by-token mode of items 1-4; "Metodologia" items
// 1-3 for the memories).
//
// One call advances every head-state by one token t (the number of tokens
// it has seen). With window W and cache size lambda:
//   1. token e = t - W - 1 leaves the window when t > W. While the cache has
//      room it joins the cache; once the cache is full, e and the lambda
//      cached pairs are scored by the self-recall error against (H, s), the
//      lambda highest (score desc, token id asc) stay and the lowest one, r,
//      is folded into the state: H += phi(k_r) v_r^T, s += phi(k_r);
//   2. the query reads one jointly normalised mixture of the window
//      [max(0, t - W), t] (softmax weights e^{a q.k}), the cache (the same
//      weights) and the linear state (phi(q)^T H, phi(q)^T s + eps), as the
//      blocked hybrid prefill does with refresh = 1;
//   3. token t enters the window ring in the row the evicted token left.
//
// Deferred fold: the fold of step 1 is not written into (H, s) by the call
// that decides it. The rejected pair is kept in the state as the pending
// pair (pend_k, pend_v) and folded by the next call's pass over H, which has
// to read and write H anyway; the call's own readout adds the fold in closed
// form, phi(q)^T phi(k_r) = (q . k_r)^2:
//   num += (q . k_r)^2 v_r,   den += (q . k_r)^2.
// H is then read and written once per token. A zero pending pair folds
// nothing (phi(0) = 0).
//
// Kernels (all counts are known on the host from t):
//   state pass  d_qk = d_v = 64, cache <= 128: one work-group per
//               head-state streams H once: pending fold, linear readout of
//               q, and the self-recall numerators of the cache candidates on
//               the bf16 matrix cores (float32-faithful split products) and
//               of the evicted pair on the vector units;
//   other shapes: a fold + readout pass over H, then the shared float32
//               scoring block over the cache + evicted candidates;
//   mix         per head-state: the rejected pair (lowest (score, -id)), cache
//               update, the closed-form fold term, the window and cache
//               softmax (online maximum), the joint division, the window
//               insert, and the new pending pair.
#include <algorithm>

#include "kla_device.hpp"
#include "kla_internal.hpp"
#include "mfma_bf16.hpp"
#include "sre_block.hpp"

namespace kla {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kKeyTile = kThreads;  // softmax keys scored per pass (online max across passes)

// Block-wide reductions (kThreads threads); every thread gets the result.
__device__ __forceinline__ float block_sum(float x, float* red) {
  x = wave_sum(x);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  float r = 0.0f;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) r += red[i];
  __syncthreads();
  return r;
}
__device__ __forceinline__ float block_max(float x, float* red) {
  x = wave_max(x);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int i = 1; i < kWaves; ++i) r = fmaxf(r, red[i]);
  __syncthreads();
  return r;
}

// ---------------------------------------------------------------- generic state pass

// One work-group per head-state: the pending pair is folded into (H, s)
// and cleared; with READ, lin[n] = (phi(q)^T H, phi(q)^T s) of the folded
// state (denominator without eps) at lin[n * lstride + 0 .. d_v].
template <int DQK, int DV, typename Tin, bool READ>
__global__ __launch_bounds__(kThreads) void hdec_fold_kernel(
    float* __restrict__ H, float* __restrict__ s, float* __restrict__ pend_k, float* __restrict__ pend_v,
    const Tin* __restrict__ q, float* __restrict__ lin, int lstride) {
  constexpr int D = phi_dim(DQK);
  constexpr int G = kThreads / DV;
  __shared__ float pq[READ ? D : 1];
  __shared__ float pk[D];
  __shared__ float qv[DQK], kv[DQK], vv[DV];
  __shared__ uint16_t tab[D];
  __shared__ float num[G][DV];
  __shared__ float red[kWaves];
  const int n = blockIdx.x;
  const int tid = threadIdx.x;
  const int c = tid % DV;
  const int g = tid / DV;
  for (int d = tid; d < DQK; d += kThreads) {
    if (READ) qv[d] = Elem<Tin>::load(q, (size_t)n * DQK + d);
    kv[d] = pend_k[(size_t)n * DQK + d];
  }
  for (int d = tid; d < DV; d += kThreads) vv[d] = pend_v[(size_t)n * DV + d];
  build_phi_table(tab, 0, D, DQK);
  __syncthreads();
  for (int f = tid; f < D; f += kThreads) {
    pk[f] = phi_of(kv, tab[f]);
    if (READ) pq[f] = phi_of(qv, tab[f]);
  }
  __syncthreads();
  float* Hn = H + (size_t)n * D * DV;
  float* sn = s + (size_t)n * D;
  const float vc = vv[c];
  float acc = 0.0f;
#pragma unroll 8
  for (int f = g; f < D; f += G) {
    const float h = Hn[(size_t)f * DV + c] + pk[f] * vc;
    Hn[(size_t)f * DV + c] = h;
    if (READ) acc += pq[f] * h;
  }
  float den = 0.0f;
  for (int f = tid; f < D; f += kThreads) {
    const float x = sn[f] + pk[f];
    sn[f] = x;
    if (READ) den += pq[f] * x;
  }
  if (READ) {
    num[g][c] = acc;
    const float dsum = block_sum(den, red);  // its barriers also publish num
    if (g == 0) {
      float x = 0.0f;
#pragma unroll
      for (int i = 0; i < G; ++i) x += num[i][c];
      lin[(size_t)n * lstride + c] = x;
    }
    if (tid == 0) lin[(size_t)n * lstride + DV] = dsum;
  }
  // every read of the pending pair went through LDS before the first barrier
  for (int d = tid; d < DQK; d += kThreads) pend_k[(size_t)n * DQK + d] = 0.0f;
  for (int d = tid; d < DV; d += kThreads) pend_v[(size_t)n * DV + d] = 0.0f;
}

// Self-recall error of the lambda + 1 candidates (cache rows, then the
// evicted window row) against the folded state, in float32.
template <int DQK, int DV>
__global__ __launch_bounds__(kThreads) void hdec_score_kernel(
    const float* __restrict__ H, const float* __restrict__ s, const float* __restrict__ cache_k,
    const float* __restrict__ cache_v, const float* __restrict__ win_k, const float* __restrict__ win_v,
    int lambda, int wrows, int slot, float* __restrict__ scores, int sstride, float eps) {
  constexpr int D = phi_dim(DQK);
  __shared__ SreShared<DQK, DV> sh;
  const int n = blockIdx.y;
  auto load_k = [&](int c, int d) {
    return c < lambda ? cache_k[((size_t)n * lambda + c) * DQK + d]
                      : win_k[((size_t)n * wrows + slot) * DQK + d];
  };
  auto load_v = [&](int c, int d) {
    return c < lambda ? cache_v[((size_t)n * lambda + c) * DV + d]
                      : win_v[((size_t)n * wrows + slot) * DV + d];
  };
  sre_block<DQK, DV>(sh, H + (size_t)n * D * DV, s + (size_t)n * D, blockIdx.x * 64, lambda + 1, load_k,
                     load_v, scores + (size_t)n * sstride, eps);
}

// ---------------------------------------------------------------- matrix-core state pass

constexpr int kFD = 64;
constexpr int kFDim = kFD * (kFD + 1) / 2;  // 2080
constexpr int kFMaxCache = 128;
constexpr int kKS = kFD + 4;                // padded LDS key rows (16-byte aligned)
// Feature order of the pass: 8 x 8 blocks (A, B), A <= B, of the pairs
// (a, b), a <= b; a block is two MFMA k-steps ("tiles") of 32 features. In
// tile t of block (A, B) the lane quarter q4 takes a = 8A + 4t + q4 and
// b = 8B .. 8B + 7: eight consecutive state rows. Diagonal blocks hold 36
// pairs in 64 slots; the slots with b < a are zero rows.
constexpr int kBlocks = 8 * 9 / 2;          // 36
constexpr int kFTiles = 2 * kBlocks;        // 72

struct BlockTable {
  uint8_t A[kBlocks], B[kBlocks];
  constexpr BlockTable() : A{}, B{} {
    int i = 0;
    for (int a = 0; a < 8; ++a)
      for (int b = a; b < 8; ++b) {
        A[i] = static_cast<uint8_t>(a);
        B[i] = static_cast<uint8_t>(b);
        ++i;
      }
  }
};
__constant__ BlockTable kBlockTab = BlockTable();

struct StateLds {
  alignas(16) float qs[kFD];
  alignas(16) float pk[kFD];
  alignas(16) float pv[kFD];
  alignas(16) float ek[kFD];
  union {
    float ck[kFMaxCache][kKS];                // cache keys (tile loop)
    float4 red[kFMaxCache / 16][4][64];       // numerator partials (after it)
  };
  float den[kWaves][kFMaxCache];
  float onum[kWaves][kFD];
  float enm[kWaves][kFD];
  float oden[kWaves];
  float eden[kWaves];
};

// Where a lane's eight features of tile T lie: first state row f0 (row of
// (a, 8B)), the first valid slot jmin, the diagonal slot jd (b == a; -1 off
// the diagonal), and the key coordinates a and 8B.
struct TileCoords {
  int f0, jmin, jd, a, b0;
};
__device__ __forceinline__ TileCoords tile_coords(int T, int q4) {
  const int blk = T >> 1;
  const int A = kBlockTab.A[blk];
  const int B = kBlockTab.B[blk];
  TileCoords c;
  c.a = 8 * A + 4 * (T & 1) + q4;
  c.b0 = 8 * B;
  c.f0 = c.a * kFD - c.a * (c.a - 1) / 2 + (c.b0 - c.a);
  c.jmin = A == B ? c.a - c.b0 : 0;
  c.jd = A == B ? c.a - c.b0 : -1;
  return c;
}

// phi over a lane's eight features of one vector x in LDS: out_j = c_j x_a x_{b0+j}.
__device__ __forceinline__ void phi8(const float* x, const TileCoords& tc, float (&out)[8]) {
  const float xa = x[tc.a];
  const float4 lo = *reinterpret_cast<const float4*>(x + tc.b0);
  const float4 hi = *reinterpret_cast<const float4*>(x + tc.b0 + 4);
  const float xs = xa * kSqrt2;
  const float xb[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
#pragma unroll
  for (int j = 0; j < 8; ++j) out[j] = (j == tc.jd ? xa : xs) * xb[j];
}

// One work-group per head-state; its four waves take the 72 tiles in turn.
// A lane (l16, q4) holds its eight state rows of a tile at columns
// 4*l16 .. 4*l16+3 (16-byte loads), adds the pending fold, writes them back
// and accumulates the float32 readouts of q and of the evicted key. The same
// registers are the B operand of the cache candidates' numerators
// phi(K_c) H on the matrix cores: the state is split exactly into three bf16
// pieces, the candidate features into two, and the product is
// p0 (h0 + h1 + h2) + p1 h0 with float32 accumulation. MT 16-row candidate
// blocks (0: no scoring in this call).
template <int MT, typename Tin>
__global__ __launch_bounds__(kThreads, 1) void hdec_state_kernel(
    float* __restrict__ H, float* __restrict__ s, const float* __restrict__ pend_k,
    const float* __restrict__ pend_v, const Tin* __restrict__ q, const float* __restrict__ cache_k,
    const float* __restrict__ cache_v, const float* __restrict__ win_k, const float* __restrict__ win_v,
    int wrows, int slot, int lambda, float* __restrict__ scores, int sstride, float* __restrict__ lin,
    int lstride, float eps) {
  constexpr int MTA = MT > 0 ? MT : 1;
  __shared__ __align__(16) StateLds sh;
  const int n = blockIdx.x;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l16 = lane & 15;
  const int q4 = lane >> 4;
  float* Hn = H + (size_t)n * kFDim * kFD;
  float* sn = s + (size_t)n * kFDim;

  // rows of slots j < jmin are not features: zero, never loaded or stored
  auto load_tile = [&](const TileCoords& tc, float4 (&h)[8], float (&sj)[8]) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      h[j] = make_float4(0.f, 0.f, 0.f, 0.f);
      sj[j] = 0.0f;
      if (j >= tc.jmin) {
        h[j] = *reinterpret_cast<const float4*>(Hn + (size_t)(tc.f0 + j) * kFD + 4 * l16);
        sj[j] = sn[tc.f0 + j];
      }
    }
  };
  TileCoords tc = tile_coords(w, q4);
  float4 h[8];
  float sj[8];
  load_tile(tc, h, sj);

  if (tid < kFD) {
    sh.qs[tid] = Elem<Tin>::load(q, (size_t)n * kFD + tid);
    sh.pk[tid] = pend_k[(size_t)n * kFD + tid];
    sh.pv[tid] = pend_v[(size_t)n * kFD + tid];
    if (MT > 0) sh.ek[tid] = win_k[((size_t)n * wrows + slot) * kFD + tid];
  }
  if (MT > 0) {
    for (int i = tid; i < 16 * MT * (kFD / 4); i += kThreads) {
      const int c = i / (kFD / 4);
      const int d4 = i % (kFD / 4);
      float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
      if (c < lambda) x = *reinterpret_cast<const float4*>(cache_k + ((size_t)n * lambda + c) * kFD + 4 * d4);
      *reinterpret_cast<float4*>(&sh.ck[c][4 * d4]) = x;
    }
  }
  __syncthreads();

  const float4 v4 = *reinterpret_cast<const float4*>(&sh.pv[4 * l16]);
  f32x4 acc[MTA][4];
#pragma unroll
  for (int mt = 0; mt < MTA; ++mt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float dacc[MTA];
#pragma unroll
  for (int mt = 0; mt < MTA; ++mt) dacc[mt] = 0.0f;
  float4 oacc = make_float4(0.f, 0.f, 0.f, 0.f);
  float4 eacc = make_float4(0.f, 0.f, 0.f, 0.f);
  float oden = 0.0f, eden = 0.0f;

#pragma unroll 1
  for (int T = w; T < kFTiles; T += kWaves) {
    float4 hn[8];
    float sjn[8];
    const bool more = T + kWaves < kFTiles;
    TileCoords tcn = tc;
    if (more) {
      tcn = tile_coords(T + kWaves, q4);
      load_tile(tcn, hn, sjn);
    }

    float pk[8], pq[8], pe[8];
    phi8(sh.pk, tc, pk);
    phi8(sh.qs, tc, pq);
    if (MT > 0) phi8(sh.ek, tc, pe);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j >= tc.jmin) {
        h[j].x += pk[j] * v4.x;
        h[j].y += pk[j] * v4.y;
        h[j].z += pk[j] * v4.z;
        h[j].w += pk[j] * v4.w;
        sj[j] += pk[j];
        *reinterpret_cast<float4*>(Hn + (size_t)(tc.f0 + j) * kFD + 4 * l16) = h[j];
      }
      oacc.x += pq[j] * h[j].x;
      oacc.y += pq[j] * h[j].y;
      oacc.z += pq[j] * h[j].z;
      oacc.w += pq[j] * h[j].w;
      oden += pq[j] * sj[j];
      if (MT > 0) {
        eacc.x += pe[j] * h[j].x;
        eacc.y += pe[j] * h[j].y;
        eacc.z += pe[j] * h[j].z;
        eacc.w += pe[j] * h[j].w;
        eden += pe[j] * sj[j];
      }
    }
    // lane l16 = j of each quarter writes s of slot j: a contiguous 32-byte run
    {
      float x = sj[0];
#pragma unroll
      for (int j = 1; j < 8; ++j) x = l16 == j ? sj[j] : x;
      if (l16 < 8 && l16 >= tc.jmin) sn[tc.f0 + l16] = x;
    }

    if (MT > 0) {
      bf16x8 ahi[MTA], alo[MTA];
#pragma unroll
      for (int mt = 0; mt < MTA; ++mt) {
        float p[8];
        phi8(sh.ck[16 * mt + l16], tc, p);
        float dd = 0.0f;
#pragma unroll
        for (int j = 0; j < 8; ++j) dd += p[j] * sj[j];
        dacc[mt] += dd;
        split2(p, ahi[mt], alo[mt]);
      }
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        float x[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = comp(h[j], nt);
        bf16x8 b0, b1, b2;
        split3(x, b0, b1, b2);
#pragma unroll
        for (int mt = 0; mt < MTA; ++mt) {
          acc[mt][nt] = mfma16x16x32(ahi[mt], b0, acc[mt][nt]);
          acc[mt][nt] = mfma16x16x32(ahi[mt], b1, acc[mt][nt]);
          acc[mt][nt] = mfma16x16x32(ahi[mt], b2, acc[mt][nt]);
          acc[mt][nt] = mfma16x16x32(alo[mt], b0, acc[mt][nt]);
        }
      }
    }
    if (more) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        h[j] = hn[j];
        sj[j] = sjn[j];
      }
      tc = tcn;
    }
  }

  // ---- vector-unit readouts: sum over the lane quarters, then over waves
  {
    float ox[4] = {oacc.x, oacc.y, oacc.z, oacc.w};
    float ex[4] = {eacc.x, eacc.y, eacc.z, eacc.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ox[i] += __shfl_xor(ox[i], 16, 64);
      ox[i] += __shfl_xor(ox[i], 32, 64);
      if (MT > 0) {
        ex[i] += __shfl_xor(ex[i], 16, 64);
        ex[i] += __shfl_xor(ex[i], 32, 64);
      }
    }
    oden += __shfl_xor(oden, 16, 64);
    oden += __shfl_xor(oden, 32, 64);
    if (MT > 0) {
      eden += __shfl_xor(eden, 16, 64);
      eden += __shfl_xor(eden, 32, 64);
    }
    if (q4 == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sh.onum[w][4 * l16 + i] = ox[i];
        if (MT > 0) sh.enm[w][4 * l16 + i] = ex[i];
      }
    }
    if (lane == 0) {
      sh.oden[w] = oden;
      if (MT > 0) sh.eden[w] = eden;
    }
  }
  if (MT > 0) {
#pragma unroll
    for (int mt = 0; mt < MTA; ++mt) {
      float d = dacc[mt];
      d += __shfl_xor(d, 16, 64);
      d += __shfl_xor(d, 32, 64);
      if (q4 == 0) sh.den[w][16 * mt + l16] = d;
    }
  }
  // numerators: the waves add into the LDS copy in turn and the last one keeps
  // the sum (the first barrier also ends every read of the cache keys, whose
  // LDS the partials reuse); with MT = 0 this only publishes the readouts
  for (int r = 0; r < kWaves; ++r) {
    __syncthreads();
    if (MT > 0 && w == r) {
#pragma unroll
      for (int mt = 0; mt < MTA; ++mt)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
          f32x4 x = acc[mt][nt];
          if (r > 0) {
            const float4 y = sh.red[mt][nt][lane];
            x[0] += y.x;
            x[1] += y.y;
            x[2] += y.z;
            x[3] += y.w;
          }
          acc[mt][nt] = x;
          if (r + 1 < kWaves) sh.red[mt][nt][lane] = make_float4(x[0], x[1], x[2], x[3]);
        }
    }
  }
  if (w == 0) {
    // wave 0: the linear readout of q, then the evicted pair's score
    float num = 0.0f, den = 0.0f;
#pragma unroll
    for (int r = 0; r < kWaves; ++r) {
      num += sh.onum[r][lane];
      den += sh.oden[r];
    }
    lin[(size_t)n * lstride + lane] = num;
    if (lane == 0) lin[(size_t)n * lstride + kFD] = den;
    if (MT > 0) {
      float en = 0.0f, ed = eps;
#pragma unroll
      for (int r = 0; r < kWaves; ++r) {
        en += sh.enm[r][lane];
        ed += sh.eden[r];
      }
      const float pred = ed != 0.0f ? en / ed : 0.0f;
      const float diff = pred - win_v[((size_t)n * wrows + slot) * kFD + lane];
      const float err = wave_sum(diff * diff);
      if (lane == 0) scores[(size_t)n * sstride + lambda] = err;
    }
  }
  if (MT > 0 && w == kWaves - 1) {
    // lane (l16, q4) holds candidates 16*mt + 4*q4 + i at state columns 4*l16 + nt
#pragma unroll
    for (int mt = 0; mt < MTA; ++mt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c = 16 * mt + 4 * q4 + i;
        const bool live = c < lambda;
        float den = eps;
#pragma unroll
        for (int r = 0; r < kWaves; ++r) den += sh.den[r][c];
        float4 vc = make_float4(0.f, 0.f, 0.f, 0.f);
        if (live) vc = *reinterpret_cast<const float4*>(cache_v + ((size_t)n * lambda + c) * kFD + 4 * l16);
        float err = 0.0f;
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
          const float pred = den != 0.0f ? acc[mt][nt][i] / den : 0.0f;
          const float diff = pred - comp(vc, nt);
          err += diff * diff;
        }
        err += __shfl_xor(err, 1, 64);
        err += __shfl_xor(err, 2, 64);
        err += __shfl_xor(err, 4, 64);
        err += __shfl_xor(err, 8, 64);
        if (l16 == 0 && live) scores[(size_t)n * sstride + c] = err;
      }
    }
  }
}

// ---------------------------------------------------------------- matrix-core state pass, 8 waves

// LDS-only work-group barrier: waits for this wave's LDS traffic, not for its
// global loads in flight.
__device__ __forceinline__ void lds_sync() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

constexpr int kThreads2 = 512;
constexpr int kPairs2 = 4;  // producer/consumer wave pairs, one per SIMD

struct State2Lds {
  alignas(16) float qs[kFD];
  alignas(16) float pk[kFD];
  alignas(16) float pv[kFD];
  alignas(16) float ek[kFD];
  union {
    struct {
      float ck[kFMaxCache][kKS];        // cache keys
      uint4 bp[kPairs2][2][12][64];     // B pieces [pair][buffer][3 * nt + piece][lane]
      float sj[kPairs2][2][4][8];       // s of each lane quarter's 8 slots
    } lp;
    float4 red[kFMaxCache / 16][4][64];  // numerator partials (after the tile loop)
  };
  float den[kPairs2][kFMaxCache];
  float onum[kPairs2][kFD];
  float enm[kPairs2][kFD];
  float oden[kPairs2];
  float eden[kPairs2];
};

// Same pass as hdec_state_kernel with two waves per SIMD. Pair p = (wave p,
// wave p + 4) walks tiles p, p + 4, ...: the producer (wave p) loads its
// tile, folds, writes it back, accumulates the readouts, splits it into the
// three bf16 B pieces and publishes them in LDS; after the barrier both
// waves take them from there. The producer runs candidate
// blocks 0..3 and the consumer blocks 4..MT-1 against the same pieces, so
// each wave keeps at most four blocks of accumulators.
template <int MT, typename Tin>
__global__ __launch_bounds__(kThreads2, 1) void hdec_state2_kernel(
    float* __restrict__ H, float* __restrict__ s, const float* __restrict__ pend_k,
    const float* __restrict__ pend_v, const Tin* __restrict__ q, const float* __restrict__ cache_k,
    const float* __restrict__ cache_v, const float* __restrict__ win_k, const float* __restrict__ win_v,
    int wrows, int slot, int lambda, float* __restrict__ scores, int sstride, float* __restrict__ lin,
    int lstride, float eps) {
  static_assert(MT > 4 && MT <= kFMaxCache / 16, "the consumer needs one to four blocks");
  __shared__ __align__(16) State2Lds sh;
  const int n = blockIdx.x;
  const int tid = threadIdx.x;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int pair = wv & 3;
  const bool prod = wv < kPairs2;
  const int lane = tid & 63;
  const int l16 = lane & 15;
  const int q4 = lane >> 4;
  float* Hn = H + (size_t)n * kFDim * kFD;
  float* sn = s + (size_t)n * kFDim;
  const int mb = prod ? 0 : 4;       // first candidate block of this wave
  const int mc = prod ? 4 : MT - 4;  // its number of blocks

  auto load_tile = [&](const TileCoords& tc, float4 (&h)[8], float (&sj)[8]) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      h[j] = make_float4(0.f, 0.f, 0.f, 0.f);
      sj[j] = 0.0f;
      if (j >= tc.jmin) {
        h[j] = *reinterpret_cast<const float4*>(Hn + (size_t)(tc.f0 + j) * kFD + 4 * l16);
        sj[j] = sn[tc.f0 + j];
      }
    }
  };
  TileCoords tc = tile_coords(pair, q4);
  float4 h[8];
  float sj[8];
  if (prod) load_tile(tc, h, sj);

  if (tid < kFD) {
    sh.qs[tid] = Elem<Tin>::load(q, (size_t)n * kFD + tid);
    sh.pk[tid] = pend_k[(size_t)n * kFD + tid];
    sh.pv[tid] = pend_v[(size_t)n * kFD + tid];
    sh.ek[tid] = win_k[((size_t)n * wrows + slot) * kFD + tid];
  }
  for (int i = tid; i < 16 * MT * (kFD / 4); i += kThreads2) {
    const int c = i / (kFD / 4);
    const int d4 = i % (kFD / 4);
    float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
    if (c < lambda) x = *reinterpret_cast<const float4*>(cache_k + ((size_t)n * lambda + c) * kFD + 4 * d4);
    *reinterpret_cast<float4*>(&sh.lp.ck[c][4 * d4]) = x;
  }
  __syncthreads();

  const float4 v4 = *reinterpret_cast<const float4*>(&sh.pv[4 * l16]);
  f32x4 acc[4][4];
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) acc[m][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float dacc[4] = {0.f, 0.f, 0.f, 0.f};
  float4 oacc = make_float4(0.f, 0.f, 0.f, 0.f);
  float4 eacc = make_float4(0.f, 0.f, 0.f, 0.f);
  float oden = 0.0f, eden = 0.0f;

  int it = 0;
#pragma unroll 1
  for (int T = pair; T < kFTiles; T += kPairs2, ++it) {
    const int buf = it & 1;
    const bool more = T + kPairs2 < kFTiles;
    const TileCoords tcn = more ? tile_coords(T + kPairs2, q4) : tc;
    float4 hn[8];
    float sjn[8];
    if (prod) {
      if (more) load_tile(tcn, hn, sjn);
      float pk[8], pq[8], pe[8];
      phi8(sh.pk, tc, pk);
      phi8(sh.qs, tc, pq);
      phi8(sh.ek, tc, pe);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (j >= tc.jmin) {
          h[j].x += pk[j] * v4.x;
          h[j].y += pk[j] * v4.y;
          h[j].z += pk[j] * v4.z;
          h[j].w += pk[j] * v4.w;
          sj[j] += pk[j];
          *reinterpret_cast<float4*>(Hn + (size_t)(tc.f0 + j) * kFD + 4 * l16) = h[j];
        }
        oacc.x += pq[j] * h[j].x;
        oacc.y += pq[j] * h[j].y;
        oacc.z += pq[j] * h[j].z;
        oacc.w += pq[j] * h[j].w;
        oden += pq[j] * sj[j];
        eacc.x += pe[j] * h[j].x;
        eacc.y += pe[j] * h[j].y;
        eacc.z += pe[j] * h[j].z;
        eacc.w += pe[j] * h[j].w;
        eden += pe[j] * sj[j];
      }
      {
        float x = sj[0];
#pragma unroll
        for (int j = 1; j < 8; ++j) x = l16 == j ? sj[j] : x;
        if (l16 < 8 && l16 >= tc.jmin) sn[tc.f0 + l16] = x;
        if (l16 < 8) sh.lp.sj[pair][buf][q4][l16] = x;
      }
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        float x[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = comp(h[j], nt);
        bf16x8 b0, b1, b2;
        split3(x, b0, b1, b2);
        sh.lp.bp[pair][buf][3 * nt][lane] = __builtin_bit_cast(uint4, b0);
        sh.lp.bp[pair][buf][3 * nt + 1][lane] = __builtin_bit_cast(uint4, b1);
        sh.lp.bp[pair][buf][3 * nt + 2][lane] = __builtin_bit_cast(uint4, b2);
      }
    }
    lds_sync();  // tile T's pieces and s are published
    if (!prod) {
#pragma unroll
      for (int j = 0; j < 8; ++j) sj[j] = sh.lp.sj[pair][buf][q4][j];
    }
    bf16x8 ahi[4], alo[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      if (m < mc) {
        float p[8];
        phi8(sh.lp.ck[16 * (mb + m) + l16], tc, p);
        float dd = 0.0f;
#pragma unroll
        for (int j = 0; j < 8; ++j) dd += p[j] * sj[j];
        dacc[m] += dd;
        split2(p, ahi[m], alo[m]);
      }
    }
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const bf16x8 b0 = __builtin_bit_cast(bf16x8, sh.lp.bp[pair][buf][3 * nt][lane]);
      const bf16x8 b1 = __builtin_bit_cast(bf16x8, sh.lp.bp[pair][buf][3 * nt + 1][lane]);
      const bf16x8 b2 = __builtin_bit_cast(bf16x8, sh.lp.bp[pair][buf][3 * nt + 2][lane]);
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        if (m < mc) {
          acc[m][nt] = mfma16x16x32(ahi[m], b0, acc[m][nt]);
          acc[m][nt] = mfma16x16x32(ahi[m], b1, acc[m][nt]);
          acc[m][nt] = mfma16x16x32(ahi[m], b2, acc[m][nt]);
          acc[m][nt] = mfma16x16x32(alo[m], b0, acc[m][nt]);
        }
      }
    }
    if (prod && more) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        h[j] = hn[j];
        sj[j] = sjn[j];
      }
    }
    tc = tcn;
  }

  // ---- vector-unit readouts (producers): over the lane quarters, then the pairs
  if (prod) {
    float ox[4] = {oacc.x, oacc.y, oacc.z, oacc.w};
    float ex[4] = {eacc.x, eacc.y, eacc.z, eacc.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ox[i] += __shfl_xor(ox[i], 16, 64);
      ox[i] += __shfl_xor(ox[i], 32, 64);
      ex[i] += __shfl_xor(ex[i], 16, 64);
      ex[i] += __shfl_xor(ex[i], 32, 64);
    }
    oden += __shfl_xor(oden, 16, 64);
    oden += __shfl_xor(oden, 32, 64);
    eden += __shfl_xor(eden, 16, 64);
    eden += __shfl_xor(eden, 32, 64);
    if (q4 == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sh.onum[pair][4 * l16 + i] = ox[i];
        sh.enm[pair][4 * l16 + i] = ex[i];
      }
    }
    if (lane == 0) {
      sh.oden[pair] = oden;
      sh.eden[pair] = eden;
    }
  }
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    if (m < mc) {
      float d = dacc[m];
      d += __shfl_xor(d, 16, 64);
      d += __shfl_xor(d, 32, 64);
      if (q4 == 0) sh.den[pair][16 * (mb + m) + l16] = d;
    }
  }
  // numerators: the pairs add into the LDS copy in turn (producers blocks
  // 0..3, consumers blocks 4..); the last pair keeps the sums. The first
  // barrier also ends every read of the keys and pieces, whose LDS the
  // partials reuse.
  for (int r = 0; r < kPairs2; ++r) {
    __syncthreads();
    if (pair == r) {
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        if (m < mc) {
#pragma unroll
          for (int nt = 0; nt < 4; ++nt) {
            f32x4 x = acc[m][nt];
            if (r > 0) {
              const float4 y = sh.red[mb + m][nt][lane];
              x[0] += y.x;
              x[1] += y.y;
              x[2] += y.z;
              x[3] += y.w;
            }
            acc[m][nt] = x;
            if (r + 1 < kPairs2) sh.red[mb + m][nt][lane] = make_float4(x[0], x[1], x[2], x[3]);
          }
        }
      }
    }
  }
  if (wv == 0) {
    // the linear readout of q, then the evicted pair's score
    float num = 0.0f, den = 0.0f, en = 0.0f, ed = eps;
#pragma unroll
    for (int r = 0; r < kPairs2; ++r) {
      num += sh.onum[r][lane];
      den += sh.oden[r];
      en += sh.enm[r][lane];
      ed += sh.eden[r];
    }
    lin[(size_t)n * lstride + lane] = num;
    if (lane == 0) lin[(size_t)n * lstride + kFD] = den;
    const float pred = ed != 0.0f ? en / ed : 0.0f;
    const float diff = pred - win_v[((size_t)n * wrows + slot) * kFD + lane];
    const float err = wave_sum(diff * diff);
    if (lane == 0) scores[(size_t)n * sstride + lambda] = err;
  }
  if (pair == kPairs2 - 1) {
    // lane (l16, q4) holds candidates 16*(mb + m) + 4*q4 + i at state columns 4*l16 + nt
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      if (m < mc) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int c = 16 * (mb + m) + 4 * q4 + i;
          const bool live = c < lambda;
          float den = eps;
#pragma unroll
          for (int r = 0; r < kPairs2; ++r) den += sh.den[r][c];
          float4 vc = make_float4(0.f, 0.f, 0.f, 0.f);
          if (live) vc = *reinterpret_cast<const float4*>(cache_v + ((size_t)n * lambda + c) * kFD + 4 * l16);
          float err = 0.0f;
#pragma unroll
          for (int nt = 0; nt < 4; ++nt) {
            const float pred = den != 0.0f ? acc[m][nt][i] / den : 0.0f;
            const float diff = pred - comp(vc, nt);
            err += diff * diff;
          }
          err += __shfl_xor(err, 1, 64);
          err += __shfl_xor(err, 2, 64);
          err += __shfl_xor(err, 4, 64);
          err += __shfl_xor(err, 8, 64);
          if (l16 == 0 && live) scores[(size_t)n * sstride + c] = err;
        }
      }
    }
  }
}

// ---------------------------------------------------------------- mix

template <int DQK, int DV>
struct MixLds {
  alignas(16) float qv[DQK];
  alignas(16) float kn[DQK];  // the new token
  alignas(16) float ek[DQK];  // the evicted token
  float vn[DV];
  float ev[DV];
  float rk[DQK];              // the rejected pair
  float rv[DV];
  float sc[kKeyTile];         // one tile's scores, then weights
  float red[kWaves];
  float num[kThreads / DV][DV];
  unsigned long long kred[kWaves];
  int rrow;
  float corr;
};

// One work-group per head-state. `refresh`: the cache is full and a token
// is evicted (scores of the lambda + 1 candidates are in `scores`); else with
// `evict` the evicted token is appended at cache row n_before.
template <int DQK, int DV, typename Tin, typename Tout>
__global__ __launch_bounds__(kThreads) void hdec_mix_kernel(
    const Tin* __restrict__ q, const Tin* __restrict__ k, const Tin* __restrict__ v, Tout* __restrict__ o,
    float* __restrict__ win_k, float* __restrict__ win_v, float* __restrict__ cache_k,
    float* __restrict__ cache_v, int32_t* __restrict__ cache_ids, float* __restrict__ pend_k,
    float* __restrict__ pend_v, int32_t* __restrict__ rejected, const float* __restrict__ scores, int sstride,
    const float* __restrict__ lin, int lstride, int lambda, int n_before, int n_after, bool refresh,
    bool evict, int wrows, int win_first, int t, int slot, int evicted_id, float scale, float eps) {
  constexpr int G = kThreads / DV;  // groups of d_v threads (one value column per thread)
  constexpr int LPK = DQK / 4;      // lanes per key in the score pass (a float4 each)
  constexpr int KPW = 64 / LPK;     // keys per wave and pass
  __shared__ MixLds<DQK, DV> sh;
  const int n = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int c = tid % DV;
  const int g = tid / DV;

  const size_t srow = (size_t)n * wrows + slot;
  for (int d = tid; d < DQK; d += kThreads) {
    sh.qv[d] = Elem<Tin>::load(q, (size_t)n * DQK + d);
    sh.kn[d] = Elem<Tin>::load(k, (size_t)n * DQK + d);
    if (evict) sh.ek[d] = win_k[srow * DQK + d];
  }
  for (int d = tid; d < DV; d += kThreads) {
    sh.vn[d] = Elem<Tin>::load(v, (size_t)n * DV + d);
    if (evict) sh.ev[d] = win_v[srow * DV + d];
  }
  if (tid == 0) sh.rrow = -1;

  // ---- the rejected pair: the last of the lambda + 1 candidates in
  // (score desc, token id asc) order
  int replaced = -1;  // the cache row the evicted pair now holds
  if (refresh) {
    unsigned long long worst = ~0ull;
    for (int i = tid; i <= lambda; i += kThreads) {
      const int id = i < lambda ? cache_ids[(size_t)n * lambda + i] : evicted_id;
      const float x = lambda > 0 ? scores[(size_t)n * sstride + i] : 0.0f;  // a lone candidate is not scored
      worst = min(worst, (unsigned long long)topk_key(x, (uint32_t)id));
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) worst = min(worst, __shfl_xor(worst, off, 64));
    if (lane == 0) sh.kred[wave] = worst;
    __syncthreads();
    unsigned long long m = sh.kred[0];
#pragma unroll
    for (int i = 1; i < kWaves; ++i) m = min(m, sh.kred[i]);
    const int rid = (int)topk_index(m);
    if (rid != evicted_id)
      for (int i = tid; i < lambda; i += kThreads)
        if (cache_ids[(size_t)n * lambda + i] == rid) sh.rrow = i;
    __syncthreads();
    const int r = sh.rrow;
    for (int d = tid; d < DQK; d += kThreads) sh.rk[d] = r >= 0 ? cache_k[((size_t)n * lambda + r) * DQK + d] : sh.ek[d];
    for (int d = tid; d < DV; d += kThreads) sh.rv[d] = r >= 0 ? cache_v[((size_t)n * lambda + r) * DV + d] : sh.ev[d];
    __syncthreads();  // row r is read before it is replaced
    // the rejected pair's fold is deferred to the next call
    for (int d = tid; d < DQK; d += kThreads) pend_k[(size_t)n * DQK + d] = sh.rk[d];
    for (int d = tid; d < DV; d += kThreads) pend_v[(size_t)n * DV + d] = sh.rv[d];
    if (r >= 0) {
      for (int d = tid; d < DQK; d += kThreads) cache_k[((size_t)n * lambda + r) * DQK + d] = sh.ek[d];
      for (int d = tid; d < DV; d += kThreads) cache_v[((size_t)n * lambda + r) * DV + d] = sh.ev[d];
      if (tid == 0) cache_ids[(size_t)n * lambda + r] = evicted_id;
    }
    if (rejected && tid == 0) rejected[n] = rid;
    replaced = r;
    // (q . k_r)^2 = phi(q)^T phi(k_r), the readout's share of the deferred fold
    if (wave == 0) {
      float x = 0.0f;
      for (int d = lane; d < DQK; d += 64) x += sh.qv[d] * sh.rk[d];
      x = wave_sum(x);
      if (lane == 0) sh.corr = x * x;
    }
  } else {
    __syncthreads();
    for (int d = tid; d < DQK; d += kThreads) pend_k[(size_t)n * DQK + d] = 0.0f;
    for (int d = tid; d < DV; d += kThreads) pend_v[(size_t)n * DV + d] = 0.0f;
    if (evict) {
      for (int d = tid; d < DQK; d += kThreads) cache_k[((size_t)n * lambda + n_before) * DQK + d] = sh.ek[d];
      for (int d = tid; d < DV; d += kThreads) cache_v[((size_t)n * lambda + n_before) * DV + d] = sh.ev[d];
      if (tid == 0) cache_ids[(size_t)n * lambda + n_before] = evicted_id;
      replaced = n_before;
    }
    if (rejected && tid == 0) rejected[n] = -1;
    if (tid == 0) sh.corr = 0.0f;
  }
  __syncthreads();
  const float corr = sh.corr;
  const float lin_num = lin[(size_t)n * lstride + c] + (refresh ? corr * sh.rv[c] : 0.0f);
  const float lin_den = lin[(size_t)n * lstride + DV] + corr;

  // ---- softmax keys: window tokens win_first .. t - 1 (ring rows), the new
  // token t, then the cache rows 0 .. n_after - 1; the row the evicted token
  // took is read from its LDS copy
  const int n_old = t - win_first;
  const int n_keys = n_old + 1 + n_after;
  auto key_row = [&](int j) -> const float* {
    if (j < n_old) return win_k + ((size_t)n * wrows + (win_first + j) % wrows) * DQK;
    if (j == n_old) return sh.kn;
    const int r = j - n_old - 1;
    return r == replaced ? sh.ek : cache_k + ((size_t)n * lambda + r) * DQK;
  };
  auto val_row = [&](int j) -> const float* {
    if (j < n_old) return win_v + ((size_t)n * wrows + (win_first + j) % wrows) * DV;
    if (j == n_old) return sh.vn;
    const int r = j - n_old - 1;
    return r == replaced ? sh.ev : cache_v + ((size_t)n * lambda + r) * DV;
  };
  const float4 q4 = *reinterpret_cast<const float4*>(&sh.qv[4 * (lane % LPK)]);
  // running maximum, starting at 0: the linear terms are scaled by e^{-m} too
  float m = 0.0f;
  float wsum = 0.0f, acc = 0.0f;
  for (int j0 = 0; j0 < n_keys; j0 += kKeyTile) {
    const int nt = min(kKeyTile, n_keys - j0);
    for (int jb = wave * KPW; jb < nt; jb += kWaves * KPW) {
      const int jl = jb + lane / LPK;
      float x = 0.0f;
      if (jl < nt) {
        const float4 k4 = *reinterpret_cast<const float4*>(key_row(j0 + jl) + 4 * (lane % LPK));
        x = q4.x * k4.x + q4.y * k4.y + q4.z * k4.z + q4.w * k4.w;
      }
#pragma unroll
      for (int off = LPK / 2; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
      if (jl < nt && lane % LPK == 0) sh.sc[jl] = x * scale;
    }
    __syncthreads();
    const float tmax = block_max(tid < nt ? sh.sc[tid] : -INFINITY, sh.red);
    const float m_new = fmaxf(m, tmax);
    const float rs = __expf(m - m_new);
    wsum *= rs;
    acc *= rs;
    if (tid < nt) {
      const float p = __expf(sh.sc[tid] - m_new);
      sh.sc[tid] = p;
      wsum += p;
    }
    __syncthreads();
    for (int j = g; j < nt; j += G) acc += sh.sc[j] * val_row(j0 + j)[c];
    __syncthreads();
    m = m_new;
  }
  const float sm_den = block_sum(wsum, sh.red);
  sh.num[g][c] = acc;
  __syncthreads();
  if (g == 0) {
    float sm_num = 0.0f;
#pragma unroll
    for (int i = 0; i < G; ++i) sm_num += sh.num[i][c];
    const float e = __expf(-m);
    const float nn = sm_num + e * lin_num;
    const float dd = sm_den + e * (lin_den + eps);
    Elem<Tout>::store(o, (size_t)n * DV + c, dd != 0.0f ? nn / dd : 0.0f);
  }
  // ---- the new token enters the window, in the evicted token's row (whose
  // values were copied to LDS before the first barrier)
  for (int d = tid; d < DQK; d += kThreads) win_k[srow * DQK + d] = sh.kn[d];
  for (int d = tid; d < DV; d += kThreads) win_v[srow * DV + d] = sh.vn[d];
}

// ---------------------------------------------------------------- host

size_t scores_bytes(const HybridDecodeArgs& a) { return align_up((size_t)a.N * (a.cache_size + 1) * sizeof(float)); }
int lin_stride(int dv) { return (dv + 1 + 3) / 4 * 4; }

bool use_matrix_pass(const HybridDecodeArgs& a) {
  return a.dqk == kFD && a.dv == kFD && a.cache_size >= 1 && a.cache_size <= kFMaxCache;
}

template <typename Tin>
hipError_t launch_state(const HybridDecodeArgs& a, int mt, int wrows, int slot, float* scores, int sstride,
                        float* lin, int lstride, hipStream_t st) {
#define KLA_STATE(M)                                                                                            \
  hipLaunchKernelGGL((hdec_state_kernel<M, Tin>), dim3(a.N), dim3(kThreads), 0, st, a.H, a.s, a.pend_k,       \
                     a.pend_v, static_cast<const Tin*>(a.q), a.cache_k, a.cache_v, a.win_k, a.win_v, wrows,   \
                     slot, a.cache_size, scores, sstride, lin, lstride, a.eps)
#define KLA_STATE2(M)                                                                                           \
  hipLaunchKernelGGL((hdec_state2_kernel<M, Tin>), dim3(a.N), dim3(kThreads2), 0, st, a.H, a.s, a.pend_k,     \
                     a.pend_v, static_cast<const Tin*>(a.q), a.cache_k, a.cache_v, a.win_k, a.win_v, wrows,   \
                     slot, a.cache_size, scores, sstride, lin, lstride, a.eps)
  // up to 64 candidates: one wave per SIMD holds every block; more: two
  switch (mt) {
    case 0: KLA_STATE(0); break;
    case 1: KLA_STATE(1); break;
    case 2: KLA_STATE(2); break;
    case 3: KLA_STATE(3); break;
    case 4: KLA_STATE(4); break;
    case 5: KLA_STATE2(5); break;
    case 6: KLA_STATE2(6); break;
    case 7: KLA_STATE2(7); break;
    case 8: KLA_STATE2(8); break;
    default: return hipErrorInvalidValue;
  }
#undef KLA_STATE
#undef KLA_STATE2
  return hipGetLastError();
}

template <int DQK, int DV, typename Tin, typename Tout>
hipError_t run_hd(const HybridDecodeArgs& a, void* ws, hipStream_t st) {
  char* p = static_cast<char*>(ws);
  float* scores = reinterpret_cast<float*>(p);
  float* lin = reinterpret_cast<float*>(p + scores_bytes(a));
  const int N = a.N, W = a.window, lam = a.cache_size, t = a.t;
  const int wrows = W + 1;
  const int slot = t % wrows;  // the evicted token's row, then the new token's
  const bool evict = t >= W + 1;
  const int evicted_id = t - W - 1;
  const int n_before = std::min(lam, std::max(0, t - W - 1));
  const bool refresh = evict && n_before == lam;
  const int n_after = std::min(lam, std::max(0, t - W));
  const int sstride = lam + 1;
  const int lstride = lin_stride(DV);
  hipError_t e;
  prof_begin(st);
  if (use_matrix_pass(a)) {
    e = launch_state<Tin>(a, refresh ? (lam + 15) / 16 : 0, wrows, slot, scores, sstride, lin, lstride, st);
  } else {
    hipLaunchKernelGGL((hdec_fold_kernel<DQK, DV, Tin, true>), dim3(N), dim3(kThreads), 0, st, a.H, a.s, a.pend_k,
                       a.pend_v, static_cast<const Tin*>(a.q), lin, lstride);
    if (refresh && lam > 0)
      hipLaunchKernelGGL((hdec_score_kernel<DQK, DV>), dim3((lam + 1 + 63) / 64, N), dim3(kThreads), 0, st, a.H,
                         a.s, a.cache_k, a.cache_v, a.win_k, a.win_v, lam, wrows, slot, scores, sstride, a.eps);
    e = hipGetLastError();
  }
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((hdec_mix_kernel<DQK, DV, Tin, Tout>), dim3(N), dim3(kThreads), 0, st,
                     static_cast<const Tin*>(a.q), static_cast<const Tin*>(a.k), static_cast<const Tin*>(a.v),
                     static_cast<Tout*>(a.o), a.win_k, a.win_v, a.cache_k, a.cache_v, a.cache_ids, a.pend_k,
                     a.pend_v, a.rejected, scores, sstride, lin, lstride, lam, n_before, n_after, refresh, evict,
                     wrows, std::max(0, t - W), t, slot, evicted_id, a.scale, a.eps);
  prof_end(st);
  return hipGetLastError();
}

template <int DQK, int DV>
hipError_t run_hd_dt(const HybridDecodeArgs& a, void* ws, hipStream_t st) {
  if (a.in_bf16)
    return a.out_bf16 ? run_hd<DQK, DV, uint16_t, uint16_t>(a, ws, st) : run_hd<DQK, DV, uint16_t, float>(a, ws, st);
  return a.out_bf16 ? run_hd<DQK, DV, float, uint16_t>(a, ws, st) : run_hd<DQK, DV, float, float>(a, ws, st);
}

}  // namespace

size_t hybrid_decode_workspace(const HybridDecodeArgs& a) {
  return scores_bytes(a) + align_up((size_t)a.N * lin_stride(a.dv) * sizeof(float));
}

hipError_t hybrid_decode_launch(const HybridDecodeArgs& a, void* ws, hipStream_t st) {
#define KLA_CASE(A, B) \
  if (a.dqk == A && a.dv == B) return run_hd_dt<A, B>(a, ws, st);
  KLA_CASE(16, 16) KLA_CASE(16, 32) KLA_CASE(16, 64)
  KLA_CASE(32, 16) KLA_CASE(32, 32) KLA_CASE(32, 64)
  KLA_CASE(64, 16) KLA_CASE(64, 32) KLA_CASE(64, 64)
#undef KLA_CASE
  return hipErrorInvalidValue;
}

hipError_t hybrid_decode_flush_launch(const HybridDecodeArgs& a, hipStream_t st) {
#define KLA_CASE(A, B)                                                                                          \
  if (a.dqk == A && a.dv == B) {                                                                                \
    hipLaunchKernelGGL((hdec_fold_kernel<A, B, float, false>), dim3(a.N), dim3(kThreads), 0, st, a.H, a.s,      \
                       a.pend_k, a.pend_v, nullptr, nullptr, 0);                                               \
    return hipGetLastError();                                                                                   \
  }
  KLA_CASE(16, 16) KLA_CASE(16, 32) KLA_CASE(16, 64)
  KLA_CASE(32, 16) KLA_CASE(32, 32) KLA_CASE(32, 64)
  KLA_CASE(64, 16) KLA_CASE(64, 32) KLA_CASE(64, 64)
#undef KLA_CASE
  return hipErrorInvalidValue;
}

}  // namespace kla
