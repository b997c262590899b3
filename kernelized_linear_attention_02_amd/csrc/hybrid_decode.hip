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
// Deferred folds: the fold of step 1 is not written into (H, s) by the call
// that decides it. The rejected pair waits in pending slot t mod P of the
// state (P = KLA_HYBRID_PENDING slots), and every call with t mod P = 0 folds
// all P slots in its pass over H and clears them; the calls between only
// read H. H is then read once per token and written once per P tokens. A
// call that does not fold adds the slots to its readouts in closed form,
// phi(x)^T phi(k_j) = (x . k_j)^2:
//   num += sum_j (x . k_j)^2 v_j,   den += sum_j (x . k_j)^2,
// and its own rejected pair r the same way. A zero slot folds nothing
// (phi(0) = 0).
//
// Carried sums: every cached pair i keeps its sums against the linear state
// (pending slots included), (phi(k_i)^T H', phi(k_i)^T s'), in the caller's
// state. A fold of pair r changes them by the same closed form,
// (k_i . k_r)^2 [v_r | 1], so the candidates of a refresh are scored from
// their sums; only the evicted pair, new to the cache, takes its sums from
// the pass over H.
//
// Kernels (all counts are known on the host from t):
//   state pass  one work-group per head-state streams H once: the pending
//               folds (every P tokens; else H is only read), linear readouts
//               of q and of the evicted key (d_qk = d_v = 64: 72 tiles in
//               block order; other shapes: the generic pass);
//   mix         per head-state: the candidates' scores from their sums, the
//               rejected pair (lowest (score, -id)), the closed-form fold
//               term for the kept pairs' sums and for the readout, the cache
//               update, the window and cache softmax (online maximum), the
//               joint division, the window insert, and the pending slot of
//               the rejected pair;
//   prime       the cached pairs' sums from (H, s) and the pending slots,
//               for a state filled from elsewhere.
#include <algorithm>
#include <mutex>

#include "kla_device.hpp"
#include "kla_internal.hpp"

namespace kla {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kPend = KLA_HYBRID_PENDING;  // pending slots, folded together every kPend tokens
constexpr int kKeyTile = 1024;  // softmax keys scored per pass (online max across passes)
constexpr int kU = 8;           // row loads in flight per lane in the softmax passes

// Four consecutive elements of a window or cache row (rows are kept in the
// step's input type; 16-byte aligned groups for float32, 8-byte for bf16).
template <typename T>
__device__ __forceinline__ float4 ld4(const T* p);
template <>
__device__ __forceinline__ float4 ld4<float>(const float* p) {
  return *reinterpret_cast<const float4*>(p);
}
template <>
__device__ __forceinline__ float4 ld4<uint16_t>(const uint16_t* p) {
  const uint2 u = *reinterpret_cast<const uint2*>(p);
  return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xFFFF0000u), __uint_as_float(u.y << 16),
                     __uint_as_float(u.y & 0xFFFF0000u));
}

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

// One work-group per head-state. With `fold` the pending slots are folded
// into (H, s) and cleared; otherwise H and s are only read and, with READ,
// the slots enter the readouts in closed form. With READ, lin[n] =
// (phi(q)^T H', phi(q)^T s') of the linear state (denominator without eps)
// at lin[n * lstride + 0 .. d_v], and, when a token leaves the window (its
// key row `slot`), the same readout of its key at esum[n * lstride + ...].
template <int DQK, int DV, typename Tin, bool READ>
__global__ __launch_bounds__(kThreads) void hdec_fold_kernel(
    float* __restrict__ H, float* __restrict__ s, float* __restrict__ pend_k, float* __restrict__ pend_v,
    const Tin* __restrict__ q, float* __restrict__ lin, int lstride, const Tin* __restrict__ win_k, int wrows,
    int slot, bool evict, bool fold, float* __restrict__ esum) {
  constexpr int D = phi_dim(DQK);
  constexpr int G = kThreads / DV;
  __shared__ float pq[READ ? D : 1];
  __shared__ float pe[READ ? D : 1];
  __shared__ float pk[kPend][D];
  __shared__ float qv[DQK], ev[DQK], kv[kPend][DQK], vv[kPend][DV];
  __shared__ uint16_t tab[D];
  __shared__ float num[G][DV];
  __shared__ float enm[G][DV];
  __shared__ float red[kWaves];
  __shared__ float wq[kPend], we[kPend];
  const int n = blockIdx.x;
  const int tid = threadIdx.x;
  const int c = tid % DV;
  const int g = tid / DV;
  const bool ev_on = READ && evict;
  for (int d = tid; d < DQK; d += kThreads) {
    if (READ) qv[d] = Elem<Tin>::load(q, (size_t)n * DQK + d);
    if (ev_on) ev[d] = Elem<Tin>::load(win_k, ((size_t)n * wrows + slot) * DQK + d);
  }
  for (int i = tid; i < kPend * DQK; i += kThreads) kv[i / DQK][i % DQK] = pend_k[(size_t)n * kPend * DQK + i];
  for (int i = tid; i < kPend * DV; i += kThreads) vv[i / DV][i % DV] = pend_v[(size_t)n * kPend * DV + i];
  build_phi_table(tab, 0, D, DQK);
  __syncthreads();
  for (int f = tid; f < D; f += kThreads) {
    if (fold)
      for (int p = 0; p < kPend; ++p) pk[p][f] = phi_of(kv[p], tab[f]);
    if (READ) pq[f] = phi_of(qv, tab[f]);
    if (ev_on) pe[f] = phi_of(ev, tab[f]);
  }
  // closed-form weights of the slots (used without a fold)
  if (READ && !fold && tid < kPend) {
    float a = 0.0f, b = 0.0f;
    for (int d = 0; d < DQK; ++d) {
      a += qv[d] * kv[tid][d];
      if (ev_on) b += ev[d] * kv[tid][d];
    }
    wq[tid] = a * a;
    we[tid] = b * b;
  }
  __syncthreads();
  float* Hn = H + (size_t)n * D * DV;
  float* sn = s + (size_t)n * D;
  float vc[kPend];
#pragma unroll
  for (int p = 0; p < kPend; ++p) vc[p] = vv[p][c];
  float acc = 0.0f, eacc = 0.0f;
#pragma unroll 4
  for (int f = g; f < D; f += G) {
    float h = Hn[(size_t)f * DV + c];
    if (fold) {
#pragma unroll
      for (int p = 0; p < kPend; ++p) h += pk[p][f] * vc[p];
      Hn[(size_t)f * DV + c] = h;
    }
    if (READ) acc += pq[f] * h;
    if (ev_on) eacc += pe[f] * h;
  }
  float den = 0.0f, eden = 0.0f;
  for (int f = tid; f < D; f += kThreads) {
    float x = sn[f];
    if (fold) {
#pragma unroll
      for (int p = 0; p < kPend; ++p) x += pk[p][f];
      sn[f] = x;
    }
    if (READ) den += pq[f] * x;
    if (ev_on) eden += pe[f] * x;
  }
  if (READ) {
    num[g][c] = acc;
    if (ev_on) enm[g][c] = eacc;
    const float dsum = block_sum(den, red);  // its barriers also publish num and enm
    const float esm = ev_on ? block_sum(eden, red) : 0.0f;
    if (g == 0) {
      float x = 0.0f, y = 0.0f;
#pragma unroll
      for (int i = 0; i < G; ++i) {
        x += num[i][c];
        if (ev_on) y += enm[i][c];
      }
      if (!fold)
#pragma unroll
        for (int p = 0; p < kPend; ++p) {
          x += wq[p] * vc[p];
          if (ev_on) y += we[p] * vc[p];
        }
      lin[(size_t)n * lstride + c] = x;
      if (ev_on) esum[(size_t)n * lstride + c] = y;
    }
    if (tid == 0) {
      float dx = dsum, ex = esm;
      if (!fold)
        for (int p = 0; p < kPend; ++p) {
          dx += wq[p];
          ex += we[p];
        }
      lin[(size_t)n * lstride + DV] = dx;
      if (ev_on) esum[(size_t)n * lstride + DV] = ex;
    }
  }
  // every read of the slots went through LDS before the first barrier
  if (fold) {
    for (int i = tid; i < kPend * DQK; i += kThreads) pend_k[(size_t)n * kPend * DQK + i] = 0.0f;
    for (int i = tid; i < kPend * DV; i += kThreads) pend_v[(size_t)n * kPend * DV + i] = 0.0f;
  }
}

// ---------------------------------------------------------------- matrix-core state pass

constexpr int kFD = 64;
constexpr int kFDim = kFD * (kFD + 1) / 2;  // 2080
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
  alignas(16) float pk[kPend][kFD];
  alignas(16) float pv[kPend][kFD];
  alignas(16) float ek[kFD];
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
// 4*l16 .. 4*l16+3 (16-byte loads, the next tile's in flight). With `fold`
// it adds the pending slots' folds and writes the rows back; otherwise H is
// only read and the slots enter the readouts in closed form. It accumulates
// the float32 readouts of q and, when a token leaves the window, of its key.
template <typename Tin, bool fold>
__global__ __launch_bounds__(kThreads) void hdec_state_kernel(
    float* __restrict__ H, float* __restrict__ s, float* __restrict__ pend_k, float* __restrict__ pend_v,
    const Tin* __restrict__ q, const Tin* __restrict__ win_k, int wrows, int slot, bool evict,
    float* __restrict__ lin, float* __restrict__ esum, int lstride) {
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
    sh.ek[tid] = evict ? Elem<Tin>::load(win_k, ((size_t)n * wrows + slot) * kFD + tid) : 0.0f;
  }
  for (int i = tid; i < kPend * kFD; i += kThreads) {
    sh.pk[i / kFD][i % kFD] = pend_k[(size_t)n * kPend * kFD + i];
    sh.pv[i / kFD][i % kFD] = pend_v[(size_t)n * kPend * kFD + i];
  }
  __syncthreads();

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

    // each lift is formed just before its use (eight values live at a time)
    float ph[8];
    if constexpr (fold) {
#pragma unroll 1
      for (int p = 0; p < kPend; ++p) {
        phi8(sh.pk[p], tc, ph);
        const float4 v4 = *reinterpret_cast<const float4*>(&sh.pv[p][4 * l16]);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          if (j >= tc.jmin) {  // slots below jmin are not features and stay zero
            h[j].x += ph[j] * v4.x;
            h[j].y += ph[j] * v4.y;
            h[j].z += ph[j] * v4.z;
            h[j].w += ph[j] * v4.w;
            sj[j] += ph[j];
          }
        }
      }
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (j >= tc.jmin) *reinterpret_cast<float4*>(Hn + (size_t)(tc.f0 + j) * kFD + 4 * l16) = h[j];
    }
    phi8(sh.qs, tc, ph);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      oacc.x += ph[j] * h[j].x;
      oacc.y += ph[j] * h[j].y;
      oacc.z += ph[j] * h[j].z;
      oacc.w += ph[j] * h[j].w;
      oden += ph[j] * sj[j];
    }
    phi8(sh.ek, tc, ph);  // zero without an evicted key
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      eacc.x += ph[j] * h[j].x;
      eacc.y += ph[j] * h[j].y;
      eacc.z += ph[j] * h[j].z;
      eacc.w += ph[j] * h[j].w;
      eden += ph[j] * sj[j];
    }
    // lane l16 = j of each quarter writes s of slot j: a contiguous 32-byte run
    if constexpr (fold) {
      float x = sj[0];
#pragma unroll
      for (int j = 1; j < 8; ++j) x = l16 == j ? sj[j] : x;
      if (l16 < 8 && l16 >= tc.jmin) sn[tc.f0 + l16] = x;
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

  // ---- readouts: sum over the lane quarters, then over waves
  {
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
        sh.onum[w][4 * l16 + i] = ox[i];
        sh.enm[w][4 * l16 + i] = ex[i];
      }
    }
    if (lane == 0) {
      sh.oden[w] = oden;
      sh.eden[w] = eden;
    }
  }
  __syncthreads();
  if (w == 0) {
    float num = 0.0f, den = 0.0f, en = 0.0f, ed = 0.0f;
#pragma unroll
    for (int r = 0; r < kWaves; ++r) {
      num += sh.onum[r][lane];
      den += sh.oden[r];
      en += sh.enm[r][lane];
      ed += sh.eden[r];
    }
    if (!fold) {
      // the slots H does not hold yet, in closed form: (x . k_j)^2 [v_j | 1]
#pragma unroll 1
      for (int p = 0; p < kPend; ++p) {
        const float kp = sh.pk[p][lane];
        const float dq = wave_sum(sh.qs[lane] * kp);
        const float de = wave_sum(sh.ek[lane] * kp);
        const float vp = sh.pv[p][lane];
        num += dq * dq * vp;
        den += dq * dq;
        en += de * de * vp;
        ed += de * de;
      }
    }
    lin[(size_t)n * lstride + lane] = num;
    if (lane == 0) lin[(size_t)n * lstride + kFD] = den;
    if (evict) {
      esum[(size_t)n * lstride + lane] = en;
      if (lane == 0) esum[(size_t)n * lstride + kFD] = ed;
    }
  }
  // the folded slots are cleared (every read of them went through LDS before
  // the first barrier)
  if (fold)
    for (int i = tid; i < kPend * kFD; i += kThreads) {
      pend_k[(size_t)n * kPend * kFD + i] = 0.0f;
      pend_v[(size_t)n * kPend * kFD + i] = 0.0f;
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
  alignas(16) float rk[DQK];  // the rejected pair
  alignas(16) float rv[DV];
  float sc[kKeyTile];         // one tile's scores, then weights
  float err[256];             // the refresh candidates' self-recall errors
  float red[kWaves];
  alignas(16) float num[kWaves][DV];
  unsigned long long kred[kWaves];
  int rrow;
  float corr;
};

// One work-group per head-state. `refresh`: the cache is full and a token
// is evicted; the lambda + 1 candidates are scored from their sums (the
// cache rows' carried sums, the evicted pair's from the state pass in
// `esum`); else with `evict` the evicted token is appended at cache row
// n_before with its sums. Candidate i's sums and value row are read by
// TPC = d_v / 16 adjacent threads, 16 columns each.
template <int DQK, int DV, typename Tin, typename Tout>
__global__ __launch_bounds__(kThreads) void hdec_mix_kernel(
    const Tin* __restrict__ q, const Tin* __restrict__ k, const Tin* __restrict__ v, Tout* __restrict__ o,
    Tin* __restrict__ win_k, Tin* __restrict__ win_v, Tin* __restrict__ cache_k,
    Tin* __restrict__ cache_v, int32_t* __restrict__ cache_ids, float* __restrict__ pend_k,
    float* __restrict__ pend_v, int32_t* __restrict__ rejected, float* __restrict__ cache_sums,
    const float* __restrict__ esum, const float* __restrict__ lin, int lstride, int lambda, int n_before,
    int n_after, bool refresh, bool evict, int wrows, int win_first, int t, int slot, int pslot, int evicted_id,
    float scale, float eps) {
  constexpr int LPK = DQK / 4;      // lanes per key in the score pass (a float4 each)
  constexpr int KPW = 64 / LPK;     // keys per wave and pass
  __shared__ MixLds<DQK, DV> sh;
  const int n = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int c = tid % DV;  // the output column of threads tid < DV

  const size_t srow = (size_t)n * wrows + slot;
  for (int d = tid; d < DQK; d += kThreads) {
    sh.qv[d] = Elem<Tin>::load(q, (size_t)n * DQK + d);
    sh.kn[d] = Elem<Tin>::load(k, (size_t)n * DQK + d);
    if (evict) sh.ek[d] = Elem<Tin>::load(win_k, srow * DQK + d);
  }
  for (int d = tid; d < DV; d += kThreads) {
    sh.vn[d] = Elem<Tin>::load(v, (size_t)n * DV + d);
    if (evict) sh.ev[d] = Elem<Tin>::load(win_v, srow * DV + d);
  }
  if (tid == 0) sh.rrow = -1;

  // ---- the rejected pair: the last of the lambda + 1 candidates in
  // (score desc, token id asc) order, score_i = || num_i / (den_i + eps) - v_i ||^2.
  // Candidate i's sums (rows of DVS floats, 16-byte aligned) are read once by
  // TPC adjacent threads, 16 columns each, and stay in their registers for
  // the update after the selection.
  constexpr int TPC = DV / 16;          // threads per candidate, 16 columns each
  constexpr int CPR = kThreads / TPC;   // candidates per round
  constexpr int NR = 256 / CPR;         // rounds for lambda + 1 <= 256 candidates
  constexpr int DPT = DQK / TPC;        // key dimensions per thread (closed-form weights)
  constexpr int DVS = DV + 4;           // row stride of the sums
  const int ci = tid / TPC, part = tid % TPC;
  int replaced = -1;  // the cache row the evicted pair now holds
  if (refresh) {
    // candidate tid's token id (lambda + 1 <= kThreads: one candidate a
    // thread), loaded beside the scoring's loads
    static_assert(kThreads >= 256, "one selection candidate per thread");
    const int myid = tid < lambda ? cache_ids[(size_t)n * lambda + tid] : evicted_id;
    float4 cs[NR][4];  // this thread's 16 columns of its candidate in each round
    float cd[NR];      // and the denominator
    if (lambda > 0) {
#pragma unroll
      for (int rr = 0; rr < NR; ++rr) {
        const int i = rr * CPR + ci;
        cd[rr] = 0.0f;
        float err = 0.0f;
        if (i <= lambda) {
          const float* sm = i < lambda ? cache_sums + ((size_t)n * lambda + i) * DVS : esum + (size_t)n * lstride;
          const Tin* vr = i < lambda ? cache_v + ((size_t)n * lambda + i) * DV : win_v + srow * DV;
#pragma unroll
          for (int j = 0; j < 4; ++j) cs[rr][j] = reinterpret_cast<const float4*>(sm + 16 * part)[j];
          cd[rr] = sm[DV];
          const float dn = cd[rr] + eps;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float4 vv4 = ld4<Tin>(vr + 16 * part + 4 * j);
            const float x[4] = {cs[rr][j].x, cs[rr][j].y, cs[rr][j].z, cs[rr][j].w};
            const float y[4] = {vv4.x, vv4.y, vv4.z, vv4.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float pred = dn != 0.0f ? x[e] / dn : 0.0f;
              const float d = pred - y[e];
              err += d * d;
            }
          }
        }
#pragma unroll
        for (int off = 1; off < TPC; off <<= 1) err += __shfl_xor(err, off, 64);
        if (i <= lambda && part == 0) sh.err[i] = err;
      }
    }
    __syncthreads();
    unsigned long long worst = ~0ull;
    if (tid <= lambda) {
      const float x = lambda > 0 ? sh.err[tid] : 0.0f;  // a lone candidate is not scored
      worst = (unsigned long long)topk_key(x, (uint32_t)myid);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) worst = min(worst, __shfl_xor(worst, off, 64));
    if (lane == 0) sh.kred[wave] = worst;
    __syncthreads();
    unsigned long long m = sh.kred[0];
#pragma unroll
    for (int i = 1; i < kWaves; ++i) m = min(m, sh.kred[i]);
    const int rid = (int)topk_index(m);
    if (rid != evicted_id && tid < lambda && myid == rid) sh.rrow = tid;
    __syncthreads();
    const int r = sh.rrow;
    for (int d = tid; d < DQK; d += kThreads)
      sh.rk[d] = r >= 0 ? Elem<Tin>::load(cache_k, ((size_t)n * lambda + r) * DQK + d) : sh.ek[d];
    for (int d = tid; d < DV; d += kThreads)
      sh.rv[d] = r >= 0 ? Elem<Tin>::load(cache_v, ((size_t)n * lambda + r) * DV + d) : sh.ev[d];
    __syncthreads();  // row r is read before it is replaced
    // the rejected pair's fold is deferred: it waits in pending slot pslot
    for (int d = tid; d < DQK; d += kThreads) pend_k[((size_t)n * kPend + pslot) * DQK + d] = sh.rk[d];
    for (int d = tid; d < DV; d += kThreads) pend_v[((size_t)n * kPend + pslot) * DV + d] = sh.rv[d];
    if (r >= 0) {
      for (int d = tid; d < DQK; d += kThreads) Elem<Tin>::store(cache_k, ((size_t)n * lambda + r) * DQK + d, sh.ek[d]);
      for (int d = tid; d < DV; d += kThreads) Elem<Tin>::store(cache_v, ((size_t)n * lambda + r) * DV + d, sh.ev[d]);
      if (tid == 0) cache_ids[(size_t)n * lambda + r] = evicted_id;
    }
    if (rejected && tid == 0) rejected[n] = rid;
    replaced = r;
    // the kept pairs' sums against the state with r folded in: their own (the
    // evicted pair, now in row r, brings its sums from the pass) plus
    // (k_i . k_r)^2 [v_r | 1]
    if (lambda > 0) {
#pragma unroll
      for (int rr = 0; rr < NR; ++rr) {
        const int i = rr * CPR + ci;
        const bool live = i < lambda;
        const bool fresh = i == r;
        float dot = 0.0f;
        if (fresh) {
#pragma unroll
          for (int j = 0; j < DPT; ++j) dot += sh.ek[DPT * part + j] * sh.rk[DPT * part + j];
        } else {
          const Tin* kr = cache_k + ((size_t)n * lambda + (live ? i : 0)) * DQK + DPT * part;
#pragma unroll
          for (int j = 0; j < DPT; j += 4) {
            const float4 x = ld4<Tin>(kr + j);
            dot += x.x * sh.rk[DPT * part + j] + x.y * sh.rk[DPT * part + j + 1] + x.z * sh.rk[DPT * part + j + 2] +
                   x.w * sh.rk[DPT * part + j + 3];
          }
        }
#pragma unroll
        for (int off = 1; off < TPC; off <<= 1) dot += __shfl_xor(dot, off, 64);
        const float wgt = dot * dot;
        if (live) {
          float4 x[4];
          float xd = cd[rr];
#pragma unroll
          for (int j = 0; j < 4; ++j) x[j] = cs[rr][j];
          if (fresh) {
            const float* src = esum + (size_t)n * lstride;
#pragma unroll
            for (int j = 0; j < 4; ++j) x[j] = reinterpret_cast<const float4*>(src + 16 * part)[j];
            xd = src[DV];
          }
          float* dst = cache_sums + ((size_t)n * lambda + i) * DVS;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float4 rv4 = *reinterpret_cast<const float4*>(&sh.rv[16 * part + 4 * j]);
            reinterpret_cast<float4*>(dst + 16 * part)[j] =
                make_float4(x[j].x + wgt * rv4.x, x[j].y + wgt * rv4.y, x[j].z + wgt * rv4.z, x[j].w + wgt * rv4.w);
          }
          if (part == 0) dst[DV] = xd + wgt;
        }
      }
    }
    // (q . k_r)^2 = phi(q)^T phi(k_r), the readout's share of the deferred fold
    if (wave == 0) {
      float x = 0.0f;
      for (int d = lane; d < DQK; d += 64) x += sh.qv[d] * sh.rk[d];
      x = wave_sum(x);
      if (lane == 0) sh.corr = x * x;
    }
  } else {
    __syncthreads();
    for (int d = tid; d < DQK; d += kThreads) pend_k[((size_t)n * kPend + pslot) * DQK + d] = 0.0f;
    for (int d = tid; d < DV; d += kThreads) pend_v[((size_t)n * kPend + pslot) * DV + d] = 0.0f;
    if (evict) {
      for (int d = tid; d < DQK; d += kThreads)
        Elem<Tin>::store(cache_k, ((size_t)n * lambda + n_before) * DQK + d, sh.ek[d]);
      for (int d = tid; d < DV; d += kThreads)
        Elem<Tin>::store(cache_v, ((size_t)n * lambda + n_before) * DV + d, sh.ev[d]);
      for (int d = tid; d <= DV; d += kThreads)
        cache_sums[((size_t)n * lambda + n_before) * (DV + 4) + d] = esum[(size_t)n * lstride + d];
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
  const int wbase = win_first % wrows;  // ring row of token win_first; j < n_old <= W keeps wbase + j < 2 wrows
  auto ring = [&](int j) { const int r = wbase + j; return r >= wrows ? r - wrows : r; };
  // four elements (from `off`) of key or value row j, 0 <= j < n_keys. The
  // memory load is issued whatever j is (a row held in LDS — the new token,
  // the evicted pair's row — loads the window's first row instead and takes
  // the LDS copy), so the kU loads of a step have no branch between them and
  // are in flight together.
  auto row4 = [&](const Tin* win, const Tin* cache, int dim, const float* lds_new, const float* lds_ev, int j,
                  int off) -> float4 {
    const int r = j - n_old - 1;
    const bool from_cache = r >= 0 && r != replaced;
    const int wj = j < n_old ? j : 0;
    const Tin* p = from_cache ? cache + ((size_t)n * lambda + r) * dim + off
                              : win + ((size_t)n * wrows + ring(wj)) * dim + off;
    const float4 g = ld4<Tin>(p);
    const float4 a = *reinterpret_cast<const float4*>(lds_new + off);
    const float4 b = *reinterpret_cast<const float4*>(lds_ev + off);
    return (j < n_old || from_cache) ? g : (j == n_old ? a : b);
  };
  auto key4 = [&](int j, int off) { return row4(win_k, cache_k, DQK, sh.kn, sh.ek, j, off); };
  auto val4 = [&](int j, int off) { return row4(win_v, cache_v, DV, sh.vn, sh.ev, j, off); };
  // Scores: LPK lanes per key (a float4 each), KPW keys per wave and step;
  // weighted sum: LPV lanes per value row (a float4 each), RPW rows per wave
  // and step. kU steps are loaded before any is used.
  constexpr int LPV = DV / 4;
  constexpr int RPW = 64 / LPV;
  constexpr int KPB = kWaves * KPW;
  constexpr int RPB = kWaves * RPW;
  const float4 q4 = *reinterpret_cast<const float4*>(&sh.qv[4 * (lane % LPK)]);
  const int vc = 4 * (lane % LPV);
  // running maximum, starting at 0: the linear terms are scaled by e^{-m} too
  float m = 0.0f;
  float wsum = 0.0f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j0 = 0; j0 < n_keys; j0 += kKeyTile) {
    const int nt = min(kKeyTile, n_keys - j0);
    for (int jb = wave * KPW + lane / LPK; jb < nt; jb += kU * KPB) {  // a key group shares jb
      float4 k4[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int jl = jb + u * KPB;
        const float4 x = key4(j0 + min(jl, nt - 1), 4 * (lane % LPK));
        k4[u] = jl < nt ? x : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int jl = jb + u * KPB;
        float x = q4.x * k4[u].x + q4.y * k4[u].y + q4.z * k4[u].z + q4.w * k4[u].w;
#pragma unroll
        for (int off = LPK / 2; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
        if (jl < nt && lane % LPK == 0) sh.sc[jl] = x * scale;
      }
    }
    __syncthreads();
    float tm = -INFINITY;
    for (int j = tid; j < nt; j += kThreads) tm = fmaxf(tm, sh.sc[j]);
    const float m_new = fmaxf(m, block_max(tm, sh.red));
    const float rs = __expf(m - m_new);
    wsum *= rs;
    acc.x *= rs;
    acc.y *= rs;
    acc.z *= rs;
    acc.w *= rs;
    for (int j = tid; j < nt; j += kThreads) {
      const float p = __expf(sh.sc[j] - m_new);
      sh.sc[j] = p;
      wsum += p;
    }
    __syncthreads();
    for (int jb = wave * RPW + lane / LPV; jb < nt; jb += kU * RPB) {
      float4 v4[kU];
      float pw[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int jl = jb + u * RPB;
        const bool in = jl < nt;
        const float4 x = val4(j0 + min(jl, nt - 1), vc);
        v4[u] = in ? x : make_float4(0.f, 0.f, 0.f, 0.f);
        pw[u] = in ? sh.sc[min(jl, nt - 1)] : 0.0f;
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        acc.x += pw[u] * v4[u].x;
        acc.y += pw[u] * v4[u].y;
        acc.z += pw[u] * v4[u].z;
        acc.w += pw[u] * v4[u].w;
      }
    }
    __syncthreads();  // the next tile's scores overwrite sc
    m = m_new;
  }
  const float sm_den = block_sum(wsum, sh.red);
#pragma unroll
  for (int off = LPV; off < 64; off <<= 1) {
    acc.x += __shfl_xor(acc.x, off, 64);
    acc.y += __shfl_xor(acc.y, off, 64);
    acc.z += __shfl_xor(acc.z, off, 64);
    acc.w += __shfl_xor(acc.w, off, 64);
  }
  if (lane < LPV) *reinterpret_cast<float4*>(&sh.num[wave][vc]) = acc;
  __syncthreads();
  if (tid < DV) {
    float sm_num = 0.0f;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) sm_num += sh.num[i][tid];
    const float e = __expf(-m);
    const float nn = sm_num + e * lin_num;
    const float dd = sm_den + e * (lin_den + eps);
    Elem<Tout>::store(o, (size_t)n * DV + tid, dd != 0.0f ? nn / dd : 0.0f);
  }
  // ---- the new token enters the window, in the evicted token's row (whose
  // values were copied to LDS before the first barrier)
  for (int d = tid; d < DQK; d += kThreads) Elem<Tin>::store(win_k, srow * DQK + d, sh.kn[d]);
  for (int d = tid; d < DV; d += kThreads) Elem<Tin>::store(win_v, srow * DV + d, sh.vn[d]);
}

// ---------------------------------------------------------------- prime

// The cached pairs' sums against the linear state of (H, s) and the pending
// slots: work-group (block of 16 rows, head-state), thread (row e, columns
// cg, cg + 16, ...): sum_f phi_f(k_e) H_f + sum_j (k_e . pend_k_j)^2
// [pend_v_j | 1], in float32.
template <int DQK, int DV, typename R>
__global__ __launch_bounds__(kThreads) void hdec_prime_kernel(const float* __restrict__ H, const float* __restrict__ s,
                                                              const float* __restrict__ pend_k,
                                                              const float* __restrict__ pend_v,
                                                              const R* __restrict__ cache_k, int lambda,
                                                              int rows, float* __restrict__ cache_sums) {
  constexpr int D = phi_dim(DQK);
  constexpr int CPT = DV / 16;  // columns per thread
  __shared__ float kk[16][DQK];
  __shared__ float pk[kPend][DQK], pv[kPend][DV];
  __shared__ uint16_t tab[D];
  const int n = blockIdx.y;
  const int tid = threadIdx.x;
  const int el = tid / 16, cg = tid % 16;
  const int e = 16 * blockIdx.x + el;
  for (int i = tid; i < 16 * DQK; i += kThreads) {
    const int r = i / DQK, d = i % DQK;
    const int ee = 16 * blockIdx.x + r;
    kk[r][d] = ee < rows ? Elem<R>::load(cache_k, ((size_t)n * lambda + ee) * DQK + d) : 0.0f;
  }
  for (int i = tid; i < kPend * DQK; i += kThreads) pk[i / DQK][i % DQK] = pend_k[(size_t)n * kPend * DQK + i];
  for (int i = tid; i < kPend * DV; i += kThreads) pv[i / DV][i % DV] = pend_v[(size_t)n * kPend * DV + i];
  build_phi_table(tab, 0, D, DQK);
  __syncthreads();
  const float* Hn = H + (size_t)n * D * DV;
  const float* sn = s + (size_t)n * D;
  float acc[CPT];
#pragma unroll
  for (int j = 0; j < CPT; ++j) acc[j] = 0.0f;
  float den = 0.0f;
  for (int f = 0; f < D; ++f) {
    const float p = phi_of(kk[el], tab[f]);
#pragma unroll
    for (int j = 0; j < CPT; ++j) acc[j] += p * Hn[(size_t)f * DV + cg + 16 * j];
    den += p * sn[f];
  }
  for (int p = 0; p < kPend; ++p) {
    float dot = 0.0f;
    for (int d = 0; d < DQK; ++d) dot += kk[el][d] * pk[p][d];
    const float wgt = dot * dot;
#pragma unroll
    for (int j = 0; j < CPT; ++j) acc[j] += wgt * pv[p][cg + 16 * j];
    den += wgt;
  }
  if (e < rows) {
    float* dst = cache_sums + ((size_t)n * lambda + e) * (DV + 4);
#pragma unroll
    for (int j = 0; j < CPT; ++j) dst[cg + 16 * j] = acc[j];
    if (cg == 0) dst[DV] = den;
  }
}

// ---------------------------------------------------------------- host

int lin_stride(int dv) { return (dv + 1 + 3) / 4 * 4; }
size_t lin_bytes(const HybridDecodeArgs& a) { return align_up((size_t)a.N * lin_stride(a.dv) * sizeof(float)); }

bool use_matrix_pass(const HybridDecodeArgs& a) { return a.dqk == kFD && a.dv == kFD; }

template <int DQK, int DV, typename Tin, typename Tout>
hipError_t run_hd(const HybridDecodeArgs& a, void* ws, hipStream_t st) {
  char* p = static_cast<char*>(ws);
  float* lin = reinterpret_cast<float*>(p);
  float* esum = reinterpret_cast<float*>(p + lin_bytes(a));
  const int N = a.N, W = a.window, lam = a.cache_size, t = a.t;
  const int wrows = W + 1;
  const int slot = t % wrows;  // the evicted token's row, then the new token's
  const bool evict = t >= W + 1;
  const int evicted_id = t - W - 1;
  const int n_before = std::min(lam, std::max(0, t - W - 1));
  const bool refresh = evict && n_before == lam;
  const int n_after = std::min(lam, std::max(0, t - W));
  const int lstride = lin_stride(DV);
  const bool fold = t % kPend == 0;  // every slot is folded into (H, s); else H is only read
  Tin* wk = static_cast<Tin*>(a.win_k);  // window and cache rows are kept in the input type
  const int pslot = t % kPend;       // the slot this call's rejected pair waits in
  prof_begin(st);
  if (use_matrix_pass(a)) {
    if (fold)
      hipLaunchKernelGGL((hdec_state_kernel<Tin, true>), dim3(N), dim3(kThreads), 0, st, a.H, a.s, a.pend_k,
                         a.pend_v, static_cast<const Tin*>(a.q), wk, wrows, slot, evict, lin, esum, lstride);
    else
      hipLaunchKernelGGL((hdec_state_kernel<Tin, false>), dim3(N), dim3(kThreads), 0, st, a.H, a.s, a.pend_k,
                         a.pend_v, static_cast<const Tin*>(a.q), wk, wrows, slot, evict, lin, esum, lstride);
  } else {
    hipLaunchKernelGGL((hdec_fold_kernel<DQK, DV, Tin, true>), dim3(N), dim3(kThreads), 0, st, a.H, a.s, a.pend_k,
                       a.pend_v, static_cast<const Tin*>(a.q), lin, lstride, wk, wrows, slot, evict, fold,
                       esum);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((hdec_mix_kernel<DQK, DV, Tin, Tout>), dim3(N), dim3(kThreads), 0, st,
                     static_cast<const Tin*>(a.q), static_cast<const Tin*>(a.k), static_cast<const Tin*>(a.v),
                     static_cast<Tout*>(a.o), wk, static_cast<Tin*>(a.win_v), static_cast<Tin*>(a.cache_k),
                     static_cast<Tin*>(a.cache_v), a.cache_ids, a.pend_k,
                     a.pend_v, a.rejected, a.cache_sums, esum, lin, lstride, lam, n_before, n_after, refresh, evict,
                     wrows, std::max(0, t - W), t, slot, pslot, evicted_id, a.scale, a.eps);
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

size_t hybrid_decode_workspace(const HybridDecodeArgs& a) { return 2 * lin_bytes(a); }

hipError_t hybrid_decode_launch(const HybridDecodeArgs& a, void* ws, hipStream_t st) {
#define KLA_CASE(A, B) \
  if (a.dqk == A && a.dv == B) return run_hd_dt<A, B>(a, ws, st);
  KLA_CASE(16, 16) KLA_CASE(16, 32) KLA_CASE(16, 64)
  KLA_CASE(32, 16) KLA_CASE(32, 32) KLA_CASE(32, 64)
  KLA_CASE(64, 16) KLA_CASE(64, 32) KLA_CASE(64, 64)
#undef KLA_CASE
  return hipErrorInvalidValue;
}

hipError_t hybrid_decode_prime_launch(const HybridDecodeArgs& a, hipStream_t st) {
  const int rows = std::min(a.cache_size, std::max(0, a.t - a.window - 1));
  if (rows == 0) return hipSuccess;
#define KLA_CASE(A, B)                                                                                             \
  if (a.dqk == A && a.dv == B) {                                                                                   \
    if (a.in_bf16)                                                                                                 \
      hipLaunchKernelGGL((hdec_prime_kernel<A, B, uint16_t>), dim3((rows + 15) / 16, a.N), dim3(kThreads), 0, st, \
                         a.H, a.s, a.pend_k, a.pend_v, static_cast<const uint16_t*>(a.cache_k), a.cache_size, rows, \
                         a.cache_sums);                                                                            \
    else                                                                                                           \
      hipLaunchKernelGGL((hdec_prime_kernel<A, B, float>), dim3((rows + 15) / 16, a.N), dim3(kThreads), 0, st,    \
                         a.H, a.s, a.pend_k, a.pend_v, static_cast<const float*>(a.cache_k), a.cache_size, rows,   \
                         a.cache_sums);                                                                            \
    return hipGetLastError();                                                                                      \
  }
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
                       a.pend_k, a.pend_v, nullptr, nullptr, 0, nullptr, 1, 0, false, true, nullptr);          \
    return hipGetLastError();                                                                                   \
  }
  KLA_CASE(16, 16) KLA_CASE(16, 32) KLA_CASE(16, 64)
  KLA_CASE(32, 16) KLA_CASE(32, 32) KLA_CASE(32, 64)
  KLA_CASE(64, 16) KLA_CASE(64, 32) KLA_CASE(64, 64)
#undef KLA_CASE
  return hipErrorInvalidValue;
}

// ---------------------------------------------------------------- static scratch

// Scratch for callers that cannot allocate (HIP graph capture, serving loops,
// harnesses that forbid device allocation): the linear readouts of the query
// and of the evicted key (two rows of d_v + 4 floats per head-state) of
// kla_hybrid_decode_step_static live in this array instead of a caller
// workspace. Each device that the library runs on holds its own copy until
// the process ends. Every call on a device uses that device's copy, so calls
// that overlap on one device race; nothing in it has to start at zero (every
// call writes what it reads).
namespace {
static __device__ __align__(256) unsigned char scratch[kHybridDecodeStaticScratch];

constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];
}  // namespace

hipError_t hybrid_decode_static_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  // once per device, with that device current: the array's device address
  // (the name itself is only a host-side stand-in)
  std::call_once(g_scratch_once[dev], [dev]() {
    void* ptr = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? ptr : nullptr;
  });
  if (g_scratch_err[dev] != hipSuccess) return g_scratch_err[dev];
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace kla
