// LoLA's three memories, token by token (LoLA page, "Estratégia de
// Inferência": the token-by-token mode of items 1-4; "Metodologia" items
// 1-3 for the memories).
//
// One call advances every head-state by one token t (the number of tokens
// it has seen). With window W and cache size lambda:
//   1. token e = t - W - 1 leaves the window when t > W. While the cache has
//      room it joins the cache; once the cache is full, e and the lambda
//      cached pairs are scored by the self-recall error against (H, s), the
//      lambda highest (score desc, token id asc) stay and the lowest one is
//      folded into the state: H += phi(k_e') v_e'^T, s += phi(k_e');
//   2. the query reads one jointly normalised mixture of the window
//      [max(0, t - W), t] (softmax weights e^{a q.k}), the cache (the same
//      weights) and the linear state (phi(q)^T H, phi(q)^T s + eps), as the
//      blocked hybrid prefill does with refresh = 1;
//   3. token t enters the window ring in the row the evicted token left.
// Kernels (all counts are known on the host from t):
//   score   : SRE of the lambda + 1 candidates (float32, shared SRE block);
//   reject  : the lowest (score, -id) candidate; the evicted pair takes its
//             cache row; the rejected pair is kept for the fold;
//   append  : while the cache fills, the evicted pair takes the next row;
//   readout : fold (when there is one) and linear readout in one pass over
//             H, then the window and cache softmax, the joint division, and
//             the window insert.
#include <algorithm>

#include "kla_device.hpp"
#include "kla_internal.hpp"
#include "sre_block.hpp"

namespace kla {
namespace {

constexpr int kThreads = 256;

template <int DQK, int DV>
__global__ __launch_bounds__(kThreads) void hdec_score_kernel(
    const float* __restrict__ H, const float* __restrict__ s, const float* __restrict__ cache_k,
    const float* __restrict__ cache_v, const float* __restrict__ win_k, const float* __restrict__ win_v,
    int lambda, int wrows, int slot, float* __restrict__ scores, int sstride, float eps) {
  constexpr int D = phi_dim(DQK);
  __shared__ SreShared<DQK, DV> sh;
  const int n = blockIdx.y;
  // candidates: cache rows 0..lambda-1, then the evicted window row
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

// The rejected candidate is the last in (score desc, token id asc) order.
template <int DQK, int DV>
__global__ __launch_bounds__(kThreads) void hdec_reject_kernel(
    const float* __restrict__ scores, int sstride, float* __restrict__ cache_k, float* __restrict__ cache_v,
    int32_t* __restrict__ cache_ids, const float* __restrict__ win_k, const float* __restrict__ win_v,
    int lambda, int wrows, int slot, int evicted_id, float* __restrict__ rej_k, float* __restrict__ rej_v,
    int32_t* __restrict__ rejected) {
  __shared__ uint64_t red[kThreads];
  __shared__ float ek[DQK], ev[DV];
  const int n = blockIdx.x;
  const int tid = threadIdx.x;
  uint64_t worst = ~0ull;
  for (int c = tid; c <= lambda; c += kThreads) {
    const int id = c < lambda ? cache_ids[(size_t)n * lambda + c] : evicted_id;
    const float sc = lambda > 0 ? scores[(size_t)n * sstride + c] : 0.0f;  // lone candidate: not scored
    worst = min(worst, topk_key(sc, (uint32_t)id));
  }
  red[tid] = worst;
  __syncthreads();
  for (int w = kThreads / 2; w > 0; w >>= 1) {
    if (tid < w) red[tid] = min(red[tid], red[tid + w]);
    __syncthreads();
  }
  const int rid = (int)topk_index(red[0]);
  // the rejected candidate's row: the evicted pair, or the cache row holding rid
  int r = lambda;
  if (rid != evicted_id)
    for (int c = 0; c < lambda; ++c)
      if (cache_ids[(size_t)n * lambda + c] == rid) r = c;
  const float* rk = r < lambda ? cache_k + ((size_t)n * lambda + r) * DQK : win_k + ((size_t)n * wrows + slot) * DQK;
  const float* rv = r < lambda ? cache_v + ((size_t)n * lambda + r) * DV : win_v + ((size_t)n * wrows + slot) * DV;
  for (int d = tid; d < DQK; d += kThreads) {
    rej_k[(size_t)n * DQK + d] = rk[d];
    ek[d] = win_k[((size_t)n * wrows + slot) * DQK + d];
  }
  for (int d = tid; d < DV; d += kThreads) {
    rej_v[(size_t)n * DV + d] = rv[d];
    ev[d] = win_v[((size_t)n * wrows + slot) * DV + d];
  }
  __syncthreads();  // every read of row r is done before it is replaced
  if (r < lambda) {
    for (int d = tid; d < DQK; d += kThreads) cache_k[((size_t)n * lambda + r) * DQK + d] = ek[d];
    for (int d = tid; d < DV; d += kThreads) cache_v[((size_t)n * lambda + r) * DV + d] = ev[d];
    if (tid == 0) cache_ids[(size_t)n * lambda + r] = evicted_id;
  }
  if (rejected && tid == 0) rejected[n] = rid;
}

template <int DQK, int DV>
__global__ void hdec_append_kernel(float* __restrict__ cache_k, float* __restrict__ cache_v,
                                   int32_t* __restrict__ cache_ids, const float* __restrict__ win_k,
                                   const float* __restrict__ win_v, int lambda, int wrows, int slot, int row,
                                   int evicted_id) {
  const int n = blockIdx.x;
  for (int d = threadIdx.x; d < DQK; d += blockDim.x)
    cache_k[((size_t)n * lambda + row) * DQK + d] = win_k[((size_t)n * wrows + slot) * DQK + d];
  for (int d = threadIdx.x; d < DV; d += blockDim.x)
    cache_v[((size_t)n * lambda + row) * DV + d] = win_v[((size_t)n * wrows + slot) * DV + d];
  if (threadIdx.x == 0) cache_ids[(size_t)n * lambda + row] = evicted_id;
}

constexpr int kKeyTile = kThreads;  // softmax keys scored per pass (online max across passes)
constexpr int kWaves = kThreads / 64;

template <int DQK, int DV>
struct ReadLds {
  static constexpr int D = phi_dim(DQK);
  float pq[D];             // phi(q)_f
  float pk[D];             // phi(k_rejected)_f (fold only)
  alignas(16) float qv[DQK];
  alignas(16) float kn[DQK];  // the new token
  float vn[DV];
  float rv[DV];            // the rejected value (fold only)
  float sc[kKeyTile];      // one tile's scores, then weights
  float red[kWaves];
  float num[kThreads / DV][DV];
  uint16_t tab[D];
};

// Block-wide reductions; every thread gets the result.
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

// One work-group per head-state.
template <int DQK, int DV, typename Tin, typename Tout>
__global__ __launch_bounds__(kThreads) void hdec_readout_kernel(
    float* __restrict__ H, float* __restrict__ s, const Tin* __restrict__ q, const Tin* __restrict__ k,
    const Tin* __restrict__ v, Tout* __restrict__ o, float* __restrict__ win_k, float* __restrict__ win_v,
    const float* __restrict__ cache_k, const float* __restrict__ cache_v, int lambda, int n_cache,
    int wrows, int win_first, int t, int slot, bool fold, const float* __restrict__ rej_k,
    const float* __restrict__ rej_v, float scale, float eps) {
  constexpr int D = phi_dim(DQK);
  constexpr int G = kThreads / DV;  // feature groups (one value column per thread)
  constexpr int LPK = DQK / 4;      // lanes per key in the score pass (a float4 each)
  constexpr int KPW = 64 / LPK;     // keys per wave and pass
  __shared__ ReadLds<DQK, DV> sh;
  const int n = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int c = tid % DV;
  const int g = tid / DV;

  for (int d = tid; d < DQK; d += kThreads) {
    sh.qv[d] = Elem<Tin>::load(q, (size_t)n * DQK + d);
    sh.kn[d] = Elem<Tin>::load(k, (size_t)n * DQK + d);
  }
  for (int d = tid; d < DV; d += kThreads) {
    sh.vn[d] = Elem<Tin>::load(v, (size_t)n * DV + d);
    if (fold) sh.rv[d] = rej_v[(size_t)n * DV + d];
  }
  build_phi_table(sh.tab, 0, D, DQK);
  __syncthreads();
  const float* rk = rej_k + (size_t)n * DQK;
  for (int f = tid; f < D; f += kThreads) {
    sh.pq[f] = phi_of(sh.qv, sh.tab[f]);
    if (fold) sh.pk[f] = phi_of(rk, sh.tab[f]);
  }
  __syncthreads();

  // ---- state: fold, then the linear readout against the folded state
  float* Hn = H + (size_t)n * D * DV;
  float* sn = s + (size_t)n * D;
  const float vr = fold ? sh.rv[c] : 0.0f;
  float lin = 0.0f;
#pragma unroll 8
  for (int f = g; f < D; f += G) {
    float h = Hn[(size_t)f * DV + c];
    if (fold) {
      h += sh.pk[f] * vr;
      Hn[(size_t)f * DV + c] = h;
    }
    lin += sh.pq[f] * h;
  }
  float den = 0.0f;
  for (int f = tid; f < D; f += kThreads) {
    float x = sn[f];
    if (fold) {
      x += sh.pk[f];
      sn[f] = x;
    }
    den += sh.pq[f] * x;
  }
  sh.num[g][c] = lin;
  const float lin_den = block_sum(den, sh.red);  // its barrier also publishes sh.num
  float lin_num = 0.0f;
#pragma unroll
  for (int i = 0; i < G; ++i) lin_num += sh.num[i][c];
  __syncthreads();

  // ---- softmax keys: window tokens win_first .. t - 1 (ring rows), the new
  // token t (kept in LDS), then the cache rows
  const int n_old = t - win_first;
  const int n_keys = n_old + 1 + n_cache;
  auto key_row = [&](int j) -> const float* {
    if (j < n_old) return win_k + ((size_t)n * wrows + (win_first + j) % wrows) * DQK;
    if (j == n_old) return sh.kn;
    return cache_k + ((size_t)n * lambda + (j - n_old - 1)) * DQK;
  };
  auto val_row = [&](int j) -> const float* {
    if (j < n_old) return win_v + ((size_t)n * wrows + (win_first + j) % wrows) * DV;
    if (j == n_old) return sh.vn;
    return cache_v + ((size_t)n * lambda + (j - n_old - 1)) * DV;
  };
  const float4 q4 = *reinterpret_cast<const float4*>(&sh.qv[4 * (lane % LPK)]);
  // Running maximum, starting at 0: the linear terms are scaled by e^{-m} too.
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
    const float r = __expf(m - m_new);
    wsum *= r;
    acc *= r;
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
  // ---- the new token enters the window, in the evicted token's row
  for (int d = tid; d < DQK; d += kThreads) win_k[((size_t)n * wrows + slot) * DQK + d] = sh.kn[d];
  for (int d = tid; d < DV; d += kThreads) win_v[((size_t)n * wrows + slot) * DV + d] = sh.vn[d];
}

__global__ void fill_i32_kernel(int32_t* p, size_t n, int32_t x) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = x;
}

struct HdWs {
  float* scores;  // [N, cache_size + 1]
  float* rej_k;   // [N, d_qk]
  float* rej_v;   // [N, d_v]
};

size_t scores_bytes(const HybridDecodeArgs& a) {
  return align_up((size_t)a.N * (a.cache_size + 1) * sizeof(float));
}

HdWs carve_hd(const HybridDecodeArgs& a, void* ws) {
  char* p = static_cast<char*>(ws);
  HdWs w;
  w.scores = reinterpret_cast<float*>(p);
  p += scores_bytes(a);
  w.rej_k = reinterpret_cast<float*>(p);
  p += align_up((size_t)a.N * a.dqk * sizeof(float));
  w.rej_v = reinterpret_cast<float*>(p);
  return w;
}

template <int DQK, int DV, typename Tin, typename Tout>
hipError_t run_hd(const HybridDecodeArgs& a, void* ws, hipStream_t st) {
  const HdWs w = carve_hd(a, ws);
  const int N = a.N, W = a.window, lam = a.cache_size, t = a.t;
  const int wrows = W + 1;
  const int slot = t % wrows;  // the evicted token's row, then the new token's
  const bool evict = t >= W + 1;
  const int evicted_id = t - W - 1;
  const int n_before = std::min(lam, std::max(0, t - W - 1));
  const bool refresh = evict && n_before == lam;
  const int n_after = std::min(lam, std::max(0, t - W));
  const int sstride = lam + 1;
  prof_begin(st);
  if (evict && !refresh) {
    hipLaunchKernelGGL((hdec_append_kernel<DQK, DV>), dim3(N), dim3(64), 0, st, a.cache_k, a.cache_v, a.cache_ids,
                       a.win_k, a.win_v, lam, wrows, slot, n_before, evicted_id);
  } else if (refresh) {
    if (lam > 0)
      hipLaunchKernelGGL((hdec_score_kernel<DQK, DV>), dim3((lam + 1 + 63) / 64, N), dim3(kThreads), 0, st, a.H,
                         a.s, a.cache_k, a.cache_v, a.win_k, a.win_v, lam, wrows, slot, w.scores, sstride, a.eps);
    hipLaunchKernelGGL((hdec_reject_kernel<DQK, DV>), dim3(N), dim3(kThreads), 0, st, w.scores, sstride,
                       a.cache_k, a.cache_v, a.cache_ids, a.win_k, a.win_v, lam, wrows, slot, evicted_id, w.rej_k,
                       w.rej_v, a.rejected);
  }
  if (!refresh && a.rejected)
    hipLaunchKernelGGL(fill_i32_kernel, dim3(1), dim3(256), 0, st, a.rejected, (size_t)N, -1);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((hdec_readout_kernel<DQK, DV, Tin, Tout>), dim3(N), dim3(kThreads), 0, st, a.H, a.s,
                     static_cast<const Tin*>(a.q), static_cast<const Tin*>(a.k), static_cast<const Tin*>(a.v),
                     static_cast<Tout*>(a.o), a.win_k, a.win_v, a.cache_k, a.cache_v, lam, n_after, wrows,
                     std::max(0, t - W), t, slot, refresh, w.rej_k, w.rej_v, a.scale, a.eps);
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
  return scores_bytes(a) + align_up((size_t)a.N * a.dqk * sizeof(float)) +
         align_up((size_t)a.N * a.dv * sizeof(float));
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

}  // namespace kla
