// Hybrid prefill with LoLA's three memories (LoLA page, "Metodologia" items
// 1-3 and "Estratégia de Inferência" items 1-4): a sliding window of exact
// softmax attention, a linear state (H, s) with the rank-one PSD lift of
// the KATA page (§2.2), and a sparse cache of the pairs the state recalls
// worst, chosen by self-recall error.
//
// This file holds the float32 vector-ALU form, for every shape the
// matrix-core form (hybrid_mfma.hip: d_qk = d_v = 64, bf16 inputs) does not
// take. Blocks of `refresh` tokens are processed in order; the selection of
// a refresh depends on the fold of the previous one, so the chain is
// sequential per head; every step runs for all heads at once:
//   score  : SRE of every candidate (cache + newly evicted) against (H, s);
//   select : order the (score, token id) keys by a bitonic sort; keep
//            cache_size, list the rest;
//   fold   : H += phi(k_i) v_i^T, s += phi(k_i) over the rejected tokens;
//   readout: for the block's queries, window and cache softmax terms and
//            the linear readout join one numerator and one denominator.
// The host knows every count in advance (they depend only on T, window,
// refresh and cache_size), so no device value is read back.
#include <algorithm>
#include <type_traits>
#include <vector>

#include "kla_device.hpp"
#include "kla_internal.hpp"
#include "sre_block.hpp"

namespace kla {
namespace {

constexpr int kThreads = 256;
constexpr int kWavesF = kThreads / 64;
constexpr int kMaxSlice = 256;

__global__ void fill_kernel_f32(float* p, size_t n, float x) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = x;
}
__global__ void fill_kernel_i32(int32_t* p, size_t n, int32_t x) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = x;
}

// cache[n][n_cache + i] = first + i for i < count (no scoring needed).
__global__ void append_kernel(int32_t* cache, int stride, int n_cache, int first, int count) {
  const int n = blockIdx.x;
  for (int i = threadIdx.x; i < count; i += blockDim.x)
    cache[(size_t)n * stride + n_cache + i] = first + i;
}

// dst[n][i] = src[n][i] for i < width.
__global__ void copy_rows_kernel(int32_t* dst, int width, const int32_t* src, int src_stride) {
  const int n = blockIdx.x;
  for (int i = threadIdx.x; i < width; i += blockDim.x)
    dst[(size_t)n * width + i] = src[(size_t)n * src_stride + i];
}

// Candidate j of head n: cache[j] for j < n_cache, else token ev0 + (j - n_cache).
__device__ __forceinline__ int cand_token(const int32_t* cache_n, int n_cache, int ev0, int j) {
  return j < n_cache ? cache_n[j] : ev0 + (j - n_cache);
}

template <int DQK, int DV, typename Tin>
__global__ __launch_bounds__(kThreads) void hyb_score_kernel(
    const float* __restrict__ H, const float* __restrict__ s, const Tin* __restrict__ k,
    const Tin* __restrict__ v, int T, const int32_t* __restrict__ cache, int cstride, int n_cache,
    int ev0, int n_cand, float* __restrict__ scores, int sstride, float eps) {
  constexpr int D = phi_dim(DQK);
  __shared__ SreShared<DQK, DV> sh;
  const int n = blockIdx.y;
  const int32_t* cn = cache + (size_t)n * cstride;
  const size_t bk = (size_t)n * T * DQK;
  const size_t bv = (size_t)n * T * DV;
  auto load_k = [&](int c, int d) {
    return Elem<Tin>::load(k, bk + (size_t)cand_token(cn, n_cache, ev0, c) * DQK + d);
  };
  auto load_v = [&](int c, int d) {
    return Elem<Tin>::load(v, bv + (size_t)cand_token(cn, n_cache, ev0, c) * DV + d);
  };
  sre_block<DQK, DV>(sh, H + (size_t)n * D * DV, s + (size_t)n * D, blockIdx.x * 64, n_cand,
                     load_k, load_v, scores + (size_t)n * sstride, eps);
}

// Keep the cache_size best candidates; write the new cache (ascending token
// ids), the rejected tokens, and the trace row.
__global__ __launch_bounds__(kThreads) void hyb_select_kernel(
    const float* __restrict__ scores, int sstride, int32_t* __restrict__ cache, int cstride,
    int n_cache, int ev0, int n_cand, int keep, int32_t* __restrict__ rejected, int rstride,
    int32_t* __restrict__ trace, size_t trace_row_stride, int block, int nblocks) {
  __shared__ uint64_t keys[256];
  __shared__ uint64_t kept[256];
  const int n = blockIdx.x;
  const int32_t* cn = cache + (size_t)n * cstride;
  for (int i = threadIdx.x; i < 256; i += blockDim.x) {
    keys[i] = i < n_cand
                  ? topk_key(scores[(size_t)n * sstride + i], (uint32_t)cand_token(cn, n_cache, ev0, i))
                  : 0ull;
  }
  bitonic_sort_desc(keys, 256);
  // kept tokens, re-sorted ascending by id (descending on 0xFFFFFFFF - id)
  for (int i = threadIdx.x; i < 256; i += blockDim.x)
    kept[i] = i < keep ? (keys[i] & 0xFFFFFFFFull) : 0ull;
  __syncthreads();
  bitonic_sort_desc(kept, 256);
  for (int i = threadIdx.x; i < n_cand - keep; i += blockDim.x)
    rejected[(size_t)n * rstride + i] = (int32_t)topk_index(keys[keep + i]);
  int32_t* cw = cache + (size_t)n * cstride;
  for (int i = threadIdx.x; i < keep; i += blockDim.x) {
    const int32_t id = (int32_t)topk_index(kept[i]);
    cw[i] = id;
    if (trace) trace[((size_t)n * nblocks + block) * trace_row_stride + i] = id;
  }
}

// H += sum_r phi(k_r) v_r^T and s += sum_r phi(k_r) over the rejected tokens;
// grid (feature slices, N).
template <int DQK, int DV, typename Tin>
__global__ __launch_bounds__(kThreads) void hyb_fold_kernel(float* __restrict__ H,
                                                            float* __restrict__ s,
                                                            const Tin* __restrict__ k,
                                                            const Tin* __restrict__ v, int T,
                                                            const int32_t* __restrict__ rejected,
                                                            int rstride, int n_rej, int Fs) {
  constexpr int D = phi_dim(DQK);
  constexpr int G = kThreads / DV;
  constexpr int J = kMaxSlice / G;
  constexpr int TB = 16;
  const int slice = blockIdx.x;
  const int n = blockIdx.y;
  const int tid = threadIdx.x;
  const int c = tid % DV;
  const int g = tid / DV;
  const int f0 = slice * Fs;
  const int fcount = min(Fs, D - f0);
  __shared__ uint16_t tab[kMaxSlice];
  __shared__ float xs[TB][DQK + 1];
  __shared__ float vs[TB][DV];
  build_phi_table(tab, f0, fcount, DQK);
  float* Hn = H + (size_t)n * D * DV;
  float h[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int fl = g + G * j;
    h[j] = fl < fcount ? Hn[(size_t)(f0 + fl) * DV + c] : 0.0f;
  }
  float sm = tid < fcount ? s[(size_t)n * D + f0 + tid] : 0.0f;
  const int32_t* rj = rejected + (size_t)n * rstride;
  const size_t bk = (size_t)n * T * DQK;
  const size_t bv = (size_t)n * T * DV;
  for (int r0 = 0; r0 < n_rej; r0 += TB) {
    const int nb = min(TB, n_rej - r0);
    __syncthreads();
    for (int i = tid; i < TB * DQK; i += kThreads) {
      const int r = i / DQK, d = i % DQK;
      xs[r][d] = r < nb ? Elem<Tin>::load(k, bk + (size_t)rj[r0 + r] * DQK + d) : 0.0f;
    }
    for (int i = tid; i < TB * DV; i += kThreads) {
      const int r = i / DV, d = i % DV;
      vs[r][d] = r < nb ? Elem<Tin>::load(v, bv + (size_t)rj[r0 + r] * DV + d) : 0.0f;
    }
    __syncthreads();
    for (int r = 0; r < nb; ++r) {
      const float vv = vs[r][c];
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const int fl = g + G * j;
        if (fl < fcount) h[j] += phi_of(xs[r], tab[fl]) * vv;
      }
      if (tid < fcount) sm += phi_of(xs[r], tab[tid]);
    }
  }
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int fl = g + G * j;
    if (fl < fcount) Hn[(size_t)(f0 + fl) * DV + c] = h[j];
  }
  if (tid < fcount) s[(size_t)n * D + f0 + tid] = sm;
}

// Output of 16 queries [t0, t0+16) of a block whose window starts at f.
// Softmax terms use a running maximum m >= 0; the linear terms are scaled by
// e^{-m} so that numerator and denominator share one normalisation.
template <int DQK, int DV, typename Tin, typename Tout>
__global__ __launch_bounds__(kThreads) void hyb_readout_kernel(
    const Tin* __restrict__ q, const Tin* __restrict__ k, const Tin* __restrict__ v,
    Tout* __restrict__ o, int T, const float* __restrict__ H, const float* __restrict__ s,
    const int32_t* __restrict__ cache, int cstride, int n_cache, int t_begin, int t_end, int f,
    float scale, float eps) {
  constexpr int D = phi_dim(DQK);
  constexpr int QB = 16;
  constexpr int KT = 64;
  constexpr int M = DV / 16;
  constexpr int FT = 32;
  const int n = blockIdx.y;
  const int t0 = t_begin + blockIdx.x * QB;
  const int nq = min(QB, t_end - t0);
  const int tid = threadIdx.x;
  const int r = tid / 16;
  const int l16 = tid % 16;

  __shared__ float qs[QB][DQK + 1];
  __shared__ float ks[KT][DQK + 1];
  __shared__ float vs[KT][DV];
  __shared__ float x[QB][KT + 1];
  __shared__ float Ht[FT][DV];
  __shared__ float st[FT];
  __shared__ uint16_t tab[D];

  const size_t bqk = (size_t)n * T * DQK;
  const size_t bv = (size_t)n * T * DV;
  const int32_t* cn = cache + (size_t)n * cstride;
  for (int i = tid; i < QB * DQK; i += kThreads) {
    const int rr = i / DQK, d = i % DQK;
    qs[rr][d] = rr < nq ? Elem<Tin>::load(q, bqk + (size_t)(t0 + rr) * DQK + d) : 0.0f;
  }
  build_phi_table(tab, 0, D, DQK);

  float m = 0.0f;  // running max, never below 0
  float l = 0.0f;
  float acc[M];
#pragma unroll
  for (int j = 0; j < M; ++j) acc[j] = 0.0f;

  // keys: cache entries, then the window [f, t0 + nq)
  const int n_win = (t0 + nq) - f;
  const int n_keys = n_cache + n_win;
  for (int k0 = 0; k0 < n_keys; k0 += KT) {
    const int nk = min(KT, n_keys - k0);
    __syncthreads();
    for (int i = tid; i < KT * DQK; i += kThreads) {
      const int rr = i / DQK, d = i % DQK;
      float val = 0.0f;
      if (rr < nk) {
        const int j = k0 + rr;
        const int tok = j < n_cache ? cn[j] : f + (j - n_cache);
        val = Elem<Tin>::load(k, bqk + (size_t)tok * DQK + d);
      }
      ks[rr][d] = val;
    }
    for (int i = tid; i < KT * DV; i += kThreads) {
      const int rr = i / DV, d = i % DV;
      float val = 0.0f;
      if (rr < nk) {
        const int j = k0 + rr;
        const int tok = j < n_cache ? cn[j] : f + (j - n_cache);
        val = Elem<Tin>::load(v, bv + (size_t)tok * DV + d);
      }
      vs[rr][d] = val;
    }
    __syncthreads();
    for (int i = tid; i < QB * KT; i += kThreads) {
      const int qq = i / KT, kk = i % KT;
      const int j = k0 + kk;
      bool ok = kk < nk && qq < nq;
      if (ok && j >= n_cache) ok = (f + (j - n_cache)) <= t0 + qq;  // causal window
      float dot = 0.0f;
#pragma unroll 16
      for (int d = 0; d < DQK; ++d) dot += qs[qq][d] * ks[kk][d];
      x[qq][kk] = ok ? scale * dot : -INFINITY;
    }
    __syncthreads();
    // tile max for query r (16 lanes of the row)
    float tm = -INFINITY;
    for (int kk = l16; kk < KT; kk += 16) tm = fmaxf(tm, x[r][kk]);
#pragma unroll
    for (int off = 8; off > 0; off >>= 1) tm = fmaxf(tm, __shfl_xor(tm, off, 16));
    const float mn = fmaxf(m, tm);
    const float corr = __expf(m - mn);
    l *= corr;
#pragma unroll
    for (int j = 0; j < M; ++j) acc[j] *= corr;
    m = mn;
#pragma unroll 4
    for (int kk = 0; kk < nk; ++kk) {
      const float p = __expf(x[r][kk] - m);
      l += p;
#pragma unroll
      for (int j = 0; j < M; ++j) acc[j] += p * vs[kk][l16 + 16 * j];
    }
  }

  // linear readout phi(q)^T [H | s]
  float lin[M];
#pragma unroll
  for (int j = 0; j < M; ++j) lin[j] = 0.0f;
  float lden = 0.0f;
  const float* Hn = H + (size_t)n * D * DV;
  const float* sn = s + (size_t)n * D;
#pragma unroll 1
  for (int f0 = 0; f0 < D; f0 += FT) {
    const int nf = min(FT, D - f0);
    __syncthreads();
    for (int i = tid; i < FT * DV; i += kThreads) {
      const int rr = i / DV, cc = i % DV;
      Ht[rr][cc] = rr < nf ? Hn[(size_t)(f0 + rr) * DV + cc] : 0.0f;
    }
    for (int i = tid; i < FT; i += kThreads) st[i] = i < nf ? sn[f0 + i] : 0.0f;
    __syncthreads();
#pragma unroll 4
    for (int rr = 0; rr < nf; ++rr) {
      const float p = phi_of(qs[r], tab[f0 + rr]);
#pragma unroll
      for (int j = 0; j < M; ++j) lin[j] += p * Ht[rr][l16 + 16 * j];
      lden += p * st[rr];
    }
  }
  if (r < nq) {
    const float e = __expf(-m);
    const float den = l + e * (lden + eps);
    const int t = t0 + r;
#pragma unroll
    for (int j = 0; j < M; ++j) {
      const float num = acc[j] + e * lin[j];
      Elem<Tout>::store(o, bv + (size_t)t * DV + l16 + 16 * j, den != 0.0f ? num / den : 0.0f);
    }
  }
}

constexpr int kCStride = 256;  // candidates per refresh, at most (cache + evicted)

struct Ws {
  float* H;
  float* s;
  int32_t* cache;
  float* scores;
  int32_t* rejected;
};

Ws carve(const HybridArgs& a, void* ws) {
  const int D = phi_dim(a.dqk);
  char* p = static_cast<char*>(ws);
  Ws w;
  if (a.HT) {
    w.H = a.HT;
  } else {
    w.H = reinterpret_cast<float*>(p);
    p += align_up((size_t)a.N * D * a.dv * sizeof(float));
  }
  if (a.sT) {
    w.s = a.sT;
  } else {
    w.s = reinterpret_cast<float*>(p);
    p += align_up((size_t)a.N * D * sizeof(float));
  }
  w.cache = reinterpret_cast<int32_t*>(p);
  p += align_up((size_t)a.N * kCStride * sizeof(int32_t));
  w.scores = reinterpret_cast<float*>(p);
  p += align_up((size_t)a.N * kCStride * sizeof(float));
  w.rejected = reinterpret_cast<int32_t*>(p);
  return w;
}

template <int DQK, int DV, typename Tin, typename Tout>
hipError_t run(const HybridArgs& a, void* ws, hipStream_t st) {
  constexpr int D = phi_dim(DQK);
  const Ws w = carve(a, ws);
  const int N = a.N;
  const int nblocks = (a.T + a.refresh - 1) / a.refresh;
  const Tin* q = static_cast<const Tin*>(a.q);
  const Tin* k = static_cast<const Tin*>(a.k);
  const Tin* v = static_cast<const Tin*>(a.v);
  Tout* o = static_cast<Tout*>(a.o);
  hipError_t e;
#define KLA_CHECK()                      \
  do {                                   \
    e = hipGetLastError();               \
    if (e != hipSuccess) return e;       \
  } while (0)
  hipLaunchKernelGGL(fill_kernel_f32, dim3(1024), dim3(256), 0, st, w.H, (size_t)N * D * DV, 0.0f);
  hipLaunchKernelGGL(fill_kernel_f32, dim3(64), dim3(256), 0, st, w.s, (size_t)N * D, 0.0f);
  hipLaunchKernelGGL(fill_kernel_i32, dim3(64), dim3(256), 0, st, w.cache, (size_t)N * kCStride, -1);
  if (a.trace && a.cache_size > 0)
    hipLaunchKernelGGL(fill_kernel_i32, dim3(1024), dim3(256), 0, st, a.trace,
                       (size_t)N * nblocks * a.cache_size, -1);
  KLA_CHECK();
  const int S = (D + kMaxSlice - 1) / kMaxSlice;
  const int Fs = (D + S - 1) / S;
  int n_cache = 0;
  int f_prev = 0;
  for (int b = 0; b < nblocks; ++b) {
    const int b0 = b * a.refresh;
    const int b1 = std::min(a.T, b0 + a.refresh);
    const int f = std::max(0, b0 - a.window);
    const int n_ev = f - f_prev;
    if (n_ev > 0) {
      const int n_cand = n_cache + n_ev;
      if (n_cand <= a.cache_size) {
        hipLaunchKernelGGL(append_kernel, dim3(N), dim3(256), 0, st, w.cache, kCStride, n_cache,
                           f_prev, n_ev);
        KLA_CHECK();
        n_cache = n_cand;
      } else {
        prof_begin(st);
        hipLaunchKernelGGL((hyb_score_kernel<DQK, DV, Tin>), dim3((n_cand + 63) / 64, N),
                           dim3(kThreads), 0, st, w.H, w.s, k, v, a.T, w.cache, kCStride, n_cache,
                           f_prev, n_cand, w.scores, kCStride, a.eps);
        hipLaunchKernelGGL(hyb_select_kernel, dim3(N), dim3(kThreads), 0, st, w.scores, kCStride,
                           w.cache, kCStride, n_cache, f_prev, n_cand, a.cache_size, w.rejected,
                           kCStride, a.trace, (size_t)a.cache_size, b, nblocks);
        prof_end(st);
        KLA_CHECK();
        hipLaunchKernelGGL((hyb_fold_kernel<DQK, DV, Tin>), dim3(S, N), dim3(kThreads), 0, st,
                           w.H, w.s, k, v, a.T, w.rejected, kCStride, n_cand - a.cache_size, Fs);
        KLA_CHECK();
        n_cache = a.cache_size;
      }
    }
    f_prev = f;
    hipLaunchKernelGGL((hyb_readout_kernel<DQK, DV, Tin, Tout>), dim3((b1 - b0 + 15) / 16, N),
                       dim3(kThreads), 0, st, q, k, v, o, a.T, w.H, w.s, w.cache, kCStride,
                       n_cache, b0, b1, f, a.scale, a.eps);
    KLA_CHECK();
  }
  if (a.cache_T && a.cache_size > 0) {
    hipLaunchKernelGGL(copy_rows_kernel, dim3(N), dim3(256), 0, st, a.cache_T, a.cache_size,
                       w.cache, kCStride);
    KLA_CHECK();
  }
#undef KLA_CHECK
  return hipSuccess;
}

template <int DQK, int DV>
hipError_t run_dt(const HybridArgs& a, void* ws, hipStream_t st) {
  if (a.in_bf16)
    return a.out_bf16 ? run<DQK, DV, uint16_t, uint16_t>(a, ws, st)
                      : run<DQK, DV, uint16_t, float>(a, ws, st);
  return a.out_bf16 ? run<DQK, DV, float, uint16_t>(a, ws, st) : run<DQK, DV, float, float>(a, ws, st);
}

}  // namespace

size_t hybrid_workspace(const HybridArgs& a) {
  if (hybrid_mfma_supported(a)) return hybrid_mfma_workspace(a);
  const int D = phi_dim(a.dqk);
  size_t b = 0;
  if (!a.HT) b += align_up((size_t)a.N * D * a.dv * sizeof(float));
  if (!a.sT) b += align_up((size_t)a.N * D * sizeof(float));
  b += align_up((size_t)a.N * kCStride * sizeof(int32_t));
  b += align_up((size_t)a.N * kCStride * sizeof(float));
  b += align_up((size_t)a.N * kCStride * sizeof(int32_t));
  return b;
}

hipError_t hybrid_launch(const HybridArgs& a, void* ws, hipStream_t st, hipStream_t aux) {
  if (hybrid_mfma_supported(a)) return hybrid_mfma_launch(a, ws, st, aux);
#define KLA_CASE(A, B) \
  if (a.dqk == A && a.dv == B) return run_dt<A, B>(a, ws, st);
  KLA_CASE(16, 16) KLA_CASE(16, 32) KLA_CASE(16, 64)
  KLA_CASE(32, 16) KLA_CASE(32, 32) KLA_CASE(32, 64)
  KLA_CASE(64, 16) KLA_CASE(64, 32) KLA_CASE(64, 64)
#undef KLA_CASE
  return hipErrorInvalidValue;
}

}  // namespace kla
