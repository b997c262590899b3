// Chunked causal prefill in float32 arithmetic on the vector ALUs.
//
// KATA page, §2.3 ("Paralelismo por Blocos"): tokens are split into chunks;
// inside a chunk the masked squared scores multiply [V | 1]; across chunks
// the state (H, s) is carried as a running prefix sum and read out by phi(Q).
//
// This is the general path: any supported (d_qk, d_v, chunk), float32 or
// bf16 inputs, float32 arithmetic throughout (1e-4 relative parity). It is
// also the state builder for decode (state-only mode, no outputs). With G > 1
// factors (KATA-Mg, KATA §2.3 "Variantes", read as G equal slices of the
// d_qk dimensions with their rank-one lifts concatenated) the features are
// the pairs inside each factor, factor by factor, and the intra-chunk weight
// is the sum of the factors' squared scores.
//
// Work split. The state of one head is D x d_v floats (D = d_qk(d_qk+1)/2),
// too large for one CU at d_qk = 64, so every head is split into S feature
// slices of at most 256 features; a work-group owns one (slice, head) pair,
// keeps its slice of H and s in registers and walks the chunks in order
// (the prefix sum is the register-resident running state). The readout of a
// slice is a partial numerator/denominator per token; a second kernel adds
// the S partials to the exact intra-chunk term and divides.
#include "kla_device.hpp"
#include "kla_internal.hpp"

namespace kla {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxSlice = 256;  // features per slice
constexpr int kTok = 16;        // token tile

// Pair (a, b) of feature f of the G-factor lift over d dimensions (G = 1:
// the rank-one lift), packed as a | (b << 8).
__device__ __forceinline__ uint16_t factor_pair(int f, int d, int G) {
  const int p = d / G;
  const int dp = p * (p + 1) / 2;
  const int fi = f / dp;
  const uint16_t ab = phi_pair(f - fi * dp, p);
  return static_cast<uint16_t>(ab + (fi * p) * 0x0101);
}

template <int DQK, int DV, typename Tin>
__global__ __launch_bounds__(kThreads) void prefill_slice_kernel(
    const Tin* __restrict__ q, const Tin* __restrict__ k, const Tin* __restrict__ v, int T,
    int chunk, int S, int Fs, const float* __restrict__ H0, const float* __restrict__ s0,
    float* __restrict__ HT, float* __restrict__ sT, float* __restrict__ part, int D, int factors) {
  constexpr int G = kThreads / DV;    // feature groups
  constexpr int J = kMaxSlice / G;    // features per thread
  constexpr int W = kThreads / 64;    // waves

  const int slice = blockIdx.x;
  const int n = blockIdx.y;
  const int tid = threadIdx.x;
  const int c = tid % DV;
  const int g = tid / DV;
  const int f0 = slice * Fs;
  const int fcount = min(Fs, D - f0);

  __shared__ uint16_t tab[kMaxSlice];
  __shared__ float xs[kTok][DQK + 1];
  __shared__ float vs[kTok][DV];
  __shared__ float red[kTok][G][DV];
  __shared__ float rden[kTok][W];

  for (int i = threadIdx.x; i < fcount; i += blockDim.x) tab[i] = factor_pair(f0 + i, DQK, factors);

  float h[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int fl = g + G * j;
    h[j] = (fl < fcount && H0) ? H0[((size_t)n * D + f0 + fl) * DV + c] : 0.0f;
  }
  float sm = (tid < fcount && s0) ? s0[(size_t)n * D + f0 + tid] : 0.0f;
  __syncthreads();

  const size_t bqk = (size_t)n * T * DQK;
  const size_t bv = (size_t)n * T * DV;

  for (int c0 = 0; c0 < T; c0 += chunk) {
    const int L = min(chunk, T - c0);
    if (part) {
      // readout of the state at the chunk start, one token tile at a time
      for (int t0 = 0; t0 < L; t0 += kTok) {
        const int nb = min(kTok, L - t0);
        for (int i = tid; i < kTok * DQK; i += kThreads) {
          const int r = i / DQK, d = i % DQK;
          xs[r][d] = r < nb ? Elem<Tin>::load(q, bqk + (size_t)(c0 + t0 + r) * DQK + d) : 0.0f;
        }
        __syncthreads();
        for (int r = 0; r < kTok; ++r) {
          float acc = 0.0f;
#pragma unroll
          for (int j = 0; j < J; ++j) {
            const int fl = g + G * j;
            if (fl < fcount) acc += phi_of(xs[r], tab[fl]) * h[j];
          }
          red[r][g][c] = acc;
          float dd = tid < fcount ? phi_of(xs[r], tab[tid]) * sm : 0.0f;
          dd = wave_sum(dd);
          if ((tid & 63) == 0) rden[r][tid >> 6] = dd;
        }
        __syncthreads();
        for (int i = tid; i < nb * (DV + 1); i += kThreads) {
          const int r = i / (DV + 1), cc = i % (DV + 1);
          float sum = 0.0f;
          if (cc < DV) {
#pragma unroll
            for (int gg = 0; gg < G; ++gg) sum += red[r][gg][cc];
          } else {
#pragma unroll
            for (int w = 0; w < W; ++w) sum += rden[r][w];
          }
          part[(((size_t)n * S + slice) * T + c0 + t0 + r) * (DV + 1) + cc] = sum;
        }
        __syncthreads();
      }
    }
    // state update with the whole chunk
    for (int t0 = 0; t0 < L; t0 += kTok) {
      const int nb = min(kTok, L - t0);
      for (int i = tid; i < kTok * DQK; i += kThreads) {
        const int r = i / DQK, d = i % DQK;
        xs[r][d] = r < nb ? Elem<Tin>::load(k, bqk + (size_t)(c0 + t0 + r) * DQK + d) : 0.0f;
      }
      for (int i = tid; i < kTok * DV; i += kThreads) {
        const int r = i / DV, d = i % DV;
        vs[r][d] = r < nb ? Elem<Tin>::load(v, bv + (size_t)(c0 + t0 + r) * DV + d) : 0.0f;
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
      __syncthreads();
    }
  }
  if (HT) {
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int fl = g + G * j;
      if (fl < fcount) HT[((size_t)n * D + f0 + fl) * DV + c] = h[j];
    }
  }
  if (sT && tid < fcount) sT[(size_t)n * D + f0 + tid] = sm;
}

// Intra-chunk term plus the S slice partials; one block per (16 queries, head).
template <int DQK, int DV, typename Tin, typename Tout>
__global__ __launch_bounds__(kThreads) void prefill_combine_kernel(
    const Tin* __restrict__ q, const Tin* __restrict__ k, const Tin* __restrict__ v,
    Tout* __restrict__ o, int T, int chunk, int S, const float* __restrict__ part, float eps, int factors) {
  constexpr int QB = 16;
  constexpr int KB = 32;
  constexpr int M = DV / 16;
  const int n = blockIdx.y;
  const int t0 = blockIdx.x * QB;
  const int tid = threadIdx.x;
  const int r = tid / 16;
  const int l16 = tid % 16;
  const int cstart = (t0 / chunk) * chunk;
  const int nq = min(QB, T - t0);

  __shared__ float qs[QB][DQK + 1];
  __shared__ float ks[KB][DQK + 1];
  __shared__ float vs[KB][DV];
  __shared__ float w[QB][KB + 1];

  const size_t bqk = (size_t)n * T * DQK;
  const size_t bv = (size_t)n * T * DV;
  for (int i = tid; i < QB * DQK; i += kThreads) {
    const int rr = i / DQK, d = i % DQK;
    qs[rr][d] = rr < nq ? Elem<Tin>::load(q, bqk + (size_t)(t0 + rr) * DQK + d) : 0.0f;
  }
  float acc[M];
#pragma unroll
  for (int m = 0; m < M; ++m) acc[m] = 0.0f;
  float den = 0.0f;

  const int kend = t0 + nq;  // keys [cstart, kend)
  for (int kt = cstart; kt < kend; kt += KB) {
    const int nk = min(KB, kend - kt);
    __syncthreads();
    for (int i = tid; i < KB * DQK; i += kThreads) {
      const int rr = i / DQK, d = i % DQK;
      ks[rr][d] = rr < nk ? Elem<Tin>::load(k, bqk + (size_t)(kt + rr) * DQK + d) : 0.0f;
    }
    for (int i = tid; i < KB * DV; i += kThreads) {
      const int rr = i / DV, d = i % DV;
      vs[rr][d] = rr < nk ? Elem<Tin>::load(v, bv + (size_t)(kt + rr) * DV + d) : 0.0f;
    }
    __syncthreads();
    for (int i = tid; i < QB * KB; i += kThreads) {
      const int qq = i / KB, kk = i % KB;
      // sum over the factors (p dimensions each) of the squared factor scores
      const int pm = DQK / factors - 1;
      float dot = 0.0f, wsum = 0.0f;
#pragma unroll
      for (int d = 0; d < DQK; ++d) {
        dot += qs[qq][d] * ks[kk][d];
        const bool end = ((d + 1) & pm) == 0;
        wsum += end ? dot * dot : 0.0f;
        dot = end ? 0.0f : dot;
      }
      const bool ok = (kk < nk) && (kt + kk <= t0 + qq) && (qq < nq);
      w[qq][kk] = ok ? wsum : 0.0f;
    }
    __syncthreads();
    for (int kk = 0; kk < nk; ++kk) {
      const float wi = w[r][kk];
#pragma unroll
      for (int m = 0; m < M; ++m) acc[m] += wi * vs[kk][l16 + 16 * m];
      den += wi;
    }
  }
  if (r < nq) {
    const int t = t0 + r;
    for (int s = 0; s < S; ++s) {
      const float* p = part + (((size_t)n * S + s) * T + t) * (DV + 1);
#pragma unroll
      for (int m = 0; m < M; ++m) acc[m] += p[l16 + 16 * m];
      den += p[DV];
    }
    const float dt = den + eps;
    const float inv = dt != 0.0f ? 1.0f / dt : 0.0f;
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const float val = dt != 0.0f ? acc[m] * inv : 0.0f;
      Elem<Tout>::store(o, bv + (size_t)t * DV + l16 + 16 * m, val);
    }
  }
}

int slices_for(int D) { return (D + kMaxSlice - 1) / kMaxSlice; }

// features of the G-factor lift over d dimensions
int factor_dim(int d, int G) {
  const int p = d / G;
  return G * p * (p + 1) / 2;
}

template <int DQK, int DV, typename Tin, typename Tout>
hipError_t launch_typed(const PrefillArgs& a, void* ws, hipStream_t st) {
  const int D = factor_dim(DQK, a.factors);
  const int S = slices_for(D);
  const int Fs = (D + S - 1) / S;
  float* part = a.o ? static_cast<float*>(ws) : nullptr;
  prof_begin(st);
  hipLaunchKernelGGL((prefill_slice_kernel<DQK, DV, Tin>), dim3(S, a.N), dim3(kThreads), 0, st,
                     static_cast<const Tin*>(a.q), static_cast<const Tin*>(a.k),
                     static_cast<const Tin*>(a.v), a.T, a.chunk, S, Fs, a.H0, a.s0, a.HT, a.sT,
                     part, D, a.factors);
  prof_end(st);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !a.o) return e;
  hipLaunchKernelGGL((prefill_combine_kernel<DQK, DV, Tin, Tout>), dim3((a.T + 15) / 16, a.N),
                     dim3(kThreads), 0, st, static_cast<const Tin*>(a.q),
                     static_cast<const Tin*>(a.k), static_cast<const Tin*>(a.v),
                     static_cast<Tout*>(a.o), a.T, a.chunk, S, part, a.eps, a.factors);
  return hipGetLastError();
}

template <int DQK, int DV>
hipError_t launch_dtypes(const PrefillArgs& a, void* ws, hipStream_t st) {
  if (a.in_bf16) {
    return a.out_bf16 ? launch_typed<DQK, DV, uint16_t, uint16_t>(a, ws, st)
                      : launch_typed<DQK, DV, uint16_t, float>(a, ws, st);
  }
  return a.out_bf16 ? launch_typed<DQK, DV, float, uint16_t>(a, ws, st)
                    : launch_typed<DQK, DV, float, float>(a, ws, st);
}

template <int DQK>
hipError_t launch_dv(const PrefillArgs& a, void* ws, hipStream_t st) {
  switch (a.dv) {
    case 16: return launch_dtypes<DQK, 16>(a, ws, st);
    case 32: return launch_dtypes<DQK, 32>(a, ws, st);
    case 64: return launch_dtypes<DQK, 64>(a, ws, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace

size_t prefill_valu_workspace(const PrefillArgs& a) {
  if (!a.o) return 0;
  const int S = slices_for(phi_dim(a.dqk));
  return align_up((size_t)a.N * S * a.T * (a.dv + 1) * sizeof(float));
}

hipError_t prefill_valu_launch(const PrefillArgs& a, void* ws, hipStream_t st) {
  if (a.factor_kind != 0 || (a.factors != 1 && a.factors != 2 && a.factors != 4)) return hipErrorInvalidValue;
  switch (a.dqk) {
    case 16: return launch_dv<16>(a, ws, st);
    case 32: return launch_dv<32>(a, ws, st);
    case 64: return launch_dv<64>(a, ws, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace kla
