// Chunked causal prefill in float32 arithmetic on the vector ALUs.
//
// KATA page, §2.3 ("Paralelismo por Blocos"): tokens are split into chunks;
// inside a chunk the masked squared scores multiply [V | 1]; across chunks
// the state (H, s) is carried as a running prefix sum and read out by phi(Q).
//
// This is the general path: any supported (d_qk, d_v, chunk), float32 or
// bf16 inputs, float32 arithmetic throughout (1e-4 relative parity). It is
// also the state builder for decode (state-only mode, no outputs). With G > 1
// factors (KATA §2.3 "Variantes", read as G equal slices of p = d_qk / G
// dimensions) it serves both multi-factor lifts:
//   KATA-Mg, the factors' rank-one lifts concatenated: the features are the
//   pairs inside each factor, factor by factor, and the intra-chunk weight
//   is the sum of the factors' squared scores, sum_i (q_i . k_i)^2;
//   KATA-Sigma-g, the lift of the summed outer products sum_i x_i x_i^T: the
//   p(p+1)/2 features are the pairs (a, b) of one factor's dimensions, each
//   summed over the factors (sum_i x_i,a x_i,b), and the intra-chunk weight
//   is sum_{i,j} (q_i . k_j)^2 - the smallest state of the variants.
//
// Work split. The state of one head is D x d_v floats (D = d_qk(d_qk+1)/2),
// too large for one CU at d_qk = 64, so every head is split into S feature
// slices of at most 256 features; a work-group owns one (slice, head) pair,
// keeps its slice of H and s in registers and walks the chunks in order
// (the prefix sum is the register-resident running state). Tokens go in
// tiles of 16: each tile's features are formed once into LDS (thread f forms
// feature f for every token), laid out so that a thread's own features are
// contiguous, and the readout and update read them as broadcast 16-byte
// loads; the next tile's rows are loaded while the current one is used. The
// readout of a slice is a partial numerator/denominator per token; a second
// kernel adds the S partials to the exact intra-chunk term and divides.
#include <algorithm>

#include "kla_device.hpp"
#include "kla_internal.hpp"

namespace kla {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxSlice = 256;  // features per slice
constexpr int kTok = 16;        // token tile

// Pair (a, b) of feature f of the G-factor lift over d dimensions (G = 1:
// the rank-one lift), packed as a | (b << 8): for the concatenated lift the
// dimensions of factor f / (p(p+1)/2); for the summed lift a pair of the
// first factor's dimensions (the feature adds the same pair of every factor).
__device__ __forceinline__ uint16_t factor_pair(int f, int d, int G, int kind) {
  const int p = d / G;
  if (kind == 1) return phi_pair(f, p);
  const int dp = p * (p + 1) / 2;
  const int fi = f / dp;
  const uint16_t ab = phi_pair(f - fi * dp, p);
  return static_cast<uint16_t>(ab + (fi * p) * 0x0101);
}

// Feature value of pair ab: the rank-one or concatenated lift reads it
// directly; the summed lift adds it over the G factors of p dimensions.
__device__ __forceinline__ float factor_phi(const float* x, uint16_t ab, int kind, int G, int p) {
  if (kind != 1) return phi_of(x, ab);
  float acc = 0.0f;
  for (int i = 0; i < G; ++i) acc += phi_of(x + i * p, ab);
  return acc;
}

template <int DQK, int DV, typename Tin>
__global__ __launch_bounds__(kThreads) void prefill_slice_kernel(
    const Tin* __restrict__ q, const Tin* __restrict__ k, const Tin* __restrict__ v, int T,
    int chunk, int S, int Fs, const float* __restrict__ H0, const float* __restrict__ s0,
    float* __restrict__ HT, float* __restrict__ sT, float* __restrict__ part, int D, int factors, int kind) {
  constexpr int G = kThreads / DV;    // feature groups
  constexpr int J = kMaxSlice / G;    // features per thread
  constexpr int W = kThreads / 64;    // waves
  static_assert(J % 4 == 0, "features per thread in float4 groups");

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
  // features of a token tile, formed once per token: feature fl = g + G j of
  // the slice at ph[r][g][j], so a thread's J features are contiguous
  __shared__ __align__(16) float ph[kTok][G][J];
  __shared__ float red[kTok][G][DV];
  __shared__ float rden[kTok][W];

  for (int i = threadIdx.x; i < fcount; i += blockDim.x) tab[i] = factor_pair(f0 + i, DQK, factors, kind);
  const int fp = DQK / factors;

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
  // features of the tile in xs (zero past the slice): thread tid forms feature tid for every token
  auto form = [&]() {
    const bool ok = tid < fcount;
    const uint16_t ab = ok ? tab[tid] : 0;
    const int gg = tid % G, jj = tid / G;
#pragma unroll 4
    for (int r = 0; r < kTok; ++r) ph[r][gg][jj] = ok ? factor_phi(xs[r], ab, kind, factors, fp) : 0.0f;
  };
  // this thread's features fill jused of its J slots; later float4 groups are skipped
  const int jused = (fcount - g + G - 1) / G;

  // The tiles in order: per chunk, the query tiles of the readout (when
  // outputs are wanted), then the key/value tiles of the update. The next
  // tile's rows are loaded into registers while the current one is used.
  constexpr int kPX = kTok * DQK / kThreads;
  constexpr int kPV = kTok * DV / kThreads;
  static_assert(kPX * kThreads == kTok * DQK && kPV * kThreads == kTok * DV, "tile loads");
  struct Tile {
    int c0, t0, upd;  // upd: 0 readout (q), 1 update (k, v)
  };
  auto first_tile = [&]() { return Tile{0, 0, part ? 0 : 1}; };
  auto next_tile = [&](Tile t) {
    const int L = min(chunk, T - t.c0);
    if (t.t0 + kTok < L) return Tile{t.c0, t.t0 + kTok, t.upd};
    if (!t.upd) return Tile{t.c0, 0, 1};
    return Tile{t.c0 + chunk, 0, part ? 0 : 1};
  };
  float px[kPX], pv[kPV];
  auto fetch = [&](Tile t) {
    const int L = t.c0 < T ? min(chunk, T - t.c0) : 0;
    const int nb = max(0, min(kTok, L - t.t0));
    const Tin* src = t.upd ? k : q;
#pragma unroll
    for (int e = 0; e < kPX; ++e) {
      const int i = tid + e * kThreads;
      const int r = i / DQK, d = i % DQK;
      px[e] = r < nb ? Elem<Tin>::load(src, bqk + (size_t)(t.c0 + t.t0 + r) * DQK + d) : 0.0f;
    }
#pragma unroll
    for (int e = 0; e < kPV; ++e) {
      const int i = tid + e * kThreads;
      const int r = i / DV, d = i % DV;
      pv[e] = (t.upd && r < nb) ? Elem<Tin>::load(v, bv + (size_t)(t.c0 + t.t0 + r) * DV + d) : 0.0f;
    }
  };
  Tile cur = first_tile();
  fetch(cur);
  while (cur.c0 < T) {
    const int L = min(chunk, T - cur.c0);
    const int nb = min(kTok, L - cur.t0);
#pragma unroll
    for (int e = 0; e < kPX; ++e) {
      const int i = tid + e * kThreads;
      xs[i / DQK][i % DQK] = px[e];
    }
    if (cur.upd) {
#pragma unroll
      for (int e = 0; e < kPV; ++e) {
        const int i = tid + e * kThreads;
        vs[i / DV][i % DV] = pv[e];
      }
    }
    const Tile nxt = next_tile(cur);
    if (nxt.c0 < T) fetch(nxt);
    __syncthreads();
    form();
    __syncthreads();
    if (!cur.upd) {
      // readout of the state at the chunk start
#pragma unroll 1
      for (int r = 0; r < kTok; ++r) {
        const float4* pr = reinterpret_cast<const float4*>(ph[r][g]);
        float acc = 0.0f;
#pragma unroll
        for (int j4 = 0; j4 < J / 4; ++j4) {
          if (4 * j4 < jused) {
            const float4 x = pr[j4];
            acc += x.x * h[4 * j4] + x.y * h[4 * j4 + 1] + x.z * h[4 * j4 + 2] + x.w * h[4 * j4 + 3];
          }
        }
        red[r][g][c] = acc;
      }
      // denominators: every token's product first, then the wave sums side by side
      {
        float dd[kTok];
#pragma unroll
        for (int r = 0; r < kTok; ++r) dd[r] = tid < fcount ? ph[r][tid % G][tid / G] * sm : 0.0f;
#pragma unroll
        for (int off = 32; off > 0; off >>= 1)
#pragma unroll
          for (int r = 0; r < kTok; ++r) dd[r] += __shfl_xor(dd[r], off, 64);
        if ((tid & 63) == 0) {
#pragma unroll
          for (int r = 0; r < kTok; ++r) rden[r][tid >> 6] = dd[r];
        }
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
        part[(((size_t)n * S + slice) * T + cur.c0 + cur.t0 + r) * (DV + 1) + cc] = sum;
      }
    } else {
      // state update with the tile's keys and values
#pragma unroll 1
      for (int r = 0; r < nb; ++r) {
        const float vv = vs[r][c];
        const float4* pr = reinterpret_cast<const float4*>(ph[r][g]);
#pragma unroll
        for (int j4 = 0; j4 < J / 4; ++j4) {
          if (4 * j4 < jused) {
            const float4 x = pr[j4];
            h[4 * j4] += x.x * vv;
            h[4 * j4 + 1] += x.y * vv;
            h[4 * j4 + 2] += x.z * vv;
            h[4 * j4 + 3] += x.w * vv;
          }
        }
        if (tid < fcount) sm += ph[r][tid % G][tid / G];
      }
    }
    __syncthreads();
    cur = nxt;
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
    Tout* __restrict__ o, int T, int chunk, int S, const float* __restrict__ part, float eps, int factors,
    int kind) {
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
      // concatenated lift: the sum over the factors (p dimensions each) of
      // the squared factor scores; summed lift: of every factor pair's
      const int p = DQK / factors;
      const int pm = p - 1;
      float wsum = 0.0f;
      if (kind == 1) {
        for (int fi = 0; fi < factors; ++fi)
          for (int fj = 0; fj < factors; ++fj) {
            float dot = 0.0f;
            for (int d = 0; d < p; ++d) dot += qs[qq][fi * p + d] * ks[kk][fj * p + d];
            wsum += dot * dot;
          }
      } else {
        float dot = 0.0f;
#pragma unroll
        for (int d = 0; d < DQK; ++d) {
          dot += qs[qq][d] * ks[kk][d];
          const bool end = ((d + 1) & pm) == 0;
          wsum += end ? dot * dot : 0.0f;
          dot = end ? 0.0f : dot;
        }
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

// Feature slices per head: enough for the features (at most kMaxSlice each)
// and, for small states or few heads, enough work-groups to fill the GPU
// (slices of at least 32 features).
// Slices per head: at most 256 features each, and more (down to 32 each)
// until the launch has about one work-group per CU (more slices repeat the
// per-tile work of every work-group and measured slower).
int slices_for(int D, int N) {
  const int s0 = (D + kMaxSlice - 1) / kMaxSlice;
  const int fill = (256 + N - 1) / N;
  return std::max(s0, std::min(fill, (D + 31) / 32));
}

// features of the G-factor lift over d dimensions (kind 0 concatenated, 1 summed)
int factor_dim(int d, int G, int kind) {
  const int p = d / G;
  return (kind == 1 ? 1 : G) * p * (p + 1) / 2;
}

template <int DQK, int DV, typename Tin, typename Tout>
hipError_t launch_typed(const PrefillArgs& a, void* ws, hipStream_t st) {
  const int D = factor_dim(DQK, a.factors, a.factor_kind);
  const int S = slices_for(D, a.N);
  const int Fs = (D + S - 1) / S;
  float* part = a.o ? static_cast<float*>(ws) : nullptr;
  prof_begin(st);
  hipLaunchKernelGGL((prefill_slice_kernel<DQK, DV, Tin>), dim3(S, a.N), dim3(kThreads), 0, st,
                     static_cast<const Tin*>(a.q), static_cast<const Tin*>(a.k),
                     static_cast<const Tin*>(a.v), a.T, a.chunk, S, Fs, a.H0, a.s0, a.HT, a.sT,
                     part, D, a.factors, a.factor_kind);
  prof_end(st);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !a.o) return e;
  hipLaunchKernelGGL((prefill_combine_kernel<DQK, DV, Tin, Tout>), dim3((a.T + 15) / 16, a.N),
                     dim3(kThreads), 0, st, static_cast<const Tin*>(a.q),
                     static_cast<const Tin*>(a.k), static_cast<const Tin*>(a.v),
                     static_cast<Tout*>(a.o), a.T, a.chunk, S, part, a.eps, a.factors, a.factor_kind);
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
  const int S = slices_for(factor_dim(a.dqk, a.factors, a.factor_kind), a.N);
  return align_up((size_t)a.N * S * a.T * (a.dv + 1) * sizeof(float));
}

hipError_t prefill_valu_launch(const PrefillArgs& a, void* ws, hipStream_t st) {
  if ((a.factor_kind != 0 && a.factor_kind != 1) || (a.factors != 1 && a.factors != 2 && a.factors != 4))
    return hipErrorInvalidValue;
  switch (a.dqk) {
    case 16: return launch_dv<16>(a, ws, st);
    case 32: return launch_dv<32>(a, ws, st);
    case 64: return launch_dv<64>(a, ws, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace kla
