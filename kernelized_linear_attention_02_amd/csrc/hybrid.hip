// Hybrid prefill with LoLA's three memories (LoLA page, "Metodologia" items
// 1-3 and "Estratégia de Inferência" items 1-4): a sliding window of exact
// softmax attention, a linear state (H, s) with the rank-one PSD lift of
// the KATA page (§2.2), and a sparse cache of the pairs the state recalls
// worst, chosen by self-recall error.
//
// Blocks of `refresh` tokens are processed in order. The selection of a
// refresh depends on the fold of the previous one, so the chain is
// sequential per head; every step runs for all heads at once:
//   score  : SRE of every candidate (cache + newly evicted) against (H, s);
//   select : order the (score, token id) keys (a bitonic sort, or ranks
//            by counting on the matrix-core path); keep cache_size, list
//            the rest;
//   fold   : H += phi(k_i) v_i^T, s += phi(k_i) over the rejected tokens;
//   readout: for the block's queries, window and cache softmax terms and
//            the linear readout join one numerator and one denominator.
// On the matrix-core path the score of refresh r reads the state before the
// fold of refresh r - 1 and adds that fold's pairs in closed form
// ((k_c . k_j)^2 weights), so the fold of r - 1 and the score of r share one
// launch (hyb_refresh_kernel).
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

// ---------------------------------------------------------------- matrix-core fold (d = 64, bf16 in)
//
// [H | s] += phi(K_r)^T [V_r | 1] over the rejected tokens, on the matrix
// cores: each wave takes 32-feature k-steps (canonical order, two 16-row
// tiles) and keeps them in MFMA accumulators seeded with the stored state.
// The feature products k_a k_b (times sqrt(2) off the diagonal) are exact
// float32 values split into three bf16 pieces p0 + p1 + p2 = p; v is bf16 on
// input, so every MFMA product is exact and the sums are float32, as in a
// float32 fold. Output column n-tile nt of lane (l16, q4) is state column
// 4 l16 + nt. Besides the float32 state, the fold writes it as readout B
// fragments (two bf16 pieces): fragment (k-step ks, n-tile nt) of lane
// (l16, q4) holds rows 32 ks + 4 q4 + i and 32 ks + 16 + 4 q4 + i (i < 4) of
// column 4 l16 + nt - exactly the lane's accumulators of the two tiles - and
// n-tile 4 holds s in lane column 0.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
constexpr int kFD = 64;
constexpr int kFPhi = kFD * (kFD + 1) / 2;   // 2080
constexpr int kFoldRows = 128;               // rejected tokens per call, at most

struct alignas(16) FoldPairs {
  uint16_t ab[kFPhi];
  constexpr FoldPairs() : ab{} {
    int f = 0;
    for (int a = 0; a < kFD; ++a)
      for (int b = a; b < kFD; ++b) ab[f++] = static_cast<uint16_t>(a | (b << 8));
  }
};
__constant__ FoldPairs kFoldPairs = FoldPairs();

__device__ __forceinline__ void split3_8(const float (&x)[8], bf16x8& p0, bf16x8& p1, bf16x8& p2) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const __bf16 a = (__bf16)x[j];
    const float r = x[j] - (float)a;
    const __bf16 b = (__bf16)r;
    p0[j] = a;
    p1[j] = b;
    p2[j] = (__bf16)(r - (float)b);
  }
}

// x ~ p0 + p1 with p0 = bf16(x), p1 = bf16(x - p0): 16 significant bits.
__device__ __forceinline__ void split2_8(const float (&x)[8], bf16x8& p0, bf16x8& p1) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const __bf16 a = (__bf16)x[j];
    p0[j] = a;
    p1[j] = (__bf16)(x[j] - (float)a);
  }
}

constexpr int kFKS = kFPhi / 32;             // 65 k-steps
constexpr int kFoldKsPerWG = 4;              // one per wave

// index of fragment (n, ks, piece, nt, lane) in uint4 units; three exact
// bf16 pieces per value (the readout uses the first two)
constexpr int kHFPieces = 3;
__device__ __forceinline__ size_t hf_index(int n, int ks, int pc, int nt, int lane) {
  return ((((size_t)n * kFKS + ks) * kHFPieces + pc) * 5 + nt) * 64 + lane;
}

struct FoldLds {
  float kt[kFD][kFoldRows + 4];
  uint16_t vt[kFD][kFoldRows + 8];
};
constexpr int kFoldWGs = (kFKS + kFoldKsPerWG - 1) / kFoldKsPerWG;  // work-groups per head

// Work-group (bx, n) of the fold: k-steps bx kFoldKsPerWG .. + kFoldKsPerWG - 1 of head n.
__device__ __forceinline__ void hyb_fold_block(FoldLds& sh, int bx, int n, float* __restrict__ H,
                                               float* __restrict__ s, uint4* __restrict__ HF,
                                               const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                                               int T, const int32_t* __restrict__ rejected, int rstride,
                                               int n_rej) {
  float (&kt)[kFD][kFoldRows + 4] = sh.kt;
  uint16_t (&vt)[kFD][kFoldRows + 8] = sh.vt;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l16 = lane & 15;
  const int q4 = lane >> 4;
  const int R = (n_rej + 31) & ~31;  // rows padded to whole k-steps (zeros)

  for (int i = tid; i < R * (kFD / 4); i += kThreads) {
    const int r = i / (kFD / 4);
    const int d4 = i % (kFD / 4);
    uint2 ku = make_uint2(0, 0), vu = ku;
    if (r < n_rej) {
      const size_t row = ((size_t)n * T + rejected[(size_t)n * rstride + r]) * kFD + 4 * d4;
      ku = *reinterpret_cast<const uint2*>(k + row);
      vu = *reinterpret_cast<const uint2*>(v + row);
    }
    kt[4 * d4 + 0][r] = __uint_as_float(ku.x << 16);
    kt[4 * d4 + 1][r] = __uint_as_float(ku.x & 0xFFFF0000u);
    kt[4 * d4 + 2][r] = __uint_as_float(ku.y << 16);
    kt[4 * d4 + 3][r] = __uint_as_float(ku.y & 0xFFFF0000u);
    vt[4 * d4 + 0][r] = (uint16_t)(vu.x & 0xFFFF);
    vt[4 * d4 + 1][r] = (uint16_t)(vu.x >> 16);
    vt[4 * d4 + 2][r] = (uint16_t)(vu.y & 0xFFFF);
    vt[4 * d4 + 3][r] = (uint16_t)(vu.y >> 16);
  }
  __syncthreads();

  bf16x8 ones;
#pragma unroll
  for (int j = 0; j < 8; ++j) ones[j] = (__bf16)(l16 == 0 ? 1.0f : 0.0f);
  float* Hn = H + (size_t)n * kFPhi * kFD;
  float* sn = s + (size_t)n * kFPhi;
#pragma unroll 1
  for (int u = 0; u < kFoldKsPerWG / kWavesF; ++u) {
    const int ks = bx * kFoldKsPerWG + u * kWavesF + w;
    if (ks >= kFKS) break;
    f32x4 acc[2][5];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int f0 = 32 * ks + 16 * t;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float4 h = *reinterpret_cast<const float4*>(Hn + (size_t)(f0 + 4 * q4 + i) * kFD + 4 * l16);
        acc[t][0][i] = h.x;
        acc[t][1][i] = h.y;
        acc[t][2][i] = h.z;
        acc[t][3][i] = h.w;
        acc[t][4][i] = l16 == 0 ? sn[f0 + 4 * q4 + i] : 0.0f;
      }
    }
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      // this lane's feature row (A operand) and its factors
      const uint16_t ab = kFoldPairs.ab[32 * ks + 16 * t + l16];
      const int fa = ab & 0xFF, fb = ab >> 8;
      const float wgt = fa == fb ? 1.0f : 1.41421356237309504880f;
      for (int kk = 0; kk < R / 32; ++kk) {
        const float4* pa = reinterpret_cast<const float4*>(&kt[fa][32 * kk + 8 * q4]);
        const float4* pb = reinterpret_cast<const float4*>(&kt[fb][32 * kk + 8 * q4]);
        const float4 a0 = pa[0], a1 = pa[1], b0 = pb[0], b1 = pb[1];
        const float p[8] = {a0.x * b0.x * wgt, a0.y * b0.y * wgt, a0.z * b0.z * wgt, a0.w * b0.w * wgt,
                            a1.x * b1.x * wgt, a1.y * b1.y * wgt, a1.z * b1.z * wgt, a1.w * b1.w * wgt};
        bf16x8 A0, A1, A2;
        split3_8(p, A0, A1, A2);
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
          // value column 4 l16 + nt of the 8 tokens 32 kk + 8 q4 + j
          const bf16x8 B = *reinterpret_cast<const bf16x8*>(&vt[4 * l16 + nt][32 * kk + 8 * q4]);
          acc[t][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A0, B, acc[t][nt], 0, 0, 0);
          acc[t][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A1, B, acc[t][nt], 0, 0, 0);
          acc[t][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A2, B, acc[t][nt], 0, 0, 0);
        }
        acc[t][4] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A0, ones, acc[t][4], 0, 0, 0);
        acc[t][4] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A1, ones, acc[t][4], 0, 0, 0);
        acc[t][4] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A2, ones, acc[t][4], 0, 0, 0);
      }
    }
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int f0 = 32 * ks + 16 * t;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        *reinterpret_cast<float4*>(Hn + (size_t)(f0 + 4 * q4 + i) * kFD + 4 * l16) =
            make_float4(acc[t][0][i], acc[t][1][i], acc[t][2][i], acc[t][3][i]);
        if (l16 == 0) sn[f0 + 4 * q4 + i] = acc[t][4][i];
      }
    }
    // readout fragments of this k-step
#pragma unroll
    for (int nt = 0; nt < 5; ++nt) {
      const float x[8] = {acc[0][nt][0], acc[0][nt][1], acc[0][nt][2], acc[0][nt][3],
                          acc[1][nt][0], acc[1][nt][1], acc[1][nt][2], acc[1][nt][3]};
      bf16x8 p0, p1, p2;
      split3_8(x, p0, p1, p2);
      HF[hf_index(n, ks, 0, nt, lane)] = __builtin_bit_cast(uint4, p0);
      HF[hf_index(n, ks, 1, nt, lane)] = __builtin_bit_cast(uint4, p1);
      HF[hf_index(n, ks, 2, nt, lane)] = __builtin_bit_cast(uint4, p2);
    }
  }
}

// ---------------------------------------------------------------- matrix-core scoring (d = 64, bf16 in)
//
// Self-recall partials of the refresh candidates (LoLA page, self-recall
// error): for candidate c and the work-group's feature k-steps,
//   num_c = sum_f phi_f(k_c) H_f,   den_c = sum_f phi_f(k_c) s_f,
// written to part[((n Z + z) pstride + c) 68 + {0..63, 64}] for the
// selection to add over z. Grid (heads, candidate blocks of 64, Z); slices
// z < zs sum the state's feature k-steps (wave w takes k-steps
// z 65 / zs + w, + 4, ...), slice zs (when Z > zs) adds the pairs folded by
// the previous refresh in closed form (hyb_score_correction). The B operands
// are the state fragments the fold wrote (three exact bf16 pieces
// h0 + h1 + h2, rows in the fold's order: lane quarter q4 holds features
// 32 ks + 4 q4 + j and 32 ks + 16 + 4 q4 + j, j < 4); the candidate features,
// in the same order, are split into two pieces p0 + p1 and the product is
// taken as p0 (h0 + h1 + h2) + p1 h0 in float32 (dropped terms below 2^-16
// relative). Denominators stay in float32 on the vector units, with s read
// back exactly from its three pieces in n-tile 4 of the fragments.
constexpr int kScoreCand = 64;
constexpr int kSZ = 5;  // score splits of the feature sum per (head, candidate block)
struct ScoreLds {
  uint16_t tab[kFPhi];
  float den[kWavesF][kScoreCand];
  union {
    float ck[kScoreCand][kFD + 1];   // candidate keys (float32), padded rows
    float4 red[4][4][64];            // numerator partials, accumulator layout
  };
};
struct CorrLds {
  uint16_t kc[kScoreCand][kFD + 8];  // candidate keys (bf16 rows)
  uint16_t kr[kFoldRows][kFD + 8];   // folded keys (bf16 rows, zero past the count)
  uint16_t vt[kFD][kFoldRows + 8];   // folded values, transposed
};
union ScoreShared {
  ScoreLds s;
  CorrLds c;
};

// Token of refresh candidate c: the cache entries, then the evicted tokens.
__device__ __forceinline__ int candidate_token(const int32_t* cache_n, int n_cache, int ev0, int c) {
  return c < n_cache ? cache_n[c] : ev0 + (c - n_cache);
}

// Slice zs of the scorer: the pairs j that the previous refresh folded, whose
// fold the state fragments it reads do not hold yet. phi(k_c) . phi(k_j) =
// (k_c . k_j)^2 (KATA §2.2), so they add
//   num_c += sum_j (k_c . k_j)^2 v_j,   den_c += sum_j (k_c . k_j)^2.
// S^T = K_j K_c^T on bf16 MFMA (exact products, float32 sums), squared in
// float32; the squares are split into three exact bf16 pieces for the product
// with V (bf16), so the numerators are float32 sums of exact products, as in
// a fold; the denominators are float32 sums. Wave w takes candidates
// 16 w .. 16 w + 15 of the block; the A operand of a 32-pair step is the two
// 16-pair score tiles as the lanes hold them (pairs 4 q4 + i of each), and
// the value fragments take the same pair order.
__device__ __forceinline__ void hyb_score_correction(
    CorrLds& sh, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, int T, int n,
    const int32_t* __restrict__ cache_n, int n_cache, int ev0, int n_cand, int cbase,
    const int32_t* __restrict__ rej_n, int n_rej, float* __restrict__ pz) {
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l16 = lane & 15;
  const int q4 = lane >> 4;
  const int R = (n_rej + 31) & ~31;
  for (int i = tid; i < kScoreCand * (kFD / 8); i += kThreads) {
    const int c = i >> 3, p = (i & 7) * 8;
    uint4 u = make_uint4(0, 0, 0, 0);
    if (cbase + c < n_cand) {
      const int tok = candidate_token(cache_n, n_cache, ev0, cbase + c);
      u = *reinterpret_cast<const uint4*>(k + ((size_t)n * T + tok) * kFD + p);
    }
    *reinterpret_cast<uint4*>(&sh.kc[c][p]) = u;
  }
  for (int i = tid; i < R * (kFD / 8); i += kThreads) {
    const int j = i >> 3, p = (i & 7) * 8;
    uint4 ku = make_uint4(0, 0, 0, 0), vu = ku;
    if (j < n_rej) {
      const size_t row = ((size_t)n * T + rej_n[j]) * kFD + p;
      ku = *reinterpret_cast<const uint4*>(k + row);
      vu = *reinterpret_cast<const uint4*>(v + row);
    }
    *reinterpret_cast<uint4*>(&sh.kr[j][p]) = ku;
    const uint32_t vw[4] = {vu.x, vu.y, vu.z, vu.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      sh.vt[p + 2 * e][j] = (uint16_t)(vw[e] & 0xFFFF);
      sh.vt[p + 2 * e + 1][j] = (uint16_t)(vw[e] >> 16);
    }
  }
  __syncthreads();

  f32x4 acc[4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float dpart = 0.0f;
  for (int jj = 0; jj < R / 32; ++jj) {
    float x[8];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int jt = 2 * jj + h;
      f32x4 s4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < kFD / 32; ++ks) {
        const bf16x8 A = *reinterpret_cast<const bf16x8*>(&sh.kr[16 * jt + l16][32 * ks + 8 * q4]);
        const bf16x8 B = *reinterpret_cast<const bf16x8*>(&sh.kc[16 * w + l16][32 * ks + 8 * q4]);
        s4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, B, s4, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float wgt = 16 * jt + 4 * q4 + i < n_rej ? s4[i] * s4[i] : 0.0f;
        dpart += wgt;
        x[4 * h + i] = wgt;
      }
    }
    bf16x8 A0, A1, A2;
    split3_8(x, A0, A1, A2);
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const uint16_t* vr = &sh.vt[16 * nt + l16][32 * jj + 4 * q4];
      const uint2 b0 = *reinterpret_cast<const uint2*>(vr);
      const uint2 b1 = *reinterpret_cast<const uint2*>(vr + 16);
      const bf16x8 B = __builtin_bit_cast(bf16x8, make_uint4(b0.x, b0.y, b1.x, b1.y));
      acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A0, B, acc[nt], 0, 0, 0);
      acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A1, B, acc[nt], 0, 0, 0);
      acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A2, B, acc[nt], 0, 0, 0);
    }
  }
  // lanes of one candidate column hold disjoint pairs
  dpart += __shfl_xor(dpart, 16, 64);
  dpart += __shfl_xor(dpart, 32, 64);
  // lane (l16, q4) holds candidates 16 w + 4 q4 + i at value column 16 nt + l16
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = 16 * w + 4 * q4 + i;
    if (cbase + c < n_cand) {
      float* pc = pz + (size_t)(cbase + c) * 68;
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) pc[16 * nt + l16] = acc[nt][i];
    }
  }
  if (q4 == 0 && cbase + 16 * w + l16 < n_cand) pz[(size_t)(cbase + 16 * w + l16) * 68 + 64] = dpart;
}

// Work-group (n, by, bz) of the scorer, bz < Z = zs + 1.
__device__ __forceinline__ void hyb_score_block(
    ScoreShared& shu, int n, int by, int bz, int Z, const uint4* __restrict__ HF, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, int T, const int32_t* __restrict__ cache, int cstride, int n_cache, int ev0,
    int n_cand, const int32_t* __restrict__ rej, int rstride, int n_rej, int zs, float* __restrict__ part,
    int pstride) {
  const int cbase = kScoreCand * by;
  if (bz == zs) {
    hyb_score_correction(shu.c, k, v, T, n, cache + (size_t)n * cstride, n_cache, ev0, n_cand, cbase,
                         rej + (size_t)n * rstride, n_rej, part + ((size_t)n * Z + zs) * pstride * 68);
    return;
  }
  ScoreLds& sh = shu.s;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l16 = lane & 15;
  const int q4 = lane >> 4;
  const int tz0 = (bz * kFKS) / zs;
  const int tz1 = ((bz + 1) * kFKS) / zs;

  // B fragments of k-step ks, and the three pieces of s for this lane's
  // features (n-tile 4, lane column 0 of the lane's quarter)
  auto load_b = [&](int ks, uint4 (&b)[3][4], uint4 (&sv)[3]) {
#pragma unroll
    for (int pc = 0; pc < 3; ++pc)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) b[pc][nt] = HF[hf_index(n, ks, pc, nt, lane)];
#pragma unroll
    for (int pc = 0; pc < 3; ++pc) sv[pc] = HF[hf_index(n, ks, pc, 4, 16 * q4)];
  };
  uint4 bf[3][4];
  uint4 sv[3];
  const int ks_first = min(tz0 + w, kFKS - 1);
  load_b(ks_first, bf, sv);

  // candidate keys: four threads per candidate, 16 dimensions each
  {
    const int c = tid >> 2;
    const int qd = tid & 3;
    float x[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) x[j] = 0.0f;
    if (cbase + c < n_cand) {
      const int tok = candidate_token(cache + (size_t)n * cstride, n_cache, ev0, cbase + c);
      const uint4* kp = reinterpret_cast<const uint4*>(k + ((size_t)n * T + tok) * kFD + 16 * qd);
      const uint4 u0 = kp[0], u1 = kp[1];
      const uint32_t uw[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        x[2 * j] = __uint_as_float(uw[j] << 16);
        x[2 * j + 1] = __uint_as_float(uw[j] & 0xFFFF0000u);
      }
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) sh.ck[c][16 * qd + j] = x[j];
  }
  for (int i = tid; i < kFPhi / 8; i += kThreads)
    reinterpret_cast<uint4*>(sh.tab)[i] = reinterpret_cast<const uint4*>(kFoldPairs.ab)[i];
  __syncthreads();

  f32x4 acc[4][4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float dacc[4] = {0.f, 0.f, 0.f, 0.f};

#pragma unroll 1
  for (int ks = tz0 + w; ks < tz1; ks += kWavesF) {
    uint4 bn[3][4];
    uint4 svn[3];
    const bool more = ks + kWavesF < tz1;
    if (more) load_b(ks + kWavesF, bn, svn);
    // this lane's eight features and their weights
    const uint2 t0 = *reinterpret_cast<const uint2*>(&sh.tab[32 * ks + 4 * q4]);
    const uint2 t1 = *reinterpret_cast<const uint2*>(&sh.tab[32 * ks + 16 + 4 * q4]);
    const uint32_t words[4] = {t0.x, t0.y, t1.x, t1.y};
    int pa[8], pb[8];
    float wt[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t u = (j & 1) ? (words[j >> 1] >> 16) : (words[j >> 1] & 0xFFFFu);
      pa[j] = u & 0xFF;
      pb[j] = u >> 8;
      wt[j] = pa[j] == pb[j] ? 1.0f : 1.41421356237309504880f;
    }
    // s from its pieces: (p0 + p1) + p2 restores the float32 value exactly
    float sj[8];
    {
      const bf16x8 s0 = __builtin_bit_cast(bf16x8, sv[0]), s1 = __builtin_bit_cast(bf16x8, sv[1]),
                   s2 = __builtin_bit_cast(bf16x8, sv[2]);
#pragma unroll
      for (int j = 0; j < 8; ++j) sj[j] = ((float)s0[j] + (float)s1[j]) + (float)s2[j];
    }
    bf16x8 B[3][4];
#pragma unroll
    for (int pc = 0; pc < 3; ++pc)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) B[pc][nt] = __builtin_bit_cast(bf16x8, bf[pc][nt]);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const float* kc = sh.ck[16 * mt + l16];
      float p[8];
      float dd = 0.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        p[j] = kc[pa[j]] * kc[pb[j]] * wt[j];
        dd += p[j] * sj[j];
      }
      dacc[mt] += dd;
      bf16x8 A0, A1;
      split2_8(p, A0, A1);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A0, B[0][nt], acc[mt][nt], 0, 0, 0);
        acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A0, B[1][nt], acc[mt][nt], 0, 0, 0);
        acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A0, B[2][nt], acc[mt][nt], 0, 0, 0);
        acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A1, B[0][nt], acc[mt][nt], 0, 0, 0);
      }
    }
    if (more) {
#pragma unroll
      for (int pc = 0; pc < 3; ++pc)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) bf[pc][nt] = bn[pc][nt];
#pragma unroll
      for (int pc = 0; pc < 3; ++pc) sv[pc] = svn[pc];
    }
  }

  // denominators: lane l16 of block mt is candidate 16 mt + l16
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    float d = dacc[mt];
    d += __shfl_xor(d, 16, 64);
    d += __shfl_xor(d, 32, 64);
    if (q4 == 0) sh.den[w][16 * mt + l16] = d;
  }
  // numerators: waves add into the LDS copy in turn; the last one keeps the
  // sum (the first barrier also ends every read of the candidate keys, whose
  // LDS the partials reuse)
  for (int r = 0; r < kWavesF; ++r) {
    __syncthreads();
    if (w == r) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
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
          if (r + 1 < kWavesF) sh.red[mt][nt][lane] = make_float4(x[0], x[1], x[2], x[3]);
        }
    }
  }
  if (w == kWavesF - 1) {
    // lane (l16, q4) holds candidates 16 mt + 4 q4 + i at state columns 4 l16 + nt
    float* pz = part + ((size_t)n * Z + bz) * pstride * 68;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c = 16 * mt + 4 * q4 + i;
        if (cbase + c < n_cand) {
          float* pc = pz + (size_t)(cbase + c) * 68;
          *reinterpret_cast<float4*>(pc + 4 * l16) =
              make_float4(acc[mt][0][i], acc[mt][1][i], acc[mt][2][i], acc[mt][3][i]);
          if (l16 == 0) {
            float den = 0.0f;
#pragma unroll
            for (int r = 0; r < kWavesF; ++r) den += sh.den[r][c];
            pc[64] = den;
          }
        }
      }
    }
  }
}

// One launch for the two halves of a refresh step that wait on the same
// work: the scoring of refresh r (work-groups 0 .. n_score - 1) and the fold
// of refresh r - 1 (the rest, decoded as (k-step block, head)). Either part
// may be empty. Per head the scoring has the correction slice of every
// candidate block, then the state slices of blocks bnew0 .. n_cblk - 1: the
// blocks before bnew0 hold only candidates whose sums over the state before
// the previous fold the previous selection carried over.
union RefreshShared {
  ScoreShared score;
  FoldLds fold;
};

__global__ __launch_bounds__(kThreads, 2) void hyb_refresh_kernel(
    // scoring of refresh r
    int n_score, int n_cblk, int bnew0, const uint4* __restrict__ HFs, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, int T, const int32_t* __restrict__ cache, int cstride, int n_cache, int ev0,
    int n_cand, const int32_t* __restrict__ rej_prev, int rstride, int n_rej_prev, float* __restrict__ part,
    int pstride,
    // fold of refresh r - 1
    float* __restrict__ H, float* __restrict__ s, uint4* __restrict__ HFf, const int32_t* __restrict__ rej_fold,
    int n_rej_fold) {
  __shared__ __align__(16) RefreshShared sh;
  const int bid = blockIdx.x;
  constexpr int Z = kSZ + 1;
  if (bid < n_score) {
    const int per_head = n_cblk + (n_cblk - bnew0) * kSZ;
    const int n = bid / per_head;
    const int i = bid % per_head;
    const int by = i < n_cblk ? i : bnew0 + (i - n_cblk) / kSZ;
    const int bz = i < n_cblk ? kSZ : (i - n_cblk) % kSZ;
    hyb_score_block(sh.score, n, by, bz, Z, HFs, k, v, T, cache, cstride, n_cache, ev0, n_cand, rej_prev, rstride,
                    n_rej_prev, kSZ, part, pstride);
  } else {
    const int f = bid - n_score;
    hyb_fold_block(sh.fold, f % kFoldWGs, f / kFoldWGs, H, s, HFf, k, v, T, rej_fold, rstride, n_rej_fold);
  }
}

// ---------------------------------------------------------------- matrix-core readout (d = 64, bf16 in)
//
// One work-group per (head, 64 queries of a block); wave w owns queries
// t0 + 16 w .. + 15 for the softmax part. Softmax keys are the cache entries
// and then the window [f, t]. Scores come from S^T = K Q^T on bf16 MFMA
// (exact products, float32 sums): lane (l16, q4) holds the scores of query
// l16 against keys 4 q4 + i of each 16-key half. Pass 1 finds each query's
// maximum m (clamped at 0, since the joint normalisation divides the linear
// terms by e^m too); pass 2 forms P = e^(tau s - m) in two bf16 pieces and
// P [V | 1], taking P's k-slots in the order the scores sit in the lanes
// (keys 4 q4 + j, then 16 + 4 q4 + j) and V in the same order. Key and value
// fragments are loaded straight from memory, one tile ahead; the softmax
// part needs no LDS and no barrier.
// The linear term phi(q)^T [H | s] reads the state fragments the fold wrote
// (two bf16 pieces, hi*hi + hi*lo + lo*hi with two-piece phi(q)); wave w
// takes the k-steps ks = w mod 4 for all 64 queries and the four partial
// sums meet in LDS at the end. Output column 4 l16 + nt sits in n-tile nt of
// lane (l16, q4), rows 4 q4 + i.
constexpr int kRW = 4;        // waves (16 queries each) per work-group
constexpr int kRT = 64 * kRW; // threads
constexpr int kRQ = 16 * kRW; // queries per work-group
constexpr int kRK = 32;       // keys per tile
constexpr int kPT = 2;        // key tiles per iteration (and in flight)
constexpr int kPF = 2;        // state k-steps per iteration (and in flight)

struct ReadoutLds {
  float qf[kRQ][kFD + 1];               // query rows (float32) for phi(q)
  uint16_t tab[kFPhi];                  // feature pairs
  float4 red[kRW][kRW][5][64];          // linear partials: [source wave][token tile][n-tile][lane]
  float mq[kRQ];                        // per-query maximum
  float den[kRQ];                       // per-query denominator
};

// Work-group (b, n, sp) of ns splits handles keys [sp * span, (sp + 1) * span)
// and state k-steps sp * kRW + w (mod ns * kRW); with ns > 1 it writes, per
// query, the partial numerator and denominator scaled by e^-m_sp, and m_sp,
// to xp[n][query][sp][66] for hyb_readout_combine_kernel.
template <typename Tout>
__global__ __launch_bounds__(kRT) void hyb_readout_mfma_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    Tout* __restrict__ o, int T, const uint4* __restrict__ HF, const int32_t* __restrict__ cache,
    int cstride, int n_cache, int t_begin, int t_end, int f, float scale, float eps, int ns,
    float* __restrict__ xp, int xq) {
  __shared__ __align__(16) ReadoutLds sh;
  const int n = blockIdx.y;
  const int sp = blockIdx.z;
  const int t0 = t_begin + kRQ * blockIdx.x;
  const int tq_end = min(t_end, t0 + kRQ);       // queries [t0, tq_end)
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l16 = lane & 15;
  const int q4 = lane >> 4;
  const int tw = t0 + 16 * w;                     // this wave's first query
  const int my_t = tw + l16;                      // query of lane (scores layout)
  const size_t base = (size_t)n * T * kFD;
  const int32_t* cn = cache + (size_t)n * cstride;
  // keys: cache, then window tokens f .. tq_end - 1
  const int n_keys = n_cache + (tq_end - f);

  for (int i = tid; i < kFPhi; i += kRT) sh.tab[i] = kFoldPairs.ab[i];
  for (int i = tid; i < kRQ * (kFD / 4); i += kRT) {
    const int r = i / (kFD / 4), d4 = i % (kFD / 4);
    uint2 u = make_uint2(0, 0);
    if (t0 + r < tq_end) u = *reinterpret_cast<const uint2*>(q + base + (size_t)(t0 + r) * kFD + 4 * d4);
    sh.qf[r][4 * d4 + 0] = __uint_as_float(u.x << 16);
    sh.qf[r][4 * d4 + 1] = __uint_as_float(u.x & 0xFFFF0000u);
    sh.qf[r][4 * d4 + 2] = __uint_as_float(u.y << 16);
    sh.qf[r][4 * d4 + 3] = __uint_as_float(u.y & 0xFFFF0000u);
  }
  // Q^T as the B operand of S^T = K Q^T: lane (l16 = query, q4) holds dims 8 q4 .. + 7 (+ 32 ks)
  bf16x8 qb[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    uint4 u = make_uint4(0, 0, 0, 0);
    if (my_t < tq_end) u = *reinterpret_cast<const uint4*>(q + base + (size_t)my_t * kFD + 32 * ks + 8 * q4);
    qb[ks] = __builtin_bit_cast(bf16x8, u);
  }
  __syncthreads();

  auto key_token = [&](int j) { return j < n_cache ? cn[j] : f + (j - n_cache); };
  // this split's keys, cut to the ones any query of the wave sees
  const int span = (((n_keys + ns - 1) / ns) + kRK - 1) / kRK * kRK;
  const int kbeg = min(n_keys, sp * span);
  const int wave_keys = max(kbeg, min(min(n_keys, kbeg + span), n_cache + (min(tq_end, tw + 16) - f)));

  // key fragments of tile j0: ka[h][ks] = key j0 + 16 h + l16, dims 32 ks + 8 q4 .. + 7
  auto load_k = [&](int j0, uint4 (&ka)[2][2]) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int j = j0 + 16 * h + l16;
      const bool ok = j < wave_keys;
      const size_t row = base + (size_t)(ok ? key_token(j) : 0) * kFD;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        ka[h][ks] = ok ? *reinterpret_cast<const uint4*>(k + row + 32 * ks + 8 * q4) : make_uint4(0, 0, 0, 0);
    }
  };
  // value rows of the 8 keys of this lane's k-slots: key 4 q4 + j (j < 4), 16 + 4 q4 + j - 4
  // (j >= 4), columns 4 l16 .. + 3
  auto load_v = [&](int j0, uint2 (&vr)[8]) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int kj = j0 + (j < 4 ? 4 * q4 + j : 16 + 4 * q4 + (j - 4));
      vr[j] = kj < wave_keys ? *reinterpret_cast<const uint2*>(v + base + (size_t)key_token(kj) * kFD + 4 * l16)
                             : make_uint2(0, 0);
    }
  };
  auto scores = [&](int j0, const uint4 (&ka)[2][2], float (&sc)[2][4]) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ka[h][ks]), qb[ks], c, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = j0 + 16 * h + 4 * q4 + i;
        // keys of this split only (wave_keys <= n_keys); cache keys precede every
        // query; window keys are causal
        const bool ok = j < wave_keys && my_t < tq_end && (j < n_cache || f + (j - n_cache) <= my_t);
        sc[h][i] = ok ? scale * c[i] : -INFINITY;
      }
    }
  };

  // ---- pass 1: per-query maximum (kPT key tiles per iteration, the next kPT in flight)
  float mx = 0.0f;  // never below 0
  {
    uint4 ka[kPT][2][2];
#pragma unroll
    for (int t = 0; t < kPT; ++t) load_k(kbeg + kRK * t, ka[t]);
    for (int j0 = kbeg; j0 < wave_keys; j0 += kRK * kPT) {
      uint4 kn[kPT][2][2];
      const bool more = j0 + kRK * kPT < wave_keys;
      if (more) {
#pragma unroll
        for (int t = 0; t < kPT; ++t) load_k(j0 + kRK * (kPT + t), kn[t]);
      }
#pragma unroll
      for (int t = 0; t < kPT; ++t) {
        float sc[2][4];
        scores(j0 + kRK * t, ka[t], sc);
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sc[h][i]);
      }
      if (more) {
#pragma unroll
        for (int t = 0; t < kPT; ++t)
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) ka[t][h][ks] = kn[t][h][ks];
      }
    }
  }
  mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
  mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
  if (q4 == 0) sh.mq[16 * w + l16] = mx;

  // ---- pass 2: P [V | 1]
  bf16x8 ones;
#pragma unroll
  for (int j = 0; j < 8; ++j) ones[j] = (__bf16)(l16 == 0 ? 1.0f : 0.0f);
  f32x4 acc[5];
#pragma unroll
  for (int nt = 0; nt < 5; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  {
    uint4 ka[kPT][2][2];
    uint2 vr[kPT][8];
#pragma unroll
    for (int t = 0; t < kPT; ++t) {
      load_k(kbeg + kRK * t, ka[t]);
      load_v(kbeg + kRK * t, vr[t]);
    }
    for (int j0 = kbeg; j0 < wave_keys; j0 += kRK * kPT) {
      uint4 kn[kPT][2][2];
      uint2 vn[kPT][8];
      const bool more = j0 + kRK * kPT < wave_keys;
      if (more) {
#pragma unroll
        for (int t = 0; t < kPT; ++t) {
          load_k(j0 + kRK * (kPT + t), kn[t]);
          load_v(j0 + kRK * (kPT + t), vn[t]);
        }
      }
#pragma unroll
      for (int t = 0; t < kPT; ++t) {
        float sc[2][4];
        scores(j0 + kRK * t, ka[t], sc);
        // P = p0 + p1 (two bf16 pieces, 16 significant bits); v and 1 are exact in bf16
        float pf[8];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int i = 0; i < 4; ++i) pf[4 * h + i] = __expf(sc[h][i] - mx);
        bf16x8 p0, p1;
        split2_8(pf, p0, p1);
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
          bf16x8 b;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const uint32_t word = (nt < 2) ? vr[t][j].x : vr[t][j].y;
            const uint16_t bits = (nt & 1) ? (uint16_t)(word >> 16) : (uint16_t)(word & 0xFFFF);
            b[j] = __builtin_bit_cast(__bf16, bits);
          }
          acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(p0, b, acc[nt], 0, 0, 0);
          acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(p1, b, acc[nt], 0, 0, 0);
        }
        acc[4] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(p0, ones, acc[4], 0, 0, 0);
        acc[4] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(p1, ones, acc[4], 0, 0, 0);
      }
      if (more) {
#pragma unroll
        for (int t = 0; t < kPT; ++t) {
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) ka[t][h][ks] = kn[t][h][ks];
#pragma unroll
          for (int j = 0; j < 8; ++j) vr[t][j] = vn[t][j];
        }
      }
    }
  }

  // ---- linear readout phi(q)^T [H | s]: this wave's k-steps, all 64 queries
  f32x4 lin[kRW][5];
#pragma unroll
  for (int tt = 0; tt < kRW; ++tt)
#pragma unroll
    for (int nt = 0; nt < 5; ++nt) lin[tt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  {
    // k-steps ks = w + kRW (kPF i + t): kPF per iteration, the next kPF in flight
    auto load_f = [&](int ks, uint4 (&x)[2][5]) {
#pragma unroll
      for (int pc = 0; pc < 2; ++pc)
#pragma unroll
        for (int nt = 0; nt < 5; ++nt)
          x[pc][nt] = ks < kFKS ? HF[hf_index(n, ks, pc, nt, lane)] : make_uint4(0, 0, 0, 0);
    };
    uint4 fr[kPF][2][5];
    const int kst = ns * kRW;  // k-step stride of this split's waves
#pragma unroll
    for (int t = 0; t < kPF; ++t) load_f(sp * kRW + w + kst * t, fr[t]);
    for (int ks0 = sp * kRW + w; ks0 < kFKS; ks0 += kst * kPF) {
      uint4 fn[kPF][2][5];
      const bool more = ks0 + kst * kPF < kFKS;
      if (more) {
#pragma unroll
        for (int t = 0; t < kPF; ++t) load_f(ks0 + kst * (kPF + t), fn[t]);
      }
#pragma unroll
      for (int t = 0; t < kPF; ++t) {
        const int ks = ks0 + kst * t;
        if (ks < kFKS) {
          // features of this lane's k-slots: 32 ks + 4 q4 + j (j < 4), 32 ks + 16 + 4 q4 + j - 4 (j >= 4)
          int fa[8], fb[8];
          float wg[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const uint16_t ab = sh.tab[32 * ks + (j < 4 ? 4 * q4 + j : 16 + 4 * q4 + (j - 4))];
            fa[j] = ab & 0xFF;
            fb[j] = ab >> 8;
            wg[j] = fa[j] == fb[j] ? 1.0f : 1.41421356237309504880f;
          }
#pragma unroll
          for (int tt = 0; tt < kRW; ++tt) {
            const float* qrow = sh.qf[16 * tt + l16];
            float p[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) p[j] = qrow[fa[j]] * qrow[fb[j]] * wg[j];
            bf16x8 A0, A1;
            split2_8(p, A0, A1);
#pragma unroll
            for (int nt = 0; nt < 5; ++nt) {
              const bf16x8 B0 = __builtin_bit_cast(bf16x8, fr[t][0][nt]);
              const bf16x8 B1 = __builtin_bit_cast(bf16x8, fr[t][1][nt]);
              lin[tt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A0, B0, lin[tt][nt], 0, 0, 0);
              lin[tt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A0, B1, lin[tt][nt], 0, 0, 0);
              lin[tt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A1, B0, lin[tt][nt], 0, 0, 0);
            }
          }
        }
      }
      if (more) {
#pragma unroll
        for (int t = 0; t < kPF; ++t)
#pragma unroll
          for (int pc = 0; pc < 2; ++pc)
#pragma unroll
            for (int nt = 0; nt < 5; ++nt) fr[t][pc][nt] = fn[t][pc][nt];
      }
    }
  }
#pragma unroll
  for (int tt = 0; tt < kRW; ++tt)
#pragma unroll
    for (int nt = 0; nt < 5; ++nt)
      sh.red[w][tt][nt][lane] = make_float4(lin[tt][nt][0], lin[tt][nt][1], lin[tt][nt][2], lin[tt][nt][3]);
  __syncthreads();
  // this wave's queries (token tile w): sum of the four partials
  f32x4 ln[5];
#pragma unroll
  for (int nt = 0; nt < 5; ++nt) {
    ln[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r = 0; r < kRW; ++r) {
      const float4 y = sh.red[r][w][nt][lane];
      ln[nt][0] += y.x;
      ln[nt][1] += y.y;
      ln[nt][2] += y.z;
      ln[nt][3] += y.w;
    }
  }

  // ---- combine: rows 4 q4 + i of the wave, columns 4 l16 + nt
  if (ns > 1) {
    // partials of this split, scaled by e^-m_sp: numerator, denominator (no eps), m_sp
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * w + 4 * q4 + i;
      if (t0 + r < tq_end) {
        const float m = sh.mq[r];
        const float e = __expf(-m);
        float* xr = xp + (((size_t)n * xq + (t0 + r - t_begin)) * ns + sp) * 66;
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) xr[4 * l16 + nt] = acc[nt][i] + e * ln[nt][i];
        if (l16 == 0) {
          xr[64] = acc[4][i] + e * ln[4][i];
          xr[65] = m;
        }
      }
    }
    return;
  }
  if (l16 == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float e = __expf(-sh.mq[16 * w + 4 * q4 + i]);
      sh.den[16 * w + 4 * q4 + i] = acc[4][i] + e * (ln[4][i] + eps);
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 16 * w + 4 * q4 + i;
    const int t = t0 + r;
    if (t < tq_end) {
      const float e = __expf(-sh.mq[r]);
      const float den = sh.den[r];
      const float inv = den != 0.0f ? 1.0f / den : 0.0f;
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
        Elem<Tout>::store(o, base + (size_t)t * kFD + 4 * l16 + nt,
                          den != 0.0f ? (acc[nt][i] + e * ln[nt][i]) * inv : 0.0f);
    }
  }
}

// Joins the ns split partials of queries [t_begin, t_end): m = max m_sp,
// o = sum e^(m_sp - m) num_sp / (sum e^(m_sp - m) den_sp + e^-m eps).
template <typename Tout>
__global__ __launch_bounds__(kThreads) void hyb_readout_combine_kernel(const float* __restrict__ xp, int xq, int ns,
                                                                     Tout* __restrict__ o, int T, int t_begin,
                                                                     int t_end, float eps) {
  const int n = blockIdx.y;
  const int idx = blockIdx.x * kThreads + threadIdx.x;  // (query, column)
  const int r = idx >> 6, c = idx & 63;
  const int t = t_begin + r;
  if (t >= t_end) return;
  const float* xr = xp + ((size_t)n * xq + r) * ns * 66;
  float m = 0.0f;
  for (int sp = 0; sp < ns; ++sp) m = fmaxf(m, xr[sp * 66 + 65]);
  float num = 0.0f, den = __expf(-m) * eps;
  for (int sp = 0; sp < ns; ++sp) {
    const float e = __expf(xr[sp * 66 + 65] - m);
    num += e * xr[sp * 66 + c];
    den += e * xr[sp * 66 + 64];
  }
  Elem<Tout>::store(o, ((size_t)n * T + t) * kFD + c, den != 0.0f ? num / den : 0.0f);
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

constexpr int kCandMax = 256;  // candidates per refresh, at most (cache + evicted)

// Matrix-core form of the selection (d = 64, bf16 token rows): the scores are
// first assembled from Z feature-split partials part[((n Z + z) pstride + c) 68
// + {0..63 numerator, 64 denominator}],
//   score_c = || num_c / (den_c + eps) - v_c ||^2   (prediction 0 when the
//   denominator is 0),
// then every candidate finds its place by counting: its rank is the number of
// larger (score, token id) keys, so ranks are distinct; the keep best go to
// the cache in ascending token order (their place is the number of kept
// tokens with a lower id) and the rest, in rank order, to the rejected list.
// The result is the one the sort of the generic form gives. The new cache goes
// to cache_out (not the cache it reads).
// Candidates c < n_carry take their sums over the state before the previous
// fold from carry_in[c] (the previous selection's totals) instead of the
// state slices, plus the correction slice Z - 1; every kept candidate's
// totals go to carry_out at its new cache position.
constexpr int kSelThreads = 1024;
__global__ __launch_bounds__(kSelThreads) void hyb_select_part_kernel(
    const float* __restrict__ part, int Z, int pstride, const uint16_t* __restrict__ v, int T,
    float eps, const int32_t* __restrict__ cache, int cstride, int32_t* __restrict__ cache_out,
    int ostride, int n_cache, int ev0, int n_cand, int keep,
    int32_t* __restrict__ rejected, int rstride, int32_t* __restrict__ trace, size_t trace_row_stride,
    int block, int nblocks, float* __restrict__ scores, int sstride, const float* __restrict__ carry_in,
    int n_carry, float* __restrict__ carry_out) {
  static_assert(kSelThreads == 4 * kCandMax, "four threads per candidate");
  __shared__ uint64_t keys[kCandMax];
  __shared__ int32_t tok[kCandMax];
  __shared__ int32_t kid[kCandMax];
  const int n = blockIdx.x;
  const int tid = threadIdx.x;
  // four adjacent threads per candidate: quarter qd of its columns, and of
  // the keys it counts against
  const int c = tid >> 2;
  const int qd = tid & 3;
  const bool live = c < n_cand;
  const int32_t* cn = cache + (size_t)n * cstride;
  if (qd == 0 && live) tok[c] = cand_token(cn, n_cache, ev0, c);
  __syncthreads();
  float err = 0.0f;
  float num[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) num[j] = 0.0f;
  float dsum = 0.0f;
  if (live) {
    auto add = [&](const float* pc) {
      const float4* p4 = reinterpret_cast<const float4*>(pc + 16 * qd);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float4 x = p4[j];
        num[4 * j] += x.x;
        num[4 * j + 1] += x.y;
        num[4 * j + 2] += x.z;
        num[4 * j + 3] += x.w;
      }
      dsum += pc[64];
    };
    if (c < n_carry) {
      add(carry_in + ((size_t)n * pstride + c) * 68);
      add(part + (((size_t)n * Z + Z - 1) * pstride + c) * 68);
    } else {
#pragma unroll 5
      for (int z = 0; z < Z; ++z) add(part + (((size_t)n * Z + z) * pstride + c) * 68);
    }
    const float den = dsum + eps;
    const uint4* vp = reinterpret_cast<const uint4*>(v + ((size_t)n * T + tok[c]) * kFD + 16 * qd);
    const uint4 va = vp[0], vb = vp[1];
    const uint32_t vw[8] = {va.x, va.y, va.z, va.w, vb.x, vb.y, vb.z, vb.w};
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const float vj = __uint_as_float((j & 1) ? (vw[j >> 1] & 0xFFFF0000u) : (vw[j >> 1] << 16));
      const float pred = den != 0.0f ? num[j] / den : 0.0f;
      const float d = pred - vj;
      err += d * d;
    }
  }
  err += __shfl_xor(err, 1, 64);
  err += __shfl_xor(err, 2, 64);
  if (qd == 0 && live) {
    keys[c] = topk_key(err, (uint32_t)tok[c]);
    if (scores) scores[(size_t)n * sstride + c] = err;
  }
  __syncthreads();
  uint64_t key = 0;
  int rank = 0;
  if (live) {
    key = keys[c];
#pragma unroll 8
    for (int j = qd; j < n_cand; j += 4) rank += keys[j] > key ? 1 : 0;
  }
  rank += __shfl_xor(rank, 1, 64);
  rank += __shfl_xor(rank, 2, 64);
  if (qd == 0 && live) kid[c] = rank < keep ? tok[c] : 0x7FFFFFFF;
  __syncthreads();
  int pos = 0;
  if (live && rank < keep) {
    const int32_t id = tok[c];
#pragma unroll 8
    for (int j = qd; j < n_cand; j += 4) pos += kid[j] < id ? 1 : 0;
  }
  pos += __shfl_xor(pos, 1, 64);
  pos += __shfl_xor(pos, 2, 64);
  if (carry_out && live && rank < keep) {
    float* co = carry_out + ((size_t)n * pstride + pos) * 68;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      *reinterpret_cast<float4*>(co + 16 * qd + 4 * j) =
          make_float4(num[4 * j], num[4 * j + 1], num[4 * j + 2], num[4 * j + 3]);
    if (qd == 0) co[64] = dsum;
  }
  if (qd == 0 && live) {
    const int32_t id = tok[c];
    if (rank >= keep) {
      rejected[(size_t)n * rstride + rank - keep] = id;
    } else {
      cache_out[(size_t)n * ostride + pos] = id;
      if (trace) trace[((size_t)n * nblocks + block) * trace_row_stride + pos] = id;
    }
  }
}

struct Ws {
  float* H;
  float* s;
  int32_t* cache;
  int32_t* cache2;  // second and third cache buffers (matrix-core path only)
  int32_t* cache3;
  float* scores;
  int32_t* rejected;
  int32_t* rejected2;  // second rejected list (matrix-core path only)
  uint4* HF[3];  // state fragments, three versions (matrix-core path only)
  float* xp;  // readout split partials [N][refresh][kRNS][66] (matrix-core path only)
  float* sp;  // score split partials [N][kSZ + 1][kCStride][68] (matrix-core path only)
  float* carry[2];  // carried candidate sums [N][kCStride][68], by refresh parity (matrix-core path only)
};

bool matrix_path(const HybridArgs& a) { return a.dqk == 64 && a.dv == 64 && a.in_bf16; }
size_t hf_bytes(const HybridArgs& a) { return align_up((size_t)a.N * kFKS * kHFPieces * 5 * 64 * sizeof(uint4)); }
constexpr int kRNS = 8;  // readout splits per (head, query block)
size_t xp_bytes(const HybridArgs& a) { return align_up((size_t)a.N * a.refresh * kRNS * 66 * sizeof(float)); }

constexpr int kCStride = kCandMax;
// plus one slice for the pairs the previous refresh folded
size_t sp_bytes(const HybridArgs& a) { return align_up((size_t)a.N * (kSZ + 1) * kCStride * 68 * sizeof(float)); }
size_t carry_bytes(const HybridArgs& a) { return align_up((size_t)a.N * kCStride * 68 * sizeof(float)); }
// every kRescore-th refresh scores every candidate against the state again,
// which bounds the rounding the carried sums gather
constexpr int kRescore = 8;

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
  w.cache2 = w.cache3 = nullptr;
  if (matrix_path(a)) {
    w.cache2 = reinterpret_cast<int32_t*>(p);
    p += align_up((size_t)a.N * kCStride * sizeof(int32_t));
    w.cache3 = reinterpret_cast<int32_t*>(p);
    p += align_up((size_t)a.N * kCStride * sizeof(int32_t));
  }
  w.scores = reinterpret_cast<float*>(p);
  p += align_up((size_t)a.N * kCStride * sizeof(float));
  w.rejected = reinterpret_cast<int32_t*>(p);
  p += align_up((size_t)a.N * kCStride * sizeof(int32_t));
  w.rejected2 = nullptr;
  for (uint4*& h : w.HF) h = nullptr;
  if (matrix_path(a)) {
    w.rejected2 = reinterpret_cast<int32_t*>(p);
    p += align_up((size_t)a.N * kCStride * sizeof(int32_t));
    for (uint4*& h : w.HF) {
      h = reinterpret_cast<uint4*>(p);
      p += hf_bytes(a);
    }
  }
  w.xp = matrix_path(a) ? reinterpret_cast<float*>(p) : nullptr;
  if (w.xp) p += xp_bytes(a);
  w.sp = matrix_path(a) ? reinterpret_cast<float*>(p) : nullptr;
  w.carry[0] = w.carry[1] = nullptr;
  if (w.sp) {
    p += sp_bytes(a);
    w.carry[0] = reinterpret_cast<float*>(p);
    p += carry_bytes(a);
    w.carry[1] = reinterpret_cast<float*>(p);
  }
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

// Events that order the caller's auxiliary stream against its main stream
// during one call. They belong to the call: created at its start and
// released at its end (a pending event is released by the runtime once it
// completes), so the library keeps nothing between calls.
struct CallEvents {
  hipEvent_t fork = nullptr, join = nullptr, ready = nullptr;
  hipEvent_t used[3] = {nullptr, nullptr, nullptr};  // slot x last read by a readout
  hipError_t create() {
    hipEvent_t* evs[6] = {&fork, &join, &ready, &used[0], &used[1], &used[2]};
    for (hipEvent_t* p : evs) {
      const hipError_t e = hipEventCreateWithFlags(p, hipEventDisableTiming);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  ~CallEvents() {
    hipEvent_t evs[6] = {fork, join, ready, used[0], used[1], used[2]};
    for (hipEvent_t e : evs)
      if (e) (void)hipEventDestroy(e);
  }
};

// The matrix-core path (d = 64, bf16 in). Scoring at refresh r reads the
// state after fold r - 2 and adds the pairs refresh r - 1 rejected in closed
// form (slice zs of the scorer), so it no longer waits for fold r - 1: the
// two run in one launch (hyb_refresh_kernel), followed by selection r. The
// refresh chain runs on the caller's stream; the readouts run on the
// caller's auxiliary stream when one is given (else on the same stream, in
// order), those of the blocks that refresh r serves once fold r is issued
// (in the launch of refresh r + 1, or alone after the last block), so they
// overlap the next refresh. Each refresh r owns slot r mod 3
// (state fragments of version r and cache r; slot 2 holds the zero state and
// the cache filled by appends before the first refresh, slot 1 the zero
// state too); the rejected lists alternate. A slot is rewritten only after
// the readouts that read it have finished (event used[slot], only needed
// with two streams); everything else is ordered by the chain's stream. The host knows every count in
// advance, so nothing is read back. Per refresh block the host issues four
// kernels (refresh, selection, readout, combine) and at most five event
// records and waits.
template <typename Tout>
hipError_t enqueue_matrix(const HybridArgs& a, void* ws, hipStream_t st, hipStream_t aux, bool prof) {
  const Ws w = carve(a, ws);
  const int N = a.N;
  const int nblocks = (a.T + a.refresh - 1) / a.refresh;
  const uint16_t* q = static_cast<const uint16_t*>(a.q);
  const uint16_t* k = static_cast<const uint16_t*>(a.k);
  const uint16_t* v = static_cast<const uint16_t*>(a.v);
  Tout* o = static_cast<Tout*>(a.o);
  hipError_t e = hipSuccess;
  // readouts go to the caller's auxiliary stream when one is given, else
  // everything runs in order on `st` and no event is needed
  const bool two = aux != nullptr && aux != st;
  const hipStream_t sb = two ? aux : st;
  CallEvents ev;
  if (two && (e = ev.create()) != hipSuccess) return e;
  CallEvents* ss = &ev;
#define KLA_TRY(x)                       \
  do {                                   \
    e = (x);                             \
    if (e != hipSuccess) return e;       \
  } while (0)
#define KLA_CHECK() KLA_TRY(hipGetLastError())
  int32_t* cache[3] = {w.cache, w.cache2, w.cache3};
  int32_t* rej[2] = {w.rejected, w.rejected2};
  bool used[3] = {false, false, false};
  hipLaunchKernelGGL(fill_kernel_f32, dim3(1024), dim3(256), 0, st, w.H, (size_t)N * kFPhi * kFD, 0.0f);
  hipLaunchKernelGGL(fill_kernel_f32, dim3(64), dim3(256), 0, st, w.s, (size_t)N * kFPhi, 0.0f);
  for (int32_t* c : cache)
    hipLaunchKernelGGL(fill_kernel_i32, dim3(64), dim3(256), 0, st, c, (size_t)N * kCStride, -1);
  for (uint4* h : w.HF)
    hipLaunchKernelGGL(fill_kernel_i32, dim3(1024), dim3(256), 0, st, reinterpret_cast<int32_t*>(h),
                       hf_bytes(a) / sizeof(int32_t), 0);
  if (a.trace && a.cache_size > 0)
    hipLaunchKernelGGL(fill_kernel_i32, dim3(1024), dim3(256), 0, st, a.trace,
                       (size_t)N * nblocks * a.cache_size, -1);
  KLA_CHECK();
  // the side stream starts after everything the caller queued so far
  if (two) {
    KLA_TRY(hipEventRecord(ss->fork, st));
    KLA_TRY(hipStreamWaitEvent(sb, ss->fork, 0));
  }
  int slot = 2;  // slot of the newest state and cache
  // everything after the fork also joins the side stream back, on error too
  const hipError_t loop_err = [&]() -> hipError_t {
    hipError_t e;
    struct Pending {
      int b0, b1, f, n_cache;
    };
    std::vector<Pending> pending;  // blocks whose readout waits for the fold of the newest refresh
    int n_cache = 0;
    int f_prev = 0;
    int r = 0;           // refreshes issued
    int n_rej_prev = 0;  // pairs rejected by refresh r - 1
    // readouts of the blocks in `pending`, reading slot x
    auto flush = [&](int x) -> hipError_t {
      if (pending.empty()) return hipSuccess;
      hipError_t e;
      if (two) {
        KLA_TRY(hipEventRecord(ss->ready, st));
        KLA_TRY(hipStreamWaitEvent(sb, ss->ready, 0));
      }
      for (const Pending& p : pending) {
        hipLaunchKernelGGL((hyb_readout_mfma_kernel<Tout>), dim3((p.b1 - p.b0 + kRQ - 1) / kRQ, N, kRNS),
                           dim3(kRT), 0, sb, q, k, v, o, a.T, w.HF[x], cache[x], kCStride, p.n_cache, p.b0, p.b1,
                           p.f, a.scale, a.eps, kRNS, w.xp, a.refresh);
        hipLaunchKernelGGL((hyb_readout_combine_kernel<Tout>),
                           dim3(((p.b1 - p.b0) * kFD + kThreads - 1) / kThreads, N), dim3(kThreads), 0, sb,
                           w.xp, a.refresh, kRNS, o, a.T, p.b0, p.b1, a.eps);
        KLA_CHECK();
      }
      if (two) {
        KLA_TRY(hipEventRecord(ss->used[x], sb));
        used[x] = true;
      }
      pending.clear();
      return hipSuccess;
    };
    // The fold of refresh r - 1 rewrites slot (r - 1) mod 3 (last read by the
    // readouts of refresh r - 4) and selection r rewrites slot r mod 3 (last
    // read by those of refresh r - 3); readouts finish in order, so waiting
    // for the latter before the fold frees both.
    auto slots_free = [&](int x) -> hipError_t {
      if (used[x]) return hipStreamWaitEvent(st, ss->used[x], 0);
      return hipSuccess;
    };
    for (int b = 0; b < nblocks; ++b) {
      const int b0 = b * a.refresh;
      const int b1 = std::min(a.T, b0 + a.refresh);
      const int f = std::max(0, b0 - a.window);
      const int n_ev = f - f_prev;
      if (n_ev > 0 && n_cache + n_ev > a.cache_size) {
        const int n_cand = n_cache + n_ev;
        const int n_rej = n_cand - a.cache_size;
        const int x_new = r % 3;          // slot of refresh r
        const int x_cur = (r + 2) % 3;    // slot of refresh r - 1 (2 before the first)
        const int x_old = (r + 1) % 3;    // slot of refresh r - 2 (the zero state for r < 2)
        // scoring r (state r - 2 + pairs of r - 1) and fold r - 1 in one launch;
        // the cached candidates' sums over state r - 2 carry over from
        // selection r - 1, except at a full re-scoring
        KLA_TRY(slots_free(x_new));
        const int n_cblk = (n_cand + kScoreCand - 1) / kScoreCand;
        const int n_carry = r % kRescore == 0 ? 0 : n_cache;
        const int bnew0 = n_carry / kScoreCand;
        const int n_score = N * (n_cblk + (n_cblk - bnew0) * kSZ);
        const int n_fold = r >= 1 ? N * kFoldWGs : 0;
        if (prof) prof_begin(st);
        hipLaunchKernelGGL(hyb_refresh_kernel, dim3(n_score + n_fold), dim3(kThreads), 0, st, n_score, n_cblk,
                           bnew0, w.HF[x_old], k, v, a.T, cache[x_cur], kCStride, n_cache, f_prev, n_cand,
                           rej[(r + 1) & 1], kCStride, r >= 1 ? n_rej_prev : 0, w.sp, kCStride, w.H, w.s,
                           w.HF[x_cur], rej[(r + 1) & 1], n_rej_prev);
        KLA_CHECK();
        // fold r - 1 is issued: the readouts of the blocks refresh r - 1 serves
        KLA_TRY(flush(x_cur));
        hipLaunchKernelGGL(hyb_select_part_kernel, dim3(N), dim3(kSelThreads), 0, st, w.sp, kSZ + 1, kCStride, v,
                           a.T, a.eps, cache[x_cur], kCStride, cache[x_new], kCStride, n_cache, f_prev, n_cand,
                           a.cache_size, rej[r & 1], kCStride, a.trace, (size_t)a.cache_size, b, nblocks,
                           w.scores, kCStride, w.carry[(r + 1) & 1], n_carry, w.carry[r & 1]);
        if (prof) prof_end(st);
        KLA_CHECK();
        n_cache = a.cache_size;
        n_rej_prev = n_rej;
        slot = x_new;
        ++r;
        pending.push_back({b0, b1, f, n_cache});
      } else {
        if (n_ev > 0) {
          // appends past the entries any queued readout reads (before the first refresh only)
          hipLaunchKernelGGL(append_kernel, dim3(N), dim3(256), 0, st, cache[slot], kCStride, n_cache, f_prev,
                             n_ev);
          KLA_CHECK();
          n_cache += n_ev;
        }
        pending.push_back({b0, b1, f, n_cache});
        // before any refresh the state is final (zero): read out at once
        if (r == 0) KLA_TRY(flush(slot));
      }
      f_prev = f;
    }
    // the fold of the last refresh alone, then the remaining readouts
    if (r >= 1) {
      KLA_TRY(slots_free(r % 3));
      hipLaunchKernelGGL(hyb_refresh_kernel, dim3(N * kFoldWGs), dim3(kThreads), 0, st, 0, 1, 0, w.HF[0], k, v, a.T,
                         cache[slot], kCStride, 0, 0, 0, rej[(r + 1) & 1], kCStride, 0, w.sp, kCStride, w.H, w.s,
                         w.HF[slot], rej[(r + 1) & 1], n_rej_prev);
      KLA_CHECK();
    }
    return flush(slot);
  }();
  // the caller's stream continues after the last readout
  if (two) {
    KLA_TRY(hipEventRecord(ss->join, sb));
    KLA_TRY(hipStreamWaitEvent(st, ss->join, 0));
  }
  if (loop_err != hipSuccess) return loop_err;
  if (a.cache_T && a.cache_size > 0) {
    hipLaunchKernelGGL(copy_rows_kernel, dim3(N), dim3(256), 0, st, a.cache_T, a.cache_size,
                       cache[slot], kCStride);
    KLA_CHECK();
  }
#undef KLA_CHECK
#undef KLA_TRY
  return hipSuccess;
}

template <typename Tout>
hipError_t run_matrix(const HybridArgs& a, void* ws, hipStream_t st, hipStream_t aux) {
  return enqueue_matrix<Tout>(a, ws, st, aux, true);
}

template <int DQK, int DV>
hipError_t run_dt(const HybridArgs& a, void* ws, hipStream_t st, hipStream_t aux) {
  if (DQK == 64 && DV == 64 && a.in_bf16)
    return a.out_bf16 ? run_matrix<uint16_t>(a, ws, st, aux) : run_matrix<float>(a, ws, st, aux);
  if (a.in_bf16)
    return a.out_bf16 ? run<DQK, DV, uint16_t, uint16_t>(a, ws, st)
                      : run<DQK, DV, uint16_t, float>(a, ws, st);
  return a.out_bf16 ? run<DQK, DV, float, uint16_t>(a, ws, st) : run<DQK, DV, float, float>(a, ws, st);
}

}  // namespace

size_t hybrid_workspace(const HybridArgs& a) {
  const int D = phi_dim(a.dqk);
  size_t b = 0;
  if (!a.HT) b += align_up((size_t)a.N * D * a.dv * sizeof(float));
  if (!a.sT) b += align_up((size_t)a.N * D * sizeof(float));
  b += align_up((size_t)a.N * kCStride * sizeof(int32_t));
  b += align_up((size_t)a.N * kCStride * sizeof(float));
  b += align_up((size_t)a.N * kCStride * sizeof(int32_t));
  if (matrix_path(a))
    b += 3 * align_up((size_t)a.N * kCStride * sizeof(int32_t)) + 3 * hf_bytes(a) + xp_bytes(a) + sp_bytes(a) +
         2 * carry_bytes(a);
  return b;
}

hipError_t hybrid_launch(const HybridArgs& a, void* ws, hipStream_t st, hipStream_t aux) {
#define KLA_CASE(A, B) \
  if (a.dqk == A && a.dv == B) return run_dt<A, B>(a, ws, st, aux);
  KLA_CASE(16, 16) KLA_CASE(16, 32) KLA_CASE(16, 64)
  KLA_CASE(32, 16) KLA_CASE(32, 32) KLA_CASE(32, 64)
  KLA_CASE(64, 16) KLA_CASE(64, 32) KLA_CASE(64, 64)
#undef KLA_CASE
  return hipErrorInvalidValue;
}

}  // namespace kla
