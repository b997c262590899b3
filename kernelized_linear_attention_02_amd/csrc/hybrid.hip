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
//   select : bitonic sort of (score, token id) keys; keep cache_size, list
//            the rest;
//   fold   : H += phi(k_i) v_i^T, s += phi(k_i) over the rejected tokens;
//   readout: for the block's queries, window and cache softmax terms and
//            the linear readout join one numerator and one denominator.
// The host knows every count in advance (they depend only on T, window,
// refresh and cache_size), so no device value is read back.
#include <algorithm>
#include <type_traits>

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
// cores: each wave takes 16-feature tiles (canonical order) and keeps a tile
// of [H | s] in MFMA accumulators seeded with the stored state. The feature
// products k_a k_b (times sqrt(2) off the diagonal) are exact float32 values
// split into three bf16 pieces p0 + p1 + p2 = p; v is bf16 on input, so every
// MFMA product is exact and the sums are float32, as in a float32 fold.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
constexpr int kFD = 64;
constexpr int kFPhi = kFD * (kFD + 1) / 2;   // 2080
constexpr int kFTiles = kFPhi / 16;          // 130
constexpr int kFoldTilesPerWG = 8;           // two per wave
constexpr int kFoldRows = 128;               // rejected tokens per call, at most

struct FoldPairs {
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

__global__ __launch_bounds__(kThreads) void hyb_fold_mfma_kernel(float* __restrict__ H, float* __restrict__ s,
                                                               const uint16_t* __restrict__ k,
                                                               const uint16_t* __restrict__ v, int T,
                                                               const int32_t* __restrict__ rejected,
                                                               int rstride, int n_rej) {
  __shared__ __align__(16) float kt[kFD][kFoldRows + 4];
  __shared__ __align__(16) uint16_t vt[kFD][kFoldRows + 8];
  const int n = blockIdx.y;
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
  for (int u = 0; u < kFoldTilesPerWG / kWavesF; ++u) {
    const int tile = blockIdx.x * kFoldTilesPerWG + u * kWavesF + w;
    if (tile >= kFTiles) break;
    const int f0 = tile * 16;
    // this lane's feature row (A operand) and its factors
    const uint16_t ab = kFoldPairs.ab[f0 + l16];
    const int fa = ab & 0xFF, fb = ab >> 8;
    const float wgt = fa == fb ? 1.0f : 1.41421356237309504880f;
    // accumulators: rows 4*q4 + i of the tile, column 16*nt + l16 (nt = 4: s in column 0)
    f32x4 acc[5];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[nt][i] = Hn[(size_t)(f0 + 4 * q4 + i) * kFD + 16 * nt + l16];
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[4][i] = l16 == 0 ? sn[f0 + 4 * q4 + i] : 0.0f;
    for (int ks = 0; ks < R / 32; ++ks) {
      const float4* pa = reinterpret_cast<const float4*>(&kt[fa][32 * ks + 8 * q4]);
      const float4* pb = reinterpret_cast<const float4*>(&kt[fb][32 * ks + 8 * q4]);
      const float4 a0 = pa[0], a1 = pa[1], b0 = pb[0], b1 = pb[1];
      const float p[8] = {a0.x * b0.x * wgt, a0.y * b0.y * wgt, a0.z * b0.z * wgt, a0.w * b0.w * wgt,
                          a1.x * b1.x * wgt, a1.y * b1.y * wgt, a1.z * b1.z * wgt, a1.w * b1.w * wgt};
      bf16x8 A0, A1, A2;
      split3_8(p, A0, A1, A2);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const bf16x8 B = *reinterpret_cast<const bf16x8*>(&vt[16 * nt + l16][32 * ks + 8 * q4]);
        acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A0, B, acc[nt], 0, 0, 0);
        acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A1, B, acc[nt], 0, 0, 0);
        acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A2, B, acc[nt], 0, 0, 0);
      }
      acc[4] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A0, ones, acc[4], 0, 0, 0);
      acc[4] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A1, ones, acc[4], 0, 0, 0);
      acc[4] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A2, ones, acc[4], 0, 0, 0);
    }
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) Hn[(size_t)(f0 + 4 * q4 + i) * kFD + 16 * nt + l16] = acc[nt][i];
    if (l16 == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) sn[f0 + 4 * q4 + i] = acc[4][i];
    }
  }
}

// ---------------------------------------------------------------- matrix-core readout (d = 64, bf16 in)
//
// One work-group per (head, 64 queries of a block); wave w owns queries
// t0 + 16 w .. + 15. Softmax keys are the cache entries and then the window
// [f, t]. Scores come from S^T = K Q^T on bf16 MFMA (exact products, float32
// sums): lane (l16, q4) holds the scores of query l16 against keys 4 q4 + i
// of each 16-key half. Pass 1 finds each query's maximum m (clamped at 0, as
// the joint normalisation divides the linear terms by e^m too); pass 2 forms
// P = e^(tau s - m) and P [V | 1] on MFMA (P in two bf16 pieces), taking P's k-slots in the order the
// scores sit in the lanes (keys 4 q4 + j, then 16 + 4 q4 + j) and V in the
// same order. The linear term phi(q)^T [H | s] streams the state through LDS
// as two-piece bf16 B fragments (hi*hi + hi*lo + lo*hi with two-piece phi(q)). Output column 4 l16 + nt sits in n-tile nt of lane
// (l16, q4), rows 4 q4 + i.
constexpr int kRW = 4;        // waves (16 queries each) per work-group
constexpr int kRT = 64 * kRW; // threads
constexpr int kRQ = 16 * kRW; // queries per work-group
constexpr int kRK = 32;       // keys per tile
constexpr int kRF = 64;       // features per staged state tile (two k-steps)
constexpr int kKVP = kRK * 8 / kRT;          // 16-byte key/value pieces per thread and tile
constexpr int kHP = kRF * (kFD / 4) / kRT;   // float4 state pieces per thread and tile

struct ReadoutLds {
  uint16_t ks[kRK][kFD + 8];            // key rows of the tile (bf16)
  uint16_t vt[kFD][kRK + 8];            // value tile, transposed (bf16)
  float qf[kRQ][kFD + 1];               // query rows (float32) for phi(q)
  uint16_t tab[kFPhi];                  // feature pairs
  uint4 hf[2][kRF / 32][5][64];         // state B fragments (hi, lo pieces) of the staged feature tile
  float mq[kRQ];                        // per-query maximum
  float den[kRQ];                       // per-query denominator
};

template <typename Tout>
__global__ __launch_bounds__(kRT) void hyb_readout_mfma_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    Tout* __restrict__ o, int T, const float* __restrict__ H, const float* __restrict__ s,
    const int32_t* __restrict__ cache, int cstride, int n_cache, int t_begin, int t_end, int f,
    float scale, float eps) {
  __shared__ __align__(16) ReadoutLds sh;
  const int n = blockIdx.y;
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

  auto key_token = [&](int j) { return j < n_cache ? cn[j] : f + (j - n_cache); };
  // key (and value) rows of tile j0 .. j0 + 31 in 16-byte pieces (row p / 8, piece p % 8),
  // loaded into registers one tile ahead, then stored to LDS
  auto load_kv = [&](int j0, bool with_v, uint4 (&ku)[kKVP], uint4 (&vu)[kKVP]) {
#pragma unroll
    for (int e = 0; e < kKVP; ++e) {
      const int pidx = tid + kRT * e, sr = pidx >> 3, sc8 = pidx & 7;
      ku[e] = make_uint4(0, 0, 0, 0);
      vu[e] = ku[e];
      if (j0 + sr < n_keys) {
        const size_t row = base + (size_t)key_token(j0 + sr) * kFD + 8 * sc8;
        ku[e] = *reinterpret_cast<const uint4*>(k + row);
        if (with_v) vu[e] = *reinterpret_cast<const uint4*>(v + row);
      }
    }
  };
  auto store_kv = [&](bool with_v, const uint4 (&ku)[kKVP], const uint4 (&vu)[kKVP]) {
#pragma unroll
    for (int e = 0; e < kKVP; ++e) {
      const int pidx = tid + kRT * e, sr = pidx >> 3, sc8 = pidx & 7;
      *reinterpret_cast<uint4*>(&sh.ks[sr][8 * sc8]) = ku[e];
      if (with_v) {
        const uint32_t vw[4] = {vu[e].x, vu[e].y, vu[e].z, vu[e].w};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          sh.vt[8 * sc8 + 2 * c][sr] = (uint16_t)(vw[c] & 0xFFFF);
          sh.vt[8 * sc8 + 2 * c + 1][sr] = (uint16_t)(vw[c] >> 16);
        }
      }
    }
  };
  // scores of this wave's queries against the staged tile: sc[h][i] = key 16 h + 4 q4 + i
  auto scores = [&](int j0, float (&sc)[2][4]) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(&sh.ks[16 * h + l16][32 * ks + 8 * q4]);
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qb[ks], c, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = j0 + 16 * h + 4 * q4 + i;
        // cache keys precede every query; window keys are causal
        const bool ok = j < n_keys && my_t < tq_end && (j < n_cache || f + (j - n_cache) <= my_t);
        sc[h][i] = ok ? scale * c[i] : -INFINITY;
      }
    }
  };
  const int wave_keys = min(n_keys, n_cache + (min(tq_end, tw + 16) - f));  // keys any query of the wave sees

  // ---- pass 1: per-query maximum
  float mx = 0.0f;  // never below 0
  uint4 kpre[kKVP], vpre[kKVP];
  load_kv(0, false, kpre, vpre);
  for (int j0 = 0; j0 < n_keys; j0 += kRK) {
    __syncthreads();
    store_kv(false, kpre, vpre);
    __syncthreads();
    if (j0 + kRK < n_keys) load_kv(j0 + kRK, false, kpre, vpre);
    if (j0 < wave_keys) {
      float sc[2][4];
      scores(j0, sc);
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sc[h][i]);
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
  load_kv(0, true, kpre, vpre);
  for (int j0 = 0; j0 < n_keys; j0 += kRK) {
    __syncthreads();
    store_kv(true, kpre, vpre);
    __syncthreads();
    if (j0 + kRK < n_keys) load_kv(j0 + kRK, true, kpre, vpre);
    if (j0 < wave_keys) {
      float sc[2][4];
      scores(j0, sc);
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
        const uint2 lo = *reinterpret_cast<const uint2*>(&sh.vt[4 * l16 + nt][4 * q4]);
        const uint2 hi = *reinterpret_cast<const uint2*>(&sh.vt[4 * l16 + nt][16 + 4 * q4]);
        const bf16x8 b = __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
        acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(p0, b, acc[nt], 0, 0, 0);
        acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(p1, b, acc[nt], 0, 0, 0);
      }
      acc[4] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(p0, ones, acc[4], 0, 0, 0);
      acc[4] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(p1, ones, acc[4], 0, 0, 0);
    }
  }

  // ---- linear readout phi(q)^T [H | s], state staged kRF features at a time
  f32x4 lin[5];
#pragma unroll
  for (int nt = 0; nt < 5; ++nt) lin[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  const float* Hn = H + (size_t)n * kFPhi * kFD;
  const float* sn = s + (size_t)n * kFPhi;
  const float* qrow = sh.qf[16 * w + l16];
  // state rows g0 .. g0 + 63 in float4 pieces p = tid + kRT m (row p / 16, columns 4 (p % 16) .. + 3),
  // one tile ahead; row r, column 4 c4 + nt goes to fragment (k-step r / 32, n-tile nt,
  // lane 16 ((r % 32) / 8) + c4, element r % 8); the normaliser fragment holds s in lane column 0
  for (int i = tid; i < 2 * (kRF / 32) * 64; i += kRT) {
    // zero the normaliser fragments once (only lane column 0 is written later)
    const int pc = i / ((kRF / 32) * 64), rest = i % ((kRF / 32) * 64);
    sh.hf[pc][rest / 64][4][rest % 64] = make_uint4(0, 0, 0, 0);
  }
  float4 hpre[kHP];
  float spre[kHP];
  auto load_h = [&](int g0) {
#pragma unroll
    for (int m = 0; m < kHP; ++m) {
      const int pidx = tid + kRT * m;
      const int r = g0 + (pidx >> 4), c4 = pidx & 15;
      hpre[m] = make_float4(0.f, 0.f, 0.f, 0.f);
      spre[m] = 0.0f;
      if (r < kFPhi) {
        hpre[m] = *reinterpret_cast<const float4*>(Hn + (size_t)r * kFD + 4 * c4);
        if (c4 == 0) spre[m] = sn[r];
      }
    }
  };
  auto put = [&](int pc, int kk, int nt, int L, int j, __bf16 x) {
    reinterpret_cast<__bf16*>(&sh.hf[pc][kk][nt][L])[j] = x;
  };
  load_h(0);
  for (int g0 = 0; g0 < kFPhi; g0 += kRF) {
    __syncthreads();
#pragma unroll
    for (int m = 0; m < kHP; ++m) {
      const int pidx = tid + kRT * m;
      const int r = pidx >> 4, c4 = pidx & 15;
      const int kk = r >> 5, L = 16 * ((r & 31) >> 3) + c4, j = r & 7;
      const float xs[4] = {hpre[m].x, hpre[m].y, hpre[m].z, hpre[m].w};
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const __bf16 a = (__bf16)xs[nt];
        put(0, kk, nt, L, j, a);
        put(1, kk, nt, L, j, (__bf16)(xs[nt] - (float)a));
      }
      if (c4 == 0) {
        const __bf16 a = (__bf16)spre[m];
        put(0, kk, 4, L, j, a);
        put(1, kk, 4, L, j, (__bf16)(spre[m] - (float)a));
      }
    }
    __syncthreads();
    if (g0 + kRF < kFPhi) load_h(g0 + kRF);
#pragma unroll
    for (int kk = 0; kk < kRF / 32; ++kk) {
      const int fr = g0 + 32 * kk + 8 * q4;
      float p[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float x = 0.0f;
        if (fr + j < kFPhi) {
          const uint16_t ab = sh.tab[fr + j];
          const int a = ab & 0xFF, bb = ab >> 8;
          x = qrow[a] * qrow[bb] * (a == bb ? 1.0f : 1.41421356237309504880f);
        }
        p[j] = x;
      }
      // phi(q) and the state in two bf16 pieces each: hi*hi + hi*lo + lo*hi
      bf16x8 A0, A1;
      split2_8(p, A0, A1);
#pragma unroll
      for (int nt = 0; nt < 5; ++nt) {
        const bf16x8 B0 = __builtin_bit_cast(bf16x8, sh.hf[0][kk][nt][lane]);
        const bf16x8 B1 = __builtin_bit_cast(bf16x8, sh.hf[1][kk][nt][lane]);
        lin[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A0, B0, lin[nt], 0, 0, 0);
        lin[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A0, B1, lin[nt], 0, 0, 0);
        lin[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A1, B0, lin[nt], 0, 0, 0);
      }
    }
  }

  // ---- combine: rows 4 q4 + i of the wave, columns 4 l16 + nt
  __syncthreads();
  if (l16 == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float e = __expf(-sh.mq[16 * w + 4 * q4 + i]);
      sh.den[16 * w + 4 * q4 + i] = acc[4][i] + e * (lin[4][i] + eps);
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
                          den != 0.0f ? (acc[nt][i] + e * lin[nt][i]) * inv : 0.0f);
    }
  }
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

struct Ws {
  float* H;
  float* s;
  int32_t* cache;
  float* scores;
  int32_t* rejected;
};

constexpr int kCStride = 256;

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
        if constexpr (DQK == 64 && DV == 64 && std::is_same<Tin, uint16_t>::value) {
          // matrix cores, float32-faithful (split bf16 operands)
          e = hybrid_score_mfma(N, w.H, w.s, k, v, a.T, w.cache, kCStride, n_cache, f_prev, n_cand,
                                w.scores, kCStride, a.eps, st);
          if (e != hipSuccess) return e;
        } else {
          hipLaunchKernelGGL((hyb_score_kernel<DQK, DV, Tin>), dim3((n_cand + 63) / 64, N),
                             dim3(kThreads), 0, st, w.H, w.s, k, v, a.T, w.cache, kCStride, n_cache,
                             f_prev, n_cand, w.scores, kCStride, a.eps);
        }
        prof_end(st);
        KLA_CHECK();
        hipLaunchKernelGGL(hyb_select_kernel, dim3(N), dim3(kThreads), 0, st, w.scores, kCStride,
                           w.cache, kCStride, n_cache, f_prev, n_cand, a.cache_size, w.rejected,
                           kCStride, a.trace, (size_t)a.cache_size, b, nblocks);
        KLA_CHECK();
        if constexpr (DQK == 64 && DV == 64 && std::is_same<Tin, uint16_t>::value) {
          hipLaunchKernelGGL(hyb_fold_mfma_kernel, dim3((kFTiles + kFoldTilesPerWG - 1) / kFoldTilesPerWG, N),
                             dim3(kThreads), 0, st, w.H, w.s, k, v, a.T, w.rejected, kCStride,
                             n_cand - a.cache_size);
        } else {
          hipLaunchKernelGGL((hyb_fold_kernel<DQK, DV, Tin>), dim3(S, N), dim3(kThreads), 0, st,
                             w.H, w.s, k, v, a.T, w.rejected, kCStride, n_cand - a.cache_size, Fs);
        }
        KLA_CHECK();
        n_cache = a.cache_size;
      }
    }
    f_prev = f;
    if constexpr (DQK == 64 && DV == 64 && std::is_same<Tin, uint16_t>::value) {
      hipLaunchKernelGGL((hyb_readout_mfma_kernel<Tout>), dim3((b1 - b0 + kRQ - 1) / kRQ, N), dim3(kRT), 0,
                         st, q, k, v, o, a.T, w.H, w.s, w.cache, kCStride, n_cache, b0, b1, f, a.scale,
                         a.eps);
    } else {
      hipLaunchKernelGGL((hyb_readout_kernel<DQK, DV, Tin, Tout>), dim3((b1 - b0 + 15) / 16, N),
                         dim3(kThreads), 0, st, q, k, v, o, a.T, w.H, w.s, w.cache, kCStride,
                         n_cache, b0, b1, f, a.scale, a.eps);
    }
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
  const int D = phi_dim(a.dqk);
  size_t b = 0;
  if (!a.HT) b += align_up((size_t)a.N * D * a.dv * sizeof(float));
  if (!a.sT) b += align_up((size_t)a.N * D * sizeof(float));
  b += align_up((size_t)a.N * kCStride * sizeof(int32_t));
  b += align_up((size_t)a.N * kCStride * sizeof(float));
  b += align_up((size_t)a.N * kCStride * sizeof(int32_t));
  return b;
}

hipError_t hybrid_launch(const HybridArgs& a, void* ws, hipStream_t st) {
#define KLA_CASE(A, B) \
  if (a.dqk == A && a.dv == B) return run_dt<A, B>(a, ws, st);
  KLA_CASE(16, 16) KLA_CASE(16, 32) KLA_CASE(16, 64)
  KLA_CASE(32, 16) KLA_CASE(32, 32) KLA_CASE(32, 64)
  KLA_CASE(64, 16) KLA_CASE(64, 32) KLA_CASE(64, 64)
#undef KLA_CASE
  return hipErrorInvalidValue;
}

}  // namespace kla
