// One decode step fused with self-recall-error scoring and top-k selection,
// for d_qk = d_v = 64 and at most 64 candidates per head-state.
//
// Decode (KATA page §1, constant-time recurrent inference; LoLA page,
// "Estratégia de Inferência", token-by-token mode):
//   s' = s + phi(k);  H' = H + phi(k) v^T;  o = phi(q)^T H' / (phi(q)^T s' + eps).
// Scoring (LoLA page, section "O Mecanismo de Erro de Auto-Recuperação"),
// against the updated state:
//   pred_c = phi(k_c)^T H' / (phi(k_c)^T s' + eps)  (0 when that is 0),
//   score_c = ||pred_c - v_c||^2,
// and selection (LoLA, "Estratégia de Inferência" item 2): the top_k highest
// scores, ties to the lower candidate index.
//
// One work-group per head-state; its four waves take the 65 tiles of 32
// features in turn. A wave streams a tile of H (32 rows x 64 floats) with
// 16-byte loads - lane (l16, q4) holds rows 8*q4 .. 8*q4+7 at columns
// 4*l16 .. 4*l16+3 - updates it in float32, writes it back, and accumulates
// the float32 readout. The same registers are then the B operand of the
// candidate numerators phi(K_c) H' on the bf16 matrix cores: the 8 rows a
// lane holds are its 8 k-values, and MFMA column n of n-block j stands for
// state column 4*n + j. The state values are split exactly into three bf16
// pieces h0 + h1 + h2, the candidate features into two, p ~ p0 + p1 (16
// significant bits), and the product is taken as p0 (h0 + h1 + h2) + p1 h0
// with float32 accumulation: the dropped terms are below 2^-16 relative, and
// a feature that is exact in bf16 (an orthonormal basis key) recalls the
// stored float32 value exactly. Denominators stay in float32 on the vector
// units. The state is read once and written once; the
// candidate keys sit in LDS.
#include "kla_device.hpp"
#include "kla_internal.hpp"
#include "mfma_bf16.hpp"

namespace kla {
namespace {

constexpr int kDim = 64;
constexpr int kD = kDim * (kDim + 1) / 2;  // 2080
constexpr int kFT = 32;                    // features per tile (one MFMA k-step)
constexpr int kTiles = kD / kFT;           // 65
constexpr int kWaves = 4;
constexpr int kThreadsF = 64 * kWaves;
constexpr int kMaxCand = 64;
static_assert(kD % kFT == 0, "tiles must cover the features exactly");

__constant__ PairTable64 kPairTable = PairTable64();

struct FusedLds {
  float qs[kDim];
  float ks[kDim];
  float vs[kDim];
  uint16_t tab[kD];
  union {
    float ck[kMaxCand][kDim + 1];    // candidate keys, padded rows (tile loop)
    float4 red[4][4][64];            // numerator partials, accumulator layout (after it)
  };
  float den[kWaves][kMaxCand];
  float onum[kWaves][kDim];
  float oden[kWaves];
  uint64_t keys[kMaxCand];
};

__device__ __forceinline__ f32x4 mfma(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return mfma16x16x32(a, b, c);
}

// State loads and stores. kStreamNT switches them to nontemporal hints,
// which measured slower on the decode workload, so they stay plain.
constexpr bool kStreamNT = false;
__device__ __forceinline__ float4 ld_state(const float* p) {
  if (kStreamNT) {
    const f32x4 x = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
    return make_float4(x[0], x[1], x[2], x[3]);
  }
  return *reinterpret_cast<const float4*>(p);
}
__device__ __forceinline__ void st_state(float* p, const float4& v) {
  if (kStreamNT) {
    const f32x4 x = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(x, reinterpret_cast<f32x4*>(p));
  } else {
    *reinterpret_cast<float4*>(p) = v;
  }
}

// Candidate source: rows of float32 arrays [N, n_cand, 64].
struct CandRows {
  const float* k;
  const float* v;
  int n_cand;
  __device__ __forceinline__ float4 k4(int n, int c, int d4) const {
    return *reinterpret_cast<const float4*>(k + ((size_t)n * n_cand + c) * kDim + 4 * d4);
  }
  __device__ __forceinline__ float4 v4(int n, int c, int d4) const {
    return *reinterpret_cast<const float4*>(v + ((size_t)n * n_cand + c) * kDim + 4 * d4);
  }
};

// Work-group (n, g) scores candidates 64 g .. 64 g + 16 MT - 1 of head-state n.
// MT: 16-candidate blocks. UPDATE: decode step first (H and s written back,
// o produced); otherwise the state is only read. SELECT: top_k selection and
// gather in the same kernel (requires n_cand <= 16 * MT, one group).
template <int MT, bool UPDATE, bool SELECT, typename Tin, typename Tout, typename Cand>
__global__ __launch_bounds__(kThreadsF, 2) void decode_sre_kernel(
    float* __restrict__ H, float* __restrict__ s, const Tin* __restrict__ q,
    const Tin* __restrict__ k, const Tin* __restrict__ v, Tout* __restrict__ o, float eps,
    Cand cand, int n_cand, int top_k, float* __restrict__ scores, int sstride,
    int32_t* __restrict__ sel, float* __restrict__ sel_k, float* __restrict__ sel_v, int sel_stride) {
  __shared__ __align__(16) FusedLds sh;
  const int n = blockIdx.x;
  const int cbase = 64 * blockIdx.y;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l16 = lane & 15;
  const int q4 = lane >> 4;
  float* Hn = H + (size_t)n * kD * kDim;
  float* sn = s + (size_t)n * kD;

  // tile ks: rows f0 .. f0 + 31; this lane's rows f0 + 8*q4 + j
  auto load_tile = [&](int ks, float4 (&h)[8], float4 (&sv)[2]) {
    const int fr = kFT * ks + 8 * q4;
#pragma unroll
    for (int j = 0; j < 8; ++j) h[j] = ld_state(Hn + (size_t)(fr + j) * kDim + 4 * l16);
    sv[0] = ld_state(sn + fr);
    sv[1] = ld_state(sn + fr + 4);
  };
  // the first tile is in flight while the block stages its inputs
  float4 h[8], sv[2];
  load_tile(w, h, sv);

  if (UPDATE && tid < kDim) {
    sh.qs[tid] = Elem<Tin>::load(q, (size_t)n * kDim + tid);
    sh.ks[tid] = Elem<Tin>::load(k, (size_t)n * kDim + tid);
    sh.vs[tid] = Elem<Tin>::load(v, (size_t)n * kDim + tid);
  }
  for (int i = tid; i < kD; i += kThreadsF) sh.tab[i] = kPairTable.ab[i];
  for (int i = tid; i < 16 * MT * (kDim / 4); i += kThreadsF) {
    const int c = i / (kDim / 4);
    const int d4 = i % (kDim / 4);
    float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
    if (cbase + c < n_cand) x = cand.k4(n, cbase + c, d4);
    sh.ck[c][4 * d4] = x.x;
    sh.ck[c][4 * d4 + 1] = x.y;
    sh.ck[c][4 * d4 + 2] = x.z;
    sh.ck[c][4 * d4 + 3] = x.w;
  }
  __syncthreads();


  float4 v4 = make_float4(0.f, 0.f, 0.f, 0.f);
  if (UPDATE) v4 = *reinterpret_cast<const float4*>(&sh.vs[4 * l16]);

  f32x4 acc[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float dacc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) dacc[mt] = 0.0f;
  float4 oacc = make_float4(0.f, 0.f, 0.f, 0.f);
  float oden = 0.0f;


#pragma unroll 1
  for (int ks = w; ks < kTiles; ks += kWaves) {
    float4 hn[8], svn[2];
    const bool more = ks + kWaves < kTiles;
    if (more) load_tile(ks + kWaves, hn, svn);

    const int fr = kFT * ks + 8 * q4;
    const uint4 pw = *reinterpret_cast<const uint4*>(&sh.tab[fr]);
    const uint32_t words[4] = {pw.x, pw.y, pw.z, pw.w};
    int pa[8], pb[8];
    float wt[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t u = (j & 1) ? (words[j >> 1] >> 16) : (words[j >> 1] & 0xFFFFu);
      pa[j] = u & 0xFF;
      pb[j] = u >> 8;
      wt[j] = pa[j] == pb[j] ? 1.0f : kSqrt2;
    }
    float sj[8] = {sv[0].x, sv[0].y, sv[0].z, sv[0].w, sv[1].x, sv[1].y, sv[1].z, sv[1].w};
    if (UPDATE) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float pk = sh.ks[pa[j]] * sh.ks[pb[j]] * wt[j];
        const float pq = sh.qs[pa[j]] * sh.qs[pb[j]] * wt[j];
        h[j].x += pk * v4.x;
        h[j].y += pk * v4.y;
        h[j].z += pk * v4.z;
        h[j].w += pk * v4.w;
        sj[j] += pk;
        st_state(Hn + (size_t)(fr + j) * kDim + 4 * l16, h[j]);
        oacc.x += pq * h[j].x;
        oacc.y += pq * h[j].y;
        oacc.z += pq * h[j].z;
        oacc.w += pq * h[j].w;
        oden += pq * sj[j];
      }
      // two lanes per quarter write its 8 values: one contiguous 128-byte run
      if (l16 < 2)
        st_state(sn + fr + 4 * l16, l16 ? make_float4(sj[4], sj[5], sj[6], sj[7])
                                        : make_float4(sj[0], sj[1], sj[2], sj[3]));
    }

    // A operands (two pieces) for every candidate block, and the float32
    // denominators
    bf16x8 ahi[MT], alo[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const float* kc = sh.ck[16 * mt + l16];
      float p[8];
      float dd = 0.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        p[j] = kc[pa[j]] * kc[pb[j]] * wt[j];
        dd += p[j] * sj[j];
      }
      dacc[mt] += dd;
      split2(p, ahi[mt], alo[mt]);
    }
    // B operands (three pieces, exact): state column 4*l16 + nt over this
    // lane's 8 rows
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      float x[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = comp(h[j], nt);
      bf16x8 b0, b1, b2;
      split3(x, b0, b1, b2);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        acc[mt][nt] = mfma(ahi[mt], b0, acc[mt][nt]);
        acc[mt][nt] = mfma(ahi[mt], b1, acc[mt][nt]);
        acc[mt][nt] = mfma(ahi[mt], b2, acc[mt][nt]);
        acc[mt][nt] = mfma(alo[mt], b0, acc[mt][nt]);
      }
    }
    if (more) {
#pragma unroll
      for (int j = 0; j < 8; ++j) h[j] = hn[j];
      sv[0] = svn[0];
      sv[1] = svn[1];
    }
  }

  // ---- readout partials: sum over the lane quarters, then over waves
  if (UPDATE) {
    float ox[4] = {oacc.x, oacc.y, oacc.z, oacc.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ox[i] += __shfl_xor(ox[i], 16, 64);
      ox[i] += __shfl_xor(ox[i], 32, 64);
    }
    oden += __shfl_xor(oden, 16, 64);
    oden += __shfl_xor(oden, 32, 64);
    if (q4 == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) sh.onum[w][4 * l16 + i] = ox[i];
    }
    if (lane == 0) sh.oden[w] = oden;
  }
  // candidate denominators: lane l16 of block mt is candidate 16*mt + l16
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    float d = dacc[mt];
    d += __shfl_xor(d, 16, 64);
    d += __shfl_xor(d, 32, 64);
    if (q4 == 0) sh.den[w][16 * mt + l16] = d;
  }
  // numerators: waves add into the LDS copy in turn; the last one keeps the sum
  // (the first barrier also ends every read of the candidate keys, whose LDS
  // the partials reuse)
  for (int r = 0; r < kWaves; ++r) {
    __syncthreads();
    if (w == r) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
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
  // (the loop's last barrier has made onum, oden and den visible)
  if (UPDATE && tid < kDim) {
    float num = 0.0f, den = eps;
#pragma unroll
    for (int r = 0; r < kWaves; ++r) {
      num += sh.onum[r][tid];
      den += sh.oden[r];
    }
    Elem<Tout>::store(o, (size_t)n * kDim + tid, den != 0.0f ? num / den : 0.0f);
  }
  if (w == kWaves - 1) {
    // lane (l16, q4) holds candidates 16*mt + 4*q4 + i at state columns 4*l16 + nt
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c = 16 * mt + 4 * q4 + i;
        const bool live = cbase + c < n_cand;
        float den = eps;
#pragma unroll
        for (int r = 0; r < kWaves; ++r) den += sh.den[r][c];
        float4 vc = make_float4(0.f, 0.f, 0.f, 0.f);
        if (live) vc = cand.v4(n, cbase + c, l16);
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
        if (l16 == 0) {
          if (live && scores) scores[(size_t)n * sstride + cbase + c] = err;
          if (SELECT) sh.keys[c] = live ? topk_key(err, (uint32_t)c) : 0ull;
        }
      }
    }
    if (SELECT)
      for (int c = 16 * MT + lane; c < kMaxCand; c += 64) sh.keys[c] = 0ull;
  }
  if (!SELECT) return;
  bitonic_sort_desc(sh.keys, kMaxCand);
  for (int i = tid; i < top_k; i += kThreadsF) sel[(size_t)n * top_k + i] = (int32_t)topk_index(sh.keys[i]);
  if (sel_k) {
    for (int i = tid; i < top_k * (kDim / 4); i += kThreadsF) {
      const int j = i / (kDim / 4);
      const int d4 = i % (kDim / 4);
      const int c = (int)topk_index(sh.keys[j]);
      const size_t dst = ((size_t)n * sel_stride + j) * kDim + 4 * d4;
      *reinterpret_cast<float4*>(sel_k + dst) = cand.k4(n, c, d4);
      *reinterpret_cast<float4*>(sel_v + dst) = cand.v4(n, c, d4);
    }
  }
}

template <int MT, bool UPDATE, typename Tin, typename Tout>
void launch_fused(int N, float* H, float* s, const void* q, const void* k, const void* v, void* o,
                  float eps, const SreArgs& sre, hipStream_t st) {
  const CandRows cand{sre.cand_k, sre.cand_v, sre.n_cand};
  hipLaunchKernelGGL((decode_sre_kernel<MT, UPDATE, true, Tin, Tout, CandRows>), dim3(N, 1), dim3(kThreadsF), 0, st,
                     H, s, static_cast<const Tin*>(q), static_cast<const Tin*>(k), static_cast<const Tin*>(v),
                     static_cast<Tout*>(o), eps, cand, sre.n_cand, sre.top_k, sre.scores, sre.n_cand, sre.sel,
                     sre.sel_k, sre.sel_v, sre.sel_stride ? sre.sel_stride : sre.top_k);
}

template <bool UPDATE, typename Tin, typename Tout>
void launch_mt(int N, float* H, float* s, const void* q, const void* k, const void* v, void* o, float eps,
               const SreArgs& sre, hipStream_t st) {
  // 16, 32 or 64 candidate rows (rows past n_cand are zero keys, not scored)
  const int mt = (sre.n_cand + 15) / 16;
  if (mt == 1) launch_fused<1, UPDATE, Tin, Tout>(N, H, s, q, k, v, o, eps, sre, st);
  else if (mt == 2) launch_fused<2, UPDATE, Tin, Tout>(N, H, s, q, k, v, o, eps, sre, st);
  else launch_fused<4, UPDATE, Tin, Tout>(N, H, s, q, k, v, o, eps, sre, st);
}

}  // namespace

bool decode_fused_supported(int dqk, int dv, const SreArgs& sre) {
  return dqk == kDim && dv == kDim && sre.n_cand >= 1 && sre.n_cand <= kMaxCand;
}

hipError_t decode_fused_launch(const DecodeArgs& a, const SreArgs& sre, hipStream_t st) {
  prof_begin(st);
  if (a.in_bf16) {
    if (a.out_bf16) launch_mt<true, uint16_t, uint16_t>(a.N, a.H, a.s, a.q, a.k, a.v, a.o, a.eps, sre, st);
    else launch_mt<true, uint16_t, float>(a.N, a.H, a.s, a.q, a.k, a.v, a.o, a.eps, sre, st);
  } else {
    if (a.out_bf16) launch_mt<true, float, uint16_t>(a.N, a.H, a.s, a.q, a.k, a.v, a.o, a.eps, sre, st);
    else launch_mt<true, float, float>(a.N, a.H, a.s, a.q, a.k, a.v, a.o, a.eps, sre, st);
  }
  prof_end(st);
  return hipGetLastError();
}

hipError_t sre_fused_launch(int N, float eps, const float* H, const float* s, const SreArgs& sre,
                            hipStream_t st) {
  prof_begin(st);
  // read-only: the kernel neither loads q, k, v nor writes H, s or o
  launch_mt<false, float, float>(N, const_cast<float*>(H), const_cast<float*>(s), nullptr, nullptr, nullptr,
                                 nullptr, eps, sre, st);
  prof_end(st);
  return hipGetLastError();
}

}  // namespace kla
