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
//
// Deferred folds (the same step with a list of pending pairs): the lift
// gives phi(x) . phi(y) = (x . y)^2 (KATA page §2.2), so the state plus
// pairs that are not yet folded in reads out as
//   phi(x)^T H + sum_j (x . k_j)^2 v_j,   phi(x)^T s + sum_j (x . k_j)^2,
// for the query and for every candidate key alike. A deferred step reads H
// and s, writes neither, and appends its pair to the list; the step whose
// pair fills the list adds all of it (rank kPend) to H and s in the same
// pass that reads them out and scores.
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
constexpr int kPend = 8;  // pending slots per head-state, folded together
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
  // pair list of the deferred modes: keys transposed (feature -> kPend
  // pairs), values by pair, and the squared dot products of the query and of
  // every candidate key with each listed key; the state's s (read-only modes
  // take it from here rather than holding it in registers)
  alignas(16) float sS[kD];
  float rnum[kWaves][kDim];  // per-wave readout sums of the read-only mode
  float rden[kWaves];
  alignas(16) float pkT[kDim][kPend];
  alignas(16) float pv[kPend][kDim];
  float wq[kPend];
  float wc[kMaxCand][kPend];
};

// Kernel modes.
//   kStep : update with the step's token, write H and s back, read out, score.
//   kScore: read H and s, score only.
//   kRead : read H and s; read out and score against them plus the list
//           (pending slots, then the token) in closed form; store the token
//           in its pending slot.
//   kFold : update with the list (the pending slots, then the token), write
//           back, read out, score.
//   kFlush: add the pending slots to H and s, write back.
enum : int { kStep = 0, kScore = 1, kFold = 2, kRead = 3, kFlush = 4 };

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

// Work-group (n, g) scores candidates 64 g .. 64 g + 16 MT - 1 of head-state n
// (MT: 16-candidate blocks, 0 for none). SELECT: top_k selection and gather
// in the same kernel (requires n_cand <= 16 * MT, one group). The deferred
// modes take the pending slots of head-state n from pend_k / pend_v
// ([N, kPend, 64] float32), n_pend of them in use (kRead: n_pend < kPend - 1;
// kFold: n_pend = kPend - 1; kFlush: n_pend <= kPend).
template <int MT, int MODE, bool SELECT, typename Tin, typename Tout, typename Cand>
__global__ __launch_bounds__(kThreadsF, 2) void decode_sre_kernel(
    float* __restrict__ H, float* __restrict__ s, const Tin* __restrict__ q,
    const Tin* __restrict__ k, const Tin* __restrict__ v, Tout* __restrict__ o, float eps,
    Cand cand, int n_cand, int top_k, float* __restrict__ scores, int sstride,
    int32_t* __restrict__ sel, float* __restrict__ sel_k, float* __restrict__ sel_v, int sel_stride,
    float* __restrict__ pend_k, float* __restrict__ pend_v, int n_pend) {
  constexpr bool kWrites = MODE == kStep || MODE == kFold || MODE == kFlush;
  constexpr bool kReadout = MODE == kStep || MODE == kFold || MODE == kRead;
  constexpr bool kToken = kReadout;
  constexpr bool kList = MODE == kFold || MODE == kRead || MODE == kFlush;
  constexpr bool kSLds = MODE == kRead || MODE == kFold;  // s from LDS
  // readout sums per wave in LDS (see read_col below) rather than in registers
  constexpr bool kLdsOut = MODE == kRead || MODE == kFold;
  constexpr int MTA = MT > 0 ? MT : 1;
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
    if (!kSLds) {
      sv[0] = ld_state(sn + fr);
      sv[1] = ld_state(sn + fr + 4);
    }
  };
  // the first tile is in flight while the block stages its inputs
  float4 h[8], sv[2];
  load_tile(w, h, sv);

  if (kToken && tid < kDim) {
    sh.qs[tid] = Elem<Tin>::load(q, (size_t)n * kDim + tid);
    sh.ks[tid] = Elem<Tin>::load(k, (size_t)n * kDim + tid);
    sh.vs[tid] = Elem<Tin>::load(v, (size_t)n * kDim + tid);
  }
  if (kList) {
    // list entry p: pending slot p (p < n_pend), the step's token (p =
    // n_pend), zero after (a zero key adds nothing)
    const size_t slot0 = (size_t)n * kPend;
    for (int i = tid; i < kPend * kDim; i += kThreadsF) {
      const int p = i / kDim, d = i % kDim;
      float kk = 0.0f, vv = 0.0f;
      if (p < n_pend) {
        kk = pend_k[(slot0 + p) * kDim + d];
        vv = pend_v[(slot0 + p) * kDim + d];
      } else if (kToken && p == n_pend) {
        kk = Elem<Tin>::load(k, (size_t)n * kDim + d);
        vv = Elem<Tin>::load(v, (size_t)n * kDim + d);
        if (MODE == kRead) {
          pend_k[(slot0 + p) * kDim + d] = kk;
          pend_v[(slot0 + p) * kDim + d] = vv;
        }
      }
      sh.pkT[d][p] = kk;
      sh.pv[p][d] = vv;
    }
  }
  for (int i = tid; i < kD; i += kThreadsF) sh.tab[i] = kPairTable.ab[i];
  if (kLdsOut) {
    sh.rnum[w][lane] = 0.0f;
    if (lane == 0) sh.rden[w] = 0.0f;
  }
  if (kSLds)
    for (int i = tid; i < kD / 4; i += kThreadsF)
      *reinterpret_cast<float4*>(&sh.sS[4 * i]) = ld_state(sn + 4 * i);
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
  if (MODE == kRead) {
    // (x . k_p)^2 for the query (vector 0) and every candidate (vectors
    // 1 ..): four threads per vector, sixteen dimensions each, all kPend
    // listed keys at once; read after the numerator reduction's first barrier
    const int part = tid & 3;
    constexpr int kVec = 1 + 16 * MT;
#pragma unroll 1
    for (int vb = 0; vb < kVec; vb += kThreadsF / 4) {
      const int vi = vb + (tid >> 2);
      const float* x = (vi == 0 || vi >= kVec) ? sh.qs : sh.ck[vi - 1];
      float dot[kPend];
#pragma unroll
      for (int p = 0; p < kPend; ++p) dot[p] = 0.0f;
#pragma unroll
      for (int dd = 0; dd < 16; ++dd) {
        const int d = 16 * part + dd;
        const float xd = x[d];
        const float4 k0 = *reinterpret_cast<const float4*>(&sh.pkT[d][0]);
        const float4 k1 = *reinterpret_cast<const float4*>(&sh.pkT[d][4]);
        dot[0] += xd * k0.x;
        dot[1] += xd * k0.y;
        dot[2] += xd * k0.z;
        dot[3] += xd * k0.w;
        dot[4] += xd * k1.x;
        dot[5] += xd * k1.y;
        dot[6] += xd * k1.z;
        dot[7] += xd * k1.w;
      }
#pragma unroll
      for (int p = 0; p < kPend; ++p) {
        dot[p] += __shfl_xor(dot[p], 1, 64);
        dot[p] += __shfl_xor(dot[p], 2, 64);
      }
      if (part == 0 && vi < kVec) {
#pragma unroll
        for (int p = 0; p < kPend; ++p) {
          if (vi == 0) sh.wq[p] = dot[p] * dot[p];
          else sh.wc[vi - 1][p] = dot[p] * dot[p];
        }
      }
    }
  }

  float4 v4 = make_float4(0.f, 0.f, 0.f, 0.f);
  if (MODE == kStep) v4 = *reinterpret_cast<const float4*>(&sh.vs[4 * l16]);
  // the list's values at this lane's four state columns
  float4 vl[kPend];
  if (MODE == kFlush) {
#pragma unroll
    for (int p = 0; p < kPend; ++p) vl[p] = *reinterpret_cast<const float4*>(&sh.pv[p][4 * l16]);
  }

  f32x4 acc[MTA][4];
#pragma unroll
  for (int mt = 0; mt < MTA; ++mt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float dacc[MTA];
#pragma unroll
  for (int mt = 0; mt < MTA; ++mt) dacc[mt] = 0.0f;
  float4 oacc = make_float4(0.f, 0.f, 0.f, 0.f);
  float oden = 0.0f;


  // One tile: the state rows in h (s in sv), the next tile's loads issued
  // into hn / svn first. The loop below alternates the two buffers, so no
  // registers are copied between tiles.
  auto tile = [&](int ks, float4 (&h)[8], float4 (&sv)[2], float4 (&hn)[8], float4 (&svn)[2]) {
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
    if (kSLds) {
      sv[0] = *reinterpret_cast<const float4*>(&sh.sS[fr]);
      sv[1] = *reinterpret_cast<const float4*>(&sh.sS[fr + 4]);
    }
    float sj[8] = {sv[0].x, sv[0].y, sv[0].z, sv[0].w, sv[1].x, sv[1].y, sv[1].z, sv[1].w};
    if (MODE == kStep) {
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
    } else if (kList && kWrites) {
      // rank-kPend update: phi_f(k_p) = k_p[a] k_p[b] wt over the listed pairs
      // (the fold reloads the list's values per tile, to leave registers to
      // the scoring)
      if (MODE == kFold) {
#pragma unroll
        for (int p = 0; p < kPend; ++p) vl[p] = *reinterpret_cast<const float4*>(&sh.pv[p][4 * l16]);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float4 a0 = *reinterpret_cast<const float4*>(&sh.pkT[pa[j]][0]);
        const float4 a1 = *reinterpret_cast<const float4*>(&sh.pkT[pa[j]][4]);
        const float4 b0 = *reinterpret_cast<const float4*>(&sh.pkT[pb[j]][0]);
        const float4 b1 = *reinterpret_cast<const float4*>(&sh.pkT[pb[j]][4]);
        const float pk[kPend] = {a0.x * b0.x * wt[j], a0.y * b0.y * wt[j], a0.z * b0.z * wt[j],
                                 a0.w * b0.w * wt[j], a1.x * b1.x * wt[j], a1.y * b1.y * wt[j],
                                 a1.z * b1.z * wt[j], a1.w * b1.w * wt[j]};
#pragma unroll
        for (int p = 0; p < kPend; ++p) {
          h[j].x += pk[p] * vl[p].x;
          h[j].y += pk[p] * vl[p].y;
          h[j].z += pk[p] * vl[p].z;
          h[j].w += pk[p] * vl[p].w;
          sj[j] += pk[p];
        }
        st_state(Hn + (size_t)(fr + j) * kDim + 4 * l16, h[j]);
      }
    }
    // kRead: the query's products. The readout's partial sums go to this
    // wave's LDS slots per tile (after a sum over the lane quarters, which
    // hold other rows of the same columns) rather than living in registers
    // through the loop.
    float pq[8];
    if (kLdsOut) {
      float dq = 0.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        pq[j] = sh.qs[pa[j]] * sh.qs[pb[j]] * wt[j];
        dq += pq[j] * sj[j];
      }
      dq += __shfl_xor(dq, 16, 64);
      dq += __shfl_xor(dq, 32, 64);
      if (lane == 0) sh.rden[w] += dq;
    }
    auto read_col = [&](int nt, const float (&x)[8]) {
      float r = 0.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j) r += pq[j] * x[j];
      r += __shfl_xor(r, 16, 64);
      r += __shfl_xor(r, 32, 64);
      if (q4 == 0) sh.rnum[w][4 * l16 + nt] += r;
    };
    if (kWrites) {
      // two lanes per quarter write its 8 values: one contiguous 128-byte run
      if (l16 < 2)
        st_state(sn + fr + 4 * l16, l16 ? make_float4(sj[4], sj[5], sj[6], sj[7])
                                        : make_float4(sj[0], sj[1], sj[2], sj[3]));
    }

    if (MT > 0) {
      // candidate blocks in groups of MH (the deferred read splits four
      // blocks in two groups so its readout fits in registers): A operands
      // (two pieces) and the float32 denominators, then per column block the
      // B operands (three pieces, exact: state column 4*l16 + nt over this
      // lane's 8 rows) and the products
      constexpr int MH = MTA;
#pragma unroll
      for (int m0 = 0; m0 < MT; m0 += MH) {
        bf16x8 ahi[MH], alo[MH];
#pragma unroll
        for (int mm = 0; mm < MH; ++mm) {
          const float* kc = sh.ck[16 * (m0 + mm) + l16];
          float p[8];
          float dd = 0.0f;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            p[j] = kc[pa[j]] * kc[pb[j]] * wt[j];
            dd += p[j] * sj[j];
          }
          dacc[m0 + mm] += dd;
          split2_pk(p, ahi[mm], alo[mm]);
        }
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
          float x[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) x[j] = comp(h[j], nt);
          if (kLdsOut && m0 == 0) read_col(nt, x);
          bf16x8 b0, b1, b2;
          split3_pk(x, b0, b1, b2);
#pragma unroll
          for (int mm = 0; mm < MH; ++mm) {
            const int mt = m0 + mm;
            acc[mt][nt] = mfma(ahi[mm], b0, acc[mt][nt]);
            acc[mt][nt] = mfma(ahi[mm], b1, acc[mt][nt]);
            acc[mt][nt] = mfma(ahi[mm], b2, acc[mt][nt]);
            acc[mt][nt] = mfma(alo[mm], b0, acc[mt][nt]);
          }
        }
      }
    } else if (kLdsOut) {
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        float x[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = comp(h[j], nt);
        read_col(nt, x);
      }
    }
  };
  float4 h2[8], sv2[2];
#pragma unroll 1
  for (int ks = w; ks < kTiles; ks += 2 * kWaves) {
    tile(ks, h, sv, h2, sv2);
    if (ks + kWaves < kTiles) tile(ks + kWaves, h2, sv2, h, sv);
  }
  if (MODE == kFlush) return;

  // ---- readout partials: sum over the lane quarters, then over waves
  if (kReadout && !kLdsOut) {
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
  // the scoring wave's candidate value rows, requested now: they arrive
  // during the reduction instead of one round trip per candidate later
  float4 vcs[MTA][4];
  if (MT > 0 && w == kWaves - 1) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c = 16 * mt + 4 * q4 + i;
        vcs[mt][i] = cbase + c < n_cand ? cand.v4(n, cbase + c, l16) : make_float4(0.f, 0.f, 0.f, 0.f);
      }
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
  // (the loop's last barrier has made onum, oden, den, wq and wc visible)
  if (kReadout && tid < kDim) {
    float num = 0.0f, den = eps;
#pragma unroll
    for (int r = 0; r < kWaves; ++r) {
      num += kLdsOut ? sh.rnum[r][tid] : sh.onum[r][tid];
      den += kLdsOut ? sh.rden[r] : sh.oden[r];
    }
    if (MODE == kRead) {
#pragma unroll
      for (int p = 0; p < kPend; ++p) {
        num += sh.wq[p] * sh.pv[p][tid];
        den += sh.wq[p];
      }
    }
    Elem<Tout>::store(o, (size_t)n * kDim + tid, den != 0.0f ? num / den : 0.0f);
  }
  if (MT > 0 && w == kWaves - 1) {
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
        float num[4] = {acc[mt][0][i], acc[mt][1][i], acc[mt][2][i], acc[mt][3][i]};
        if (MODE == kRead) {
#pragma unroll
          for (int p = 0; p < kPend; ++p) {
            const float wgt = sh.wc[c][p];
            const float4 vp = *reinterpret_cast<const float4*>(&sh.pv[p][4 * l16]);
            den += wgt;
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) num[nt] += wgt * comp(vp, nt);
          }
        }
        const float4 vc = vcs[mt][i];
        float err = 0.0f;
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
          const float pred = den != 0.0f ? num[nt] / den : 0.0f;
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
  // the 64 keys, one per lane of one wave, sorted in registers (bitonic
  // network over lane exchanges, no work-group barrier per stage)
  __syncthreads();
  if (w == 0) {
    uint64_t x = sh.keys[lane];
#pragma unroll
    for (int kk = 2; kk <= kMaxCand; kk <<= 1) {
#pragma unroll
      for (int j = kk >> 1; j > 0; j >>= 1) {
        const uint32_t lo = __shfl_xor((uint32_t)x, j, 64);
        const uint32_t hi = __shfl_xor((uint32_t)(x >> 32), j, 64);
        const uint64_t y = ((uint64_t)hi << 32) | lo;
        // descending inside blocks with (lane & kk) == 0, ascending
        // otherwise: the lower lane of a pair keeps the larger key there
        const bool keep_max = ((lane & j) == 0) == ((lane & kk) == 0);
        x = keep_max ? (x > y ? x : y) : (x < y ? x : y);
      }
    }
    sh.keys[lane] = x;
  }
  __syncthreads();
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

template <int MT, int MODE, bool SELECT, typename Tin, typename Tout>
void launch_fused(int N, float* H, float* s, const void* q, const void* k, const void* v, void* o,
                  float eps, const SreArgs& sre, float* pend_k, float* pend_v, int n_pend, hipStream_t st) {
  const CandRows cand{sre.cand_k, sre.cand_v, sre.n_cand};
  hipLaunchKernelGGL((decode_sre_kernel<MT, MODE, SELECT, Tin, Tout, CandRows>), dim3(N, 1), dim3(kThreadsF), 0,
                     st, H, s, static_cast<const Tin*>(q), static_cast<const Tin*>(k), static_cast<const Tin*>(v),
                     static_cast<Tout*>(o), eps, cand, sre.n_cand, sre.top_k, sre.scores, sre.n_cand, sre.sel,
                     sre.sel_k, sre.sel_v, sre.sel_stride ? sre.sel_stride : sre.top_k, pend_k, pend_v, n_pend);
}

template <int MODE, typename Tin, typename Tout>
void launch_mt(int N, float* H, float* s, const void* q, const void* k, const void* v, void* o, float eps,
               const SreArgs* sre, float* pend_k, float* pend_v, int n_pend, hipStream_t st) {
  if (!sre) {
    launch_fused<0, MODE, false, Tin, Tout>(N, H, s, q, k, v, o, eps, SreArgs{}, pend_k, pend_v, n_pend, st);
    return;
  }
  // 16, 32 or 64 candidate rows (rows past n_cand are zero keys, not scored)
  const int mt = (sre->n_cand + 15) / 16;
  if (mt == 1) launch_fused<1, MODE, true, Tin, Tout>(N, H, s, q, k, v, o, eps, *sre, pend_k, pend_v, n_pend, st);
  else if (mt == 2)
    launch_fused<2, MODE, true, Tin, Tout>(N, H, s, q, k, v, o, eps, *sre, pend_k, pend_v, n_pend, st);
  else launch_fused<4, MODE, true, Tin, Tout>(N, H, s, q, k, v, o, eps, *sre, pend_k, pend_v, n_pend, st);
}

template <int MODE>
void launch_dtypes(const DecodeArgs& a, const SreArgs* sre, float* pend_k, float* pend_v, int n_pend,
                   hipStream_t st) {
  if (a.in_bf16) {
    if (a.out_bf16)
      launch_mt<MODE, uint16_t, uint16_t>(a.N, a.H, a.s, a.q, a.k, a.v, a.o, a.eps, sre, pend_k, pend_v, n_pend, st);
    else launch_mt<MODE, uint16_t, float>(a.N, a.H, a.s, a.q, a.k, a.v, a.o, a.eps, sre, pend_k, pend_v, n_pend, st);
  } else {
    if (a.out_bf16)
      launch_mt<MODE, float, uint16_t>(a.N, a.H, a.s, a.q, a.k, a.v, a.o, a.eps, sre, pend_k, pend_v, n_pend, st);
    else launch_mt<MODE, float, float>(a.N, a.H, a.s, a.q, a.k, a.v, a.o, a.eps, sre, pend_k, pend_v, n_pend, st);
  }
}

}  // namespace

bool decode_fused_supported(int dqk, int dv, const SreArgs& sre) {
  return dqk == kDim && dv == kDim && sre.n_cand >= 1 && sre.n_cand <= kMaxCand;
}

hipError_t decode_fused_launch(const DecodeArgs& a, const SreArgs& sre, hipStream_t st) {
  prof_begin(st);
  launch_dtypes<kStep>(a, &sre, nullptr, nullptr, 0, st);
  prof_end(st);
  return hipGetLastError();
}

hipError_t sre_fused_launch(int N, float eps, const float* H, const float* s, const SreArgs& sre,
                            hipStream_t st) {
  prof_begin(st);
  // read-only: the kernel neither loads q, k, v nor writes H, s or o
  launch_mt<kScore, float, float>(N, const_cast<float*>(H), const_cast<float*>(s), nullptr, nullptr, nullptr,
                                  nullptr, eps, &sre, nullptr, nullptr, 0, st);
  prof_end(st);
  return hipGetLastError();
}

int decode_pending_slots() { return kPend; }

hipError_t decode_deferred_launch(const DecodeArgs& a, const SreArgs* sre, float* pend_k, float* pend_v,
                                  int n_pend, hipStream_t st) {
  prof_begin(st);
  // the token that takes the last slot folds the whole list into H and s
  if (n_pend == kPend - 1) launch_dtypes<kFold>(a, sre, pend_k, pend_v, n_pend, st);
  else launch_dtypes<kRead>(a, sre, pend_k, pend_v, n_pend, st);
  prof_end(st);
  return hipGetLastError();
}

hipError_t decode_flush_launch(int N, float* H, float* s, const float* pend_k, const float* pend_v, int n_pend,
                               hipStream_t st) {
  if (n_pend == 0) return hipSuccess;
  launch_fused<0, kFlush, false, float, float>(N, H, s, nullptr, nullptr, nullptr, nullptr, 0.0f, SreArgs{},
                                               const_cast<float*>(pend_k), const_cast<float*>(pend_v), n_pend, st);
  return hipGetLastError();
}

}  // namespace kla
