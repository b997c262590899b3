// Hybrid prefill on the matrix cores (d_qk = d_v = 64, bf16 inputs): the
// LoLA page's three memories ("Metodologia" items 1-3, "Estratégia de
// Inferência" items 1-4) — a sliding window of exact softmax attention, a
// linear state (H, s) under the rank-one PSD lift of the KATA page (§2.2),
// and a sparse cache of the pairs the state recalls worst (self-recall
// error), refreshed every block of `refresh` tokens.
//
// The selection at refresh r scores every candidate (cache r - 1 plus the
// tokens block b_r evicts) against the state S_{r-1} that holds every pair
// rejected before. Only that chain is sequential; everything sized by the
// state is taken off it with one identity: phi(x) . phi(k_j) = (x . k_j)^2,
// so a candidate's sums over S_{r-1} are its sums over an older state
// version S_v plus the closed-form terms (x . k_j)^2 [v_j | 1] of the pairs
// rejected after v. Per refresh the chain runs one launch per head
// (hyb_chain_kernel): the cached candidates carry their sums over S_{r-2}
// from the previous selection and add the pairs refresh r - 1 rejected; the
// new candidates take their sums over a state version two batches old
// (scored off the chain) and add the pairs rejected since; then the scores,
// ranks, the new cache and the rejected list. Every kL refreshes (a batch),
// a second stream of the caller's (or the same stream, in order) runs:
//   fold    : the batch's rejected pairs into (H, s), writing the next state
//             version as three-piece bf16 fragments;
//   score   : the candidates that batch m + 2 will evict, against it;
//   readout : the batch's blocks — window and cache softmax terms and the
//             linear term against the previous state version plus the
//             closed-form terms of the batch's pairs up to the block's
//             refresh — in one launch, and the split partials' combine.
// The host knows every count in advance (they depend only on T, window,
// refresh and cache_size), so nothing is read back.
#include <algorithm>
#include <vector>

#include "kla_device.hpp"
#include "kla_internal.hpp"
#include "mfma_bf16.hpp"

namespace kla {
namespace {

constexpr int kFD = 64;
constexpr int kFPhi = kFD * (kFD + 1) / 2;  // 2080 features
constexpr int kFKS = kFPhi / 32;            // 65 feature k-steps of 32
constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kCandMax = 256;  // candidates per refresh, at most (cache + evicted)
constexpr int kCStride = kCandMax;
constexpr int kPairMax = 128;  // pairs one refresh rejects, at most (refresh <= 128)
constexpr int kL = 4;          // refreshes per batch
constexpr int kRingB = 4;      // batches the cache, carry and rejected rings hold
constexpr int kRing = kL * kRingB;
constexpr int kBaseSlots = 3;  // batches of new-candidate state sums in flight
constexpr int kSZ = 4;         // feature splits of the state sums per (head, candidate block)
constexpr int kScoreCand = 64;
constexpr int kRNS = 4;   // readout splits per (head, query block)
constexpr int kRB = 8;    // blocks per readout launch, at most
constexpr int kHFPieces = 3;

__constant__ PairTable64 kPairs = PairTable64();

__global__ void fill_f32_kernel(float* p, size_t n, float x) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = x;
}
__global__ void fill_i32_kernel(int32_t* p, size_t n, int32_t x) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = x;
}
// row n of ids: 0 .. count - 1 (the cache before the first refresh holds the
// tokens evicted so far, in order)
__global__ void iota_rows_kernel(int32_t* ids, int stride, int count) {
  for (int i = threadIdx.x; i < count; i += blockDim.x) ids[(size_t)blockIdx.x * stride + i] = i;
}
__global__ void copy_rows_kernel(int32_t* dst, int width, const int32_t* src, int src_stride) {
  for (int i = threadIdx.x; i < width; i += blockDim.x)
    dst[(size_t)blockIdx.x * width + i] = src[(size_t)blockIdx.x * src_stride + i];
}

// State fragments: index of (head n, k-step ks, piece pc, n-tile nt, lane) in
// uint4 units. Lane (l16, q4) of k-step ks holds features 32 ks + 4 q4 + j
// and 32 ks + 16 + 4 q4 + j (j < 4) of state column 4 l16 + nt (n-tile 4:
// column 0 is s, the rest zero), as three exact bf16 pieces of the float32
// value.
__device__ __forceinline__ size_t hf_index(int n, int ks, int pc, int nt, int lane) {
  return ((((size_t)n * kFKS + ks) * kHFPieces + pc) * 5 + nt) * 64 + lane;
}

// Rejected lists of several refreshes, each in a slot of the ring
// rej[slot][head][kCStride]; pair g of the concatenation is entry g - (sum of
// the earlier counts) of the set it falls in.
struct PairSets {
  int n;
  int slot[2 * kL];
  int cnt[2 * kL];
};

// Copies the concatenated token ids of `ps` for head n into dst (count
// returned). Every thread of the block calls it.
__device__ __forceinline__ int gather_pair_tokens(const PairSets& ps, const int32_t* __restrict__ rej, int N, int n,
                                                  int32_t* dst) {
  const int nt = blockDim.x;  // read once (it is reloaded after every store otherwise)
  int off = 0;
#pragma unroll
  for (int s = 0; s < 2 * kL; ++s) {
    if (s < ps.n) {
      const int32_t* src = rej + ((size_t)ps.slot[s] * N + n) * kCStride;
      for (int i = threadIdx.x; i < ps.cnt[s]; i += nt) dst[off + i] = src[i];
      off += ps.cnt[s];
    }
  }
  return off;
}

// bf16 value words: b[j] = column (4 l16 + nt) of row j, from rows of four
// columns 4 l16 .. + 3 (uint2 each).
__device__ __forceinline__ bf16x8 value_operand(const uint2 (&vr)[8], int nt) {
  bf16x8 b;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t word = (nt < 2) ? vr[j].x : vr[j].y;
    const uint16_t bits = (nt & 1) ? (uint16_t)(word >> 16) : (uint16_t)(word & 0xFFFF);
    b[j] = __builtin_bit_cast(__bf16, bits);
  }
  return b;
}

// k-slot j of a 32-row step holds row 4 q4 + j (j < 4) or 16 + 4 q4 + j - 4:
// the rows whose products lane (l16, q4) holds in the two 16-row halves of a
// product S^T = K X^T.
__device__ __forceinline__ int kslot_row(int q4, int j) { return j < 4 ? 4 * q4 + j : 16 + 4 * q4 + (j - 4); }

// ---------------------------------------------------------------- the refresh chain

// Closed-form sums of 16 rows x (candidates or queries, B operand xb: row
// l16, dims 32 ks + 8 q4 .. + 7) over pairs [g0, g1) of a token list:
//   num_x += sum_j (x . k_j)^2 v_j,   den_x += sum_j (x . k_j)^2.
// S^T = K_j X^T on bf16 MFMA (exact products, float32 sums), squared in
// float32, split into PIECES exact (3) or 16-bit (2) bf16 pieces for the
// product with V (bf16, exact). acc[nt] lane (l16, q4): rows 4 q4 + i, value
// column 4 l16 + nt; den: lane (l16, q4) holds part of row l16's sum (the
// caller adds over q4). `live` masks rows (their weights are zeroed). The
// next 32-pair step's rows are loaded while the current one is computed
// (always issued, the last step reloaded, so the wait counts stay exact).
template <int PIECES>
__device__ __forceinline__ void closed_form_pairs(const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                                                  size_t base, const int32_t* __restrict__ ptok, int g0, int g1,
                                                  const bf16x8 (&xb)[2], bool live, f32x4 (&acc)[4],
                                                  float& den) {
  const int lane = threadIdx.x & 63;
  const int l16 = lane & 15;
  const int q4 = lane >> 4;
  if (g0 >= g1) return;
  auto load = [&](int j0, uint4 (&ka)[2][2], uint2 (&vr)[8]) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int g = j0 + 16 * h + l16;
      const bool ok = g < g1;
      const size_t row = base + (size_t)(ok ? ptok[g] : ptok[g0]) * kFD;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const uint4 u = *reinterpret_cast<const uint4*>(k + row + 32 * ks + 8 * q4);
        ka[h][ks] = ok ? u : make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int g = j0 + kslot_row(q4, j);
      const bool ok = g < g1;
      const uint2 u = *reinterpret_cast<const uint2*>(v + base + (size_t)(ok ? ptok[g] : ptok[g0]) * kFD + 4 * l16);
      vr[j] = ok ? u : make_uint2(0, 0);
    }
  };
  uint4 ka[2][2];
  uint2 vr[8];
  load(g0, ka, vr);
  for (int j0 = g0; j0 < g1; j0 += 32) {
    uint4 kn[2][2];
    uint2 vn[8];
    load(j0 + 32 < g1 ? j0 + 32 : j0, kn, vn);
    float x[8];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      f32x4 s4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) s4 = mfma16x16x32(__builtin_bit_cast(bf16x8, ka[h][ks]), xb[ks], s4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float wgt = live ? s4[i] * s4[i] : 0.0f;
        den += wgt;
        x[4 * h + i] = wgt;
      }
    }
    if (PIECES == 3) {
      bf16x8 A0, A1, A2;
      split3(x, A0, A1, A2);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const bf16x8 B = value_operand(vr, nt);
        acc[nt] = mfma16x16x32(A0, B, acc[nt]);
        acc[nt] = mfma16x16x32(A1, B, acc[nt]);
        acc[nt] = mfma16x16x32(A2, B, acc[nt]);
      }
    } else {
      bf16x8 A0, A1;
      split2(x, A0, A1);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const bf16x8 B = value_operand(vr, nt);
        acc[nt] = mfma16x16x32(A0, B, acc[nt]);
        acc[nt] = mfma16x16x32(A1, B, acc[nt]);
      }
    }
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) ka[h][ks] = kn[h][ks];
#pragma unroll
    for (int j = 0; j < 8; ++j) vr[j] = vn[j];
  }
}

struct ChainArgs {
  const uint16_t* k;
  const uint16_t* v;
  int T, N;
  float eps;
  int keep;                 // cache_size
  const int32_t* cache_in;  // cache of the previous refresh, [N][kCStride], n_cache entries
  int n_cache;
  const float* carry_in;    // its entries' sums over the state before the previous fold, [N][kCStride][68]
  int ev0, n_ev;            // tokens ev0 .. ev0 + n_ev - 1 are evicted at this refresh
  const float* base;        // new candidate c's sums over an older state version at
  int base_stride;          //   base + (n base_stride + c) 68; NULL: the zero state
  const int32_t* rej;       // rejected-list ring [kRing][N][kCStride]
  PairSets prev;            // pairs of the previous refresh (cached candidates)
  PairSets since;           // pairs rejected after the base's state version (new candidates)
  int32_t* cache_out;
  float* carry_out;
  int32_t* rej_out;
  int32_t* trace;
  size_t trace_row_stride;
  int block, nblocks;
};

constexpr int kChainThreads = 1024;
constexpr int kChainWaves = kChainThreads / 64;
constexpr int kItemsMax = kChainWaves + 1;
constexpr int kRound = 256;          // pairs staged in LDS at a time
constexpr int kRowH = kFD + 8;       // staged row stride (bf16), 144 bytes
struct ChainLds {
  uint16_t pk[kRound][kRowH];        // staged pair keys
  uint16_t pv[kRound][kRowH];        // staged pair values
  float red[kItemsMax][16][68];      // per work item: 16 candidates' numerators (64) and denominator
  int32_t ptok[kPairMax + 2 * kL * kPairMax];  // previous refresh's pairs (padded to 32), then the later ones
  uint64_t keys[kCandMax];
  int32_t tok[kCandMax];
  int32_t kid[kCandMax];
  int32_t rank[kCandMax];
  int32_t pos[kCandMax];
};

// Token ids of the sets of `ps` for head n into dst; every thread of the
// (1024-thread) block issues its loads (at most one per set) before it
// stores any.
__device__ __forceinline__ int chain_gather(const PairSets& ps, const int32_t* __restrict__ rej, int N, int n,
                                            int32_t* dst) {
  static_assert(kChainThreads >= kPairMax, "one entry per thread and set");
  const int tid = threadIdx.x;
  int32_t x[2 * kL];
#pragma unroll
  for (int s = 0; s < 2 * kL; ++s)
    x[s] = (s < ps.n && tid < ps.cnt[s]) ? rej[((size_t)ps.slot[s] * N + n) * kCStride + tid] : 0;
  int off = 0;
#pragma unroll
  for (int s = 0; s < 2 * kL; ++s) {
    if (s < ps.n) {
      if (tid < ps.cnt[s]) dst[off + tid] = x[s];
      off += ps.cnt[s];
    }
  }
  return off;
}

// One refresh of every head (one work-group each): closed-form terms, scores,
// selection. The pair list is the previous refresh's pairs (padded to 32),
// then the pairs rejected after the new candidates' state version; rounds of
// 256 pairs are staged in LDS (keys and values, bf16) and shared by every
// work item. Candidates are cut into tiles of 16 (cached tiles, which take
// the first part of the list, then new ones, which take the second); a work
// item is one tile and a share of its pairs, and the waves take the items in
// turn (new tiles, which have the longer lists, get the spare waves). For a
// 32-pair step, S^T = K_j X^T on bf16 MFMA (exact products, float32 sums),
// the squares are split into three exact bf16 pieces for the product with V
// (bf16), so the numerators are float32 sums of exact products, as in a fold.
// Then four threads per candidate add its item partials to its carried or
// state sums,
//   score_c = || num_c / (den_c + eps) - v_c ||^2   (prediction 0 when the
//   denominator is 0),
// and each candidate's rank is the number of larger (score, token id) keys
// (wave ballots); the keep best go to the cache in ascending token order
// (their place is the number of kept tokens with a lower id) with their
// sums, the rest in rank order to the rejected list — the order the sort of
// the generic form gives.
__global__ __launch_bounds__(kChainThreads) void hyb_chain_kernel(const ChainArgs a) {
  __shared__ __align__(16) ChainLds sh;
  const int n = blockIdx.x;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l16 = lane & 15;
  const int q4 = lane >> 4;
  const int n_cand = a.n_cache + a.n_ev;
  const size_t base = (size_t)n * a.T * kFD;
  {
    const int32_t* cin = a.cache_in + (size_t)n * kCStride;
    if (tid < n_cand) sh.tok[tid] = tid < a.n_cache ? cin[tid] : a.ev0 + (tid - a.n_cache);
  }
  const int np_prev = chain_gather(a.prev, a.rej, a.N, n, sh.ptok);
  const int p0 = (np_prev + 31) & ~31;  // first pair of the new candidates' list
  if (tid >= np_prev && tid < p0) sh.ptok[tid] = 0;  // padding: a valid token, never counted
  const int np_since = chain_gather(a.since, a.rej, a.N, n, sh.ptok + p0);
  const int np_all = p0 + np_since;
  // four adjacent threads per candidate (after the closed-form terms):
  // quarter qd of its columns; its carried or state sums are loaded now
  const int c = tid >> 2;
  const int qd = tid & 3;
  const bool live = c < n_cand;
  float4 pre[4] = {make_float4(0.f, 0.f, 0.f, 0.f), make_float4(0.f, 0.f, 0.f, 0.f),
                   make_float4(0.f, 0.f, 0.f, 0.f), make_float4(0.f, 0.f, 0.f, 0.f)};
  float pre_den = 0.0f;
  {
    const float* row = nullptr;
    if (live && c < a.n_cache) row = a.carry_in + ((size_t)n * kCStride + c) * 68;
    if (live && c >= a.n_cache && a.base) row = a.base + ((size_t)n * a.base_stride + (c - a.n_cache)) * 68;
    if (row) {
#pragma unroll
      for (int j = 0; j < 4; ++j) pre[j] = reinterpret_cast<const float4*>(row + 16 * qd)[j];
      pre_den = row[64];
    }
  }
  __syncthreads();

  const int ncT = (a.n_cache + 15) / 16;
  const int neT = (a.n_ev + 15) / 16;
  const int P = neT > 0 ? max(1, (kChainWaves - ncT) / neT) : 1;
  const int n_items = ncT + neT * P;
  // work item of this wave in slot s: tile, pair range [g0, g1) of the list
  auto item = [&](int it, int& c0, int& c_end, int& g0, int& g1) {
    const bool cached = it < ncT;
    const int tile = cached ? it : (it - ncT) / P;
    const int part = cached ? 0 : (it - ncT) % P;
    const int parts = cached ? 1 : P;
    c0 = cached ? 16 * tile : a.n_cache + 16 * tile;
    c_end = cached ? a.n_cache : n_cand;
    const int np = cached ? np_prev : np_since;
    const int off = cached ? 0 : p0;
    const int nch = (np + 31) / 32;
    g0 = off + 32 * (part * nch / parts);
    g1 = off + min(np, 32 * ((part + 1) * nch / parts));
  };
  const int n_rounds = (np_all + kRound - 1) / kRound;
  for (int slot = 0; slot * kChainWaves < n_items; ++slot) {
    const int it = w + slot * kChainWaves;
    int c0 = 0, c_end = 0, g0 = 0, g1 = 0;
    if (it < n_items) item(it, c0, c_end, g0, g1);
    const int cc = c0 + l16;
    const bool rl = it < n_items && cc < c_end;
    bf16x8 xb[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const uint4 u =
          rl ? *reinterpret_cast<const uint4*>(a.k + base + (size_t)sh.tok[cc] * kFD + 32 * ks + 8 * q4)
             : make_uint4(0, 0, 0, 0);
      xb[ks] = __builtin_bit_cast(bf16x8, u);
    }
    f32x4 acc[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float den = 0.0f;
    for (int rd = 0; rd < n_rounds; ++rd) {
      const int r0 = rd * kRound;
      // stage pairs r0 .. r0 + 255: four threads per pair, 32 bytes of its key and value each
      {
        const int r = tid >> 2, part = tid & 3;
        const int g = r0 + r;
        const int tk = g < np_all ? sh.ptok[g] : 0;
        const uint4* kp = reinterpret_cast<const uint4*>(a.k + base + (size_t)tk * kFD + 16 * part);
        const uint4* vp = reinterpret_cast<const uint4*>(a.v + base + (size_t)tk * kFD + 16 * part);
        const uint4 k0 = kp[0], k1 = kp[1], v0 = vp[0], v1 = vp[1];
        __syncthreads();  // the previous round's reads are done
        uint4* kd = reinterpret_cast<uint4*>(&sh.pk[r][16 * part]);
        uint4* vd = reinterpret_cast<uint4*>(&sh.pv[r][16 * part]);
        kd[0] = k0;
        kd[1] = k1;
        vd[0] = v0;
        vd[1] = v1;
      }
      __syncthreads();
      const int a0 = max(g0, r0), a1 = min(g1, r0 + kRound);
      for (int j0 = a0; j0 < a1; j0 += 32) {
        const int rj = j0 - r0;
        float x[8];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const bool ok = j0 + 16 * h + l16 < a1;
          f32x4 s4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            uint4 u = *reinterpret_cast<const uint4*>(&sh.pk[rj + 16 * h + l16][32 * ks + 8 * q4]);
            if (!ok) u = make_uint4(0, 0, 0, 0);
            s4 = mfma16x16x32(__builtin_bit_cast(bf16x8, u), xb[ks], s4);
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float wgt = rl ? s4[i] * s4[i] : 0.0f;
            den += wgt;
            x[4 * h + i] = wgt;
          }
        }
        uint2 vr[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int kr = kslot_row(q4, j);
          uint2 u = *reinterpret_cast<const uint2*>(&sh.pv[rj + kr][4 * l16]);
          vr[j] = j0 + kr < a1 ? u : make_uint2(0, 0);
        }
        bf16x8 A0, A1, A2;
        split3(x, A0, A1, A2);
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
          const bf16x8 B = value_operand(vr, nt);
          acc[nt] = mfma16x16x32(A0, B, acc[nt]);
          acc[nt] = mfma16x16x32(A1, B, acc[nt]);
          acc[nt] = mfma16x16x32(A2, B, acc[nt]);
        }
      }
    }
    if (it < n_items) {
      den += __shfl_xor(den, 16, 64);
      den += __shfl_xor(den, 32, 64);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) sh.red[it][4 * q4 + i][4 * l16 + nt] = acc[nt][i];
      if (q4 == 0) sh.red[it][l16][64] = den;
    }
  }
  __syncthreads();

  float num[16];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    num[4 * j] = pre[j].x;
    num[4 * j + 1] = pre[j].y;
    num[4 * j + 2] = pre[j].z;
    num[4 * j + 3] = pre[j].w;
  }
  float dsum = pre_den;
  float err = 0.0f;
  if (live) {
    const uint4* vp = reinterpret_cast<const uint4*>(a.v + base + (size_t)sh.tok[c] * kFD + 16 * qd);
    const uint4 va = vp[0], vb = vp[1];
    auto add = [&](const float* pc) {
#pragma unroll
      for (int j = 0; j < 16; ++j) num[j] += pc[16 * qd + j];
      dsum += pc[64];
    };
    if (c < a.n_cache) {
      add(&sh.red[c / 16][c % 16][0]);
    } else {
      const int e = c - a.n_cache;
      for (int p = 0; p < P; ++p) add(&sh.red[ncT + (e / 16) * P + p][e % 16][0]);
    }
    const float dn = dsum + a.eps;
    const uint32_t vw[8] = {va.x, va.y, va.z, va.w, vb.x, vb.y, vb.z, vb.w};
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const float vj = __uint_as_float((j & 1) ? (vw[j >> 1] & 0xFFFF0000u) : (vw[j >> 1] << 16));
      const float pred = dn != 0.0f ? num[j] / dn : 0.0f;
      const float d = pred - vj;
      err += d * d;
    }
  }
  err += __shfl_xor(err, 1, 64);
  err += __shfl_xor(err, 2, 64);
  if (qd == 0 && live) sh.keys[c] = topk_key(err, (uint32_t)sh.tok[c]);
  __syncthreads();
  // ranks: wave w takes candidates w, w + 16, ...; lane l holds keys l, 64 + l, ...
  {
    uint64_t kk[kCandMax / 64];
#pragma unroll
    for (int i = 0; i < kCandMax / 64; ++i) kk[i] = 64 * i + lane < n_cand ? sh.keys[64 * i + lane] : 0ull;
    for (int cw = w; cw < n_cand; cw += kChainWaves) {
      // key cw from the lane that holds it
      uint64_t kx = kk[0];
#pragma unroll
      for (int i = 1; i < kCandMax / 64; ++i)
        if ((cw >> 6) == i) kx = kk[i];
      const uint32_t khi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(kx >> 32), cw & 63);
      const uint32_t klo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)kx, cw & 63);
      const uint64_t key = ((uint64_t)khi << 32) | (uint64_t)klo;
      int rk = 0;
#pragma unroll
      for (int i = 0; i < kCandMax / 64; ++i) rk += __popcll(__ballot(kk[i] > key));
      if (lane == 0) {
        sh.rank[cw] = rk;
        sh.kid[cw] = rk < a.keep ? sh.tok[cw] : 0x7FFFFFFF;
      }
    }
  }
  __syncthreads();
  // places of the kept tokens: the number of kept tokens with a lower id
  {
    int32_t ki[kCandMax / 64];
#pragma unroll
    for (int i = 0; i < kCandMax / 64; ++i) ki[i] = 64 * i + lane < n_cand ? sh.kid[64 * i + lane] : 0x7FFFFFFF;
    for (int cw = w; cw < n_cand; cw += kChainWaves) {
      int32_t kx = ki[0];
#pragma unroll
      for (int i = 1; i < kCandMax / 64; ++i)
        if ((cw >> 6) == i) kx = ki[i];
      const int32_t id = __builtin_amdgcn_readlane(kx, cw & 63);
      int ps = 0;
#pragma unroll
      for (int i = 0; i < kCandMax / 64; ++i) ps += __popcll(__ballot(ki[i] < id));
      if (lane == 0) sh.pos[cw] = ps;
    }
  }
  __syncthreads();
  if (!live) return;
  const int rank = sh.rank[c];
  if (rank < a.keep) {
    const int pos = sh.pos[c];
    float* co = a.carry_out + ((size_t)n * kCStride + pos) * 68;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      *reinterpret_cast<float4*>(co + 16 * qd + 4 * j) =
          make_float4(num[4 * j], num[4 * j + 1], num[4 * j + 2], num[4 * j + 3]);
    if (qd == 0) {
      co[64] = dsum;
      a.cache_out[(size_t)n * kCStride + pos] = sh.tok[c];
      if (a.trace) a.trace[((size_t)n * a.nblocks + a.block) * a.trace_row_stride + pos] = sh.tok[c];
    }
  } else if (qd == 0) {
    a.rej_out[(size_t)n * kCStride + rank - a.keep] = sh.tok[c];
  }
}

// ---------------------------------------------------------------- fold (off the chain)

constexpr int kFoldRows = 128;  // pairs staged at a time
struct FoldLds {
  uint16_t kt[kFD][kFoldRows + 8];  // staged keys, transposed (bf16)
  uint16_t vt[kFD][kFoldRows + 8];  // staged values, transposed
  int32_t tok[kL * kPairMax];       // the batch's pairs, set after set
};
constexpr int kFoldWGs = (kFKS + kWaves - 1) / kWaves;  // work-groups per head, one k-step per wave

// Work-group (bx, n) of the fold: H += sum_j phi(k_j) v_j^T, s += sum_j phi(k_j)
// over the pairs of `sets`, for k-step 4 bx + w of head n. Each wave's
// accumulators are seeded with the stored float32 state, take the pairs 128
// at a time (staged in LDS, two threads per row), and go back to H, s and,
// as three exact bf16 pieces, to the fragments of the next state version.
// Feature products are float32 (from bf16 keys), split exactly into three
// bf16 pieces, and v is bf16, so every MFMA product is exact and the sums
// are float32.
__device__ __forceinline__ void fold_block(FoldLds& sh, int bx, int n, float* __restrict__ H,
                                           float* __restrict__ s, uint4* __restrict__ HF,
                                           const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, int T,
                                           const int32_t* __restrict__ rej, int N, const PairSets& sets) {
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l16 = lane & 15;
  const int q4 = lane >> 4;
  const int ks = bx * kWaves + w;
  const bool act = ks < kFKS;
  const int total = gather_pair_tokens(sets, rej, N, n, sh.tok);
  float* Hn = H + (size_t)n * kFPhi * kFD;
  float* sn = s + (size_t)n * kFPhi;
  f32x4 acc[2][5];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int f0 = 32 * ks + 16 * t;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float4 h = make_float4(0.f, 0.f, 0.f, 0.f);
      float sv = 0.0f;
      if (act) {
        h = *reinterpret_cast<const float4*>(Hn + (size_t)(f0 + 4 * q4 + i) * kFD + 4 * l16);
        if (l16 == 0) sv = sn[f0 + 4 * q4 + i];
      }
      acc[t][0][i] = h.x;
      acc[t][1][i] = h.y;
      acc[t][2][i] = h.z;
      acc[t][3][i] = h.w;
      acc[t][4][i] = sv;
    }
  }
  bf16x8 ones;
#pragma unroll
  for (int j = 0; j < 8; ++j) ones[j] = (__bf16)(l16 == 0 ? 1.0f : 0.0f);
  // this lane's two feature rows (A operands) and their factors
  int fa[2], fb[2];
  float wgt[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const uint16_t ab = act ? kPairs.ab[32 * ks + 16 * t + l16] : 0;
    fa[t] = ab & 0xFF;
    fb[t] = ab >> 8;
    wgt[t] = fa[t] == fb[t] ? 1.0f : kSqrt2;
  }
  __syncthreads();
  for (int r0 = 0; r0 < total; r0 += kFoldRows) {
    const int R = min(kFoldRows, total - r0);
    // row r of the round, half hf of its key and value (zeros past the count)
    {
      const int r = tid >> 1, hf = tid & 1;
      const bool ok = r < R;
      const size_t row = ((size_t)n * T + (ok ? sh.tok[min(r0 + r, kL * kPairMax - 1)] : 0)) * kFD + 32 * hf;
      uint4 ku[4], vu[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        ku[j] = ok ? reinterpret_cast<const uint4*>(k + row)[j] : make_uint4(0, 0, 0, 0);
        vu[j] = ok ? reinterpret_cast<const uint4*>(v + row)[j] : make_uint4(0, 0, 0, 0);
      }
      if (r0 > 0) __syncthreads();  // the previous round's reads are done
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t kw[4] = {ku[j].x, ku[j].y, ku[j].z, ku[j].w};
        const uint32_t vw[4] = {vu[j].x, vu[j].y, vu[j].z, vu[j].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int d = 32 * hf + 8 * j + 2 * e;
          sh.kt[d][r] = (uint16_t)(kw[e] & 0xFFFF);
          sh.kt[d + 1][r] = (uint16_t)(kw[e] >> 16);
          sh.vt[d][r] = (uint16_t)(vw[e] & 0xFFFF);
          sh.vt[d + 1][r] = (uint16_t)(vw[e] >> 16);
        }
      }
    }
    __syncthreads();
    if (act) {
      const int KS = (R + 31) / 32;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        for (int kk = 0; kk < KS; ++kk) {
          const uint4 ua = *reinterpret_cast<const uint4*>(&sh.kt[fa[t]][32 * kk + 8 * q4]);
          const uint4 ub = *reinterpret_cast<const uint4*>(&sh.kt[fb[t]][32 * kk + 8 * q4]);
          const uint32_t wa[4] = {ua.x, ua.y, ua.z, ua.w}, wb[4] = {ub.x, ub.y, ub.z, ub.w};
          float p[8];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            p[2 * e] = __uint_as_float(wa[e] << 16) * __uint_as_float(wb[e] << 16) * wgt[t];
            p[2 * e + 1] = __uint_as_float(wa[e] & 0xFFFF0000u) * __uint_as_float(wb[e] & 0xFFFF0000u) * wgt[t];
          }
          bf16x8 A0, A1, A2;
          split3(p, A0, A1, A2);
#pragma unroll
          for (int nt = 0; nt < 4; ++nt) {
            // value column 4 l16 + nt of the 8 pairs 32 kk + 8 q4 + j
            const bf16x8 B = *reinterpret_cast<const bf16x8*>(&sh.vt[4 * l16 + nt][32 * kk + 8 * q4]);
            acc[t][nt] = mfma16x16x32(A0, B, acc[t][nt]);
            acc[t][nt] = mfma16x16x32(A1, B, acc[t][nt]);
            acc[t][nt] = mfma16x16x32(A2, B, acc[t][nt]);
          }
          acc[t][4] = mfma16x16x32(A0, ones, acc[t][4]);
          acc[t][4] = mfma16x16x32(A1, ones, acc[t][4]);
          acc[t][4] = mfma16x16x32(A2, ones, acc[t][4]);
        }
      }
    }
  }
  if (!act) return;
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
#pragma unroll
  for (int nt = 0; nt < 5; ++nt) {
    const float x[8] = {acc[0][nt][0], acc[0][nt][1], acc[0][nt][2], acc[0][nt][3],
                        acc[1][nt][0], acc[1][nt][1], acc[1][nt][2], acc[1][nt][3]};
    bf16x8 p0, p1, p2;
    split3(x, p0, p1, p2);
    HF[hf_index(n, ks, 0, nt, lane)] = __builtin_bit_cast(uint4, p0);
    HF[hf_index(n, ks, 1, nt, lane)] = __builtin_bit_cast(uint4, p1);
    HF[hf_index(n, ks, 2, nt, lane)] = __builtin_bit_cast(uint4, p2);
  }
}

// ---------------------------------------------------------------- state sums of future candidates (off the chain)

// Evicted tokens of the refreshes of one batch.
struct EvictBatch {
  int nr;
  int ev0[kL];
  int n_ev[kL];
};

struct ScoreLds {
  uint16_t tab[kFPhi];
  float den[kWaves][kScoreCand];
  union {
    float ck[kScoreCand][kFD + 1];  // candidate keys (float32), padded rows
    float4 red[4][4][64];           // numerator partials, accumulator layout
  };
};

// Work-group (by * kSZ + bz, refresh i of the batch, head n): the sums of
// candidates 64 by .. + 63 of refresh i (tokens ev0_i + c) over feature
// split bz of a state version (LoLA page, self-recall error):
//   num_c = sum_f phi_f(k_c) H_f,   den_c = sum_f phi_f(k_c) s_f,
// to part[((n kSZ + bz) pstride + i evs + c) 68 + {0..63, 64}]. Wave w takes
// k-steps bz 65 / kSZ + w, + 4, ...; the B operands are the version's
// fragments (three exact pieces h0 + h1 + h2), the candidate features, in
// the fragments' feature order, are split into two pieces and the product is
// p0 (h0 + h1 + h2) + p1 h0 in float32 (dropped terms below 2^-16
// relative). Denominators stay in float32 on the vector units, with s read
// back exactly from its three pieces in n-tile 4.
__global__ __launch_bounds__(kThreads, 2) void hyb_state_sums_kernel(const uint4* __restrict__ HF,
                                                                     const uint16_t* __restrict__ k, int T,
                                                                     const EvictBatch eb, int evs,
                                                                     float* __restrict__ part) {
  __shared__ __align__(16) ScoreLds sh;
  const int n = blockIdx.z;
  const int i = blockIdx.y;
  const int by = blockIdx.x / kSZ;
  const int bz = blockIdx.x % kSZ;
  int ev0 = eb.ev0[0], n_cand = eb.n_ev[0];
#pragma unroll
  for (int u = 1; u < kL; ++u)
    if (i == u) {
      ev0 = eb.ev0[u];
      n_cand = eb.n_ev[u];
    }
  const int cbase = kScoreCand * by;
  if (i >= eb.nr || cbase >= n_cand) return;
  const int pstride = kL * evs;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l16 = lane & 15;
  const int q4 = lane >> 4;
  const int tz0 = (bz * kFKS) / kSZ;
  const int tz1 = ((bz + 1) * kFKS) / kSZ;

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
  load_b(min(tz0 + w, kFKS - 1), bf, sv);

  // candidate keys: four threads per candidate, 16 dimensions each
  {
    const int c = tid >> 2;
    const int qd = tid & 3;
    float x[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) x[j] = 0.0f;
    if (cbase + c < n_cand) {
      const uint4* kp =
          reinterpret_cast<const uint4*>(k + ((size_t)n * T + ev0 + cbase + c) * kFD + 16 * qd);
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
  for (int t = tid; t < kFPhi / 8; t += kThreads)
    reinterpret_cast<uint4*>(sh.tab)[t] = reinterpret_cast<const uint4*>(kPairs.ab)[t];
  __syncthreads();

  f32x4 acc[4][4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float dacc[4] = {0.f, 0.f, 0.f, 0.f};

#pragma unroll 1
  for (int ks = tz0 + w; ks < tz1; ks += kWaves) {
    uint4 bn[3][4];
    uint4 svn[3];
    const bool more = ks + kWaves < tz1;
    if (more) load_b(ks + kWaves, bn, svn);
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
      wt[j] = pa[j] == pb[j] ? 1.0f : kSqrt2;
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
      split2(p, A0, A1);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        acc[mt][nt] = mfma16x16x32(A0, B[0][nt], acc[mt][nt]);
        acc[mt][nt] = mfma16x16x32(A0, B[1][nt], acc[mt][nt]);
        acc[mt][nt] = mfma16x16x32(A0, B[2][nt], acc[mt][nt]);
        acc[mt][nt] = mfma16x16x32(A1, B[0][nt], acc[mt][nt]);
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
  for (int r = 0; r < kWaves; ++r) {
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
          if (r + 1 < kWaves) sh.red[mt][nt][lane] = make_float4(x[0], x[1], x[2], x[3]);
        }
    }
  }
  if (w == kWaves - 1) {
    // lane (l16, q4) holds candidates 16 mt + 4 q4 + i at state columns 4 l16 + nt
    float* pz = part + (((size_t)n * kSZ + bz) * pstride + (size_t)i * evs) * 68;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int c = 16 * mt + 4 * q4 + ii;
        if (cbase + c < n_cand) {
          float* pc = pz + (size_t)(cbase + c) * 68;
          *reinterpret_cast<float4*>(pc + 4 * l16) =
              make_float4(acc[mt][0][ii], acc[mt][1][ii], acc[mt][2][ii], acc[mt][3][ii]);
          if (l16 == 0) {
            float den = 0.0f;
#pragma unroll
            for (int r = 0; r < kWaves; ++r) den += sh.den[r][c];
            pc[64] = den;
          }
        }
      }
    }
  }
}

// out[n][c] = sum_z part[n][z][c] for c < count (68 floats each): the state
// sums of a batch's new candidates, one row per candidate for the chain.
__global__ __launch_bounds__(kThreads) void hyb_sum_splits_kernel(const float* __restrict__ part, int pstride,
                                                                  float* __restrict__ out, int count) {
  const int n = blockIdx.y;
  const int i = blockIdx.x * kThreads + threadIdx.x;  // (candidate, float4)
  if (i >= count * 17) return;
  const int c = i / 17, q = i % 17;
  float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int z = 0; z < kSZ; ++z) {
    const float4 y = reinterpret_cast<const float4*>(part + (((size_t)n * kSZ + z) * pstride + c) * 68)[q];
    x.x += y.x;
    x.y += y.y;
    x.z += y.z;
    x.w += y.w;
  }
  reinterpret_cast<float4*>(out + ((size_t)n * pstride + c) * 68)[q] = x;
}

// ---------------------------------------------------------------- readout (off the chain)
//
// A launch reads out up to kRB blocks of `refresh` tokens with two kernels,
// joined by a third. For query t of block z:
//   keys   (work-group (query block, head, kRNS z + sp)): the softmax terms
//          over split sp's share of the block's keys (cache entries, then
//          the window [f, t]) and of the closed-form pairs (those rejected
//          after the state version, up to the block's refresh); writes
//          num_sp, den_sp scaled by e^-m_sp, and m_sp, to xp;
//   state  (work-group (query block and k-step range g, head, z)):
//          phi(q)^T [H | s] over range g's feature k-steps of the state
//          version, unscaled, to lp;
//   combine: m = max m_sp, o = (sum e^(m_sp - m) num_sp + e^-m sum_g lin_g)
//          / (sum e^(m_sp - m) den_sp + e^-m (sum_g lin_g,den + eps)).
// The keys kernel: wave w owns queries t0 + 16 w .. + 15. Scores come from
// S^T = K Q^T on bf16 MFMA (exact products, float32 sums): lane (l16, q4)
// holds the scores of query l16 against keys 4 q4 + i of each 16-key half.
// One pass over the keys keeps each query's running maximum m (clamped at
// 0, since the joint normalisation divides the linear terms by e^m too),
// rescales what it has accumulated when m grows, and adds P = e^(tau s - m)
// in two bf16 pieces times [V | 1]; the closed-form pairs add
// (q . k_j)^2 [v_j | 1] (weights in two bf16 pieces), scaled by e^-m.
constexpr int kRW = 4;         // waves (16 queries each) per work-group
constexpr int kRT = 64 * kRW;  // threads
constexpr int kRQ = 16 * kRW;  // queries per work-group
constexpr int kRK = 32;        // keys per tile
constexpr int kPT = 2;         // key tiles per iteration (and in flight)
constexpr int kSR = 4;         // k-step ranges of the state term

struct ReadoutBlocks {
  int nb;
  int t_begin[kRB], t_end[kRB], f[kRB], n_cache[kRB];
  int npairs[kRB];  // closed-form pairs: a prefix of the launch's pair sets
  int qoff[kRB];    // first row of the block in xp and lp
  const int32_t* cache[kRB];
};

__device__ __forceinline__ void readout_keys_block(int32_t* ptok, int qblk, int n, int z, int sp,
                                                   const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                                   const uint16_t* __restrict__ v, int T, const ReadoutBlocks& rb,
                                                   const PairSets& cf, const int32_t* __restrict__ rej, int N,
                                                   float scale, float* __restrict__ xp, int xq) {
  if (z >= rb.nb) return;
  const int t_begin = rb.t_begin[z], t_end = rb.t_end[z], f = rb.f[z], n_cache = rb.n_cache[z],
            ncf = rb.npairs[z], qoff = rb.qoff[z];
  const int32_t* cache = rb.cache[z];
  const int t0 = t_begin + kRQ * qblk;
  if (t0 >= t_end) return;
  const int tq_end = min(t_end, t0 + kRQ);  // queries [t0, tq_end)
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l16 = lane & 15;
  const int q4 = lane >> 4;
  const int tw = t0 + 16 * w;  // this wave's first query
  const int my_t = tw + l16;   // query of lane (scores layout)
  const size_t base = (size_t)n * T * kFD;
  const int32_t* cn = cache + (size_t)n * kCStride;
  // keys: cache, then window tokens f .. tq_end - 1
  const int n_keys = n_cache + (tq_end - f);
  if (ncf > 0) gather_pair_tokens(cf, rej, N, n, ptok);
  // Q^T as the B operand of S^T = K Q^T: lane (l16 = query, q4) holds dims 8 q4 .. + 7 (+ 32 ks)
  bf16x8 qb[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    uint4 u = make_uint4(0, 0, 0, 0);
    if (my_t < tq_end) u = *reinterpret_cast<const uint4*>(q + base + (size_t)my_t * kFD + 32 * ks + 8 * q4);
    qb[ks] = __builtin_bit_cast(bf16x8, u);
  }
  if (ncf > 0) __syncthreads();

  auto key_token = [&](int j) { return j < n_cache ? cn[j] : f + (j - n_cache); };
  // this split's keys, cut to the ones any query of the wave sees
  const int span = (((n_keys + kRNS - 1) / kRNS) + kRK - 1) / kRK * kRK;
  const int kbeg = min(n_keys, sp * span);
  const int wave_keys = max(kbeg, min(min(n_keys, kbeg + span), n_cache + (min(tq_end, tw + 16) - f)));

  // key fragments of tile j0: ka[h][ks] = key j0 + 16 h + l16, dims 32 ks + 8 q4 .. + 7
  auto load_k = [&](int j0, uint4 (&ka)[2][2]) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int j = j0 + 16 * h + l16;
      const bool ok = j < wave_keys;
      const size_t row = base + (size_t)(ok ? key_token(j) : 0) * kFD;
      // loaded whatever ok is (row 0 of the head otherwise) and selected
      // after, so the tile's loads carry no branch and issue together
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const uint4 x = *reinterpret_cast<const uint4*>(k + row + 32 * ks + 8 * q4);
        ka[h][ks] = ok ? x : make_uint4(0, 0, 0, 0);
      }
    }
  };
  // value rows of the 8 keys of this lane's k-slots, columns 4 l16 .. + 3
  // (the same unconditional loads)
  auto load_v = [&](int j0, uint2 (&vr)[8]) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int kj = j0 + kslot_row(q4, j);
      const bool ok = kj < wave_keys;
      const uint2 x = *reinterpret_cast<const uint2*>(v + base + (size_t)(ok ? key_token(kj) : 0) * kFD + 4 * l16);
      vr[j] = ok ? x : make_uint2(0, 0);
    }
  };
  auto scores = [&](int j0, const uint4 (&ka)[2][2], float (&sc)[2][4]) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) c = mfma16x16x32(__builtin_bit_cast(bf16x8, ka[h][ks]), qb[ks], c);
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

  // ---- one pass over the split's keys (kPT tiles per iteration, the next kPT
  // in flight) with a running per-query maximum m (never below 0): a tile that
  // raises it rescales the accumulated P [V | 1] by e^(m_old - m_new), then
  // adds P = e^(tau s - m) (two bf16 pieces) times [V | 1]
  bf16x8 ones;
#pragma unroll
  for (int j = 0; j < 8; ++j) ones[j] = (__bf16)(l16 == 0 ? 1.0f : 0.0f);
  f32x4 acc[5];
#pragma unroll
  for (int nt = 0; nt < 5; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float mx = 0.0f;  // lane (l16, q4): query l16's running maximum
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
        float tm = mx;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int i = 0; i < 4; ++i) tm = fmaxf(tm, sc[h][i]);
        tm = fmaxf(tm, __shfl_xor(tm, 16, 64));
        tm = fmaxf(tm, __shfl_xor(tm, 32, 64));
        const float alpha = __expf(mx - tm);
        mx = tm;
        // accumulator rows 4 q4 + i are queries 4 q4 + i: their factors sit in lanes 4 q4 + i
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float ai = __shfl(alpha, 4 * q4 + i, 64);
#pragma unroll
          for (int nt = 0; nt < 5; ++nt) acc[nt][i] *= ai;
        }
        float pf[8];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int i = 0; i < 4; ++i) pf[4 * h + i] = __expf(sc[h][i] - mx);
        bf16x8 p0, p1;
        split2(pf, p0, p1);
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
          const bf16x8 b = value_operand(vr[t], nt);
          acc[nt] = mfma16x16x32(p0, b, acc[nt]);
          acc[nt] = mfma16x16x32(p1, b, acc[nt]);
        }
        acc[4] = mfma16x16x32(p0, ones, acc[4]);
        acc[4] = mfma16x16x32(p1, ones, acc[4]);
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

  // ---- closed-form pairs: this split's share, all queries of the wave
  f32x4 cfa[4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) cfa[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float cfd = 0.0f;
  if (ncf > 0) {
    const int cspan = (((ncf + kRNS - 1) / kRNS) + 31) / 32 * 32;
    const int g0 = min(ncf, sp * cspan);
    const int g1 = min(ncf, g0 + cspan);
    closed_form_pairs<2>(k, v, base, ptok, g0, g1, qb, my_t < tq_end, cfa, cfd);
  }
  cfd += __shfl_xor(cfd, 16, 64);
  cfd += __shfl_xor(cfd, 32, 64);

  // ---- partials of this split, scaled by e^-m_sp: numerator, denominator (no eps), m_sp;
  // query 4 q4 + i of the wave (rows of the accumulators) sits in lane 4 q4 + i of mx and cfd
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 16 * w + 4 * q4 + i;
    const float m = __shfl(mx, 4 * q4 + i, 64);
    const float cd = __shfl(cfd, 4 * q4 + i, 64);
    if (t0 + r < tq_end) {
      const float e = __expf(-m);
      float* xr = xp + (((size_t)n * xq + qoff + (t0 + r - t_begin)) * kRNS + sp) * 66;
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) xr[4 * l16 + nt] = acc[nt][i] + e * cfa[nt][i];
      if (l16 == 0) {
        xr[64] = acc[4][i] + e * cd;
        xr[65] = m;
      }
    }
  }
}

// The state term: work-group (query block qb and range g as kSR qb + g, head
// n, block z) takes feature k-steps [g 65 / kSR, (g + 1) 65 / kSR) of the
// state version for the block's 64 queries; wave w takes the range's k-steps
// w, w + 4, ... for all four 16-query tiles (two-piece fragments,
// hi*hi + hi*lo + lo*hi with two-piece phi(q)), and the four partials of a
// tile meet in LDS, one tile at a time. Output column 4 l16 + nt sits in
// n-tile nt of lane (l16, q4), rows 4 q4 + i.
struct StateLds {
  float qf[kRQ][kFD + 1];  // query rows (float32) for phi(q)
  uint16_t tab[kFPhi];     // feature pairs
  float4 red[kRW][5][64];  // one token tile's partials from the four waves
};

__device__ __forceinline__ void readout_state_block(StateLds& sh, int qblk, int g, int n, int z,
                                                    const uint16_t* __restrict__ q, int T,
                                                    const uint4* __restrict__ HF, const ReadoutBlocks& rb,
                                                    float* __restrict__ lp, int xq) {
  if (z >= rb.nb) return;
  const int t_begin = rb.t_begin[z], t_end = rb.t_end[z], qoff = rb.qoff[z];
  const int t0 = t_begin + kRQ * qblk;
  if (t0 >= t_end) return;
  const int tq_end = min(t_end, t0 + kRQ);
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l16 = lane & 15;
  const int q4 = lane >> 4;
  const size_t base = (size_t)n * T * kFD;
  for (int i = tid; i < kFPhi / 8; i += kRT)
    reinterpret_cast<uint4*>(sh.tab)[i] = reinterpret_cast<const uint4*>(kPairs.ab)[i];
  for (int i = tid; i < kRQ * (kFD / 4); i += kRT) {
    const int r = i / (kFD / 4), d4 = i % (kFD / 4);
    uint2 u = make_uint2(0, 0);
    if (t0 + r < tq_end) u = *reinterpret_cast<const uint2*>(q + base + (size_t)(t0 + r) * kFD + 4 * d4);
    sh.qf[r][4 * d4 + 0] = __uint_as_float(u.x << 16);
    sh.qf[r][4 * d4 + 1] = __uint_as_float(u.x & 0xFFFF0000u);
    sh.qf[r][4 * d4 + 2] = __uint_as_float(u.y << 16);
    sh.qf[r][4 * d4 + 3] = __uint_as_float(u.y & 0xFFFF0000u);
  }
  __syncthreads();

  const int k0 = (g * kFKS) / kSR, k1 = ((g + 1) * kFKS) / kSR;
  f32x4 lin[kRW][5];
#pragma unroll
  for (int tt = 0; tt < kRW; ++tt)
#pragma unroll
    for (int nt = 0; nt < 5; ++nt) lin[tt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto load_f = [&](int ks, uint4 (&x)[2][5]) {
#pragma unroll
    for (int pc = 0; pc < 2; ++pc)
#pragma unroll
      for (int nt = 0; nt < 5; ++nt) x[pc][nt] = HF[hf_index(n, min(ks, kFKS - 1), pc, nt, lane)];
  };
  uint4 fr[2][5];
  load_f(k0 + w, fr);
  for (int ks = k0 + w; ks < k1; ks += kRW) {
    uint4 fn[2][5];
    const bool more = ks + kRW < k1;
    if (more) load_f(ks + kRW, fn);
    // features of this lane's k-slots: 32 ks + kslot_row(q4, j)
    int fa[8], fb[8];
    float wg[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint16_t ab = sh.tab[32 * ks + kslot_row(q4, j)];
      fa[j] = ab & 0xFF;
      fb[j] = ab >> 8;
      wg[j] = fa[j] == fb[j] ? 1.0f : kSqrt2;
    }
#pragma unroll
    for (int tt = 0; tt < kRW; ++tt) {
      const float* qrow = sh.qf[16 * tt + l16];
      float p[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) p[j] = qrow[fa[j]] * qrow[fb[j]] * wg[j];
      bf16x8 A0, A1;
      split2(p, A0, A1);
#pragma unroll
      for (int nt = 0; nt < 5; ++nt) {
        const bf16x8 B0 = __builtin_bit_cast(bf16x8, fr[0][nt]);
        const bf16x8 B1 = __builtin_bit_cast(bf16x8, fr[1][nt]);
        lin[tt][nt] = mfma16x16x32(A0, B0, lin[tt][nt]);
        lin[tt][nt] = mfma16x16x32(A0, B1, lin[tt][nt]);
        lin[tt][nt] = mfma16x16x32(A1, B0, lin[tt][nt]);
      }
    }
    if (more) {
#pragma unroll
      for (int pc = 0; pc < 2; ++pc)
#pragma unroll
        for (int nt = 0; nt < 5; ++nt) fr[pc][nt] = fn[pc][nt];
    }
  }
  // token tile tt's four partials meet in LDS; wave tt keeps the sum
  f32x4 ln[5];
#pragma unroll
  for (int tt = 0; tt < kRW; ++tt) {
#pragma unroll
    for (int nt = 0; nt < 5; ++nt)
      sh.red[w][nt][lane] = make_float4(lin[tt][nt][0], lin[tt][nt][1], lin[tt][nt][2], lin[tt][nt][3]);
    __syncthreads();
    if (w == tt) {
#pragma unroll
      for (int nt = 0; nt < 5; ++nt) {
        ln[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int r = 0; r < kRW; ++r) {
          const float4 y = sh.red[r][nt][lane];
          ln[nt][0] += y.x;
          ln[nt][1] += y.y;
          ln[nt][2] += y.z;
          ln[nt][3] += y.w;
        }
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 16 * w + 4 * q4 + i;
    if (t0 + r < tq_end) {
      float* lr = lp + (((size_t)n * xq + qoff + (t0 + r - t_begin)) * kSR + g) * 65;
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) lr[4 * l16 + nt] = ln[nt][i];
      if (l16 == 0) lr[64] = ln[4][i];
    }
  }
}

// Joins the kRNS key partials and the ng state ranges of every block of a launch.
template <typename Tout>
__global__ __launch_bounds__(kThreads) void hyb_readout_combine_kernel(const float* __restrict__ xp,
                                                                     const float* __restrict__ lp, int ng, int xq,
                                                                     const ReadoutBlocks rb, Tout* __restrict__ o,
                                                                     int T, float eps) {
  const int n = blockIdx.y;
  const int z = blockIdx.z;
  if (z >= rb.nb) return;
  const int t_begin = rb.t_begin[z], t_end = rb.t_end[z], qoff = rb.qoff[z];
  const int idx = blockIdx.x * kThreads + threadIdx.x;  // (query, column)
  const int r = idx >> 6, c = idx & 63;
  const int t = t_begin + r;
  if (t >= t_end) return;
  const size_t row = (size_t)n * xq + qoff + r;
  const float* xr = xp + row * kRNS * 66;
  float m = 0.0f;
  for (int sp = 0; sp < kRNS; ++sp) m = fmaxf(m, xr[sp * 66 + 65]);
  float num = 0.0f, den = 0.0f;
  for (int sp = 0; sp < kRNS; ++sp) {
    const float e = __expf(xr[sp * 66 + 65] - m);
    num += e * xr[sp * 66 + c];
    den += e * xr[sp * 66 + 64];
  }
  float lnum = 0.0f, lden = eps;
  const float* lr = lp + row * kSR * 65;
  for (int g = 0; g < ng; ++g) {
    lnum += lr[g * 65 + c];
    lden += lr[g * 65 + 64];
  }
  const float e = __expf(-m);
  num += e * lnum;
  den += e * lden;
  Elem<Tout>::store(o, ((size_t)n * T + t) * kFD + c, den != 0.0f ? num / den : 0.0f);
}

// Launches of the batch work: the fold (work-group (k-step block, head)),
// then the readout key terms (work-group (query block, head, kRNS block +
// split)) and state terms (work-group (kSR query block + range, head,
// block)).
__global__ __launch_bounds__(kThreads) void hyb_fold_kernel(float* __restrict__ H, float* __restrict__ s,
                                                            uint4* __restrict__ HF, const uint16_t* __restrict__ k,
                                                            const uint16_t* __restrict__ v, int T,
                                                            const int32_t* __restrict__ rej, int N,
                                                            const PairSets sets) {
  __shared__ __align__(16) FoldLds sh;
  fold_block(sh, blockIdx.x, blockIdx.y, H, s, HF, k, v, T, rej, N, sets);
}

struct ReadoutArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  int T, N;
  const uint4* HF;  // the state version read; NULL: the zero state
  ReadoutBlocks rb;
  PairSets cf;
  const int32_t* rej;
  float scale;
  float* xp;
  float* lp;
  int xq;
};

__global__ __launch_bounds__(kRT) void hyb_readout_keys_kernel(const ReadoutArgs a) {
  __shared__ int32_t ptok[kL * kPairMax];
  readout_keys_block(ptok, blockIdx.x, blockIdx.y, blockIdx.z / kRNS, blockIdx.z % kRNS, a.q, a.k, a.v, a.T, a.rb,
                     a.cf, a.rej, a.N, a.scale, a.xp, a.xq);
}

__global__ __launch_bounds__(kRT, 2) void hyb_readout_state_kernel(const ReadoutArgs a) {
  __shared__ __align__(16) StateLds sh;
  readout_state_block(sh, blockIdx.x / kSR, blockIdx.x % kSR, blockIdx.y, blockIdx.z, a.q, a.T, a.HF, a.rb, a.lp,
                      a.xq);
}

// ---------------------------------------------------------------- host side

struct Refresh {
  int block, n_cache, ev0, n_ev, n_rej;
};
struct Block {
  int t0, t1, f, n_cache, r;  // r: the refresh that serves it (-1: none yet)
};

struct Plan {
  std::vector<Refresh> R;
  std::vector<Block> B;
  int n_pre = 0;  // cache entries before the first refresh (tokens 0 .. n_pre - 1)
  int evs = 64;   // candidate stride of a refresh in the state sums
};

// The block loop's counts (LoLA page, "Estratégia de Inferência"): at block
// b the window frontier moves to f = max(0, b refresh - window); the tokens
// it passes are appended to the cache while it has room, else they and the
// cache are the candidates of a refresh that keeps cache_size of them.
Plan make_plan(const HybridArgs& a) {
  Plan p;
  const int nblocks = (a.T + a.refresh - 1) / a.refresh;
  int n_cache = 0, f_prev = 0;
  for (int b = 0; b < nblocks; ++b) {
    const int t0 = b * a.refresh;
    const int t1 = std::min(a.T, t0 + a.refresh);
    const int f = std::max(0, t0 - a.window);
    const int n_ev = f - f_prev;
    if (n_ev > 0 && n_cache + n_ev > a.cache_size) {
      p.R.push_back({b, n_cache, f_prev, n_ev, n_cache + n_ev - a.cache_size});
      n_cache = a.cache_size;
    } else if (n_ev > 0) {
      n_cache += n_ev;
    }
    p.B.push_back({t0, t1, f, n_cache, (int)p.R.size() - 1});
    f_prev = f;
  }
  p.n_pre = p.R.empty() ? n_cache : p.R[0].n_cache;
  p.evs = (a.refresh + 63) / 64 * 64;
  return p;
}

struct Ws {
  float* H;
  float* s;
  uint4* HF[2];
  int32_t* cache;  // [kRing + 1][N][kCStride]; slot kRing: before the first refresh
  float* carry;    // [kRing + 1][N][kCStride][68]
  int32_t* rej;    // [kRing][N][kCStride]
  float* part;     // [N][kSZ][kL evs][68]: state sums of a batch's new candidates, by feature split
  float* base;     // [kBaseSlots][N][kL evs][68]: their sums
  float* xp;       // [N][kRB refresh][kRNS][66]
  float* lp;       // [N][kRB refresh][kSR][65]
};

size_t hf_bytes(const HybridArgs& a) { return align_up((size_t)a.N * kFKS * kHFPieces * 5 * 64 * sizeof(uint4)); }
size_t cache_bytes(const HybridArgs& a) { return align_up((size_t)(kRing + 1) * a.N * kCStride * sizeof(int32_t)); }
size_t carry_bytes(const HybridArgs& a) {
  return align_up((size_t)(kRing + 1) * a.N * kCStride * 68 * sizeof(float));
}
size_t rej_bytes(const HybridArgs& a) { return align_up((size_t)kRing * a.N * kCStride * sizeof(int32_t)); }
int evs_of(const HybridArgs& a) { return (a.refresh + 63) / 64 * 64; }
size_t base_slot_floats(const HybridArgs& a) { return (size_t)a.N * kL * evs_of(a) * 68; }
size_t part_bytes(const HybridArgs& a) { return align_up(kSZ * base_slot_floats(a) * sizeof(float)); }
size_t base_bytes(const HybridArgs& a) { return align_up(kBaseSlots * base_slot_floats(a) * sizeof(float)); }
size_t xp_bytes(const HybridArgs& a) { return align_up((size_t)a.N * kRB * a.refresh * kRNS * 66 * sizeof(float)); }
size_t lp_bytes(const HybridArgs& a) { return align_up((size_t)a.N * kRB * a.refresh * kSR * 65 * sizeof(float)); }

Ws carve(const HybridArgs& a, void* ws) {
  char* p = static_cast<char*>(ws);
  auto take = [&](size_t bytes) {
    char* r = p;
    p += bytes;
    return r;
  };
  Ws w;
  w.H = a.HT ? a.HT : reinterpret_cast<float*>(take(align_up((size_t)a.N * kFPhi * kFD * sizeof(float))));
  w.s = a.sT ? a.sT : reinterpret_cast<float*>(take(align_up((size_t)a.N * kFPhi * sizeof(float))));
  for (uint4*& h : w.HF) h = reinterpret_cast<uint4*>(take(hf_bytes(a)));
  w.cache = reinterpret_cast<int32_t*>(take(cache_bytes(a)));
  w.carry = reinterpret_cast<float*>(take(carry_bytes(a)));
  w.rej = reinterpret_cast<int32_t*>(take(rej_bytes(a)));
  w.part = reinterpret_cast<float*>(take(part_bytes(a)));
  w.base = reinterpret_cast<float*>(take(base_bytes(a)));
  w.xp = reinterpret_cast<float*>(take(xp_bytes(a)));
  w.lp = reinterpret_cast<float*>(take(lp_bytes(a)));
  return w;
}

// Events of one call, created at its start and released at its end (a
// pending event is released by the runtime once it completes), so the
// library keeps nothing between calls.
struct CallEvents {
  hipEvent_t ev[6] = {nullptr, nullptr, nullptr, nullptr, nullptr, nullptr};
  hipEvent_t& fork() { return ev[0]; }
  hipEvent_t& join() { return ev[1]; }
  hipEvent_t& chain() { return ev[2]; }
  hipEvent_t& sums(int m) { return ev[3 + m % kBaseSlots]; }
  hipError_t create() {
    for (hipEvent_t& e : ev) {
      const hipError_t r = hipEventCreateWithFlags(&e, hipEventDisableTiming);
      if (r != hipSuccess) return r;
    }
    return hipSuccess;
  }
  ~CallEvents() {
    for (hipEvent_t e : ev)
      if (e) (void)hipEventDestroy(e);
  }
};

// Issue order (the caller's stream `st` runs the chain, `sb` the batch work;
// both are `st` without an auxiliary stream):
//   for each batch m: [st waits for the state sums of batch m (from batch
//   m - 2)] chain launches of batch m; [sb waits for them] fold of batch m
//   (state version m into HF[m % 2]); state sums of batch m + 2's evicted
//   tokens; [event]; readouts of batch m's blocks against version m - 1 and
//   the batch's pairs up to each block's refresh.
// Ring slots: refresh r writes cache / carry / rejected slot r mod kRing.
// Before batch m's chain starts, the batch work of m - 2 has issued its state
// sums, so every readout of batch m - 3 and before is done (sb is in order)
// and the slots batch m rewrites (those of m - 4) are free; the state sums of
// batch m + 2 go to slot (m + 2) mod 3, last read by batch m - 1's chain,
// which the fold of batch m already waited for.
template <typename Tout>
hipError_t enqueue(const HybridArgs& a, void* ws, hipStream_t st, hipStream_t aux) {
  const Plan plan = make_plan(a);
  const Ws w = carve(a, ws);
  const int N = a.N;
  const int nblocks = (int)plan.B.size();
  const int nR = (int)plan.R.size();
  const int M = (nR + kL - 1) / kL;
  const int evs = plan.evs;
  const uint16_t* q = static_cast<const uint16_t*>(a.q);
  const uint16_t* k = static_cast<const uint16_t*>(a.k);
  const uint16_t* v = static_cast<const uint16_t*>(a.v);
  Tout* o = static_cast<Tout*>(a.o);
  const bool two = aux != nullptr && aux != st;
  const hipStream_t sb = two ? aux : st;
  CallEvents ev;
  hipError_t e = hipSuccess;
  if (two && (e = ev.create()) != hipSuccess) return e;
#define KLA_TRY(x)                 \
  do {                             \
    e = (x);                       \
    if (e != hipSuccess) return e; \
  } while (0)
#define KLA_CHECK() KLA_TRY(hipGetLastError())
  auto cache_slot = [&](int r) { return w.cache + (size_t)(r >= 0 ? r % kRing : kRing) * N * kCStride; };
  auto carry_slot = [&](int r) { return w.carry + (size_t)(r >= 0 ? r % kRing : kRing) * N * kCStride * 68; };
  auto rej_slot = [&](int r) { return w.rej + (size_t)(r % kRing) * N * kCStride; };
  auto base_slot = [&](int m) { return w.base + (size_t)(m % kBaseSlots) * base_slot_floats(a); };
  // pair sets of refreshes r0 .. r1 - 1
  auto sets_of = [&](int r0, int r1) {
    PairSets ps{};
    ps.n = std::max(0, r1 - r0);
    for (int i = 0; i < ps.n; ++i) {
      ps.slot[i] = (r0 + i) % kRing;
      ps.cnt[i] = plan.R[r0 + i].n_rej;
    }
    return ps;
  };

  hipLaunchKernelGGL(fill_f32_kernel, dim3(1024), dim3(256), 0, st, w.H, (size_t)N * kFPhi * kFD, 0.0f);
  hipLaunchKernelGGL(fill_f32_kernel, dim3(64), dim3(256), 0, st, w.s, (size_t)N * kFPhi, 0.0f);
  hipLaunchKernelGGL(fill_i32_kernel, dim3(64), dim3(256), 0, st, cache_slot(-1), (size_t)N * kCStride, -1);
  if (plan.n_pre > 0) hipLaunchKernelGGL(iota_rows_kernel, dim3(N), dim3(256), 0, st, cache_slot(-1), kCStride, plan.n_pre);
  hipLaunchKernelGGL(fill_f32_kernel, dim3(256), dim3(256), 0, st, carry_slot(-1), (size_t)N * kCStride * 68, 0.0f);
  if (a.trace && a.cache_size > 0)
    hipLaunchKernelGGL(fill_i32_kernel, dim3(1024), dim3(256), 0, st, a.trace, (size_t)N * nblocks * a.cache_size,
                       -1);
  KLA_CHECK();
  // the side stream starts after everything the caller queued so far
  if (two) {
    KLA_TRY(hipEventRecord(ev.fork(), st));
    KLA_TRY(hipStreamWaitEvent(sb, ev.fork(), 0));
  }
  const hipError_t loop_err = [&]() -> hipError_t {
    hipError_t e;
    // Batch work of batch m (m < 0: the blocks before the first refresh):
    // the fold of its pairs into state version m (m >= 0) and the readouts
    // of blocks [i0, i1) against version m - 1 (the zero state for m < 1)
    // and the batch's pairs up to each block's refresh, in launches of at
    // most kRB blocks; `mid` issues the work that waits for the fold, before
    // the first readouts.
    auto batch_work = [&](int i0, int i1, int m, const auto& mid) -> hipError_t {
      hipError_t e;
      const uint4* HF = m >= 1 ? w.HF[(m - 1) % 2] : nullptr;
      const PairSets cf = m >= 0 ? sets_of(m * kL, std::min(nR, (m + 1) * kL)) : PairSets{};
      bool first = true;
      for (int j0 = i0; first || j0 < i1; j0 += kRB) {
        ReadoutBlocks rb{};
        rb.nb = std::max(0, std::min(kRB, i1 - j0));
        int qmax = 0;
        for (int z = 0; z < rb.nb; ++z) {
          const Block& bl = plan.B[j0 + z];
          rb.t_begin[z] = bl.t0;
          rb.t_end[z] = bl.t1;
          rb.f[z] = bl.f;
          rb.n_cache[z] = bl.n_cache;
          rb.qoff[z] = z * a.refresh;
          rb.cache[z] = cache_slot(bl.r);
          int np = 0;
          if (m >= 0)
            for (int r = m * kL; r <= bl.r; ++r) np += plan.R[r].n_rej;
          rb.npairs[z] = np;
          qmax = std::max(qmax, bl.t1 - bl.t0);
        }
        for (int z = rb.nb; z < kRB; ++z) rb.cache[z] = cache_slot(-1);
        const int nqb = (qmax + kRQ - 1) / kRQ;
        if (first && m >= 0) {
          hipLaunchKernelGGL(hyb_fold_kernel, dim3(kFoldWGs, N), dim3(kThreads), 0, sb, w.H, w.s, w.HF[m % 2], k, v,
                             a.T, w.rej, N, cf);
          KLA_CHECK();
        }
        if (first) KLA_TRY(mid());
        first = false;
        if (rb.nb > 0) {
          ReadoutArgs ra{};
          ra.q = q;
          ra.k = k;
          ra.v = v;
          ra.T = a.T;
          ra.N = N;
          ra.HF = HF;
          ra.rb = rb;
          ra.cf = cf;
          ra.rej = w.rej;
          ra.scale = a.scale;
          ra.xp = w.xp;
          ra.lp = w.lp;
          ra.xq = kRB * a.refresh;
          hipLaunchKernelGGL(hyb_readout_keys_kernel, dim3(nqb, N, kRNS * rb.nb), dim3(kRT), 0, sb, ra);
          if (HF) hipLaunchKernelGGL(hyb_readout_state_kernel, dim3(nqb * kSR, N, rb.nb), dim3(kRT), 0, sb, ra);
        }
        KLA_CHECK();
        if (rb.nb > 0)
          hipLaunchKernelGGL((hyb_readout_combine_kernel<Tout>), dim3((qmax * kFD + kThreads - 1) / kThreads, N, rb.nb),
                             dim3(kThreads), 0, sb, w.xp, w.lp, HF ? kSR : 0, kRB * a.refresh, rb, o, a.T, a.eps);
        KLA_CHECK();
      }
      return hipSuccess;
    };
    // blocks before the first refresh: the zero state
    int i_blk = 0;
    while (i_blk < nblocks && plan.B[i_blk].r < 0) ++i_blk;
    KLA_TRY(batch_work(0, i_blk, -1, [] { return hipSuccess; }));
    for (int m = 0; m < M; ++m) {
      const int r0 = m * kL;
      const int r1 = std::min(nR, r0 + kL);
      if (two && m >= 2) KLA_TRY(hipStreamWaitEvent(st, ev.sums(m - 2), 0));
      for (int r = r0; r < r1; ++r) {
        const Refresh& R = plan.R[r];
        ChainArgs c{};
        c.k = k;
        c.v = v;
        c.T = a.T;
        c.N = N;
        c.eps = a.eps;
        c.keep = a.cache_size;
        c.cache_in = cache_slot(r - 1);
        c.n_cache = R.n_cache;
        c.carry_in = carry_slot(r - 1);
        c.ev0 = R.ev0;
        c.n_ev = R.n_ev;
        c.base = m >= 2 ? base_slot(m) + (size_t)(r - r0) * evs * 68 : nullptr;
        c.base_stride = kL * evs;
        c.rej = w.rej;
        c.prev = r >= 1 ? sets_of(r - 1, r) : PairSets{};
        c.since = sets_of(m >= 2 ? (m - 1) * kL : 0, r);
        c.cache_out = cache_slot(r);
        c.carry_out = carry_slot(r);
        c.rej_out = rej_slot(r);
        c.trace = a.trace;
        c.trace_row_stride = (size_t)a.cache_size;
        c.block = R.block;
        c.nblocks = nblocks;
        prof_begin(st);
        hipLaunchKernelGGL(hyb_chain_kernel, dim3(N), dim3(kChainThreads), 0, st, c);
        prof_end(st);
        KLA_CHECK();
      }
      if (two) {
        KLA_TRY(hipEventRecord(ev.chain(), st));
        KLA_TRY(hipStreamWaitEvent(sb, ev.chain(), 0));
      }
      // after the fold: the state sums of the tokens batch m + 2 evicts
      auto sums = [&]() -> hipError_t {
        hipError_t e;
        if (m + 2 < M) {
          EvictBatch eb{};
          const int s0 = (m + 2) * kL;
          eb.nr = std::min(nR, s0 + kL) - s0;
          int ev_max = 0;
          for (int i = 0; i < eb.nr; ++i) {
            eb.ev0[i] = plan.R[s0 + i].ev0;
            eb.n_ev[i] = plan.R[s0 + i].n_ev;
            ev_max = std::max(ev_max, eb.n_ev[i]);
          }
          hipLaunchKernelGGL(hyb_state_sums_kernel, dim3(((ev_max + kScoreCand - 1) / kScoreCand) * kSZ, eb.nr, N),
                             dim3(kThreads), 0, sb, w.HF[m % 2], k, a.T, eb, evs, w.part);
          hipLaunchKernelGGL(hyb_sum_splits_kernel, dim3((kL * evs * 17 + kThreads - 1) / kThreads, N),
                             dim3(kThreads), 0, sb, w.part, kL * evs, base_slot(m + 2), kL * evs);
          KLA_CHECK();
        }
        if (two) KLA_TRY(hipEventRecord(ev.sums(m), sb));
        return hipSuccess;
      };
      int i_end = i_blk;
      while (i_end < nblocks && plan.B[i_end].r < r1) ++i_end;
      KLA_TRY(batch_work(i_blk, i_end, m, sums));
      i_blk = i_end;
    }
    return hipSuccess;
  }();
  // the caller's stream continues after the last readout
  if (two) {
    const hipError_t r1 = hipEventRecord(ev.join(), sb);
    const hipError_t r2 = r1 == hipSuccess ? hipStreamWaitEvent(st, ev.join(), 0) : r1;
    if (loop_err == hipSuccess && r2 != hipSuccess) return r2;
  }
  if (loop_err != hipSuccess) return loop_err;
  if (a.cache_T && a.cache_size > 0) {
    hipLaunchKernelGGL(copy_rows_kernel, dim3(N), dim3(256), 0, st, a.cache_T, a.cache_size, cache_slot(nR - 1),
                       kCStride);
    KLA_CHECK();
  }
#undef KLA_CHECK
#undef KLA_TRY
  return hipSuccess;
}

}  // namespace

bool hybrid_mfma_supported(const HybridArgs& a) { return a.dqk == 64 && a.dv == 64 && a.in_bf16; }

size_t hybrid_mfma_workspace(const HybridArgs& a) {
  size_t b = 0;
  if (!a.HT) b += align_up((size_t)a.N * kFPhi * kFD * sizeof(float));
  if (!a.sT) b += align_up((size_t)a.N * kFPhi * sizeof(float));
  return b + 2 * hf_bytes(a) + cache_bytes(a) + carry_bytes(a) + rej_bytes(a) + part_bytes(a) + base_bytes(a) + xp_bytes(a) +
         lp_bytes(a);
}

hipError_t hybrid_mfma_launch(const HybridArgs& a, void* ws, hipStream_t st, hipStream_t aux) {
  return a.out_bf16 ? enqueue<uint16_t>(a, ws, st, aux) : enqueue<float>(a, ws, st, aux);
}

}  // namespace kla
