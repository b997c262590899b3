// Chunked causal prefill on the bf16 matrix cores (d_qk = d_v = 64).
//
// KATA page, §2.3 ("Paralelismo por Blocos"; the linear chunked-state
// operating point): inside a chunk, masked (Q K^T)∘(Q K^T) scores multiply
// [V | 1]; across chunks the state (H, s) is a running prefix sum, read out by
// phi(Q) and updated by phi(K)^T [V | 1]. The lift is the rank-one PSD feature
// of KATA §2.2, phi(x)_ab = x_a x_b (times sqrt(2) off the diagonal).
//
// Feature tiles. The 64 dimensions form four blocks of 16. A tile is 16
// ordered pairs sharing b: row r is a = 16 X + r, with b = 16 Y + j, for one of
// the ten block pairs X <= Y and j = 0..15, so 160 tiles. Off the diagonal
// blocks (X < Y) each unordered pair appears once and carries the weight 2 of
// phi(q)_ab phi(k)_ab = 2 q_a q_b k_a k_b; a diagonal block (X = Y) holds all
// 256 ordered pairs of its dimensions, each pair and its mirror, with weight
// 1, which sums to the same. The kernels keep G(a, b) = sum_t k_a k_b v_t and
// s(a, b) = sum_t k_a k_b (no sqrt(2)); the ABI's vec_sym layout is converted
// on import and export.
//
// Multi-factor lift (KATA-Mg, KATA §2.3 "Variantes", read as G equal factors
// of 64 / G dimensions with their rank-one lifts concatenated): its features
// are the pairs inside one factor, i.e. the tiles of the block pairs inside
// the factors (G = 2: six of the ten, G = 4: the four diagonal blocks); the
// finish kernel then sums the factors' squared scores.
//
// Slices. A work-group owns one head and the tiles of one value of j (16
// slices per head) or two (8 slices) across the block pairs, so the tile
// structure inside a work-group is fixed at compile time and only j varies.
//
// State kernel, eight waves, stepping through 64-token sub-chunks; each step
// has two barriers: between them the update waves publish the state and the
// readout waves flush their partials, around them every wave computes on the
// staged sub-chunk while the next one is staged into the other buffer:
//   update waves (4) hold their tiles of G and s in MFMA accumulators (fp32)
//   for the whole sequence and add phi(K)^T [V | 1] per 32 tokens (MFMA
//   16x16x32 bf16; a column of ones gives s). In the A operand a lane holds
//   feature row r for eight tokens: it keeps k_a in registers and takes k_b
//   from the lane of its 16-lane row that loaded it, by a DPP row broadcast
//   folded into the multiply. At each chunk end they publish the state as bf16
//   B fragments in LDS.
//   readout waves (4): each takes 32 tokens and half of the tiles and reads
//   out num = phi(Q) G and den = phi(Q) s (a fifth MFMA n-tile whose first
//   column is s) against the state of the chunk start; a lane holds one token
//   and forms its products from q values in registers. The two waves sharing
//   tokens trade halves through LDS, and each writes one summed bf16 partial
//   of a 16-token tile to a workspace [head, chunk, slice, token tile,
//   16 x (d_v + 1)] in the MFMA accumulator order, so that both its writes and
//   the finish kernel's reads are whole 512-byte runs per wave. They also
//   stage the sub-chunks (q as fp32 rows, k as fp32 columns, v as bf16
//   columns) from loads issued one sub-step ahead.
// A head's work-groups are placed on one XCD (work-groups are dealt to the 8
// XCDs in turn), so their shared q, k and v reads meet in one L2.
//
// Finish kernel. One work-group per (head, chunk): the exact intra-chunk
// term A [V | 1] with A = lower-triangular (Q K^T)^2 (MFMA; for G factors the
// sum of the factors' squared scores), plus the sum of the slice partials,
// divided, cast to the output type.
#include <algorithm>

#include "kla_device.hpp"
#include "kla_internal.hpp"

namespace kla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kDim = 64;                          // d_qk = d_v
constexpr int kAcc = kDim + 1;                    // accumulator row: num | den
// Slice partials of one 16-token tile (bf16): the numerators in MFMA
// accumulator order [n-tile][lane][4 tokens], then the 16 denominators.
constexpr int kTileAcc = 16 * kAcc;


__device__ __forceinline__ float bf16f(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

__device__ __forceinline__ f32x4 mfma(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 pack8(const float* p) {
  bf16x8 r;
#pragma unroll
  for (int j = 0; j < 8; ++j) r[j] = (__bf16)p[j];
  return r;
}

// x from lane J of this lane's 16-lane row (DPP row broadcast).
template <int J>
__device__ __forceinline__ float row_bcast(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x150 + J, 0xF, 0xF, true));
}

// Work-group -> (head, slice); a head's slices share one XCD when N % 8 == 0.
__device__ __forceinline__ void wg_identity(int N, int S, int& n, int& slice) {
  const int wg = blockIdx.x;
  if ((N & 7) == 0) {
    const int xcd = wg & 7;
    const int r = wg >> 3;
    n = (r / S) * 8 + xcd;
    slice = r % S;
  } else {
    n = wg / S;
    slice = wg % S;
  }
}

// ------------------------------------------------------------ tile structure

constexpr int kUW = 4;                            // update waves (own G, s)
constexpr int kRW = 4;                            // readout waves
constexpr int kThreads3 = 64 * (kUW + kRW);
constexpr int kCS = 64;                           // staged sub-chunk (tokens), at most
constexpr int kQS = kDim + 4;                     // q row stride (floats)
constexpr int kKS = kCS + 4;                      // k^T row stride (floats)

// Block pairs X <= Y in order (0,0) (0,1) (0,2) (0,3) (1,1) (1,2) (1,3) (2,2) (2,3) (3,3).
__host__ __device__ constexpr int bp_x(int bp) { return bp < 4 ? 0 : bp < 7 ? 1 : bp < 9 ? 2 : 3; }
__host__ __device__ constexpr int bp_y(int bp) { return bp < 4 ? bp : bp < 7 ? bp - 3 : bp < 9 ? bp - 5 : 3; }

// Block pairs of the lift with G factors (KATA-Mg, concatenated factor lifts:
// only pairs of dimensions inside one factor of 64 / G dimensions are
// features): G = 1 all ten, G = 2 the six inside the halves, G = 4 the four
// diagonal blocks.
__host__ __device__ constexpr int factor_bps(int G) { return G == 1 ? 10 : G == 2 ? 6 : 4; }
__host__ __device__ constexpr int factor_bp(int G, int i) {
  return G == 1 ? i : G == 2 ? (i < 2 ? i : i == 2 ? 4 : i + 4) : (i == 0 ? 0 : i == 1 ? 4 : i == 2 ? 7 : 9);
}

// The tiles of one slice. S = 8: tile u is (block pair u / 2, j = j0 + u % 2)
// with j0 = 2 * slice; S = 16: tile u is (block pair u, j = slice), block
// pairs taken from the factor structure's list. Readout pairs are tiles
// (2p, 2p + 1); update wave w and readout half h take contiguous shares.
template <int S, int G>
struct Slice {
  static_assert(S == 8 || S == 16, "slices per head");
  static_assert(G == 1 || G == 2 || G == 4, "factors");
  static constexpr int kBP = factor_bps(G);
  static constexpr int kTiles = S == 8 ? 2 * kBP : kBP;
  static constexpr int kPairs = kTiles / 2;
  static constexpr int kJ = S == 8 ? 2 : 1;  // values of j in a slice
  __host__ __device__ static constexpr int bp(int u) { return factor_bp(G, S == 8 ? u >> 1 : u); }
  __host__ __device__ static constexpr int jj(int u) { return S == 8 ? (u & 1) : 0; }
  __host__ __device__ static constexpr int X(int u) { return bp_x(bp(u)); }
  __host__ __device__ static constexpr int Y(int u) { return bp_y(bp(u)); }
  // update wave w owns tiles [upd_first(w), upd_first(w) + upd_count(w))
  __host__ __device__ static constexpr int upd_count(int w) { return kTiles / 4 + (w < kTiles % 4 ? 1 : 0); }
  __host__ __device__ static constexpr int upd_first(int w) { return w * (kTiles / 4) + (w < kTiles % 4 ? w : kTiles % 4); }
  // readout half h owns pairs [rd_first(h), rd_first(h) + rd_count(h))
  __host__ __device__ static constexpr int rd_first(int h) { return h * ((kPairs + 1) / 2); }
  __host__ __device__ static constexpr int rd_count(int h) { return h == 0 ? (kPairs + 1) / 2 : kPairs / 2; }
  __host__ __device__ static constexpr bool upd_uses_x(int w, int b) {
    for (int u = upd_first(w); u < upd_first(w) + upd_count(w); ++u)
      if (X(u) == b) return true;
    return false;
  }
  __host__ __device__ static constexpr bool upd_uses_y(int w, int b) {
    for (int u = upd_first(w); u < upd_first(w) + upd_count(w); ++u)
      if (Y(u) == b) return true;
    return false;
  }
  __host__ __device__ static constexpr bool rd_uses_x(int h, int b) {
    for (int u = 2 * rd_first(h); u < 2 * (rd_first(h) + rd_count(h)); ++u)
      if (X(u) == b) return true;
    return false;
  }
};

// Index of feature (a, b), a <= b in one factor, in the ABI's state layout:
// the factors' vec_sym blocks in order, each upper-triangular row-major.
template <int G>
__device__ __forceinline__ int feat_abi(int a, int b) {
  constexpr int p = kDim / G;
  const int f = a / p;
  const int i = a - f * p, j = b - f * p;
  return f * (p * (p + 1) / 2) + i * p - i * (i - 1) / 2 + (j - i);
}

template <int S, int G>
struct StateLds {
  // staged sub-chunks, double buffered (the next is staged during this one)
  float qs[2][kCS][kQS];                          // q rows (fp32)
  float kt[2][kDim][kKS];                         // k transposed (fp32)
  uint16_t vt[2][kDim][kCS + 8];                  // v transposed (bf16)
  uint4 hs[Slice<S, G>::kPairs][4][64];           // G at the chunk start, bf16 B fragments
  uint4 ss[Slice<S, G>::kPairs][4];               // s as bf16 per pair and lane quarter
  f32x4 xs[kRW][5][64];                           // readout trade: one token tile's accumulators
};

// LDS-only work-group barrier: waits for this wave's LDS traffic, not for
// outstanding global loads or atomics.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
}

// One 16-byte group (8 dims) of q, k and v for one token of the next
// sub-chunk. The loads are unconditional (a token past the end reads the last
// row and is zeroed at staging), so that no branch has to wait for them.
struct Prefetch {
  uint4 q, k, v;
  bool ok;
};

__device__ __forceinline__ Prefetch prefetch(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                             const uint16_t* __restrict__ v, size_t row0, int n0, int T, int t,
                                             int grp) {
  Prefetch p;
  const size_t off = (row0 + min(n0 + t, T - 1)) * kDim + 8 * grp;
  p.q = *reinterpret_cast<const uint4*>(q + off);
  p.k = *reinterpret_cast<const uint4*>(k + off);
  p.v = *reinterpret_cast<const uint4*>(v + off);
  p.ok = n0 + t < T;
  return p;
}

// Staging: thread (token t, 8-dim group grp) writes q as fp32 rows, k as
// fp32 columns and v as bf16 columns.
// FULL: every token of the sub-chunk exists, so nothing is zeroed.
template <bool FULL, class Lds>
__device__ __forceinline__ void stage(Lds& sh, const Prefetch& p, int t, int grp, int buf) {
  const uint4 z = make_uint4(0, 0, 0, 0);
  const bool ok = FULL || p.ok;
  const uint4 pq = ok ? p.q : z, pk = ok ? p.k : z, pv = ok ? p.v : z;
  const uint32_t qw[4] = {pq.x, pq.y, pq.z, pq.w};
  const uint32_t kw[4] = {pk.x, pk.y, pk.z, pk.w};
  const uint32_t vw[4] = {pv.x, pv.y, pv.z, pv.w};
  const int d0 = 8 * grp;
  const float4 lo = make_float4(bf16f(qw[0] & 0xFFFF), bf16f(qw[0] >> 16), bf16f(qw[1] & 0xFFFF), bf16f(qw[1] >> 16));
  const float4 hi = make_float4(bf16f(qw[2] & 0xFFFF), bf16f(qw[2] >> 16), bf16f(qw[3] & 0xFFFF), bf16f(qw[3] >> 16));
  *reinterpret_cast<float4*>(&sh.qs[buf][t][d0]) = lo;
  *reinterpret_cast<float4*>(&sh.qs[buf][t][d0 + 4]) = hi;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    sh.kt[buf][d0 + 2 * e][t] = bf16f(kw[e] & 0xFFFF);
    sh.kt[buf][d0 + 2 * e + 1][t] = bf16f(kw[e] >> 16);
    sh.vt[buf][d0 + 2 * e][t] = (uint16_t)(vw[e] & 0xFFFF);
    sh.vt[buf][d0 + 2 * e + 1][t] = (uint16_t)(vw[e] >> 16);
  }
}

// Everything a wave of the state kernel needs about its work-group.
struct StateCtx {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  int T, NC, S, n, slice, j0;
  int D;  // features per head in the ABI layout
  const float* H0;
  const float* s0;
  float* HT;
  float* sT;
  uint16_t* part;  // slice partials [head, chunk, slice, token tile, kTileAcc], or NULL
};

// ------------------------------------------------------------- update waves

template <int C, int CS, int S, int G, int W>
__device__ __forceinline__ void update_wave(StateLds<S, G>& sh, const StateCtx& cx) {
  using SL = Slice<S, G>;
  constexpr int U0 = SL::upd_first(W);
  constexpr int NU = SL::upd_count(W);
  constexpr int SUB = C / CS;
  const int lane = threadIdx.x & 63;
  const int l16 = lane & 15;
  const int q4 = lane >> 4;
  const int nsteps = cx.NC * SUB;
  const float inv_sqrt2 = 0.70710678118654752f;

  // G (value n-tiles 0..3) and s (n-tile 4, column 0) of each owned tile;
  // lane (l16, q4) holds rows 4 q4 + i, column l16 of an n-tile
  f32x4 h[NU][5];
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    const int a0 = 16 * SL::X(U0 + u) + 4 * q4;
    const int b = 16 * SL::Y(U0 + u) + cx.j0 + SL::jj(U0 + u);
#pragma unroll
    for (int nt = 0; nt < 5; ++nt) h[u][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int a = a0 + i;
      const size_t f = (size_t)cx.n * cx.D + feat_abi<G>(min(a, b), max(a, b));
      const float sc = a != b ? inv_sqrt2 : 1.0f;
      if (cx.H0) {
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) h[u][nt][i] = cx.H0[f * kDim + 16 * nt + l16] * sc;
      }
      if (cx.s0 && l16 == 0) h[u][4][i] = cx.s0[f] * sc;
    }
  }

  // B operand of the s n-tile: column 0 is all ones
  bf16x8 ones;
#pragma unroll
  for (int i = 0; i < 8; ++i) ones[i] = (__bf16)(l16 == 0 ? 1.0f : 0.0f);

  auto publish = [&]() {
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int pr = (U0 + u) >> 1;
      const int half = (U0 + u) & 1;
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        bf16x4 x;
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = (__bf16)h[u][nt][i];
        *reinterpret_cast<bf16x4*>(reinterpret_cast<char*>(&sh.hs[pr][nt][lane]) + 8 * half) = x;
      }
      if (l16 == 0) {
        bf16x4 x;
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = (__bf16)h[u][4][i];
        *reinterpret_cast<bf16x4*>(reinterpret_cast<char*>(&sh.ss[pr][q4]) + 8 * half) = x;
      }
    }
  };
  publish();  // the state at the start of chunk 0

  // k_b sources: lane j' < kJ of each row holds k[token][16 Y + j0 + j']; the
  // other lanes keep whatever they held (only these lanes are broadcast)
  float kr[4][8];
#pragma unroll
  for (int b = 0; b < 4; ++b)
#pragma unroll
    for (int i = 0; i < 8; ++i) kr[b][i] = 0.0f;

  lds_barrier();  // (B0) initial state published, first sub-chunk staged
  for (int st = 0; st < nsteps; ++st) {
    const int buf = st & 1;
#pragma unroll
    for (int ks = 0; ks < CS / 32; ++ks) {
      const int t0 = ks * 32 + 8 * q4;
      bf16x8 vb[4];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) vb[nt] = *reinterpret_cast<const bf16x8*>(&sh.vt[buf][16 * nt + l16][t0]);
      float ka[4][8];
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        if (SL::upd_uses_x(W, b)) {
          const float4* p = reinterpret_cast<const float4*>(&sh.kt[buf][16 * b + l16][t0]);
          const float4 x0 = p[0], x1 = p[1];
          ka[b][0] = x0.x; ka[b][1] = x0.y; ka[b][2] = x0.z; ka[b][3] = x0.w;
          ka[b][4] = x1.x; ka[b][5] = x1.y; ka[b][6] = x1.z; ka[b][7] = x1.w;
        }
      }
      if (l16 < SL::kJ) {
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          if (SL::upd_uses_y(W, b)) {
            const float4* p = reinterpret_cast<const float4*>(&sh.kt[buf][16 * b + cx.j0 + l16][t0]);
            const float4 x0 = p[0], x1 = p[1];
            kr[b][0] = x0.x; kr[b][1] = x0.y; kr[b][2] = x0.z; kr[b][3] = x0.w;
            kr[b][4] = x1.x; kr[b][5] = x1.y; kr[b][6] = x1.z; kr[b][7] = x1.w;
          }
        }
      }
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        const int X = SL::X(U0 + u);
        const int Y = SL::Y(U0 + u);
        const int J = SL::jj(U0 + u);
        float p[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) p[i] = ka[X][i] * (J == 0 ? row_bcast<0>(kr[Y][i]) : row_bcast<1>(kr[Y][i]));
        const bf16x8 A = pack8(p);
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) h[u][nt] = mfma(A, vb[nt], h[u][nt]);
        h[u][4] = mfma(A, ones, h[u][4]);
      }
    }
    lds_barrier();  // (B2) sub-chunk consumed, readouts done
    if (st % SUB == SUB - 1) publish();
    lds_barrier();  // (B1) state published, next sub-chunk staged
  }

  // final state in the ABI layout (sqrt(2) on the off-diagonal features);
  // of a diagonal block's ordered pairs only a <= b is written
  const float sqrt2 = 1.41421356237309504880f;
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    const int a0 = 16 * SL::X(U0 + u) + 4 * q4;
    const int b = 16 * SL::Y(U0 + u) + cx.j0 + SL::jj(U0 + u);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int a = a0 + i;
      if (a > b) continue;
      const size_t f = (size_t)cx.n * cx.D + feat_abi<G>(a, b);
      const float sc = a < b ? sqrt2 : 1.0f;
      if (cx.HT) {
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) cx.HT[f * kDim + 16 * nt + l16] = h[u][nt][i] * sc;
      }
      if (cx.sT && l16 == 0) cx.sT[f] = h[u][4][i] * sc;
    }
  }
}

// ------------------------------------------------------------ readout waves

template <int C, int CS, int S, int G, int W>
__device__ __forceinline__ void readout_wave(StateLds<S, G>& sh, const StateCtx& cx) {
  using SL = Slice<S, G>;
  constexpr int HF = W & 1;                       // half of the pairs
  constexpr int TP = W >> 1;                      // token tiles 2 TP, 2 TP + 1 of a sub-chunk
  constexpr int P0 = SL::rd_first(HF);
  constexpr int NP = SL::rd_count(HF);
  constexpr int SUB = C / CS;
  constexpr bool kActive = 32 * TP < CS;
  const int lane = threadIdx.x & 63;
  const int l16 = lane & 15;
  const int q4 = lane >> 4;
  const size_t row0 = (size_t)cx.n * cx.T;
  const int nsteps = cx.NC * SUB;
  const bool active = kActive && cx.part != nullptr;

  // the own token tile (2 TP + HF) of the previous sub-step, kept across its
  // closing barrier until the partner's half has been added
  f32x4 keep[5];
#pragma unroll
  for (int nt = 0; nt < 5; ++nt) keep[nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto flush = [&](int st) {
    // add the partner's half of the own token tile, write the slice partial
    const f32x4* xs = &sh.xs[W ^ 1][0][0];
#pragma unroll
    for (int nt = 0; nt < 5; ++nt) {
      const f32x4 o = xs[nt * 64 + lane];
#pragma unroll
      for (int i = 0; i < 4; ++i) keep[nt][i] += o[i];
    }
    const int c = st / SUB;
    const int tt = ((st % SUB) * CS) / 16 + 2 * TP + HF;
    uint16_t* pc = cx.part + ((((size_t)cx.n * cx.NC + c) * cx.S + cx.slice) * (C / 16) + tt) * kTileAcc;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      bf16x4 b;
#pragma unroll
      for (int i = 0; i < 4; ++i) b[i] = (__bf16)keep[nt][i];
      *reinterpret_cast<bf16x4*>(pc + (nt * 64 + lane) * 4) = b;
    }
    if (l16 == 0) {
      bf16x4 b;
#pragma unroll
      for (int i = 0; i < 4; ++i) b[i] = (__bf16)keep[4][i];
      *reinterpret_cast<bf16x4*>(pc + 4 * 64 * 4 + 4 * q4) = b;
    }
  };

  // The readout waves stage the sub-chunks for the whole work-group (wave W:
  // 8-dim groups 2W and 2W + 1 of every token): the next sub-chunk into the
  // other buffer while this one is computed, with its loads issued a whole
  // sub-step earlier.
  auto pre = [&](int st, Prefetch (&p)[2]) {
    const int n0 = (st / SUB) * C + (st % SUB) * CS;
#pragma unroll
    for (int g = 0; g < 2; ++g) p[g] = prefetch(cx.q, cx.k, cx.v, row0, n0, cx.T, lane, 2 * W + g);
  };
  auto stage2 = [&](const Prefetch (&p)[2], int buf, int st) {
    if (lane < CS) {
      if ((st / SUB) * C + (st % SUB) * CS + CS <= cx.T) {  // uniform: a full sub-chunk
        stage<true>(sh, p[0], lane, 2 * W, buf);
        stage<true>(sh, p[1], lane, 2 * W + 1, buf);
      } else {
        stage<false>(sh, p[0], lane, 2 * W, buf);
        stage<false>(sh, p[1], lane, 2 * W + 1, buf);
      }
    }
  };
  Prefetch pf[2];
  pre(0, pf);
  stage2(pf, 0, 0);
  pre(1, pf);  // past the end: clamped reads, never staged
  lds_barrier();  // (B0)

  for (int st = 0; st < nsteps; ++st) {
    const int buf = st & 1;
    if (st + 1 < nsteps) {
      stage2(pf, buf ^ 1, st + 1);
      pre(st + 2, pf);
    }
    if (active) {
      // q factors of this lane's token in each of the two token tiles:
      // qa[tt][X] = q[16 X + 4 q4 + 0..3], qb[tt][u] = w_u q[16 Y_u + j_u]
      float qa[2][4][4];
      float qb[2][2 * NP];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const float* qrow = sh.qs[buf][32 * TP + 16 * tt + l16];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          if (SL::rd_uses_x(HF, b)) {
            const float4 x = *reinterpret_cast<const float4*>(qrow + 16 * b + 4 * q4);
            qa[tt][b][0] = x.x; qa[tt][b][1] = x.y; qa[tt][b][2] = x.z; qa[tt][b][3] = x.w;
          }
        }
#pragma unroll
        for (int u = 0; u < 2 * NP; ++u) {
          const int t = 2 * P0 + u;
          const float w = SL::X(t) < SL::Y(t) ? 2.0f : 1.0f;
          qb[tt][u] = w * qrow[16 * SL::Y(t) + cx.j0 + SL::jj(t)];
        }
      }
      // n-tiles 0..3: numerators; n-tile 4: the denominator in column 0
      f32x4 acc[2][5];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int nt = 0; nt < 5; ++nt) acc[tt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        const int pr = P0 + p;
        bf16x8 B[5];
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) B[nt] = __builtin_bit_cast(bf16x8, sh.hs[pr][nt][lane]);
        // s of this lane's k-slots in column 0, zero elsewhere
        const uint4 sw = sh.ss[pr][q4];
        B[4] = __builtin_bit_cast(bf16x8, l16 == 0 ? sw : make_uint4(0, 0, 0, 0));
        const int X0 = SL::X(2 * pr);
        const int X1 = SL::X(2 * pr + 1);
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          float f[8];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            f[i] = qa[tt][X0][i] * qb[tt][2 * p];
            f[4 + i] = qa[tt][X1][i] * qb[tt][2 * p + 1];
          }
          const bf16x8 A = pack8(f);
#pragma unroll
          for (int nt = 0; nt < 5; ++nt) acc[tt][nt] = mfma(A, B[nt], acc[tt][nt]);
        }
      }
      // hand the partner its token tile, keep the own one
      f32x4* xs = &sh.xs[W][0][0];
#pragma unroll
      for (int nt = 0; nt < 5; ++nt) {
        xs[nt * 64 + lane] = acc[1 - HF][nt];
        keep[nt] = acc[HF][nt];
      }
    }
    lds_barrier();  // (B2)
    if (active) flush(st);
    lds_barrier();  // (B1)
  }
}

// C: the chunk (intra-chunk region of the output); the state kernel stages it
// in sub-chunks of CS tokens, all read out against the state at the chunk start.
template <int C, int S, int G>
__global__ __launch_bounds__(kThreads3, 1) void prefill_state_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, int N, int T,
    const float* __restrict__ H0, const float* __restrict__ s0, float* __restrict__ HT, float* __restrict__ sT,
    uint16_t* __restrict__ part) {
  constexpr int CS = C < kCS ? C : kCS;
  static_assert(C % CS == 0 && CS % 32 == 0, "chunk must be a multiple of the sub-chunk");
  __shared__ __align__(16) StateLds<S, G> sh;
  StateCtx cx;
  cx.q = q;
  cx.k = k;
  cx.v = v;
  cx.T = T;
  cx.NC = (T + C - 1) / C;
  cx.S = S;
  cx.D = G * (kDim / G) * (kDim / G + 1) / 2;
  wg_identity(N, S, cx.n, cx.slice);
  cx.j0 = S == 8 ? 2 * cx.slice : cx.slice;
  cx.H0 = H0;
  cx.s0 = s0;
  cx.HT = HT;
  cx.sT = sT;
  cx.part = part;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  switch (wv) {
    case 0: update_wave<C, CS, S, G, 0>(sh, cx); break;
    case 1: update_wave<C, CS, S, G, 1>(sh, cx); break;
    case 2: update_wave<C, CS, S, G, 2>(sh, cx); break;
    case 3: update_wave<C, CS, S, G, 3>(sh, cx); break;
    case 4: readout_wave<C, CS, S, G, 0>(sh, cx); break;
    case 5: readout_wave<C, CS, S, G, 1>(sh, cx); break;
    case 6: readout_wave<C, CS, S, G, 2>(sh, cx); break;
    default: readout_wave<C, CS, S, G, 3>(sh, cx); break;
  }
}

template <int C>
struct FinishLds {
  uint16_t qs[C][kDim + 8];
  uint16_t ks[C][kDim + 8];
  uint16_t vt[kDim][C + 8];
};

// Weights of one 16-key x 16-query tile, key-major: the lane with query
// column l16 and group q4 gets keys 4 q4 + i of the tile. (q . k)^2, or for
// G factors the sum of the factors' squared scores.
template <int C, int G>
__device__ __forceinline__ f32x4 finish_weights(const FinishLds<C>& sh, int kq, int mq, int l16, int q4) {
  f32x4 w4 = {0.f, 0.f, 0.f, 0.f};
  if constexpr (G == 4) {
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      const s16x4 A = *reinterpret_cast<const s16x4*>(&sh.ks[kq * 16 + l16][16 * f + 4 * q4]);
      const s16x4 B = *reinterpret_cast<const s16x4*>(&sh.qs[mq * 16 + l16][16 * f + 4 * q4]);
      const f32x4 s4 = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(A, B, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
      w4 += s4 * s4;
    }
  } else {
    f32x4 s4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < kDim / 32; ++ks) {
      const bf16x8 A = *reinterpret_cast<const bf16x8*>(&sh.ks[kq * 16 + l16][ks * 32 + 8 * q4]);
      const bf16x8 B = *reinterpret_cast<const bf16x8*>(&sh.qs[mq * 16 + l16][ks * 32 + 8 * q4]);
      s4 = mfma(A, B, G == 2 ? f32x4{0.f, 0.f, 0.f, 0.f} : s4);
      if (G == 2) w4 += s4 * s4;
    }
    if (G == 1) w4 = s4 * s4;
  }
  return w4;
}

// One work-group per (chunk, head): intra-chunk term + accumulator -> output.
// The weights are formed transposed (keys as MFMA rows), so the accumulator
// of two 16-key tiles already is the A operand of the 32-key step of A [V | 1]
// when its k-slots are read as keys 4 q4 + i (i < 4) of the first tile and
// 4 q4 + i - 4 of the second; the value fragments take the same key order.
// The weights never leave registers.
template <int C, typename Tout, int G>
__global__ __launch_bounds__(kThreads) void prefill_finish_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ part, int S,
    Tout* __restrict__ o, int T, float eps) {
  __shared__ __align__(16) FinishLds<C> sh;
  const int c0 = blockIdx.x * C;
  const int n = blockIdx.y;
  const int L = min(C, T - c0);
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l16 = lane & 15;
  const int q4 = lane >> 4;
  const size_t row0 = (size_t)n * T + c0;

  for (int idx = tid; idx < C * 8; idx += kThreads) {
    const int t = idx >> 3;
    const int p = (idx & 7) * 8;
    uint4 qv = make_uint4(0, 0, 0, 0), kv = qv, vv = qv;
    if (t < L) {
      qv = *reinterpret_cast<const uint4*>(q + (row0 + t) * kDim + p);
      kv = *reinterpret_cast<const uint4*>(k + (row0 + t) * kDim + p);
      vv = *reinterpret_cast<const uint4*>(v + (row0 + t) * kDim + p);
    }
    *reinterpret_cast<uint4*>(&sh.qs[t][p]) = qv;
    *reinterpret_cast<uint4*>(&sh.ks[t][p]) = kv;
    const uint32_t vw[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      sh.vt[p + 2 * e][t] = (uint16_t)(vw[e] & 0xFFFF);
      sh.vt[p + 2 * e + 1][t] = (uint16_t)(vw[e] >> 16);
    }
  }
  __syncthreads();

  for (int mq = w; mq < C / 16; mq += kWaves) {
    f32x4 ra[4];
#pragma unroll
    for (int nt4 = 0; nt4 < 4; ++nt4) ra[nt4] = f32x4{0.f, 0.f, 0.f, 0.f};
    // this lane's query (column) and its running denominator over its keys
    const int qi = mq * 16 + l16;
    float dpart = 0.0f;
    for (int ks = 0; ks <= (mq >> 1); ++ks) {
      bf16x8 A;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int kq = 2 * ks + h;
        const f32x4 w4 = finish_weights<C, G>(sh, kq, mq, l16, q4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int ki = kq * 16 + 4 * q4 + i;
          const float a = (ki <= qi && ki < L) ? w4[i] : 0.0f;
          dpart += a;
          A[4 * h + i] = (__bf16)a;
        }
      }
#pragma unroll
      for (int nt4 = 0; nt4 < 4; ++nt4) {
        const uint16_t* vr = &sh.vt[16 * nt4 + l16][ks * 32 + 4 * q4];
        const bf16x4 b0 = *reinterpret_cast<const bf16x4*>(vr);
        const bf16x4 b1 = *reinterpret_cast<const bf16x4*>(vr + 16);
        const bf16x8 B = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
        ra[nt4] = mfma(A, B, ra[nt4]);
      }
    }
    // the lanes of one query column hold disjoint keys: add the four groups,
    // then fetch the denominators of the accumulator rows 4 q4 + i
    dpart += __shfl_xor(dpart, 16, 64);
    dpart += __shfl_xor(dpart, 32, 64);
    // lane holds O_in[query mq*16 + 4*q4 + i][value 16*nt4 + l16]; the slice
    // partials hold four consecutive tokens of one column as bf16
    float den[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) den[i] = __shfl(dpart, 4 * q4 + i, 64) + eps;
    const uint16_t* pc = part + ((size_t)(n * gridDim.x + blockIdx.x) * S * (C / 16) + mq) * kTileAcc;
    // the slices' loads are independent: keep several in flight
#pragma unroll 4
    for (int s = 0; s < S; ++s) {
      const uint16_t* ps = pc + (size_t)s * (C / 16) * kTileAcc;
#pragma unroll
      for (int nt4 = 0; nt4 < 4; ++nt4) {
        const bf16x4 b = *reinterpret_cast<const bf16x4*>(ps + (nt4 * 64 + lane) * 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) ra[nt4][i] += (float)b[i];
      }
      const bf16x4 b = *reinterpret_cast<const bf16x4*>(ps + 4 * 64 * 4 + 4 * q4);
#pragma unroll
      for (int i = 0; i < 4; ++i) den[i] += (float)b[i];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = mq * 16 + 4 * q4 + i;
      if (t < L) {
        const float inv = den[i] != 0.0f ? 1.0f / den[i] : 0.0f;
#pragma unroll
        for (int nt4 = 0; nt4 < 4; ++nt4)
          Elem<Tout>::store(o, (row0 + t) * kDim + 16 * nt4 + l16, den[i] != 0.0f ? ra[nt4][i] * inv : 0.0f);
      }
    }
  }
}

// Slices per head: 16 (one value of j each) while that keeps at most 256
// work-groups, else 8.
int slices_for(int N) { return N <= 16 ? 16 : 8; }

// The chunk the kernels run: a request for 32 runs as 64. The chunk only
// decides which part of each output is summed exactly (the intra-chunk
// term) and which through the bf16 state; after a 32-token first chunk the
// state-side rounding can reach the bf16 tolerance on small outputs, and 64
// halves it.
int run_chunk(int chunk) { return chunk == 32 ? 64 : chunk; }

size_t part_bytes(const PrefillArgs& a) {
  const int S = slices_for(a.N);
  const int C = run_chunk(a.chunk);
  const size_t nc = (a.T + C - 1) / C;
  return align_up((size_t)a.N * nc * S * kAcc * C * sizeof(uint16_t));
}

template <int C, int S, int G>
void launch_state(const PrefillArgs& a, uint16_t* part, hipStream_t st) {
  hipLaunchKernelGGL((prefill_state_kernel<C, S, G>), dim3(S * a.N), dim3(kThreads3), 0, st,
                     static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                     static_cast<const uint16_t*>(a.v), a.N, a.T, a.H0, a.s0, a.HT, a.sT, part);
}

template <int C, int G>
hipError_t launch_c(const PrefillArgs& a, void* ws, hipStream_t st) {
  uint16_t* part = a.o ? static_cast<uint16_t*>(ws) : nullptr;
  const int S = slices_for(a.N);
  prof_begin(st);
  if (S == 16) launch_state<C, 16, G>(a, part, st);
  else launch_state<C, 8, G>(a, part, st);
  prof_end(st);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !part) return e;
  const dim3 grid((a.T + C - 1) / C, a.N);
  if (a.out_bf16)
    hipLaunchKernelGGL((prefill_finish_kernel<C, uint16_t, G>), grid, dim3(kThreads), 0, st,
                       static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                       static_cast<const uint16_t*>(a.v), part, S, static_cast<uint16_t*>(a.o), a.T, a.eps);
  else
    hipLaunchKernelGGL((prefill_finish_kernel<C, float, G>), grid, dim3(kThreads), 0, st,
                       static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                       static_cast<const uint16_t*>(a.v), part, S, static_cast<float*>(a.o), a.T, a.eps);
  return hipGetLastError();
}

template <int G>
hipError_t launch_g(const PrefillArgs& a, void* ws, hipStream_t st) {
  switch (run_chunk(a.chunk)) {
    case 64: return launch_c<64, G>(a, ws, st);
    case 128: return launch_c<128, G>(a, ws, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace

bool prefill_mfma_supported(const PrefillArgs& a) {
  return a.in_bf16 && a.dqk == kDim && a.dv == kDim && (a.chunk == 32 || a.chunk == 64 || a.chunk == 128) &&
         a.factor_kind == 0 && (a.factors == 1 || a.factors == 2 || a.factors == 4);
}

size_t prefill_mfma_workspace(const PrefillArgs& a) { return a.o ? part_bytes(a) : 0; }

hipError_t prefill_mfma_launch(const PrefillArgs& a, void* ws, hipStream_t st) {
  switch (a.factors) {
    case 1: return launch_g<1>(a, ws, st);
    case 2: return launch_g<2>(a, ws, st);
    case 4: return launch_g<4>(a, ws, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace kla
