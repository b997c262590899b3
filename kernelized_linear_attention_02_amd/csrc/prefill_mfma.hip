// Chunked causal prefill on the matrix cores (d_qk = d_v = 64, bf16 inputs).
//
// KATA page, §2.3 ("Paralelismo por Blocos"; the linear chunked-state
// operating point): inside a chunk, masked (Q K^T)∘(Q K^T) scores multiply
// V; across chunks the state H is a running prefix sum, read out by phi(Q)
// and updated by phi(K)^T V. The lift is the rank-one PSD feature of KATA
// §2.2, phi(x)_ab = x_a x_b (times sqrt(2) off the diagonal), so
// phi(q).phi(k) = (q.k)^2. The normaliser phi(q)^T s equals q^T S q with
// S = sum_t k_t k_t^T (the keys' Gram matrix, which holds s up to the sqrt(2)
// scaling), so it is formed from S in float32.
//
// Feature tiles. The 64 dimensions form four blocks of 16. A tile is 16
// ordered pairs sharing b: row r is a = 16 X + r, with b = 16 Y + j, for one
// of the ten block pairs X <= Y and j = 0..15. Rows of a diagonal block with
// a > b are mirrors of rows with a < b: they are accumulated (the tile's
// shape needs them) but carry weight 0 in the readout and never cross the
// ABI, so every feature a <= b has exactly one owner. The kernels keep
// G(a, b) = sum_t k_a k_b v_t; the ABI's vec_sym layout (sqrt(2) off the
// diagonal) is converted on import and export.
//
// Work split. A head's features are cut into SF slices (the tiles of 16 / SF
// values of j) and its 64 value columns into two halves: one work-group per
// (head, slice, half), 2 SF work-groups per head, all on one XCD (work-groups
// are dealt to the 8 XCDs in turn) so their q, k, v reads meet in one L2.
//
// Precision. The feature products and the state are float16 (11-bit
// significands) with exact power-of-two scales that keep every value in
// float16 range whatever the inputs: each sub-chunk's keys are scaled by
// 2^-ek (largest |k| below 1) and its values by 2^(2 ek - G), where the
// running exponent G >= 2 ek + log2 max|v| of every sub-chunk seen; the
// accumulators hold H 2^-G (rescaled when G grows). Queries are scaled per
// token (undone before the partials are written). The published state is
// scaled by 2^-P so that a bound on its largest weighted entry stays below
// 2^15.
// Accumulation is float32 throughout; the slice partials are float32.
//
// State kernel, eight waves, stepping through sub-chunks of up to 64 tokens;
// each step has two barriers: between them the update waves publish the
// state (at chunk ends), the readout waves write their partials and stage
// the next sub-chunk; around them every wave computes on the staged one.
//   update waves (4) hold their tiles of G for the whole sequence in MFMA
//   accumulators and add phi(K)^T V per 32 tokens (mfma 16x16x32 f16): a lane
//   of the A operand holds feature row r for eight tokens and forms them as
//   packed float16 products of its k_a and k_b, k_b coming from lane 0 of its
//   16-lane row by a DPP broadcast. In the first value half's work-group each
//   wave also accumulates one X block of the keys' Gram matrix for the
//   slice's columns b (the staged float16 keys hold the bf16 keys exactly up
//   to the sub-chunk's power of two: exact products, float32 sums). At each
//   chunk end they publish the weighted state (2 off the diagonal, 1 on it, 0
//   for mirror rows) as float16 B fragments in LDS and the Gram matrix to
//   memory.
//   readout waves (4): each takes 32 tokens and half of the tile pairs and
//   reads out phi(Q) G against the state of the chunk start; a lane holds one
//   token and forms its products from q values in registers. The two waves
//   sharing tokens trade halves through LDS, and each writes one float32
//   partial [16 tokens x 32 columns] per token tile in the MFMA accumulator
//   order. They also stage the sub-chunks (q rows, k columns, v columns of
//   the work-group's half), in two passes: the scales' maxima before the
//   middle barrier, the scaled values after it.
//
// Finish kernel. One work-group per (head, chunk): the exact intra-chunk term
// (squared scores as two bf16 pieces times V), the denominator's state term
// q^T S q from the Gram matrix of the chunk start (two bf16 pieces on the
// matrix cores, float32 sums), the sum of the slice partials, divided, cast
// to the output type.
#include <algorithm>
#include <climits>

#include "kla_device.hpp"
#include "kla_internal.hpp"

namespace kla {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kDim = 64;      // d_qk = d_v
constexpr int kCols = 32;     // value columns per work-group (two per head)
constexpr int kUW = 4;        // update waves
constexpr int kRW = 4;        // readout (and staging) waves
constexpr int kThreads3 = 64 * (kUW + kRW);
constexpr int kCS = 64;       // staged sub-chunk (tokens), at most
constexpr int kPad = 8;       // halves of padding per LDS row
constexpr int kNoExp = INT_MIN / 4;
// float32 partials of one 16-token tile: 4 column n-tiles x 64 lanes x 4 tokens
constexpr int kTilePart = 4 * 64 * 4;

__device__ __forceinline__ float bf16f(uint32_t h) { return __uint_as_float(h << 16); }

__device__ __forceinline__ f32x4 mfma_h(const f16x8& a, const f16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_b(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// e with m 2^-e in [0.5, 1) for m > 0 (so |x| <= m gives |x| 2^-e < 1);
// kNoExp for m = 0.
__device__ __forceinline__ int exp_above(float m) {
  if (!(m > 0.0f)) return kNoExp;
  const int be = (int)((__float_as_uint(m) >> 23) & 0xFF);
  return be == 0 ? -126 : be - 126;
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}

// x from lane 0 of this lane's 16-lane row (DPP row broadcast).
__device__ __forceinline__ uint32_t row_bcast0(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x150, 0xF, 0xF, true);
}

__device__ __forceinline__ f16x2 as_h2(uint32_t x) { return __builtin_bit_cast(f16x2, x); }
__device__ __forceinline__ uint32_t as_u(f16x2 x) { return __builtin_bit_cast(uint32_t, x); }

// Largest |x| of bf16 values as a bf16 bit pattern: |x| orders like the low
// 15 bits of the pattern (packed 16-bit maxima).
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ u16x2 abs_pair(uint32_t x) { return __builtin_bit_cast(u16x2, x & 0x7FFF7FFFu); }
__device__ __forceinline__ u16x2 absmax_pairs(uint4 w) {
  return __builtin_elementwise_max(__builtin_elementwise_max(abs_pair(w.x), abs_pair(w.y)),
                                   __builtin_elementwise_max(abs_pair(w.z), abs_pair(w.w)));
}
__device__ __forceinline__ uint32_t pair_max(u16x2 m) { return max((uint32_t)m[0], (uint32_t)m[1]); }

// Eight bf16 values times 2^e, rounded to float16 (nearest even).
__device__ __forceinline__ uint4 bf16x8_to_f16_scaled(uint4 w, int e) {
  const uint32_t in[4] = {w.x, w.y, w.z, w.w};
  uint32_t out[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float lo = __builtin_ldexpf(bf16f(in[i] & 0xFFFFu), e);
    const float hi = __builtin_ldexpf(bf16f(in[i] >> 16), e);
    out[i] = as_u(f16x2{(_Float16)lo, (_Float16)hi});
  }
  return make_uint4(out[0], out[1], out[2], out[3]);
}

// Work-group -> (head, feature slice, value half); a head's work-groups share
// one XCD when N % 8 == 0.
__device__ __forceinline__ void wg_identity(int N, int SF, int& n, int& sf, int& ch) {
  const int wg = blockIdx.x;
  const int per = 2 * SF;
  int local;
  if ((N & 7) == 0) {
    const int r = wg >> 3;
    n = (r / per) * 8 + (wg & 7);
    local = r % per;
  } else {
    n = wg / per;
    local = wg % per;
  }
  sf = local >> 1;
  ch = local & 1;
}

// ------------------------------------------------------------ tile structure

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

// The tiles of one feature slice: SF = 4 slices hold j = 4 sf + jj (jj < 4),
// SF = 8 slices j = 2 sf + jj (jj < 2), each over the factor structure's
// block pairs. Tile u is (jj = u / kBP, block pair u % kBP); update wave w
// owns tiles [w kNU, (w + 1) kNU), which share one jj; readout pair p is
// tiles (2p, 2p + 1), and readout half h owns pairs [h kNP, (h + 1) kNP).
template <int SF, int G>
struct Slice {
  static_assert(SF == 4 || SF == 8, "feature slices per head");
  static_assert(G == 1 || G == 2 || G == 4, "factors");
  static constexpr int kBP = factor_bps(G);
  static constexpr int kJ = 16 / SF;
  static constexpr int kTiles = kJ * kBP;
  static constexpr int kPairs = kTiles / 2;
  static constexpr int kNU = kTiles / kUW;
  static constexpr int kNP = kPairs / 2;
  static_assert(kTiles % kUW == 0 && kPairs % 2 == 0 && kBP % kNU == 0, "tile split");
  static constexpr int kNB = 4 * kJ;  // Gram columns b of a slice
  __host__ __device__ static constexpr int jj(int u) { return u / kBP; }
  __host__ __device__ static constexpr int bp(int u) { return factor_bp(G, u % kBP); }
  __host__ __device__ static constexpr int X(int u) { return bp_x(bp(u)); }
  __host__ __device__ static constexpr int Y(int u) { return bp_y(bp(u)); }
  __host__ __device__ static constexpr bool upd_uses_x(int w, int x) {
    for (int u = w * kNU; u < (w + 1) * kNU; ++u)
      if (X(u) == x) return true;
    return false;
  }
  __host__ __device__ static constexpr bool upd_uses_y(int w, int y) {
    for (int u = w * kNU; u < (w + 1) * kNU; ++u)
      if (Y(u) == y) return true;
    return false;
  }
  __host__ __device__ static constexpr bool rd_uses_x(int h, int x) {
    for (int u = 2 * h * kNP; u < 2 * (h + 1) * kNP; ++u)
      if (X(u) == x) return true;
    return false;
  }
  __host__ __device__ static constexpr bool rd_uses_y(int h, int y) {
    for (int u = 2 * h * kNP; u < 2 * (h + 1) * kNP; ++u)
      if (Y(u) == y) return true;
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

template <int G>
__host__ __device__ __forceinline__ bool same_factor(int a, int b) {
  constexpr int p = kDim / G;
  return a / p == b / p;
}

template <int SF, int G>
struct StateLds {
  uint4 hs[Slice<SF, G>::kPairs][2][64];  // weighted state, float16 B fragments
  f32x4 xs[kRW][2][64];                   // readout trade: one token tile's accumulators
  // staged sub-chunks, double buffered (the next is staged during this one)
  _Float16 qs[2][kCS][kDim + kPad];       // q rows, scaled per token
  _Float16 kt[2][kDim][kCS + kPad];       // k columns, scaled per sub-chunk
  _Float16 vt[2][kCols][kCS + kPad];      // v columns of the work-group's half, scaled
  int qe[2][kCS];                         // per-token query exponent
  int sc[2][2];                           // per buffer: key exponent ek, state exponent G
  float qmx[kRW][kCS];                    // staging: per wave and token, max |q| over its dims
  float kvmx[kRW][2];                     // staging: per wave, max |k| and max |v|
  float umx[kUW];                         // per update wave, max |imported state|
  int pub_e;                              // exponent of the published state (G + P)
};

// LDS-only work-group barrier: waits for this wave's LDS traffic, not for
// outstanding global loads.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
}

// One token's share of a sub-chunk for staging wave W: q and k dims
// 16 W .. 16 W + 15, v dims 32 ch + 8 W .. + 7. The loads are unconditional (a
// token past the end reads the last row and is zeroed), so that no branch
// has to wait for them.
struct Prefetch {
  uint4 q[2], k[2], v;
  bool ok;
};

__device__ __forceinline__ Prefetch prefetch(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                             const uint16_t* __restrict__ v, size_t row0, int n0, int T, int t,
                                             int W, int ch) {
  Prefetch p;
  const size_t row = (row0 + min(n0 + t, T - 1)) * kDim;
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    p.q[g] = *reinterpret_cast<const uint4*>(q + row + 16 * W + 8 * g);
    p.k[g] = *reinterpret_cast<const uint4*>(k + row + 16 * W + 8 * g);
  }
  p.v = *reinterpret_cast<const uint4*>(v + row + kCols * ch + 8 * W);
  p.ok = n0 + t < T;
  return p;
}

// Everything a wave of the state kernel needs about its work-group.
struct StateCtx {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  int T, NC, n, sf, ch, j0;
  int D;  // features per head in the ABI layout
  const float* H0;
  const float* s0;
  float* HT;
  float* sT;
  float* part;  // slice partials [head, chunk, slice, token tile, kTilePart], or NULL
  float* Sg;    // Gram matrix at each chunk start [head, chunk, 64, 64], or NULL
};

// Staging, first pass (before the middle barrier): maxima of the prefetched
// values. Lane t < CS holds token t.
template <int CS, class Lds>
__device__ __forceinline__ void stage_max(Lds& sh, const Prefetch& p, int W, int lane) {
  const bool act = lane < CS && p.ok;
  uint32_t qm = 0, km = 0, vm = 0;
  if (act) {
    qm = pair_max(__builtin_elementwise_max(absmax_pairs(p.q[0]), absmax_pairs(p.q[1])));
    km = pair_max(__builtin_elementwise_max(absmax_pairs(p.k[0]), absmax_pairs(p.k[1])));
    vm = pair_max(absmax_pairs(p.v));
  }
  if (lane < CS) sh.qmx[W][lane] = bf16f(qm);
  const float kw = wave_max(bf16f(km));
  const float vw = wave_max(bf16f(vm));
  if (lane == 0) {
    sh.kvmx[W][0] = kw;
    sh.kvmx[W][1] = vw;
  }
}

// The running state exponent: once the accumulators may hold something (an
// imported state, or a sub-chunk with nonzero keys and values) it only grows;
// before that it follows the first nonzero sub-chunk.
struct ExpTrack {
  int G = 0;
  bool live = false;
  __device__ void see(int E) {
    G = live ? max(G, E) : E;
    live = true;
  }
};

// Staging, second pass (after the middle barrier): scales and scaled values
// into buffer `buf`.
template <int CS, class Lds>
__device__ __forceinline__ void stage_write(Lds& sh, const Prefetch& p, int W, int lane, int buf, ExpTrack& g) {
  const float kall = fmaxf(fmaxf(sh.kvmx[0][0], sh.kvmx[1][0]), fmaxf(sh.kvmx[2][0], sh.kvmx[3][0]));
  const float vall = fmaxf(fmaxf(sh.kvmx[0][1], sh.kvmx[1][1]), fmaxf(sh.kvmx[2][1], sh.kvmx[3][1]));
  const int ekr = exp_above(kall), ev = exp_above(vall);
  // a sub-chunk whose keys or values are all zero adds nothing: its values
  // are staged as zeros and the exponent does not move
  const bool contributes = ekr != kNoExp && ev != kNoExp;
  if (contributes) g.see(2 * ekr + ev);
  const int ek = ekr == kNoExp ? 0 : ekr;
  if (lane < CS) {
    const int t = lane;
    const uint4 z = make_uint4(0, 0, 0, 0);
    const uint4 q0 = p.ok ? p.q[0] : z, q1 = p.ok ? p.q[1] : z;
    const uint4 k0 = p.ok ? p.k[0] : z, k1 = p.ok ? p.k[1] : z;
    const uint4 vv = p.ok && contributes ? p.v : z;
    const float qm = fmaxf(fmaxf(sh.qmx[0][t], sh.qmx[1][t]), fmaxf(sh.qmx[2][t], sh.qmx[3][t]));
    const int eqr = exp_above(qm);
    const int eq = eqr == kNoExp ? 0 : eqr;
    *reinterpret_cast<uint4*>(&sh.qs[buf][t][16 * W]) = bf16x8_to_f16_scaled(q0, -eq);
    *reinterpret_cast<uint4*>(&sh.qs[buf][t][16 * W + 8]) = bf16x8_to_f16_scaled(q1, -eq);
    if (W == 0) sh.qe[buf][t] = eq;
    const uint4 kh0 = bf16x8_to_f16_scaled(k0, -ek), kh1 = bf16x8_to_f16_scaled(k1, -ek);
    const uint32_t kh[8] = {kh0.x, kh0.y, kh0.z, kh0.w, kh1.x, kh1.y, kh1.z, kh1.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int d = 16 * W + 2 * e;
      sh.kt[buf][d][t] = as_h2(kh[e])[0];
      sh.kt[buf][d + 1][t] = as_h2(kh[e])[1];
    }
    const uint4 vh = bf16x8_to_f16_scaled(vv, contributes ? 2 * ek - g.G : 0);
    const uint32_t vw[4] = {vh.x, vh.y, vh.z, vh.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      sh.vt[buf][8 * W + 2 * e][t] = as_h2(vw[e])[0];
      sh.vt[buf][8 * W + 2 * e + 1][t] = as_h2(vw[e])[1];
    }
  }
  if (W == 0 && lane == 0) {
    sh.sc[buf][0] = ek;
    sh.sc[buf][1] = g.G;
  }
}

// ------------------------------------------------------------- update waves

template <int C, int CS, int SF, int G, int W>
__device__ __forceinline__ void update_wave(StateLds<SF, G>& sh, const StateCtx& cx) {
  using SL = Slice<SF, G>;
  constexpr int U0 = W * SL::kNU;
  constexpr int NU = SL::kNU;
  constexpr int JJ = SL::jj(U0);  // one value of j per update wave
  constexpr int SUB = C / CS;
  const int lane = threadIdx.x & 63;
  const int l16 = lane & 15;
  const int q4 = lane >> 4;
  const int nsteps = cx.NC * SUB;
  const int j = cx.j0 + JJ;
  const float inv_sqrt2 = 0.70710678118654752f;
  const bool gram_wg = cx.ch == 0;  // the first value half also forms the Gram matrix

  // Gram column of this lane: the slice's b values 16 Y + j0 + jj
  const int gb = 16 * (l16 / SL::kJ) + cx.j0 + (l16 % SL::kJ);
  const bool gb_ok = l16 < SL::kNB;

  // G (value n-tiles 0, 1 of the work-group's half) of each owned tile;
  // lane (l16, q4) holds rows 4 q4 + i, column l16 of an n-tile
  f32x4 h[NU][2];
  f32x4 gram = {0.f, 0.f, 0.f, 0.f};  // float32 Gram matrix (true scale)
  f32x4 gsub = {0.f, 0.f, 0.f, 0.f};  // this sub-chunk's part, in the staged key scale
  float hmax = 0.0f;
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    const int a0 = 16 * SL::X(U0 + u) + 4 * q4;
    const int b = 16 * SL::Y(U0 + u) + j;
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) h[u][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (cx.H0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int a = a0 + i;
        if (a > b) continue;  // mirror rows of a diagonal block are never imported
        const size_t f = (size_t)cx.n * cx.D + feat_abi<G>(a, b);
        const float scl = a != b ? inv_sqrt2 : 1.0f;
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          const float x = cx.H0[f * kDim + kCols * cx.ch + 16 * nt + l16] * scl;
          h[u][nt][i] = x;
          hmax = fmaxf(hmax, fabsf(x));
        }
      }
    }
  }
  if (gram_wg && cx.s0 && gb_ok) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int a = 16 * W + 4 * q4 + i;
      if (a <= gb && same_factor<G>(a, gb))
        gram[i] = cx.s0[(size_t)cx.n * cx.D + feat_abi<G>(a, gb)] * (a != gb ? inv_sqrt2 : 1.0f);
    }
  }
  hmax = wave_max(hmax);
  if (lane == 0) sh.umx[W] = hmax;

  int Gu = 0;  // the accumulators hold G 2^-Gu
  // Bound on |h| in current units: the imported state plus one per token
  // (each token adds k'_a k'_b v'' with every factor below 1), scaled with
  // the accumulators. Uniform across the wave.
  float hb = 0.0f;
  // publish the state at the start of chunk c; m bounds |h| in current units
  auto publish = [&](int c, float m) {
    // the largest weighted entry stays below 2^15 in float16
    const int em = exp_above(2.0f * m);
    const int P = em == kNoExp ? 0 : em - 15;
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int X = SL::X(U0 + u), Y = SL::Y(U0 + u);
      const int pr = (U0 + u) >> 1;
      const int half = (U0 + u) & 1;
      // readout weight of each row: 2 off the diagonal blocks; on them 2 for
      // a < b, 1 for a = b, 0 for the mirror rows a > b
      float wr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * q4 + i;
        const float w = X < Y ? 2.0f : (r < j ? 2.0f : (r == j ? 1.0f : 0.0f));
        wr[i] = __builtin_ldexpf(w, -P);
      }
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const f16x2 lo = {(_Float16)(h[u][nt][0] * wr[0]), (_Float16)(h[u][nt][1] * wr[1])};
        const f16x2 hi = {(_Float16)(h[u][nt][2] * wr[2]), (_Float16)(h[u][nt][3] * wr[3])};
        uint2* dst = reinterpret_cast<uint2*>(reinterpret_cast<char*>(&sh.hs[pr][nt][lane]) + 8 * half);
        *dst = make_uint2(as_u(lo), as_u(hi));
      }
    }
    if (W == 0 && lane == 0) sh.pub_e = Gu + P;
    // the Gram matrix at the start of chunk c: each entry a <= b is written by
    // its owner at (a, b) and (b, a)
    if (gram_wg && cx.Sg && c < cx.NC && gb_ok) {
      float* S = cx.Sg + ((size_t)cx.n * cx.NC + c) * kDim * kDim;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int a = 16 * W + 4 * q4 + i;
        if (a <= gb) {
          S[a * kDim + gb] = gram[i];
          S[gb * kDim + a] = gram[i];
        }
      }
    }
  };

  lds_barrier();  // (B0a) state maxima and the first sub-chunk's maxima posted
  lds_barrier();  // (B0b) first sub-chunk staged with its exponents
  Gu = __builtin_amdgcn_readfirstlane(sh.sc[0][1]);
  {
    const float s = __builtin_ldexpf(1.0f, -Gu);
#pragma unroll
    for (int u = 0; u < NU; ++u)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) h[u][nt] *= s;
    const float m = fmaxf(fmaxf(sh.umx[0], sh.umx[1]), fmaxf(sh.umx[2], sh.umx[3]));
    hb = m * s;
    publish(0, hb);  // the state at the start of chunk 0
  }
  lds_barrier();  // (B0c) initial state published

  for (int st = 0; st < nsteps; ++st) {
    const int buf = st & 1;
    const int Gn = __builtin_amdgcn_readfirstlane(sh.sc[buf][1]);
    if (Gn != Gu) {  // uniform: the state exponent moved
      const float s = __builtin_ldexpf(1.0f, Gu - Gn);
#pragma unroll
      for (int u = 0; u < NU; ++u)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) h[u][nt] *= s;
      hb *= s;
      Gu = Gn;
    }
#pragma unroll
    for (int ks = 0; ks < CS / 32; ++ks) {
      const int t0 = ks * 32 + 8 * q4;
      f16x8 vb[2];
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) vb[nt] = *reinterpret_cast<const f16x8*>(&sh.vt[buf][16 * nt + l16][t0]);
      uint4 ka[4];
#pragma unroll
      for (int x = 0; x < 4; ++x)
        if (SL::upd_uses_x(W, x)) ka[x] = *reinterpret_cast<const uint4*>(&sh.kt[buf][16 * x + l16][t0]);
      uint4 kb[4];
#pragma unroll
      for (int y = 0; y < 4; ++y) {
        if (SL::upd_uses_y(W, y)) {
          uint4 src = make_uint4(0, 0, 0, 0);
          if (l16 == 0) src = *reinterpret_cast<const uint4*>(&sh.kt[buf][16 * y + j][t0]);
          kb[y] = make_uint4(row_bcast0(src.x), row_bcast0(src.y), row_bcast0(src.z), row_bcast0(src.w));
        }
      }
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        const uint4 xa = ka[SL::X(U0 + u)];
        const uint4 xb = kb[SL::Y(U0 + u)];
        const uint32_t p0 = as_u(as_h2(xa.x) * as_h2(xb.x));
        const uint32_t p1 = as_u(as_h2(xa.y) * as_h2(xb.y));
        const uint32_t p2 = as_u(as_h2(xa.z) * as_h2(xb.z));
        const uint32_t p3 = as_u(as_h2(xa.w) * as_h2(xb.w));
        const f16x8 A = __builtin_bit_cast(f16x8, make_uint4(p0, p1, p2, p3));
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) h[u][nt] = mfma_h(A, vb[nt], h[u][nt]);
      }
      if (gram_wg) {
        const f16x8 A = *reinterpret_cast<const f16x8*>(&sh.kt[buf][16 * W + l16][t0]);
        f16x8 B = __builtin_bit_cast(f16x8, make_uint4(0, 0, 0, 0));
        if (gb_ok) B = *reinterpret_cast<const f16x8*>(&sh.kt[buf][gb][t0]);
        gsub = mfma_h(A, B, gsub);
      }
    }
    if (gram_wg) {
      // the sub-chunk's keys were staged times 2^-ek: exact products, so the
      // float32 Gram matrix gets them back times 4^ek
      const float s = __builtin_ldexpf(1.0f, 2 * __builtin_amdgcn_readfirstlane(sh.sc[buf][0]));
      gram += gsub * s;
      gsub = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    hb += (float)CS;
    const bool chunk_end = st % SUB == SUB - 1;
    lds_barrier();  // (B2) sub-chunk consumed, readouts done
    if (chunk_end) publish(st / SUB + 1, hb);
    lds_barrier();  // (B1) state published, next sub-chunk staged
  }

  // final state in the ABI layout (sqrt(2) on the off-diagonal features)
  const float sqrt2 = 1.41421356237309504880f;
  if (cx.HT) {
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int a0 = 16 * SL::X(U0 + u) + 4 * q4;
      const int b = 16 * SL::Y(U0 + u) + j;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int a = a0 + i;
        if (a > b) continue;
        const size_t f = (size_t)cx.n * cx.D + feat_abi<G>(a, b);
        const float scl = __builtin_ldexpf(a < b ? sqrt2 : 1.0f, Gu);
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) cx.HT[f * kDim + kCols * cx.ch + 16 * nt + l16] = h[u][nt][i] * scl;
      }
    }
  }
  if (gram_wg && cx.sT && gb_ok) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int a = 16 * W + 4 * q4 + i;
      if (a <= gb && same_factor<G>(a, gb))
        cx.sT[(size_t)cx.n * cx.D + feat_abi<G>(a, gb)] = gram[i] * (a < gb ? sqrt2 : 1.0f);
    }
  }
}

// ------------------------------------------------------------ readout waves

template <int C, int CS, int SF, int G, int W>
__device__ __forceinline__ void readout_wave(StateLds<SF, G>& sh, const StateCtx& cx) {
  using SL = Slice<SF, G>;
  constexpr int HF = W & 1;   // half of the pairs
  constexpr int TP = W >> 1;  // token tiles 2 TP, 2 TP + 1 of a sub-chunk
  constexpr int P0 = HF * SL::kNP;
  constexpr int NP = SL::kNP;
  constexpr int SUB = C / CS;
  constexpr bool kActive = 32 * TP < CS;
  const int lane = threadIdx.x & 63;
  const int l16 = lane & 15;
  const int q4 = lane >> 4;
  const size_t row0 = (size_t)cx.n * cx.T;
  const int nsteps = cx.NC * SUB;
  const bool active = kActive && cx.part != nullptr;

  f32x4 keep[2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) keep[nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto flush = [&](int st, int buf, int pe) {
    // add the partner's half of the own token tile, undo the scales
    // (per-token query exponent, published-state exponent) and write the
    // float32 partial
    const f32x4* xs = &sh.xs[W ^ 1][0][0];
    const int tl = 16 * (2 * TP + HF) + 4 * q4;  // tokens tl + i of the sub-chunk
    float f[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = __builtin_ldexpf(1.0f, 2 * sh.qe[buf][tl + i] + pe);
    const int c = st / SUB;
    const int tt = ((st % SUB) * CS) / 16 + 2 * TP + HF;
    float* pc = cx.part + ((((size_t)cx.n * cx.NC + c) * SF + cx.sf) * (C / 16) + tt) * kTilePart;
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const f32x4 o = xs[nt * 64 + lane];
      f32x4 r;
#pragma unroll
      for (int i = 0; i < 4; ++i) r[i] = (keep[nt][i] + o[i]) * f[i];
      *reinterpret_cast<f32x4*>(pc + ((2 * cx.ch + nt) * 64 + lane) * 4) = r;
    }
  };

  auto pre = [&](int st) {
    const int n0 = (st / SUB) * C + (st % SUB) * CS;
    return prefetch(cx.q, cx.k, cx.v, row0, n0, cx.T, lane, W, cx.ch);
  };
  ExpTrack g;
  Prefetch pf = pre(0);
  stage_max<CS>(sh, pf, W, lane);
  lds_barrier();  // (B0a)
  if (cx.H0) {
    // an imported state: the exponent starts where the accumulators hold it
    // below 2^100 and then only grows
    const float m = fmaxf(fmaxf(sh.umx[0], sh.umx[1]), fmaxf(sh.umx[2], sh.umx[3]));
    const int e = exp_above(m);
    if (e != kNoExp) g.see(e - 100);
  }
  stage_write<CS>(sh, pf, W, lane, 0, g);
  if (nsteps > 1) pf = pre(1);
  lds_barrier();  // (B0b)
  lds_barrier();  // (B0c)

  for (int st = 0; st < nsteps; ++st) {
    const int buf = st & 1;
    const int pe = sh.pub_e;  // published before this step's middle barrier
    if (st + 1 < nsteps) stage_max<CS>(sh, pf, W, lane);
    if (active) {
      // q' factors of this lane's token in each of the two token tiles:
      // qa[tt][X] = q'[16 X + 4 q4 + 0..3], qb[tt][Y] = q'[16 Y + j0 + 0..kJ-1]
      uint2 qa[2][4];
      uint32_t qb[2][4][SL::kJ / 2];  // packed pairs of q'_b
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const _Float16* qrow = sh.qs[buf][32 * TP + 16 * tt + l16];
#pragma unroll
        for (int x = 0; x < 4; ++x)
          if (SL::rd_uses_x(HF, x)) qa[tt][x] = *reinterpret_cast<const uint2*>(qrow + 16 * x + 4 * q4);
#pragma unroll
        for (int y = 0; y < 4; ++y) {
          if (SL::rd_uses_y(HF, y)) {
            if constexpr (SL::kJ == 4) {
              const uint2 w2 = *reinterpret_cast<const uint2*>(qrow + 16 * y + cx.j0);
              qb[tt][y][0] = w2.x;
              qb[tt][y][1] = w2.y;
            } else {
              qb[tt][y][0] = *reinterpret_cast<const uint32_t*>(qrow + 16 * y + cx.j0);
            }
          }
        }
      }
      f32x4 acc[2][2];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) acc[tt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        const int pr = P0 + p;
        f16x8 B[2];
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) B[nt] = __builtin_bit_cast(f16x8, sh.hs[pr][nt][lane]);
        const int u0 = 2 * pr, u1 = 2 * pr + 1;
        const int X0 = SL::X(u0), X1 = SL::X(u1), Y0 = SL::Y(u0), Y1 = SL::Y(u1);
        const int J0 = SL::jj(u0), J1 = SL::jj(u1);
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          // q'_b of each tile, broadcast to both halves (an op_sel of the
          // packed multiply)
          const f16x2 c0 = as_h2(qb[tt][Y0][J0 >> 1]), c1 = as_h2(qb[tt][Y1][J1 >> 1]);
          const f16x2 bb0 = (J0 & 1) ? __builtin_shufflevector(c0, c0, 1, 1) : __builtin_shufflevector(c0, c0, 0, 0);
          const f16x2 bb1 = (J1 & 1) ? __builtin_shufflevector(c1, c1, 1, 1) : __builtin_shufflevector(c1, c1, 0, 0);
          const uint32_t p0 = as_u(as_h2(qa[tt][X0].x) * bb0);
          const uint32_t p1 = as_u(as_h2(qa[tt][X0].y) * bb0);
          const uint32_t p2 = as_u(as_h2(qa[tt][X1].x) * bb1);
          const uint32_t p3 = as_u(as_h2(qa[tt][X1].y) * bb1);
          const f16x8 A = __builtin_bit_cast(f16x8, make_uint4(p0, p1, p2, p3));
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) acc[tt][nt] = mfma_h(A, B[nt], acc[tt][nt]);
        }
      }
      // hand the partner its token tile, keep the own one
      f32x4* xs = &sh.xs[W][0][0];
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        xs[nt * 64 + lane] = acc[1 - HF][nt];
        keep[nt] = acc[HF][nt];
      }
    }
    lds_barrier();  // (B2)
    if (st + 1 < nsteps) {
      stage_write<CS>(sh, pf, W, lane, buf ^ 1, g);
      if (st + 2 < nsteps) pf = pre(st + 2);
    }
    if (active) flush(st, buf, pe);
    lds_barrier();  // (B1)
  }
}

// C: the chunk (intra-chunk region of the output); the state kernel stages it
// in sub-chunks of CS tokens, all read out against the state at the chunk start.
template <int C, int SF, int G>
__global__ __launch_bounds__(kThreads3, 1) void prefill_state_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, int N, int T,
    const float* __restrict__ H0, const float* __restrict__ s0, float* __restrict__ HT, float* __restrict__ sT,
    float* __restrict__ part, float* __restrict__ Sg) {
  constexpr int CS = C < kCS ? C : kCS;
  static_assert(C % CS == 0 && CS % 32 == 0, "chunk must be a multiple of the sub-chunk");
  __shared__ __align__(16) StateLds<SF, G> sh;
  StateCtx cx;
  cx.q = q;
  cx.k = k;
  cx.v = v;
  cx.T = T;
  cx.NC = (T + C - 1) / C;
  cx.D = G * (kDim / G) * (kDim / G + 1) / 2;
  wg_identity(N, SF, cx.n, cx.sf, cx.ch);
  cx.j0 = Slice<SF, G>::kJ * cx.sf;
  cx.H0 = H0;
  cx.s0 = s0;
  cx.HT = HT;
  cx.sT = sT;
  cx.part = part;
  cx.Sg = Sg;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  switch (wv) {
    case 0: update_wave<C, CS, SF, G, 0>(sh, cx); break;
    case 1: update_wave<C, CS, SF, G, 1>(sh, cx); break;
    case 2: update_wave<C, CS, SF, G, 2>(sh, cx); break;
    case 3: update_wave<C, CS, SF, G, 3>(sh, cx); break;
    case 4: readout_wave<C, CS, SF, G, 0>(sh, cx); break;
    case 5: readout_wave<C, CS, SF, G, 1>(sh, cx); break;
    case 6: readout_wave<C, CS, SF, G, 2>(sh, cx); break;
    default: readout_wave<C, CS, SF, G, 3>(sh, cx); break;
  }
}

// ------------------------------------------------------------ finish kernel

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
      s4 = mfma_b(A, B, G == 2 ? f32x4{0.f, 0.f, 0.f, 0.f} : s4);
      if (G == 2) w4 += s4 * s4;
    }
    if (G == 1) w4 = s4 * s4;
  }
  return w4;
}

// One work-group per (chunk, head): intra-chunk term, the denominator's state
// term q^T S q from the Gram matrix of the chunk start, the sum of the slice
// partials -> output. The intra-chunk weights are formed transposed (keys as
// MFMA rows), so the accumulator of two 16-key tiles already is the A operand
// of the 32-key step of A V when its k-slots are read as keys 4 q4 + i (i < 4)
// of the first tile and 4 q4 + i - 4 of the second; the value fragments take
// the same key order. The weights never leave registers.
template <int C, typename Tout, int G>
__global__ __launch_bounds__(kThreads) void prefill_finish_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const float* __restrict__ part, const float* __restrict__ Sg, int SF, Tout* __restrict__ o, int T,
    float eps) {
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

  // the Gram matrix at the chunk start as B fragments of two bf16 pieces:
  // lane (column 16 nt + l16, dims 32 ks + 8 q4 + e); S is symmetric, so the
  // fragment is row 16 nt + l16 of S. For G factors only the factors'
  // diagonal blocks count (phi(q).s = sum over factors of q_f^T S_ff q_f).
  bf16x8 Shi[2][4], Slo[2][4];
  {
    const float* S = Sg + ((size_t)n * gridDim.x + blockIdx.x) * kDim * kDim;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const int col = 16 * nt + l16;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const float4* src = reinterpret_cast<const float4*>(S + col * kDim + 32 * ks + 8 * q4);
        const float4 x0 = src[0], x1 = src[1];
        const float xv[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int d = 32 * ks + 8 * q4 + e;
          const float x = same_factor<G>(d, col) ? xv[e] : 0.0f;
          const __bf16 hi = (__bf16)x;
          Shi[ks][nt][e] = hi;
          Slo[ks][nt][e] = (__bf16)(x - (float)hi);
        }
      }
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
      // the float32 weights as two bf16 pieces (hi + lo carries 16
      // significant bits), so the numerator is formed from the same
      // weights the float32 denominator sums
      bf16x8 A, Alo;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int kq = 2 * ks + h;
        const f32x4 w4 = finish_weights<C, G>(sh, kq, mq, l16, q4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int ki = kq * 16 + 4 * q4 + i;
          const float a = (ki <= qi && ki < L) ? w4[i] : 0.0f;
          dpart += a;
          const __bf16 hi = (__bf16)a;
          A[4 * h + i] = hi;
          Alo[4 * h + i] = (__bf16)(a - (float)hi);
        }
      }
#pragma unroll
      for (int nt4 = 0; nt4 < 4; ++nt4) {
        const uint16_t* vr = &sh.vt[16 * nt4 + l16][ks * 32 + 4 * q4];
        const bf16x4 b0 = *reinterpret_cast<const bf16x4*>(vr);
        const bf16x4 b1 = *reinterpret_cast<const bf16x4*>(vr + 16);
        const bf16x8 B = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
        ra[nt4] = mfma_b(A, B, ra[nt4]);
        ra[nt4] = mfma_b(Alo, B, ra[nt4]);
      }
    }
    // the lanes of one query column hold disjoint keys: add the four groups,
    // then fetch the denominators of the accumulator rows 4 q4 + i
    dpart += __shfl_xor(dpart, 16, 64);
    dpart += __shfl_xor(dpart, 32, 64);
    float den[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) den[i] = __shfl(dpart, 4 * q4 + i, 64) + eps;
    // the state term of the denominator: M = Q S (float32 sums of exact
    // products of q with the two pieces of S), then q . M per query
    {
      f32x4 M[4];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) M[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const bf16x8 Aq = *reinterpret_cast<const bf16x8*>(&sh.qs[mq * 16 + l16][32 * ks + 8 * q4]);
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
          M[nt] = mfma_b(Aq, Shi[ks][nt], M[nt]);
          M[nt] = mfma_b(Aq, Slo[ks][nt], M[nt]);
        }
      }
      // lane holds M[query mq*16 + 4 q4 + i][column 16 nt + l16]
      float dx[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint16_t* qr = sh.qs[mq * 16 + 4 * q4 + i];
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) dx[i] += bf16f(qr[16 * nt + l16]) * M[nt][i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int o2 = 8; o2 > 0; o2 >>= 1) dx[i] += __shfl_xor(dx[i], o2, 64);
        den[i] += dx[i];
      }
    }
    // lane holds O_in[query mq*16 + 4*q4 + i][value 16*nt4 + l16]; the slice
    // partials are float32 in the same order
    const float* pc = part + ((size_t)(n * gridDim.x + blockIdx.x) * SF * (C / 16) + mq) * kTilePart;
#pragma unroll 4
    for (int s = 0; s < SF; ++s) {
      const float* ps = pc + (size_t)s * (C / 16) * kTilePart;
#pragma unroll
      for (int nt4 = 0; nt4 < 4; ++nt4) ra[nt4] += *reinterpret_cast<const f32x4*>(ps + (nt4 * 64 + lane) * 4);
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

// Feature slices per head: 8 while that keeps at most 256 work-groups
// (two per slice), else 4.
int slices_for(int N) { return N <= 16 ? 8 : 4; }

size_t part_bytes(const PrefillArgs& a) {
  const int SF = slices_for(a.N);
  const size_t nc = (a.T + a.chunk - 1) / a.chunk;
  return align_up((size_t)a.N * nc * SF * (a.chunk / 16) * kTilePart * sizeof(float));
}

size_t gram_bytes(const PrefillArgs& a) {
  const size_t nc = (a.T + a.chunk - 1) / a.chunk;
  return align_up((size_t)a.N * nc * kDim * kDim * sizeof(float));
}

template <int C, int SF, int G>
void launch_state(const PrefillArgs& a, float* part, float* Sg, hipStream_t st) {
  hipLaunchKernelGGL((prefill_state_kernel<C, SF, G>), dim3(2 * SF * a.N), dim3(kThreads3), 0, st,
                     static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                     static_cast<const uint16_t*>(a.v), a.N, a.T, a.H0, a.s0, a.HT, a.sT, part, Sg);
}

template <int C, int G>
hipError_t launch_c(const PrefillArgs& a, void* ws, hipStream_t st) {
  float* part = a.o ? static_cast<float*>(ws) : nullptr;
  float* Sg = a.o ? reinterpret_cast<float*>(static_cast<char*>(ws) + part_bytes(a)) : nullptr;
  const int SF = slices_for(a.N);
  prof_begin(st);
  if (SF == 8) launch_state<C, 8, G>(a, part, Sg, st);
  else launch_state<C, 4, G>(a, part, Sg, st);
  prof_end(st);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !part) return e;
  const dim3 grid((a.T + C - 1) / C, a.N);
  if (a.out_bf16)
    hipLaunchKernelGGL((prefill_finish_kernel<C, uint16_t, G>), grid, dim3(kThreads), 0, st,
                       static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                       static_cast<const uint16_t*>(a.v), part, Sg, SF, static_cast<uint16_t*>(a.o), a.T, a.eps);
  else
    hipLaunchKernelGGL((prefill_finish_kernel<C, float, G>), grid, dim3(kThreads), 0, st,
                       static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                       static_cast<const uint16_t*>(a.v), part, Sg, SF, static_cast<float*>(a.o), a.T, a.eps);
  return hipGetLastError();
}

template <int G>
hipError_t launch_g(const PrefillArgs& a, void* ws, hipStream_t st) {
  switch (a.chunk) {
    case 32: return launch_c<32, G>(a, ws, st);
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

size_t prefill_mfma_workspace(const PrefillArgs& a) { return a.o ? part_bytes(a) + gram_bytes(a) : 0; }

hipError_t prefill_mfma_launch(const PrefillArgs& a, void* ws, hipStream_t st) {
  switch (a.factors) {
    case 1: return launch_g<1>(a, ws, st);
    case 2: return launch_g<2>(a, ws, st);
    case 4: return launch_g<4>(a, ws, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace kla
