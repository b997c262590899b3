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
// running exponent G is at least 2 ek + log2 max|v| of every sub-chunk seen
// and large enough that a running bound on every accumulated entry stays
// below 2^14 in units of 2^G; the accumulators hold H 2^-G (rescaled when G
// grows), so the published state, weighted by at most 2, fits float16 as it
// is. Queries are scaled per token (undone before the partials are
// written). Accumulation is float32 throughout; the slice partials are
// float32.
//
// Staging kernel. One work-group per (head, sub-chunk of up to 64 tokens)
// converts the sub-chunk once: the exponents, q rows times 2^-eq (per
// token), k columns times 2^-ek and v columns times 2^-ev (its own largest
// |v|), as float16 in the layout the state kernel copies into LDS.
//
// State kernel, eight waves, stepping through the staged sub-chunks with one
// barrier per step; the staging buffers, the published state and the
// readout trade are double-buffered so no wave waits on another within a
// step.
//   update waves (4) hold their tiles of G for the whole sequence in MFMA
//   accumulators and add phi(K)^T V per 32 tokens (mfma 16x16x32 f16): a lane
//   of the A operand holds feature row r for eight tokens and forms them as
//   packed float16 products of its k_a and of k_b (an LDS broadcast read:
//   the same address on all 16 lanes of a row). In the first value half's
//   work-group each wave also accumulates one X block of the keys' Gram
//   matrix for the slice's columns b (the staged float16 keys hold the bf16
//   keys exactly up to the sub-chunk's power of two: exact products, float32
//   sums). At each chunk end they publish the state of the next chunk's start
//   as float16 B fragments in LDS (diagonal-block rows weighted 2 for a < b,
//   1 for a = b, 0 for the mirror rows), each tile right after its last
//   product, and the Gram matrix to memory.
//   readout waves (4): each takes 32 tokens and half of the tile pairs and
//   reads out phi(Q) G against the state of the chunk start; a lane holds one
//   token and forms its products from q values in registers (q_b doubled for
//   the off-diagonal blocks, whose features weigh 2). The two waves sharing
//   tokens trade halves through LDS, and each writes one float32 partial
//   [16 tokens x 32 columns] per token tile in the MFMA accumulator order,
//   a step later. They also copy the staged sub-chunks into LDS (v scaled to
//   the running exponent) and track the exponents; each sub-chunk is loaded
//   two steps ahead and written one step ahead.
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
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

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

// Largest of the wave's values (all >= 0: they order like their bit
// patterns), on every lane: DPP shifts within rows of 16, then across rows.
__device__ __forceinline__ float wave_max(float x) {
  int v = __float_as_int(x);
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false));  // row_shr:1
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false));  // row_shr:2
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false));  // row_shr:4
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false));  // row_shr:8
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false));  // row_bcast:15
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false));  // row_bcast:31
  return __int_as_float(__builtin_amdgcn_readlane(v, 63));
}

__device__ __forceinline__ f16x2 as_h2(uint32_t x) { return __builtin_bit_cast(f16x2, x); }
__device__ __forceinline__ uint32_t as_u(f16x2 x) { return __builtin_bit_cast(uint32_t, x); }

// Largest |x| of bf16 values as a bf16 bit pattern: |x| orders like the low
// 15 bits of the pattern (packed 16-bit maxima).
__device__ __forceinline__ u16x2 abs_pair(uint32_t x) { return __builtin_bit_cast(u16x2, x & 0x7FFF7FFFu); }
__device__ __forceinline__ u16x2 absmax_pairs(uint4 w) {
  return __builtin_elementwise_max(__builtin_elementwise_max(abs_pair(w.x), abs_pair(w.y)),
                                   __builtin_elementwise_max(abs_pair(w.z), abs_pair(w.w)));
}
__device__ __forceinline__ uint32_t pair_max(u16x2 m) { return max((uint32_t)m[0], (uint32_t)m[1]); }

// Eight bf16 values times 2^e, rounded to float16 (nearest even).
__device__ __forceinline__ uint4 bf16x8_to_f16_scaled_fp(uint4 w, int e) {
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

// The same for scaled values below 1 (every use here), by exponent
// arithmetic on the bit patterns: a bf16 significand fits float16's, so a
// value of float16's normal range is exact; the exponent field is lowered by
// 112 - e with saturation at zero, which flushes what falls below float16's
// normal range (magnitudes under 2^-14) to zero. Needs 112 - e >= 1 (bf16
// subnormals then flush too); below -143, where every value underflows, the
// shift saturates at 255.
__device__ __forceinline__ uint4 bf16x8_to_f16_scaled(uint4 w, int e) {
  if (e > 111) return bf16x8_to_f16_scaled_fp(w, e);
  const unsigned short k = (unsigned short)(min(112 - e, 255) << 7);
  const u16x2 K = {k, k};
  const uint32_t in[4] = {w.x, w.y, w.z, w.w};
  uint32_t out[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const u16x2 m = __builtin_bit_cast(u16x2, in[i] & 0x7FFF7FFFu);
    const u16x2 t = __builtin_elementwise_sub_sat(m, K);
    const u16x2 f = t << (u16x2){3, 3};
    out[i] = (in[i] & 0x80008000u) | __builtin_bit_cast(uint32_t, f);
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

// Lift variants, by the template parameter G: G > 0 the concatenation of G
// factors' rank-one lifts (KATA-Mg; G = 1 the rank-one lift itself), G < 0
// the summed lift of -G factors (KATA-Sigma-g: feature (a, b) of one
// factor's dimensions is sum_f x_(f p + a) x_(f p + b), p = 64 / -G).
__host__ __device__ constexpr int nfac(int G) { return G < 0 ? -G : G; }
__host__ __device__ constexpr bool summed(int G) { return G < 0; }
__host__ __device__ constexpr int fdim(int G) { return kDim / nfac(G); }
// blocks of 16 dimensions between one factor and the next
__host__ __device__ constexpr int fstride(int G) { return fdim(G) / 16; }

// Block pairs of the lift with G factors (KATA-Mg, concatenated factor lifts:
// only pairs of dimensions inside one factor of 64 / G dimensions are
// features): G = 1 all ten, G = 2 the six inside the halves, G = 4 the four
// diagonal blocks. The summed lifts keep the first factor's pairs: three
// (G = -2) or one (G = -4); each of their features adds the same pair of
// blocks of every factor.
__host__ __device__ constexpr int factor_bps(int G) {
  return G == 1 ? 10 : G == 2 ? 6 : G == 4 ? 4 : G == -2 ? 3 : 1;
}
__host__ __device__ constexpr int factor_bp(int G, int i) {
  return G == 1    ? i
         : G == 2  ? (i < 2 ? i : i == 2 ? 4 : i + 4)
         : G == 4  ? (i == 0 ? 0 : i == 1 ? 4 : i == 2 ? 7 : 9)
         : G == -2 ? (i < 2 ? i : 4)
                   : 0;
}

// The tiles of one feature slice: SF = 4 slices hold j = 4 sf + jj (jj < 4),
// SF = 8 slices j = 2 sf + jj (jj < 2), each over the factor structure's
// block pairs. Tile u is (jj = u / kBP, block pair u % kBP); update wave w
// owns tiles [w kNU, (w + 1) kNU), which share one jj; readout pair p is
// tiles (2p, 2p + 1), and readout half h owns pairs [h kNP, (h + 1) kNP).
template <int SF, int G>
struct Slice {
  static_assert(SF == 4 || SF == 8, "feature slices per head");
  static_assert(G == 1 || G == 2 || G == 4 || G == -2 || G == -4, "factors");
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
  // the summed lifts also read the same blocks of the other factors
  static constexpr int kNF = summed(G) ? nfac(G) : 1;
  __host__ __device__ static constexpr bool upd_uses_x(int w, int x) {
    for (int u = w * kNU; u < (w + 1) * kNU; ++u)
      for (int f = 0; f < kNF; ++f)
        if (X(u) + f * fstride(G) == x) return true;
    return false;
  }
  __host__ __device__ static constexpr bool upd_uses_y(int w, int y) {
    for (int u = w * kNU; u < (w + 1) * kNU; ++u)
      for (int f = 0; f < kNF; ++f)
        if (Y(u) + f * fstride(G) == y) return true;
    return false;
  }
  __host__ __device__ static constexpr bool rd_uses_x(int h, int x) {
    for (int u = 2 * h * kNP; u < 2 * (h + 1) * kNP; ++u)
      for (int f = 0; f < kNF; ++f)
        if (X(u) + f * fstride(G) == x) return true;
    return false;
  }
  __host__ __device__ static constexpr bool rd_uses_y(int h, int y) {
    for (int u = 2 * h * kNP; u < 2 * (h + 1) * kNP; ++u)
      for (int f = 0; f < kNF; ++f)
        if (Y(u) + f * fstride(G) == y) return true;
    return false;
  }
};

// Index of feature (a, b), a <= b in one factor, in the ABI's state layout:
// the factors' vec_sym blocks in order, each upper-triangular row-major (the
// summed lifts: one such block, a and b in the first factor).
template <int G>
__device__ __forceinline__ int feat_abi(int a, int b) {
  constexpr int p = fdim(G);
  const int f = a / p;
  const int i = a - f * p, j = b - f * p;
  return f * (p * (p + 1) / 2) + i * p - i * (i - 1) / 2 + (j - i);
}

// Whether the keys' Gram entry (a, b) belongs to the state: a pair inside
// one factor, or for the summed lifts a pair inside the first factor (the
// entry then holds the sum over the factors).
template <int G>
__host__ __device__ __forceinline__ bool same_factor(int a, int b) {
  constexpr int p = fdim(G);
  if (summed(G)) return a < p && b < p;
  return a / p == b / p;
}

template <int SF, int G>
struct StateLds {
  // published state of the chunk start, by chunk parity: float16 B fragments
  // (diagonal-block rows weighted 2 / 1 / 0, other tiles unweighted)
  uint4 hs[2][Slice<SF, G>::kPairs][2][64];
  f32x4 xs[2][kRW][2][64];                // readout trade, by step parity
  // staged sub-chunks, by step parity (sub-chunk s + 1 is staged during s)
  _Float16 qs[2][kCS][kDim + kPad];       // q rows, scaled per token
  _Float16 kt[2][kDim][kCS + kPad];       // k columns, scaled per sub-chunk
  _Float16 vt[2][kCols][kCS + kPad];      // v columns of the work-group's half, scaled
  int qe[2][kCS];                         // per-token query exponent
  int sc[2][2];                           // per buffer: key exponent ek, state exponent G
  float umx[kUW];                         // per update wave, max |imported state|
  int pub_e[2];                           // exponent of the published state, by chunk parity
};

// LDS-only work-group barrier: waits for this wave's LDS traffic, not for
// outstanding global loads.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
}

// The staged sub-chunks come from the staging kernel below: per head and
// sub-chunk of CS tokens, float16 q rows (scaled per token), k columns
// (scaled per sub-chunk) and v columns (scaled by their own maximum), plus
// the exponents. The readout waves copy a sub-chunk into LDS as 16-byte
// pieces: 8 CS of q, 8 CS of k and 4 CS of the work-group's v half, dealt
// round-robin to the 256 lanes r of the four readout waves.
template <int CS>
struct Stage {
  static constexpr int kHalves = 3 * kDim * CS;  // per head and sub-chunk
  static constexpr int kExps = 4 * CS;           // per token: eq, ek, ev, 0
  static constexpr int kPieces = 20 * CS;
  static constexpr int kPerLane = (kPieces + 255) / 256;
};

template <int CS>
struct StageLoad {
  uint4 c[Stage<CS>::kPerLane];
  int eq;      // query exponent of token r (r < CS)
  int ek, ev;  // the sub-chunk's key and value exponents
};

template <int CS>
__device__ __forceinline__ StageLoad<CS> load_stage(const uint16_t* __restrict__ blk, const int* __restrict__ ex,
                                                    int ch, int r) {
  constexpr int RW = CS / 8;  // pieces per k or v column
  StageLoad<CS> L;
  const int4 e4 = *reinterpret_cast<const int4*>(ex + 4 * min(r, CS - 1));
  L.eq = e4.x;
  L.ek = e4.y;
  L.ev = e4.z;
#pragma unroll
  for (int i = 0; i < Stage<CS>::kPerLane; ++i) {
    const int c = r + 256 * i;
    if (c < 8 * CS) {
      L.c[i] = *reinterpret_cast<const uint4*>(blk + (c >> 3) * kDim + 8 * (c & 7));
    } else if (c < 16 * CS) {
      const int e = c - 8 * CS;
      L.c[i] = *reinterpret_cast<const uint4*>(blk + kDim * CS + (e / RW) * CS + 8 * (e % RW));
    } else if (c < 20 * CS) {
      const int e = c - 16 * CS;
      L.c[i] = *reinterpret_cast<const uint4*>(blk + 2 * kDim * CS + (kCols * ch + e / RW) * CS + 8 * (e % RW));
    }
  }
  return L;
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
  const uint16_t* stage;  // staged sub-chunks [head, sub-chunk, kStageHalves]
  const int* exps;        // their exponents [head, sub-chunk, kStageExps]
  int NS;                 // sub-chunks per head
};

// The running state exponent G: the accumulators hold the state times 2^-G.
// It only grows once the accumulators may hold something (an imported state,
// or a sub-chunk with nonzero keys and values); before that it follows the
// first nonzero sub-chunk. It is at least the exponent of every sub-chunk's
// largest possible term (so the scaled values stay below 1), and large
// enough that a running bound b on every accumulated entry, in units of 2^G,
// stays below 2^14: weighted by at most 2, the published state then fits
// float16 without a further scale.
struct ExpTrack {
  int G = 0;
  bool live = false;
  float b = 0.0f;
  __device__ void start(float m) {  // an imported state whose largest entry is m > 0
    G = exp_above(m) - 14;
    b = __builtin_ldexpf(m, -G);
    live = true;
  }
  // n tokens whose every term is below 2^E
  __device__ void add(int E, int n) {
    if (!live) {
      G = E;
      b = 0.0f;
      live = true;
    } else if (E > G) {
      b = __builtin_ldexpf(b, G - E);
      G = E;
    }
    b += __builtin_ldexpf((float)n, E - G);
    if (b >= 16384.0f) {
      const int up = exp_above(b) - 14;
      b = __builtin_ldexpf(b, -up);
      G += up;
    }
  }
};

// Writes a loaded sub-chunk into staging buffer `buf` (v times vs).
template <int CS, class Lds>
__device__ __forceinline__ void write_stage(Lds& sh, const StageLoad<CS>& L, int r, int buf, f16x2 vs) {
  constexpr int RW = CS / 8;
#pragma unroll
  for (int i = 0; i < Stage<CS>::kPerLane; ++i) {
    const int c = r + 256 * i;
    if (c < 8 * CS) {
      *reinterpret_cast<uint4*>(&sh.qs[buf][c >> 3][8 * (c & 7)]) = L.c[i];
    } else if (c < 16 * CS) {
      const int e = c - 8 * CS;
      *reinterpret_cast<uint4*>(&sh.kt[buf][e / RW][8 * (e % RW)]) = L.c[i];
    } else if (c < 20 * CS) {
      const int e = c - 16 * CS;
      const uint4 v = L.c[i];
      const uint4 vv = make_uint4(as_u(as_h2(v.x) * vs), as_u(as_h2(v.y) * vs), as_u(as_h2(v.z) * vs),
                                  as_u(as_h2(v.w) * vs));
      *reinterpret_cast<uint4*>(&sh.vt[buf][e / RW][8 * (e % RW)]) = vv;
    }
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
  // the first value half also forms the Gram matrix (for the summed lifts
  // only its first factor's rows, each the sum over the factors)
  const bool gram_wg = cx.ch == 0 && (!summed(G) || W < fstride(G));

  // Gram column of this lane: the slice's b values 16 Y + j0 + jj
  const int gb = 16 * (l16 / SL::kJ) + cx.j0 + (l16 % SL::kJ);
  const bool gb_ok = l16 < SL::kNB && (!summed(G) || gb < fdim(G));

  // readout weight of the rows 4 q4 .. 4 q4 + 3 of a diagonal-block tile
  // (column j): 2 for a < b, 1 for a = b, 0 for the mirror rows a > b
  f16x2 wdiag[2];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 4 * q4 + i;
    wdiag[i >> 1][i & 1] = (_Float16)(r < j ? 2.0f : (r == j ? 1.0f : 0.0f));
  }

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
  // publish the state at the start of chunk c (float16, diagonal-block rows
  // weighted; the exponent bound keeps every weighted entry below 2^15)
  // publish tile u of the state at the start of chunk c (float16,
  // diagonal-block rows weighted; the exponent bound keeps every weighted
  // entry below 2^15)
  auto publish_tile = [&](int c, int u) {
    const int pb = c & 1;
    const int X = SL::X(U0 + u), Y = SL::Y(U0 + u);
    const int pr = (U0 + u) >> 1;
    const int half = (U0 + u) & 1;
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      f16x2 lo = {(_Float16)h[u][nt][0], (_Float16)h[u][nt][1]};
      f16x2 hi = {(_Float16)h[u][nt][2], (_Float16)h[u][nt][3]};
      if (X == Y) {
        lo *= wdiag[0];
        hi *= wdiag[1];
      }
      uint2* dst = reinterpret_cast<uint2*>(reinterpret_cast<char*>(&sh.hs[pb][pr][nt][lane]) + 8 * half);
      *dst = make_uint2(as_u(lo), as_u(hi));
    }
  };
  // the rest of a publish: the exponent and the Gram matrix at the start of
  // chunk c (each entry a <= b is written by its owner at (a, b) and (b, a))
  auto publish_rest = [&](int c) {
    if (W == 0 && lane == 0) sh.pub_e[c & 1] = Gu;
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
  auto publish = [&](int c) {
#pragma unroll
    for (int u = 0; u < NU; ++u) publish_tile(c, u);
    publish_rest(c);
  };

  lds_barrier();  // (P1) state maxima and the first sub-chunks' maxima posted
  lds_barrier();  // (P2) first sub-chunk staged with its exponents
  Gu = __builtin_amdgcn_readfirstlane(sh.sc[0][1]);
  {
    const float s = __builtin_ldexpf(1.0f, -Gu);
#pragma unroll
    for (int u = 0; u < NU; ++u)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) h[u][nt] *= s;
    publish(0);  // the state at the start of chunk 0
  }
  lds_barrier();  // (P3) initial state published

  for (int st = 0; st < nsteps; ++st) {
    const int buf = st & 1;
    // every operand of the sub-chunk, loaded at once: value fragments, the
    // key rows a of the owned tiles' blocks, and k_b for each b block (the
    // same address on all lanes of a 16-lane row: an LDS broadcast)
    constexpr int KS = CS / 32;
    f16x8 vb[KS][2];
    uint4 ka[KS][4], kb[KS][4];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int t0 = ks * 32 + 8 * q4;
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) vb[ks][nt] = *reinterpret_cast<const f16x8*>(&sh.vt[buf][16 * nt + l16][t0]);
#pragma unroll
      for (int x = 0; x < 4; ++x)
        if (SL::upd_uses_x(W, x)) ka[ks][x] = *reinterpret_cast<const uint4*>(&sh.kt[buf][16 * x + l16][t0]);
#pragma unroll
      for (int y = 0; y < 4; ++y)
        if (SL::upd_uses_y(W, y)) kb[ks][y] = *reinterpret_cast<const uint4*>(&sh.kt[buf][16 * y + j][t0]);
    }
    const int Gn = __builtin_amdgcn_readfirstlane(sh.sc[buf][1]);
    if (Gn != Gu) {  // uniform: the state exponent moved
      const float s = __builtin_ldexpf(1.0f, Gu - Gn);
#pragma unroll
      for (int u = 0; u < NU; ++u)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) h[u][nt] *= s;
      Gu = Gn;
    }
    // at a chunk end the state of the next chunk's start is published into
    // the other buffer (this chunk's readout still reads its own), each tile
    // a few tiles behind its last product so its accumulators are done
    const bool pub = st % SUB == SUB - 1;
    const int cn = st / SUB + 1;
    constexpr int kLag = 2;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int t0 = ks * 32 + 8 * q4;
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        const uint4 xa = ka[ks][SL::X(U0 + u)];
        const uint4 xb = kb[ks][SL::Y(U0 + u)];
        f16x2 p0 = as_h2(xa.x) * as_h2(xb.x);
        f16x2 p1 = as_h2(xa.y) * as_h2(xb.y);
        f16x2 p2 = as_h2(xa.z) * as_h2(xb.z);
        f16x2 p3 = as_h2(xa.w) * as_h2(xb.w);
        // summed lifts: the same pair of blocks of the other factors
#pragma unroll
        for (int f = 1; f < SL::kNF; ++f) {
          const uint4 ya = ka[ks][SL::X(U0 + u) + f * fstride(G)];
          const uint4 yb = kb[ks][SL::Y(U0 + u) + f * fstride(G)];
          p0 += as_h2(ya.x) * as_h2(yb.x);
          p1 += as_h2(ya.y) * as_h2(yb.y);
          p2 += as_h2(ya.z) * as_h2(yb.z);
          p3 += as_h2(ya.w) * as_h2(yb.w);
        }
        const f16x8 A = __builtin_bit_cast(f16x8, make_uint4(as_u(p0), as_u(p1), as_u(p2), as_u(p3)));
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) h[u][nt] = mfma_h(A, vb[ks][nt], h[u][nt]);
        if (ks == KS - 1 && u >= kLag && pub) publish_tile(cn, u - kLag);
      }
      if (gram_wg) {
#pragma unroll
        for (int f = 0; f < SL::kNF; ++f) {
          const int off = 16 * f * fstride(G);
          const f16x8 A = *reinterpret_cast<const f16x8*>(&sh.kt[buf][16 * W + off + l16][t0]);
          f16x8 B = __builtin_bit_cast(f16x8, make_uint4(0, 0, 0, 0));
          if (gb_ok) B = *reinterpret_cast<const f16x8*>(&sh.kt[buf][gb + off][t0]);
          gsub = mfma_h(A, B, gsub);
        }
      }
    }
    if (gram_wg) {
      // the sub-chunk's keys were staged times 2^-ek: exact products, so the
      // float32 Gram matrix gets them back times 4^ek
      const float s = __builtin_ldexpf(1.0f, 2 * __builtin_amdgcn_readfirstlane(sh.sc[buf][0]));
      gram += gsub * s;
      gsub = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    if (pub) {
#pragma unroll
      for (int u = NU > kLag ? NU - kLag : 0; u < NU; ++u) publish_tile(cn, u);
      publish_rest(cn);
    }
    lds_barrier();  // (B) one barrier per sub-chunk
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
  const int tl = 16 * (2 * TP + HF) + 4 * q4;  // tokens tl + i of the own token tile

  f32x4 keep[2];  // own token tile of the previous step, awaiting the partner's half
  float fq[4];    // its scales 2^(2 eq + pe)
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) keep[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 4; ++i) fq[i] = 1.0f;

  // add the partner's half of the own token tile of step st (traded through
  // xs[st & 1]), undo the scales and write the float32 partial
  auto flush = [&](int st, f32x4 k0, f32x4 k1, const float* f) {
    const f32x4 kk[2] = {k0, k1};
    const f32x4* xs = &sh.xs[st & 1][W ^ 1][0][0];
    const int c = st / SUB;
    const int tt = ((st % SUB) * CS) / 16 + 2 * TP + HF;
    float* pc = cx.part + ((((size_t)cx.n * cx.NC + c) * SF + cx.sf) * (C / 16) + tt) * kTilePart;
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const f32x4 o = xs[nt * 64 + lane];
      f32x4 r;
#pragma unroll
      for (int i = 0; i < 4; ++i) r[i] = (kk[nt][i] + o[i]) * f[i];
      *reinterpret_cast<f32x4*>(pc + ((2 * cx.ch + nt) * 64 + lane) * 4) = r;
    }
  };

  // read out the tokens of step st against the state of its chunk start
  auto compute = [&](int st) {
    const int buf = st & 1;
    const int c = st / SUB;
    const int pb = c & 1;
    const int pe = sh.pub_e[pb];
#pragma unroll
    for (int i = 0; i < 4; ++i) fq[i] = __builtin_ldexpf(1.0f, 2 * sh.qe[buf][tl + i] + pe);
    // q' factors of this lane's token in each of the two token tiles:
    // qa[tt][X] = q'[16 X + 4 q4 + 0..3], qb[tt][Y] = q'[16 Y + j0 + 0..kJ-1]
    // (qb2 = 2 qb, the weight of the off-diagonal features)
    uint2 qa[2][4];
    uint32_t qb[2][4][SL::kJ / 2], qb2[2][4][SL::kJ / 2];
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
#pragma unroll
          for (int e = 0; e < SL::kJ / 2; ++e) qb2[tt][y][e] = as_u(as_h2(qb[tt][y][e]) + as_h2(qb[tt][y][e]));
        }
      }
    }
    f32x4 acc[2][2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) acc[tt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    // the state fragments of all pairs, loaded ahead of the products
    f16x8 Bv[NP][2];
#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) Bv[p][nt] = __builtin_bit_cast(f16x8, sh.hs[pb][P0 + p][nt][lane]);
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int pr = P0 + p;
      const f16x8* B = Bv[p];
      const int u0 = 2 * pr, u1 = 2 * pr + 1;
      const int X0 = SL::X(u0), X1 = SL::X(u1), Y0 = SL::Y(u0), Y1 = SL::Y(u1);
      const int J0 = SL::jj(u0), J1 = SL::jj(u1);
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        // q'_b of each tile (doubled off the diagonal blocks), broadcast to
        // both halves (an op_sel of the packed multiply)
        f16x2 p0 = {}, p1 = {}, p2 = {}, p3 = {};
        // summed lifts: the same pair of blocks of every factor
#pragma unroll
        for (int f = 0; f < SL::kNF; ++f) {
          const int o = f * fstride(G);
          const f16x2 c0 = as_h2(X0 < Y0 ? qb2[tt][Y0 + o][J0 >> 1] : qb[tt][Y0 + o][J0 >> 1]);
          const f16x2 c1 = as_h2(X1 < Y1 ? qb2[tt][Y1 + o][J1 >> 1] : qb[tt][Y1 + o][J1 >> 1]);
          const f16x2 bb0 = (J0 & 1) ? __builtin_shufflevector(c0, c0, 1, 1) : __builtin_shufflevector(c0, c0, 0, 0);
          const f16x2 bb1 = (J1 & 1) ? __builtin_shufflevector(c1, c1, 1, 1) : __builtin_shufflevector(c1, c1, 0, 0);
          if (f == 0) {
            p0 = as_h2(qa[tt][X0].x) * bb0;
            p1 = as_h2(qa[tt][X0].y) * bb0;
            p2 = as_h2(qa[tt][X1].x) * bb1;
            p3 = as_h2(qa[tt][X1].y) * bb1;
          } else {
            p0 += as_h2(qa[tt][X0 + o].x) * bb0;
            p1 += as_h2(qa[tt][X0 + o].y) * bb0;
            p2 += as_h2(qa[tt][X1 + o].x) * bb1;
            p3 += as_h2(qa[tt][X1 + o].y) * bb1;
          }
        }
        const f16x8 A = __builtin_bit_cast(f16x8, make_uint4(as_u(p0), as_u(p1), as_u(p2), as_u(p3)));
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) acc[tt][nt] = mfma_h(A, B[nt], acc[tt][nt]);
      }
    }
    // hand the partner its token tile, keep the own one
    f32x4* xs = &sh.xs[buf][W][0][0];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      xs[nt * 64 + lane] = acc[1 - HF][nt];
      keep[nt] = acc[HF][nt];
    }
  };

  // Staging: sub-chunk x's data is loaded at the start of step x - 1 and
  // written to LDS at its end, after the wave's matrix work, so the loads are
  // consumed in the step that issued them. Every readout wave runs the same
  // exponent sequence; wave 0 publishes it with the query exponents.
  const int r = 64 * W + lane;
  ExpTrack g;
  auto blk = [&](int x) { return cx.stage + ((size_t)cx.n * cx.NS + x) * Stage<CS>::kHalves; };
  auto exps = [&](int x) { return cx.exps + ((size_t)cx.n * cx.NS + x) * Stage<CS>::kExps; };
  // exponents of a loaded sub-chunk: advance G, post them to buffer buf,
  // return the v factor
  auto advance = [&](const StageLoad<CS>& L, int buf) {
    const int ekr = __builtin_amdgcn_readfirstlane(L.ek);
    const int ev = __builtin_amdgcn_readfirstlane(L.ev);
    const bool contributes = ekr != kNoExp && ev != kNoExp;
    // a summed lift's features add -G products: their bound is -G times larger
    if (contributes) g.add(2 * ekr + ev + (summed(G) ? (nfac(G) == 2 ? 1 : 2) : 0), CS);
    const int ek = ekr == kNoExp ? 0 : ekr;
    // v was staged times 2^-ev; the update needs it times 2^(2 ek - G)
    const _Float16 f = contributes ? (_Float16)__builtin_ldexpf(1.0f, 2 * ek + ev - g.G) : (_Float16)0.0f;
    if (W == 0) {
      if (lane < CS) sh.qe[buf][lane] = L.eq;
      if (lane == 0) {
        sh.sc[buf][0] = ek;
        sh.sc[buf][1] = g.G;
      }
    }
    return f16x2{f, f};
  };

  // sub-chunk x is loaded during step x - 2 (into register set x & 1) and
  // written to LDS at the end of step x - 1; loads past the last sub-chunk
  // read the last one again (never written)
  const int last = cx.NS - 1;
  StageLoad<CS> La = load_stage<CS>(blk(0), exps(0), cx.ch, r);
  StageLoad<CS> Lb = load_stage<CS>(blk(min(1, last)), exps(min(1, last)), cx.ch, r);
  lds_barrier();  // (P1) imported state maxima posted
  if (cx.H0) {
    const float m = fmaxf(fmaxf(sh.umx[0], sh.umx[1]), fmaxf(sh.umx[2], sh.umx[3]));
    if (m > 0.0f) g.start(m);
  }
  write_stage(sh, La, r, 0, advance(La, 0));
  La = load_stage<CS>(blk(min(2, last)), exps(min(2, last)), cx.ch, r);
  lds_barrier();  // (P2)
  lds_barrier();  // (P3)

  // Ln: sub-chunk st + 1 (loaded a step ago) to write, then receives st + 3
  // The matrix work comes last in the step, so that right after the barrier
  // the update waves' operand reads are not queued behind this wave's reads
  // of the published state.
  auto step = [&](int st, StageLoad<CS>& Ln) {
    if (st >= 1 && active) flush(st - 1, keep[0], keep[1], fq);
    if (st + 1 < cx.NS) write_stage(sh, Ln, r, (st + 1) & 1, advance(Ln, (st + 1) & 1));
    Ln = load_stage<CS>(blk(min(st + 3, last)), exps(min(st + 3, last)), cx.ch, r);
    if (active) compute(st);
    lds_barrier();  // (B)
  };
  int st = 0;
  for (; st + 1 < nsteps; st += 2) {
    step(st, Lb);
    step(st + 1, La);
  }
  if (st < nsteps) step(st, Lb);
  if (active) flush(nsteps - 1, keep[0], keep[1], fq);
}

// ------------------------------------------------------------ staging kernel

// Work-group (g, head) handles sub-chunks g R .. g R + R - 1 of CS tokens:
// the scales and scaled float16 values the state kernel reads (see Stage).
// Thread (t, qd) holds dims 16 qd .. 16 qd + 15 of token t's q, k and v; with
// more than one sub-chunk per work-group, the next sub-chunk's rows are
// loaded while the current one is converted and written. Every element is
// converted once here instead of once per work-group of its head. One
// sub-chunk per work-group measured fastest (of 1, 2 and 4 on 4 x 8 x 4096:
// the most work-groups in flight).
constexpr int kStageR = 1;  // sub-chunks per staging work-group

template <int CS>
__global__ __launch_bounds__(4 * CS) void prefill_stage_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, int T,
    int NS, uint16_t* __restrict__ stage, int* __restrict__ exps) {
  constexpr int NW = 4 * CS / 64;
  constexpr int RW = CS / 8;
  __shared__ __align__(16) _Float16 tk[kDim][CS + kPad];
  __shared__ __align__(16) _Float16 tv[kDim][CS + kPad];
  __shared__ float red[2][2][NW];
  const int n = blockIdx.y;
  const int x0 = blockIdx.x * kStageR;
  const int x1 = min(x0 + kStageR, NS);
  const int tid = threadIdx.x, t = tid >> 2, qd = tid & 3;
  const uint4 z = make_uint4(0, 0, 0, 0);
  struct Rows {
    uint4 q[2], k[2], v[2];
  };
  // rows past the end read the last row (unconditional loads) and are zeroed
  // when used
  auto load = [&](int x, Rows& R) {
    const size_t row = ((size_t)n * T + min(x * CS + t, T - 1)) * kDim + 16 * qd;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      R.q[h] = *reinterpret_cast<const uint4*>(q + row + 8 * h);
      R.k[h] = *reinterpret_cast<const uint4*>(k + row + 8 * h);
      R.v[h] = *reinterpret_cast<const uint4*>(v + row + 8 * h);
    }
  };
  // sub-chunk x from `cur`; the next one is loaded into `nxt` first
  auto body = [&](int x, Rows& cur, Rows& nxt) {
    const int par = (x - x0) & 1;  // the reduction slots alternate
    if (x + 1 < x1) load(x + 1, nxt);
    if (x * CS + t >= T) {
#pragma unroll
      for (int h = 0; h < 2; ++h) cur.q[h] = cur.k[h] = cur.v[h] = z;
    }
    // the token's largest |q| over the four threads holding it (adjacent lanes)
    uint32_t qm = pair_max(__builtin_elementwise_max(absmax_pairs(cur.q[0]), absmax_pairs(cur.q[1])));
    qm = max(qm, (uint32_t)__builtin_amdgcn_mov_dpp((int)qm, 0xB1, 0xF, 0xF, false));  // quad_perm 1,0,3,2
    qm = max(qm, (uint32_t)__builtin_amdgcn_mov_dpp((int)qm, 0x4E, 0xF, 0xF, false));  // quad_perm 2,3,0,1
    const int eqr = exp_above(bf16f(qm));
    const int eq = eqr == kNoExp ? 0 : eqr;
    // the sub-chunk's largest |k| and |v|
    const float km =
        wave_max(bf16f(pair_max(__builtin_elementwise_max(absmax_pairs(cur.k[0]), absmax_pairs(cur.k[1])))));
    const float vm =
        wave_max(bf16f(pair_max(__builtin_elementwise_max(absmax_pairs(cur.v[0]), absmax_pairs(cur.v[1])))));
    if ((tid & 63) == 0) {
      red[par][0][tid >> 6] = km;
      red[par][1][tid >> 6] = vm;
    }
    __syncthreads();  // maxima posted; the previous sub-chunk's transposes read
    float kall = red[par][0][0], vall = red[par][1][0];
#pragma unroll
    for (int w = 1; w < NW; ++w) {
      kall = fmaxf(kall, red[par][0][w]);
      vall = fmaxf(vall, red[par][1][w]);
    }
    const int ekr = exp_above(kall), evr = exp_above(vall);
    const int ek = ekr == kNoExp ? 0 : ekr, ev = evr == kNoExp ? 0 : evr;
    uint16_t* blk = stage + ((size_t)n * NS + x) * Stage<CS>::kHalves;
#pragma unroll
    for (int h = 0; h < 2; ++h)
      *reinterpret_cast<uint4*>(blk + t * kDim + 16 * qd + 8 * h) = bf16x8_to_f16_scaled(cur.q[h], -eq);
    // k and v columns, transposed through LDS
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint4 kh = bf16x8_to_f16_scaled(cur.k[h], -ek), vh = bf16x8_to_f16_scaled(cur.v[h], -ev);
      const uint32_t kw[4] = {kh.x, kh.y, kh.z, kh.w}, vw[4] = {vh.x, vh.y, vh.z, vh.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int d = 16 * qd + 8 * h + 2 * e;
        tk[d][t] = as_h2(kw[e])[0];
        tk[d + 1][t] = as_h2(kw[e])[1];
        tv[d][t] = as_h2(vw[e])[0];
        tv[d + 1][t] = as_h2(vw[e])[1];
      }
    }
    int* e = exps + ((size_t)n * NS + x) * Stage<CS>::kExps;
    if (qd == 0) *reinterpret_cast<int4*>(e + 4 * t) = make_int4(eq, ekr, evr, 0);
    __syncthreads();  // transposes written
    for (int c = tid; c < kDim * RW; c += 4 * CS) {
      const int d = c / RW, j = c % RW;
      *reinterpret_cast<uint4*>(blk + kDim * CS + d * CS + 8 * j) = *reinterpret_cast<const uint4*>(&tk[d][8 * j]);
      *reinterpret_cast<uint4*>(blk + 2 * kDim * CS + d * CS + 8 * j) =
          *reinterpret_cast<const uint4*>(&tv[d][8 * j]);
    }
  };
  Rows A, B;
  load(x0, A);
  int x = x0;
  for (; x + 1 < x1; x += 2) {
    body(x, A, B);
    body(x + 1, B, A);
  }
  if (x < x1) body(x, A, B);
}

// C: the chunk (intra-chunk region of the output); the state kernel steps
// through it in staged sub-chunks of CS tokens, all read out against the
// state at the chunk start.
template <int C, int SF, int G>
__global__ __launch_bounds__(kThreads3, 1) void prefill_state_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, int N, int T,
    const float* __restrict__ H0, const float* __restrict__ s0, float* __restrict__ HT, float* __restrict__ sT,
    float* __restrict__ part, float* __restrict__ Sg, const uint16_t* __restrict__ stage,
    const int* __restrict__ exps) {
  constexpr int CS = C < kCS ? C : kCS;
  static_assert(C % CS == 0 && CS % 32 == 0, "chunk must be a multiple of the sub-chunk");
  __shared__ __align__(16) StateLds<SF, G> sh;
  StateCtx cx;
  cx.q = q;
  cx.k = k;
  cx.v = v;
  cx.T = T;
  cx.NC = (T + C - 1) / C;
  cx.D = (summed(G) ? 1 : G) * fdim(G) * (fdim(G) + 1) / 2;
  wg_identity(N, SF, cx.n, cx.sf, cx.ch);
  cx.j0 = Slice<SF, G>::kJ * cx.sf;
  cx.H0 = H0;
  cx.s0 = s0;
  cx.HT = HT;
  cx.sT = sT;
  cx.part = part;
  cx.Sg = Sg;
  cx.stage = stage;
  cx.exps = exps;
  cx.NS = cx.NC * (C / CS);  // staged sub-chunks per head (whole chunks)
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // the update waves carry the longer dependent chain of each step: let them
  // issue first when both kinds of wave are ready on a SIMD
  if (wv < kUW) __builtin_amdgcn_s_setprio(2);
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
// G factors the sum of the factors' squared scores, or for the summed lifts
// the sum over every pair of factors (i, j) of (q_i . k_j)^2
// (phi(q) . phi(k) of the summed lift).
template <int C, int G>
__device__ __forceinline__ f32x4 finish_weights(const FinishLds<C>& sh, int kq, int mq, int l16, int q4) {
  f32x4 w4 = {0.f, 0.f, 0.f, 0.f};
  if constexpr (G == -2) {
#pragma unroll
    for (int fk = 0; fk < 2; ++fk)
#pragma unroll
      for (int fq = 0; fq < 2; ++fq) {
        const bf16x8 A = *reinterpret_cast<const bf16x8*>(&sh.ks[kq * 16 + l16][32 * fk + 8 * q4]);
        const bf16x8 B = *reinterpret_cast<const bf16x8*>(&sh.qs[mq * 16 + l16][32 * fq + 8 * q4]);
        const f32x4 s4 = mfma_b(A, B, f32x4{0.f, 0.f, 0.f, 0.f});
        w4 += s4 * s4;
      }
  } else if constexpr (G == -4) {
#pragma unroll
    for (int fk = 0; fk < 4; ++fk)
#pragma unroll
      for (int fq = 0; fq < 4; ++fq) {
        const s16x4 A = *reinterpret_cast<const s16x4*>(&sh.ks[kq * 16 + l16][16 * fk + 4 * q4]);
        const s16x4 B = *reinterpret_cast<const s16x4*>(&sh.qs[mq * 16 + l16][16 * fq + 4 * q4]);
        const f32x4 s4 = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(A, B, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
        w4 += s4 * s4;
      }
  } else if constexpr (G == 4) {
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
  // For the summed lifts the state kernel wrote the first factor's block,
  // already summed over the factors (A = sum_f S_ff), and
  // phi(q).s = sum_f q_f^T A q_f: every diagonal block holds A.
  bf16x8 Shi[2][4], Slo[2][4];
  {
    const float* S = Sg + ((size_t)n * gridDim.x + blockIdx.x) * kDim * kDim;
    constexpr int p = fdim(G);
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const int col = 16 * nt + l16;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int d0 = 32 * ks + 8 * q4;
        const float4* src = reinterpret_cast<const float4*>(
            summed(G) ? S + (col % p) * kDim + (d0 % p) : S + col * kDim + d0);
        float4 x0 = make_float4(0.f, 0.f, 0.f, 0.f), x1 = x0;
        if (!summed(G) || d0 / p == col / p) {
          x0 = src[0];
          x1 = src[1];
        }
        const float xv[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int d = 32 * ks + 8 * q4 + e;
          const float x = (summed(G) || same_factor<G>(d, col)) ? xv[e] : 0.0f;
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

bool summed_lift(const PrefillArgs& a) { return a.factor_kind == 1 && a.factors > 1; }

// Feature slices per head: 8 while that keeps at most 256 work-groups
// (two per slice), else 4; 4 for the summed lifts (their 3 or 1 block pairs
// per value of j fill four update waves only with four values of j).
int slices_for(const PrefillArgs& a) { return (a.N <= 16 && !summed_lift(a)) ? 8 : 4; }

size_t part_bytes(const PrefillArgs& a) {
  const int SF = slices_for(a);
  const size_t nc = (a.T + a.chunk - 1) / a.chunk;
  return align_up((size_t)a.N * nc * SF * (a.chunk / 16) * kTilePart * sizeof(float));
}

size_t gram_bytes(const PrefillArgs& a) {
  const size_t nc = (a.T + a.chunk - 1) / a.chunk;
  return align_up((size_t)a.N * nc * kDim * kDim * sizeof(float));
}

int sub_chunk(int chunk) { return chunk < kCS ? chunk : kCS; }

// Staged sub-chunks per head: whole chunks (the state kernel steps through
// every sub-chunk of the last, partial chunk; tokens past T stage as zeros).
size_t staged_sub_chunks(const PrefillArgs& a) {
  return (size_t)((a.T + a.chunk - 1) / a.chunk) * (a.chunk / sub_chunk(a.chunk));
}

size_t stage_bytes(const PrefillArgs& a) {
  return align_up((size_t)a.N * staged_sub_chunks(a) * 3 * kDim * sub_chunk(a.chunk) * sizeof(uint16_t));
}

size_t exps_bytes(const PrefillArgs& a) {
  return align_up((size_t)a.N * staged_sub_chunks(a) * 4 * sub_chunk(a.chunk) * sizeof(int));
}

template <int C, int SF, int G>
void launch_state(const PrefillArgs& a, float* part, float* Sg, const uint16_t* stage, const int* exps,
                  hipStream_t st) {
  hipLaunchKernelGGL((prefill_state_kernel<C, SF, G>), dim3(2 * SF * a.N), dim3(kThreads3), 0, st,
                     static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                     static_cast<const uint16_t*>(a.v), a.N, a.T, a.H0, a.s0, a.HT, a.sT, part, Sg, stage, exps);
}

template <int C, int G>
hipError_t launch_c(const PrefillArgs& a, void* ws, hipStream_t st) {
  constexpr int CS = C < kCS ? C : kCS;
  char* p = static_cast<char*>(ws);
  uint16_t* stage = reinterpret_cast<uint16_t*>(p);
  int* exps = reinterpret_cast<int*>(p + stage_bytes(a));
  char* rest = p + stage_bytes(a) + exps_bytes(a);
  float* part = a.o ? reinterpret_cast<float*>(rest) : nullptr;
  float* Sg = a.o ? reinterpret_cast<float*>(rest + part_bytes(a)) : nullptr;
  const int SF = slices_for(a);
  const int ns = (int)staged_sub_chunks(a);
  hipLaunchKernelGGL((prefill_stage_kernel<CS>), dim3((ns + kStageR - 1) / kStageR, a.N), dim3(4 * CS), 0, st,
                     static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                     static_cast<const uint16_t*>(a.v), a.T, ns, stage, exps);
  prof_begin(st);
  if constexpr (summed(G)) {
    launch_state<C, 4, G>(a, part, Sg, stage, exps, st);
  } else {
    if (SF == 8) launch_state<C, 8, G>(a, part, Sg, stage, exps, st);
    else launch_state<C, 4, G>(a, part, Sg, stage, exps, st);
  }
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
         (a.factor_kind == 0 || a.factor_kind == 1) && (a.factors == 1 || a.factors == 2 || a.factors == 4);
}

size_t prefill_mfma_workspace(const PrefillArgs& a) {
  return stage_bytes(a) + exps_bytes(a) + (a.o ? part_bytes(a) + gram_bytes(a) : 0);
}

hipError_t prefill_mfma_launch(const PrefillArgs& a, void* ws, hipStream_t st) {
  if (summed_lift(a)) {
    if (a.factors == 2) return launch_g<-2>(a, ws, st);
    if (a.factors == 4) return launch_g<-4>(a, ws, st);
    return hipErrorInvalidValue;
  }
  switch (a.factors) {
    case 1: return launch_g<1>(a, ws, st);
    case 2: return launch_g<2>(a, ws, st);
    case 4: return launch_g<4>(a, ws, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace kla
