// Chunked causal prefill on the bf16 matrix cores (d_qk = d_v = 64).
//
// KATA page, §2.3 ("Paralelismo por Blocos"; the linear chunked-state
// operating point): inside a chunk, masked (Q K^T)∘(Q K^T) scores multiply
// [V | 1]; across chunks the state (H, s) is a running prefix sum, read out by
// phi(Q) and updated by phi(K)^T [V | 1]. The lift is the rank-one PSD feature
// of KATA §2.2, phi(x)_ab = x_a x_b (times sqrt(2) off the diagonal).
//
// Feature order inside the kernels. Features (a, b), a <= b, are addressed by
// (a, e = b - a) and grouped in 4x4 blocks of that triangle: tile (i, j) holds
// a = 4i + g, e = 4j + c for g, c in 0..3, as tile row r = 4g + c. The 136
// tiles cover the 2080 features; the 16 tiles on the anti-diagonal are only
// partly inside the triangle (b > 63), and their outside rows stay zero
// because the k rows beyond the last dimension read as zero. The internal
// state keeps x_a x_b without the sqrt(2); the readout uses 2 q_a q_b off the
// diagonal instead, and the state is rescaled when it crosses the ABI.
//
// State kernel. A work-group owns one head and a contiguous range of tiles
// (a feature slice) and walks the chunks in order, a staged sub-chunk of q,
// k and v at a time. Its four update waves split the tiles and keep their
// slice of H in MFMA accumulators (fp32) and of s in LDS:
//   update   H += phi(K)^T V (MFMA 16x16x32 bf16), s += phi(K)^T 1;
// at each chunk end they publish the state as bf16 MFMA B fragments in LDS
// (double buffered). Its four readout waves each take a 16-token tile and
// read out against the state of the chunk start:
//   readout  num_x = phi(Q) H (MFMA), den_x = phi(Q) s (bf16 dot products),
// partial over the slice, written as bf16 to a workspace [head, chunk,
// slice, token tile, 16 x (d_v + 1)] in the MFMA accumulator order, so that
// both its writes and the finish kernel's reads are whole 512-byte runs per
// wave. A head's work-groups are placed on one XCD
// (work-groups are dealt to the 8 XCDs in turn), so their shared q, k and v
// reads meet in one L2.
//
// Finish kernel. One work-group per (head, chunk): the exact intra-chunk
// term A [V | 1] with A = lower-triangular (Q K^T)^2 (MFMA), plus the sum of
// the slice partials, divided, cast to the output type.
#include <algorithm>

#include "kla_device.hpp"
#include "kla_internal.hpp"

namespace kla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kDim = 64;                          // d_qk = d_v
constexpr int kD = kDim * (kDim + 1) / 2;         // 2080
constexpr int kBlk = kDim / 4;                    // 16 blocks per side
constexpr int kTiles = kBlk * (kBlk + 1) / 2;     // 136
constexpr int kTW = 5;                            // tiles per wave, at most
constexpr int kMinSlices = 8;                     // tiles per work-group <= 17
constexpr int kKR = kDim + 4;                     // k^T rows; 64..67 are zero
constexpr int kAcc = kDim + 1;                    // accumulator row: num | den
// Slice partials of one 16-token tile (bf16): the numerators in MFMA
// accumulator order [n-tile][lane][4 tokens], then the 16 denominators.
constexpr int kTileAcc = 16 * kAcc;

__device__ __forceinline__ void tile_coords(int t, int& i, int& j) {
  int start = 0;
  i = 0;
  while (start + (kBlk - i) <= t) {
    start += kBlk - i;
    ++i;
  }
  j = t - start;
}

__device__ __forceinline__ int feat_index(int a, int b) { return a * kDim - a * (a - 1) / 2 + (b - a); }

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

__device__ __forceinline__ bf16x8 join(const bf16x4& lo, const bf16x4& hi) {
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Sum of 8 bf16 products a_j * b_j added to c (four v_dot2 steps).
__device__ __forceinline__ float dot8(const bf16x8& a, const bf16x8& b, float c) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    bf16x2 x = {a[2 * j], a[2 * j + 1]};
    bf16x2 y = {b[2 * j], b[2 * j + 1]};
    c = __builtin_amdgcn_fdot2_f32_bf16(x, y, c, false);
  }
  return c;
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

constexpr int kUW = 4;                            // update waves (own H)
constexpr int kRW = 4;                            // readout waves (own token tiles)
constexpr int kThreads3 = 64 * (kUW + kRW);
constexpr int kWG = kUW * kTW;                    // tiles per work-group, at most (>= 17)
constexpr int kPairs = (kTiles / kMinSlices + 1) / 2;   // readout k-steps: 9
constexpr int kCS = 64;                           // staged sub-chunk (tokens)

static_assert(kTiles / kMinSlices + 1 <= kWG, "a work-group's tiles must fit its update waves");

template <int CS>
struct StateLds {
  // q and k transposed (fp32, rows 64..67 zero); the row paddings spread the
  // readout's and the update's reads over the LDS banks
  float qt[kKR][CS + 16];
  float kt[kKR][CS + 12];
  uint16_t vt[kDim][CS + 8];                      // v transposed (bf16)
  uint4 hs[2][kPairs][4][64];                     // H as bf16 B fragments, double buffer
  uint4 ss[2][kPairs][4];                         // s as bf16 per pair and lane quarter
  float s[kUW][kTW][16];                          // s slice per update-wave tile (fp32)
};

// LDS-only work-group barrier: waits for this wave's LDS traffic, not for
// outstanding global loads or atomics.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
}

// One 16-byte group (8 dims) of q, k and v for one token of the next sub-chunk.
struct Prefetch {
  uint4 q, k, v;
};

template <int CS>
__device__ __forceinline__ Prefetch prefetch(const uint16_t* __restrict__ q,
                                             const uint16_t* __restrict__ k,
                                             const uint16_t* __restrict__ v, size_t row, int L,
                                             int t, int grp) {
  Prefetch p;
  p.q = make_uint4(0, 0, 0, 0);
  p.k = p.q;
  p.v = p.q;
  if (t < L) {
    const size_t off = (row + t) * kDim + 8 * grp;
    p.q = *reinterpret_cast<const uint4*>(q + off);
    p.k = *reinterpret_cast<const uint4*>(k + off);
    p.v = *reinterpret_cast<const uint4*>(v + off);
  }
  return p;
}

template <int CS>
__device__ __forceinline__ void stage(StateLds<CS>& sh, const Prefetch& p, int t, int grp) {
  const uint32_t qw[4] = {p.q.x, p.q.y, p.q.z, p.q.w};
  const uint32_t kw[4] = {p.k.x, p.k.y, p.k.z, p.k.w};
  const uint32_t vw[4] = {p.v.x, p.v.y, p.v.z, p.v.w};
  const int d0 = 8 * grp;
  float4 lo, hi;
  lo.x = bf16f(qw[0] & 0xFFFF); lo.y = bf16f(qw[0] >> 16);
  lo.z = bf16f(qw[1] & 0xFFFF); lo.w = bf16f(qw[1] >> 16);
  hi.x = bf16f(qw[2] & 0xFFFF); hi.y = bf16f(qw[2] >> 16);
  hi.z = bf16f(qw[3] & 0xFFFF); hi.w = bf16f(qw[3] >> 16);
  sh.qt[d0][t] = lo.x;
  sh.qt[d0 + 1][t] = lo.y;
  sh.qt[d0 + 2][t] = lo.z;
  sh.qt[d0 + 3][t] = lo.w;
  sh.qt[d0 + 4][t] = hi.x;
  sh.qt[d0 + 5][t] = hi.y;
  sh.qt[d0 + 6][t] = hi.z;
  sh.qt[d0 + 7][t] = hi.w;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    sh.kt[d0 + 2 * e][t] = bf16f(kw[e] & 0xFFFF);
    sh.kt[d0 + 2 * e + 1][t] = bf16f(kw[e] >> 16);
    sh.vt[d0 + 2 * e][t] = (uint16_t)(vw[e] & 0xFFFF);
    sh.vt[d0 + 2 * e + 1][t] = (uint16_t)(vw[e] >> 16);
  }
}

// Publish an update wave's H tiles (bf16 B fragments) and s (bf16).
__device__ __forceinline__ void publish_state(uint4 (*hs)[4][64], uint4 (*ss)[4],
                                              const f32x4 (&h)[kTW][4], const float (*s_w)[16],
                                              int lw0, int ntw, int lane) {
#pragma unroll
  for (int u = 0; u < kTW; ++u) {
    if (u < ntw) {
      const int lt = lw0 + u;
      const int pr = lt >> 1;
      const int half = lt & 1;
#pragma unroll
      for (int nt4 = 0; nt4 < 4; ++nt4) {
        bf16x4 b;
#pragma unroll
        for (int i = 0; i < 4; ++i) b[i] = (__bf16)h[u][nt4][i];
        *reinterpret_cast<bf16x4*>(reinterpret_cast<char*>(&hs[pr][nt4][lane]) + 8 * half) = b;
      }
      if (lane < 16) {
        const __bf16 x = (__bf16)s_w[u][lane];
        reinterpret_cast<uint16_t*>(&ss[pr][lane >> 2])[4 * half + (lane & 3)] =
            __builtin_bit_cast(uint16_t, x);
      }
    }
  }
}

// C: the chunk (intra-chunk region of the output); the state kernel stages it
// in sub-chunks of CS tokens, all read out against the state at the chunk start.
template <int C, int CS, int NP>
__global__ __launch_bounds__(kThreads3, 1) void prefill_state_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, int N, int T, int S, const float* __restrict__ H0,
    const float* __restrict__ s0, float* __restrict__ HT, float* __restrict__ sT,
    uint16_t* __restrict__ part) {
  static_assert(C % CS == 0 && CS % 32 == 0, "chunk must be a multiple of the sub-chunk");
  constexpr int SUB = C / CS;                 // sub-steps per chunk
  constexpr int MT = CS / 16;                 // token tiles per sub-chunk
  static_assert(NP <= kPairs, "pair count");
  __shared__ __align__(16) StateLds<CS> sh;
  const int NC = (T + C - 1) / C;

  int n, slice;
  wg_identity(N, S, n, slice);
  const int tid = threadIdx.x;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool upd = wv < kUW;                  // update wave, else readout wave
  const int w = upd ? wv : wv - kUW;
  const int lane = tid & 63;
  const int l16 = lane & 15;
  const int q4 = lane >> 4;
  // staging role: token = lane, 8-dim group = wave
  const int st_t = lane;
  const int st_g = wv;

  const int tb = (slice * kTiles) / S;
  const int nt = ((slice + 1) * kTiles) / S - tb;
  const int base = nt / kUW;
  const int extra = nt % kUW;
  const int ntw = upd ? base + (w < extra ? 1 : 0) : 0;
  const int lw0 = w * base + min(w, extra);

  // zero pads and both fragment buffers
  for (int i = tid; i < CS * 4; i += kThreads3) sh.qt[kDim + (i & 3)][i >> 2] = 0.0f;
  for (int i = tid; i < 4 * (CS + 12); i += kThreads3) sh.kt[kDim + i / (CS + 12)][i % (CS + 12)] = 0.0f;
  for (int i = tid; i < 2 * kPairs * 4 * 64; i += kThreads3) (&sh.hs[0][0][0][0])[i] = make_uint4(0, 0, 0, 0);
  for (int i = tid; i < 2 * kPairs * 4; i += kThreads3) (&sh.ss[0][0][0])[i] = make_uint4(0, 0, 0, 0);

  const float inv_sqrt2 = 0.70710678118654752f;
  const size_t row0 = (size_t)n * T;
  const int nsteps = ((T + C - 1) / C) * SUB;

  // first sub-chunk in flight while the state is set up
  Prefetch pf = prefetch<CS>(q, k, v, row0, min(CS, T), st_t, st_g);

  if (upd) {
    // -------------------------------------------------------------- update waves
    int ti[kTW], tj[kTW];
#pragma unroll
    for (int u = 0; u < kTW; ++u) {
      ti[u] = 0;
      tj[u] = 0;
      if (u < ntw) tile_coords(tb + lw0 + u, ti[u], tj[u]);
    }
    f32x4 h[kTW][4];
#pragma unroll
    for (int u = 0; u < kTW; ++u) {
#pragma unroll
      for (int nt4 = 0; nt4 < 4; ++nt4) h[u][nt4] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (H0 && u < ntw) {
#pragma unroll
        for (int nt4 = 0; nt4 < 4; ++nt4) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int a = 4 * ti[u] + q4;
            const int b = a + 4 * tj[u] + i;
            if (b < kDim)
              h[u][nt4][i] = H0[((size_t)n * kD + feat_index(a, b)) * kDim + 16 * nt4 + l16] *
                             (a < b ? inv_sqrt2 : 1.0f);
          }
        }
      }
    }
    if (lane < 16) {
#pragma unroll
      for (int u = 0; u < kTW; ++u) {
        float x = 0.0f;
        if (s0 && u < ntw) {
          const int a = 4 * ti[u] + (lane >> 2);
          const int b = a + 4 * tj[u] + (lane & 3);
          if (b < kDim) x = s0[(size_t)n * kD + feat_index(a, b)] * (a < b ? inv_sqrt2 : 1.0f);
        }
        sh.s[w][u][lane] = x;
      }
    }
    lds_barrier();  // zero fill done
    publish_state(sh.hs[1], sh.ss[1], h, sh.s[w], lw0, ntw, lane);

    const int g = l16 >> 2;
    const int cc = l16 & 3;
    for (int st = 0; st < nsteps; ++st) {
      const int c0 = (st / SUB) * C + (st % SUB) * CS;
      if (st_t < CS) stage<CS>(sh, pf, st_t, st_g);
      lds_barrier();  // (B1) sub-chunk staged
      if (st + 1 < nsteps) {
        const int n0 = ((st + 1) / SUB) * C + ((st + 1) % SUB) * CS;
        pf = prefetch<CS>(q, k, v, row0 + n0, min(CS, T - n0), st_t, st_g);
      }
      float dsum[kTW];
#pragma unroll
      for (int u = 0; u < kTW; ++u) dsum[u] = 0.0f;
#pragma unroll
      for (int ks = 0; ks < CS / 32; ++ks) {
        bf16x8 vb[4];
#pragma unroll
        for (int nt4 = 0; nt4 < 4; ++nt4)
          vb[nt4] = *reinterpret_cast<const bf16x8*>(&sh.vt[16 * nt4 + l16][ks * 32 + 8 * q4]);
#pragma unroll
        for (int u = 0; u < kTW; ++u) {
          if (u < ntw) {
            const int a = 4 * ti[u] + g;
            const int b = a + 4 * tj[u] + cc;
            const float4* ka = reinterpret_cast<const float4*>(&sh.kt[a][ks * 32 + 8 * q4]);
            const float4* kb = reinterpret_cast<const float4*>(&sh.kt[b][ks * 32 + 8 * q4]);
            const float4 a0 = ka[0], a1 = ka[1], b0 = kb[0], b1 = kb[1];
            float p[8] = {a0.x * b0.x, a0.y * b0.y, a0.z * b0.z, a0.w * b0.w,
                          a1.x * b1.x, a1.y * b1.y, a1.z * b1.z, a1.w * b1.w};
            dsum[u] += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
            const bf16x8 A = pack8(p);
#pragma unroll
            for (int nt4 = 0; nt4 < 4; ++nt4) h[u][nt4] = mfma(A, vb[nt4], h[u][nt4]);
          }
        }
      }
#pragma unroll
      for (int u = 0; u < kTW; ++u) {
        float d = dsum[u];
        d += __shfl_xor(d, 16, 64);
        d += __shfl_xor(d, 32, 64);
        if (q4 == 0 && u < ntw) sh.s[w][u][l16] += d;
      }
      if (st % SUB == SUB - 1) {
        const int c = st / SUB;
        publish_state(sh.hs[c & 1], sh.ss[c & 1], h, sh.s[w], lw0, ntw, lane);
      }
      (void)c0;
      lds_barrier();  // (B2) sub-chunk consumed
    }

    // final state in the ABI layout (sqrt(2) on the off-diagonal rows)
    const float sqrt2 = 1.41421356237309504880f;
    if (HT) {
#pragma unroll
      for (int u = 0; u < kTW; ++u) {
        if (u < ntw) {
#pragma unroll
          for (int nt4 = 0; nt4 < 4; ++nt4) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int a = 4 * ti[u] + q4;
              const int b = a + 4 * tj[u] + i;
              if (b < kDim)
                HT[((size_t)n * kD + feat_index(a, b)) * kDim + 16 * nt4 + l16] =
                    h[u][nt4][i] * (a < b ? sqrt2 : 1.0f);
            }
          }
        }
      }
    }
    if (sT && lane < 16) {
      for (int u = 0; u < ntw; ++u) {
        const int a = 4 * ti[u] + (lane >> 2);
        const int b = a + 4 * tj[u] + (lane & 3);
        if (b < kDim) sT[(size_t)n * kD + feat_index(a, b)] = sh.s[w][u][lane] * (a < b ? sqrt2 : 1.0f);
      }
    }
  } else {
    // -------------------------------------------------------------- readout waves
    int gi[2 * NP], gj[2 * NP];  // coordinates of the work-group's tiles
#pragma unroll
    for (int u = 0; u < 2 * NP; ++u) {
      gi[u] = 0;
      gj[u] = 0;
      if (u < nt) tile_coords(tb + u, gi[u], gj[u]);
    }
    lds_barrier();  // zero fill done (matches the update waves' first barrier)
    for (int st = 0; st < nsteps; ++st) {
      const int c = st / SUB;
      const int c0 = c * C + (st % SUB) * CS;
      const int L = min(CS, T - c0);
      if (st_t < CS) stage<CS>(sh, pf, st_t, st_g);
      lds_barrier();  // (B1)
      if (st + 1 < nsteps) {
        const int n0 = ((st + 1) / SUB) * C + ((st + 1) % SUB) * CS;
        pf = prefetch<CS>(q, k, v, row0 + n0, min(CS, T - n0), st_t, st_g);
      }
      if (part && w < MT) {
        const int pb = (c + 1) & 1;  // the state at the chunk start
        f32x4 ra[4];
#pragma unroll
        for (int nt4 = 0; nt4 < 4; ++nt4) ra[nt4] = f32x4{0.f, 0.f, 0.f, 0.f};
        float dn = 0.0f;
        const int qcol = w * 16 + l16;
        // absent tiles have zero fragments in hs/ss, so they add nothing
#pragma unroll
        for (int pr = 0; pr < NP; ++pr) {
          bf16x8 B[4];
#pragma unroll
          for (int nt4 = 0; nt4 < 4; ++nt4) B[nt4] = __builtin_bit_cast(bf16x8, sh.hs[pb][pr][nt4][lane]);
          const bf16x8 sv = __builtin_bit_cast(bf16x8, sh.ss[pb][pr][q4]);
          const int ae = 4 * gi[2 * pr] + q4;
          const int be = 4 * (gi[2 * pr] + gj[2 * pr]) + q4;
          const int ao = 4 * gi[2 * pr + 1] + q4;
          const int bo = 4 * (gi[2 * pr + 1] + gj[2 * pr + 1]) + q4;
          // doubled off-diagonal weight; the diagonal feature (first column of
          // a tile with j == 0) keeps 1
          const float qe = 2.0f * sh.qt[ae][qcol];
          const float qo = 2.0f * sh.qt[ao][qcol];
          const float de = gj[2 * pr] == 0 ? 0.5f : 1.0f;
          const float dd = gj[2 * pr + 1] == 0 ? 0.5f : 1.0f;
          float p[8];
#pragma unroll
          for (int cc = 0; cc < 4; ++cc) {
            p[cc] = qe * sh.qt[be + cc][qcol];
            p[4 + cc] = qo * sh.qt[bo + cc][qcol];
          }
          p[0] *= de;
          p[4] *= dd;
          const bf16x8 A = pack8(p);
          dn = dot8(A, sv, dn);
#pragma unroll
          for (int nt4 = 0; nt4 < 4; ++nt4) ra[nt4] = mfma(A, B[nt4], ra[nt4]);
        }
        // lane holds num for tokens w*16 + 4*q4 + i, column 16*nt4 + l16;
        // the partial block of this token tile keeps that layout (bf16)
        const int tt = ((st % SUB) * CS) / 16 + w;
        uint16_t* pc = part + ((((size_t)n * NC + c) * S + slice) * (C / 16) + tt) * kTileAcc;
#pragma unroll
        for (int nt4 = 0; nt4 < 4; ++nt4) {
          bf16x4 b;
#pragma unroll
          for (int i = 0; i < 4; ++i) b[i] = (__bf16)ra[nt4][i];
          *reinterpret_cast<bf16x4*>(pc + (nt4 * 64 + lane) * 4) = b;
        }
        dn += __shfl_xor(dn, 16, 64);
        dn += __shfl_xor(dn, 32, 64);
        if (q4 == 0) pc[4 * 64 * 4 + l16] = __builtin_bit_cast(uint16_t, (__bf16)dn);
        (void)L;
      }
      lds_barrier();  // (B2)
    }
  }
}


template <int C>
struct FinishLds {
  uint16_t qs[C][kDim + 8];
  uint16_t ks[C][kDim + 8];
  uint16_t vt[kDim][C + 8];
  uint16_t at[C][C + 8];
  float den[C];
};

// One work-group per (chunk, head): intra-chunk term + accumulator -> output.
template <int C, typename Tout>
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
  for (int i = tid; i < C; i += kThreads) sh.den[i] = 0.0f;
  __syncthreads();

  // A = lower-triangular (Q K^T)^2 for the query tiles of this wave; each
  // query tile mq needs key tiles up to the end of its 32-key step.
  for (int mq = w; mq < C / 16; mq += kWaves) {
    const int kmax = ((mq >> 1) << 1) + 1;  // last key tile of the 32-key step
    float den_part[4] = {0.f, 0.f, 0.f, 0.f};
    for (int kq = 0; kq <= kmax && kq < C / 16; ++kq) {
      f32x4 s4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < kDim / 32; ++ks) {
        const bf16x8 A = *reinterpret_cast<const bf16x8*>(&sh.qs[mq * 16 + l16][ks * 32 + 8 * q4]);
        const bf16x8 B = *reinterpret_cast<const bf16x8*>(&sh.ks[kq * 16 + l16][ks * 32 + 8 * q4]);
        s4 = mfma(A, B, s4);
      }
      // lane holds S[query mq*16 + 4*q4 + i][key kq*16 + l16]
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int qi = mq * 16 + 4 * q4 + i;
        const int ki = kq * 16 + l16;
        const float sq = s4[i] * s4[i];
        const float a = (ki <= qi && ki < L) ? sq : 0.0f;
        den_part[i] += a;
        sh.at[qi][ki] = __builtin_bit_cast(uint16_t, (__bf16)a);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float d = den_part[i];
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) d += __shfl_xor(d, off, 64);
      if (l16 == 0) sh.den[mq * 16 + 4 * q4 + i] = d;
    }
  }
  __syncthreads();

  for (int mq = w; mq < C / 16; mq += kWaves) {
    f32x4 ra[4];
#pragma unroll
    for (int nt4 = 0; nt4 < 4; ++nt4) ra[nt4] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int ks = 0; ks <= (mq >> 1); ++ks) {
      const bf16x8 A = *reinterpret_cast<const bf16x8*>(&sh.at[mq * 16 + l16][ks * 32 + 8 * q4]);
#pragma unroll
      for (int nt4 = 0; nt4 < 4; ++nt4) {
        const bf16x8 B = *reinterpret_cast<const bf16x8*>(&sh.vt[16 * nt4 + l16][ks * 32 + 8 * q4]);
        ra[nt4] = mfma(A, B, ra[nt4]);
      }
    }
    // lane holds O_in[query mq*16 + 4*q4 + i][value 16*nt4 + l16]; the slice
    // partials hold four consecutive tokens of one column as bf16
    float den[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) den[i] = sh.den[mq * 16 + 4 * q4 + i] + eps;
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

int cu_count() {
  static int cached = 0;
  if (cached == 0) {
    int dev = 0;
    int cus = 256;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && cus > 0)
      cached = cus;
    else
      cached = 256;
  }
  return cached;
}

int slices_for(int N) {
  const int want = (cu_count() + N - 1) / N;
  return std::min(kTiles, std::max(kMinSlices, want));
}

// pairs per readout pass for S slices (tiles per work-group rounded up, halved)
int pairs_for(int S) { return ((kTiles + S - 1) / S + 1) / 2; }

size_t part_bytes(const PrefillArgs& a) {
  const int S = slices_for(a.N);
  const size_t nc = (a.T + a.chunk - 1) / a.chunk;
  return align_up((size_t)a.N * nc * S * kAcc * a.chunk * sizeof(uint16_t));
}

template <int C, int NP>
void launch_state(const PrefillArgs& a, int S, uint16_t* part, hipStream_t st) {
  hipLaunchKernelGGL((prefill_state_kernel<C, (C < kCS ? C : kCS), NP>), dim3(S * a.N), dim3(kThreads3), 0, st,
                     static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                     static_cast<const uint16_t*>(a.v), a.N, a.T, S, a.H0, a.s0, a.HT, a.sT, part);
}

template <int C>
hipError_t launch_c(const PrefillArgs& a, void* ws, hipStream_t st) {
  uint16_t* part = a.o ? static_cast<uint16_t*>(ws) : nullptr;
  const int S = slices_for(a.N);
  const int np = pairs_for(S);
  prof_begin(st);
  if (np > 5) launch_state<C, kPairs>(a, S, part, st);
  else if (np > 3) launch_state<C, 5>(a, S, part, st);
  else if (np > 1) launch_state<C, 3>(a, S, part, st);
  else launch_state<C, 1>(a, S, part, st);
  prof_end(st);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !part) return e;
  const dim3 grid((a.T + C - 1) / C, a.N);
  if (a.out_bf16)
    hipLaunchKernelGGL((prefill_finish_kernel<C, uint16_t>), grid, dim3(kThreads), 0, st,
                       static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                       static_cast<const uint16_t*>(a.v), part, S, static_cast<uint16_t*>(a.o), a.T, a.eps);
  else
    hipLaunchKernelGGL((prefill_finish_kernel<C, float>), grid, dim3(kThreads), 0, st,
                       static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                       static_cast<const uint16_t*>(a.v), part, S, static_cast<float*>(a.o), a.T, a.eps);
  return hipGetLastError();
}

}  // namespace

bool prefill_mfma_supported(const PrefillArgs& a) {
  return a.in_bf16 && a.dqk == kDim && a.dv == kDim &&
         (a.chunk == 32 || a.chunk == 64 || a.chunk == 128);
}

size_t prefill_mfma_workspace(const PrefillArgs& a) { return a.o ? part_bytes(a) : 0; }

hipError_t prefill_mfma_launch(const PrefillArgs& a, void* ws, hipStream_t st) {
  switch (a.chunk) {
    case 32: return launch_c<32>(a, ws, st);
    case 64: return launch_c<64>(a, ws, st);
    case 128: return launch_c<128>(a, ws, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace kla
