// Causal prefill in the quadratic form on the bf16 matrix cores (d_qk = d_v
// = 64, bf16 inputs).
//
// KATA page, §2.3, the quadratic of its two operating points: a
// FlashAttention-style forward that never forms the state. With the rank-one
// PSD lift, phi(q) . phi(k) = (q . k)^2, so for every query t
//   num_t = sum_{i <= t} (q_t . k_i)^2 v_i,   den_t = sum_{i <= t} (q_t . k_i)^2,
//   o_t = num_t / (den_t + eps)   (0 when that is 0),
// the same outputs as the chunked state form. The weights are squares, never
// negative and never exponentiated, so no running maximum is needed.
//
// One work-group per head and pair of 256-query blocks (x, nqb - 1 - x),
// the heavy one first, so that every work-group does the same causal work;
// wave w owns queries 32 w .. 32 w + 31 of a block as two 16-query tiles.
// Keys come in blocks of 64, staged in LDS (double buffered: k rows, v
// transposed) while the previous block computes, with the next three blocks
// in flight from memory. Per key block a wave
//   * forms S^T = K Q^T on MFMA 16x16x32 bf16 (float32 sums): lane (l16, q4)
//     holds the scores of query l16 against keys 4 q4 + i of each 16-key tile;
//   * squares them in float32 (causal mask only on the blocks that reach
//     past the wave's first query) and rounds them to bf16 as the B operand
//     of O^T = V^T P^T, taking P's k-slots in the order they sit in the lanes
//     (keys 4 q4 + j of tile 2p, then of tile 2p + 1) and V^T's in the same
//     order, so no value moves between lanes; the denominators are float32
//     sums of the unrounded weights on the vector units (the backward needs
//     them accurate: it divides by them again).
// Each K and V fragment read from LDS serves both query tiles of the wave.
// On request the row denominators den_t + eps are stored as well (float32),
// for the backward.
//
// Multi-factor variants (KATA §2.3, "Variantes"; the reading: the 64
// dimensions split into G equal factors). KATA-Mg concatenates the factors'
// rank-one lifts, so the weight is sum_i (q_i . k_i)^2; KATA-Sigma-g lifts the
// summed outer products, so it is sum_{i,j} (q_i . k_j)^2. Only the weights
// change: for G = 2 the two 32-dimension k-steps of the score product are the
// factors (their products are kept apart, and Sigma-2 adds the two crossed
// ones); for G = 4 the scores of each factor pair come from
// mfma_f32_16x16x16_bf16, whose k-range is one 16-dimension factor.
#include <algorithm>
#include <type_traits>

#include "kla_device.hpp"
#include "kla_internal.hpp"
#include "quad_tiles.hpp"

namespace kla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kQD = 64;           // d_qk = d_v
constexpr int kQW = 8;            // waves per work-group
constexpr int kQT = 64 * kQW;     // threads
constexpr int kBQ = 32 * kQW;     // queries per work-group
constexpr int kBK = 64;           // keys per block
constexpr int kKS = kQD + 8;      // k row stride (bf16)
constexpr int kVS = kBK + 8;      // v^T row stride (bf16)

struct QuadLds {
  uint16_t k[2][kBK][kKS];        // key rows
  uint16_t vt[2][kQD][kVS];       // values transposed: [dim][key]
};

__device__ __forceinline__ f32x4 mfma(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
// 16x16x16: lane (l16, q4) holds k-values 4 q4 .. 4 q4 + 3 of its row (A) or column (B)
__device__ __forceinline__ f32x4 mfma16(const s16x4& a, const s16x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 sq(const f32x4& x) { return x * x; }

// Factor structure of the weights: KIND 0 concatenated lifts (KATA-Mg), 1
// summed lifts (KATA-Sigma-g); G factors (G = 1: the rank-one lift).
template <int KIND, int G>
struct Factors {
  static_assert(G == 1 || G == 2 || G == 4, "factors");
  // query operands of one 16-query tile: G <= 2: [k-step] bf16x8; G = 4: [factor] 4 x bf16
  struct Q {
    bf16x8 f[2];
    s16x4 h[4];
  };
  static __device__ __forceinline__ Q load_q(const uint16_t* __restrict__ row, bool ok, int q4) {
    Q r;
    if constexpr (G == 4) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint2 u = make_uint2(0, 0);
        if (ok) u = *reinterpret_cast<const uint2*>(row + 16 * i + 4 * q4);
        r.h[i] = __builtin_bit_cast(s16x4, u);
      }
    } else {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        uint4 u = make_uint4(0, 0, 0, 0);
        if (ok) u = *reinterpret_cast<const uint4*>(row + 32 * ks + 8 * q4);
        r.f[ks] = __builtin_bit_cast(bf16x8, u);
      }
    }
    return r;
  }
  // weights of keys 16 kt + 4 q4 + i (rows of S^T) against query l16; krow is
  // key row 16 kt + l16 in LDS
  static __device__ __forceinline__ void weights(const uint16_t* krow, int q4, const Q (&qf)[2], f32x4 (&w)[2]) {
    const f32x4 z = f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (G == 4) {
      s16x4 a[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) a[j] = *reinterpret_cast<const s16x4*>(krow + 16 * j + 4 * q4);
#pragma unroll
      for (int tq = 0; tq < 2; ++tq) {
        f32x4 acc = z;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            if (KIND == 0 && i != j) continue;
            acc += sq(mfma16(a[j], qf[tq].h[i], z));
          }
        }
        w[tq] = acc;
      }
    } else {
      bf16x8 a[2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) a[ks] = *reinterpret_cast<const bf16x8*>(krow + 32 * ks + 8 * q4);
#pragma unroll
      for (int tq = 0; tq < 2; ++tq) {
        if constexpr (G == 1) {
          w[tq] = sq(mfma(a[1], qf[tq].f[1], mfma(a[0], qf[tq].f[0], z)));
        } else {
          f32x4 acc = sq(mfma(a[0], qf[tq].f[0], z)) + sq(mfma(a[1], qf[tq].f[1], z));
          if (KIND == 1) acc += sq(mfma(a[1], qf[tq].f[0], z)) + sq(mfma(a[0], qf[tq].f[1], z));
          w[tq] = acc;
        }
      }
    }
  }
};

// One thread's share of a key block: key tid % kBK, dims kDPT g .. kDPT g + kDPT - 1
// of k and v with g = tid / kBK.
constexpr int kDPT = kQD * kBK / kQT;  // dims per staging thread
constexpr int kU4 = kDPT / 8;     // 16-byte groups per thread and tensor
struct KVLoad {
  uint4 k[kU4], v[kU4];
};

__device__ __forceinline__ KVLoad load_kv(const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                                          size_t row0, int key, int T, int w) {
  KVLoad r;
#pragma unroll
  for (int j = 0; j < kU4; ++j) r.k[j] = r.v[j] = make_uint4(0, 0, 0, 0);
  if (key < T) {
    const size_t off = (row0 + key) * kQD + kDPT * w;
    const uint4* kp = reinterpret_cast<const uint4*>(k + off);
    const uint4* vp = reinterpret_cast<const uint4*>(v + off);
#pragma unroll
    for (int j = 0; j < kU4; ++j) {
      r.k[j] = kp[j];
      r.v[j] = vp[j];
    }
  }
  return r;
}

// Key rows as they are, values transposed with the column permutation of
// vt_col (see quad_tiles.hpp).
__device__ __forceinline__ void stage_kv(QuadLds& sh, int buf, const KVLoad& r, int key, int w) {
#pragma unroll
  for (int j = 0; j < kU4; ++j) {
    *reinterpret_cast<uint4*>(&sh.k[buf][key][kDPT * w + 8 * j]) = r.k[j];
    store_transposed8(&sh.vt[buf][0][0], kVS, r.v[j], key, kDPT * w + 8 * j);
  }
}

template <typename Tout, int KIND, int G>
__global__ __launch_bounds__(kQT, 1) void prefill_quad_kernel(const uint16_t* __restrict__ q,
                                                              const uint16_t* __restrict__ k,
                                                              const uint16_t* __restrict__ v,
                                                              Tout* __restrict__ o, float* __restrict__ den,
                                                              int T, float eps) {
  __shared__ __align__(16) QuadLds sh;
  const int nqb = (T + kBQ - 1) / kBQ;
  const int n = blockIdx.y;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l16 = lane & 15;
  const int q4 = lane >> 4;
  const size_t row0 = (size_t)n * T;
  // query blocks nqb - 1 - x and x: every work-group does the same causal work
  for (int rep = 0; rep < 2; ++rep) {
    const int qb = rep == 0 ? nqb - 1 - (int)blockIdx.x : (int)blockIdx.x;
    if (rep == 1 && qb >= nqb - 1 - (int)blockIdx.x) break;
    const int qw0 = qb * kBQ + 32 * w;              // this wave's first query
    const int q_last = min(T, (qb + 1) * kBQ) - 1;  // the block's last query
    const int nkb = q_last / kBK + 1;               // key blocks with keys <= q_last

    // Q as the B operand of S^T = K Q^T (per query tile)
    using F = Factors<KIND, G>;
    typename F::Q qf[2];
#pragma unroll
    for (int tq = 0; tq < 2; ++tq) {
      const int t = qw0 + 16 * tq + l16;
      qf[tq] = F::load_q(q + (row0 + min(t, T - 1)) * kQD, t < T, q4);
    }

    const int skey = tid % kBK;  // staging role
    const int sgrp = tid / kBK;
    // blocks 1..3 in flight in three register slots (block b in slot b mod 3)
    // while block 0 is staged; each key block's compute is far shorter than
    // a memory round trip
    KVLoad pf0 = load_kv(k, v, row0, skey, T, sgrp);
    stage_kv(sh, 0, pf0, skey, sgrp);
    KVLoad pf1 = load_kv(k, v, row0, kBK + skey, T, sgrp);
    KVLoad pf2 = load_kv(k, v, row0, 2 * kBK + skey, T, sgrp);
    pf0 = load_kv(k, v, row0, 3 * kBK + skey, T, sgrp);
    __syncthreads();

    f32x4 acc[2][4];  // O^T: [query tile][dim tile], lane holds dims 16 dt + 4 q4 + i of query l16
    float dsv[2];     // float32 sums of the weights of query l16 over this lane's keys
#pragma unroll
    for (int tq = 0; tq < 2; ++tq) {
      dsv[tq] = 0.0f;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) acc[tq][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    // one key block; MASKED: apply the causal mask (blocks with keys above a query of the wave)
    auto key_block = [&](int kb, auto masked_c) {
      constexpr bool MASKED = decltype(masked_c)::value;
      const int buf = kb & 1;
      const int k0 = kb * kBK;
      // weights (squared scores, summed over factor pairs) for kBK / 16 key
      // tiles x 2 query tiles
      f32x4 s[kBK / 16][2];
#pragma unroll
      for (int kt = 0; kt < kBK / 16; ++kt) F::weights(&sh.k[buf][16 * kt + l16][0], q4, qf, s[kt]);
      // P = S^2 as the bf16 B operands of O^T = V^T P^T
      bf16x8 pb[kBK / 32][2];  // [key pair][query tile]
#pragma unroll
      for (int tq = 0; tq < 2; ++tq) {
        const int t = qw0 + 16 * tq + l16;
#pragma unroll
        for (int kt = 0; kt < kBK / 16; ++kt) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float p = s[kt][tq][i];
            if (MASKED && k0 + 16 * kt + 4 * q4 + i > t) p = 0.0f;
            dsv[tq] += p;
            pb[kt >> 1][tq][4 * (kt & 1) + i] = (__bf16)p;
          }
        }
      }
#pragma unroll
      for (int p2 = 0; p2 < kBK / 32; ++p2) {
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          // V^T rows 16 dt + l16, keys 32 p2 + 4 q4 + j and 32 p2 + 16 + 4 q4 + j
          // (columns 32 p2 + 8 q4 .. + 7)
          const bf16x8 av = *reinterpret_cast<const bf16x8*>(&sh.vt[buf][16 * dt + l16][32 * p2 + 8 * q4]);
#pragma unroll
          for (int tq = 0; tq < 2; ++tq) acc[tq][dt] = mfma(av, pb[p2][tq], acc[tq][dt]);
        }
      }
    };

    // blocks below kb_mask have no key above the wave's first query
    const int kb_mask = min(nkb, (qw0 + 1) / kBK);
    // block kb, then stage block kb + 1 from its slot and load block kb + 4 into it
    auto step = [&](int kb, KVLoad& slot) {
      if (kb < kb_mask) key_block(kb, std::false_type{});
      else key_block(kb, std::true_type{});
      if (kb + 1 < nkb) {
        stage_kv(sh, (kb & 1) ^ 1, slot, skey, sgrp);
        if (kb + 4 < nkb) slot = load_kv(k, v, row0, (kb + 4) * kBK + skey, T, sgrp);
      }
      __syncthreads();
    };
    for (int kb = 0; kb < nkb; kb += 3) {
      step(kb, pf1);
      if (kb + 1 < nkb) step(kb + 1, pf2);
      if (kb + 2 < nkb) step(kb + 2, pf0);
    }

    // denominators: the four lane quarters of query l16 hold disjoint keys
#pragma unroll
    for (int tq = 0; tq < 2; ++tq) {
      const int t = qw0 + 16 * tq + l16;
      float dsum = dsv[tq];
      dsum += __shfl_xor(dsum, 16, 64);
      dsum += __shfl_xor(dsum, 32, 64);
      if (t >= T) continue;
      const float d = dsum + eps;
      if (den && q4 == 0) den[row0 + t] = d;
      const float inv = d != 0.0f ? 1.0f / d : 0.0f;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          Elem<Tout>::store(o, (row0 + t) * kQD + 16 * dt + 4 * q4 + i, d != 0.0f ? acc[tq][dt][i] * inv : 0.0f);
      }
    }
  }  // rep
}

template <int KIND, int G>
void launch_quad(const PrefillArgs& a, dim3 grid, hipStream_t st) {
  if (a.out_bf16)
    hipLaunchKernelGGL((prefill_quad_kernel<uint16_t, KIND, G>), grid, dim3(kQT), 0, st,
                       static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                       static_cast<const uint16_t*>(a.v), static_cast<uint16_t*>(a.o), a.den, a.T, a.eps);
  else
    hipLaunchKernelGGL((prefill_quad_kernel<float, KIND, G>), grid, dim3(kQT), 0, st,
                       static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                       static_cast<const uint16_t*>(a.v), static_cast<float*>(a.o), a.den, a.T, a.eps);
}

}  // namespace

bool prefill_quad_supported(const PrefillArgs& a) {
  return a.in_bf16 && a.dqk == kQD && a.dv == kQD && (a.factor_kind == 0 || a.factor_kind == 1) &&
         (a.factors == 1 || a.factors == 2 || a.factors == 4);
}

hipError_t prefill_quad_launch(const PrefillArgs& a, hipStream_t st) {
  if (!prefill_quad_supported(a) || a.T < 1 || !a.o) return hipErrorInvalidValue;
  const int nqb = (a.T + kBQ - 1) / kBQ;
  const dim3 grid((nqb + 1) / 2, a.N);
  prof_begin(st);
  switch (a.factor_kind * 8 + a.factors) {
    case 0 * 8 + 1:
    case 1 * 8 + 1: launch_quad<0, 1>(a, grid, st); break;
    case 0 * 8 + 2: launch_quad<0, 2>(a, grid, st); break;
    case 1 * 8 + 2: launch_quad<1, 2>(a, grid, st); break;
    case 0 * 8 + 4: launch_quad<0, 4>(a, grid, st); break;
    case 1 * 8 + 4: launch_quad<1, 4>(a, grid, st); break;
    default: prof_end(st); return hipErrorInvalidValue;
  }
  prof_end(st);
  return hipGetLastError();
}

}  // namespace kla
