// Recurrent decode step, self-recall-error scoring and top-k selection.
//
// Decode (KATA page §1: constant-time recurrent inference over a fixed-size
// state; LoLA page, "Estratégia de Inferência", token-by-token mode):
//   s += phi(k); H += phi(k) v^T; o = phi(q)^T H / (phi(q)^T s + eps).
// The state of each head-state is read once and written once, streamed
// row by row (a row = d_v contiguous floats) with 16-byte accesses.
//
// Self-recall error (LoLA page, section "O Mecanismo de Erro de
// Auto-Recuperação"): pred = phi(k_c)^T H / phi(k_c)^T s, score =
// ||pred - v_c||^2, in float32. Selection (LoLA, "Estratégia de
// Inferência" item 2): the highest scores are kept; ties go to the lower
// candidate index. A bitonic network sorts packed (score, index) keys.
#include "kla_device.hpp"
#include "kla_internal.hpp"
#include "sre_block.hpp"

namespace kla {
namespace {

constexpr int kThreads = 256;

template <int DQK, int DV, typename Tin, typename Tout>
__global__ __launch_bounds__(kThreads) void decode_kernel(float* __restrict__ H,
                                                          float* __restrict__ s,
                                                          const Tin* __restrict__ q,
                                                          const Tin* __restrict__ k,
                                                          const Tin* __restrict__ v,
                                                          Tout* __restrict__ o, float eps) {
  constexpr int D = phi_dim(DQK);
  constexpr int C4 = DV / 4;     // float4 per state row
  constexpr int R = kThreads / C4;  // rows per sweep
  constexpr int W = kThreads / 64;
  const int n = blockIdx.x;
  const int tid = threadIdx.x;
  const int c4 = tid % C4;
  const int rg = tid / C4;

  __shared__ float qs[DQK];
  __shared__ float ks[DQK];
  __shared__ float vs[DV];
  __shared__ uint16_t tab[D];
  __shared__ float red[R][DV];
  __shared__ float rden[W];

  for (int i = tid; i < DQK; i += kThreads) {
    qs[i] = Elem<Tin>::load(q, (size_t)n * DQK + i);
    ks[i] = Elem<Tin>::load(k, (size_t)n * DQK + i);
  }
  for (int i = tid; i < DV; i += kThreads) vs[i] = Elem<Tin>::load(v, (size_t)n * DV + i);
  build_phi_table(tab, 0, D, DQK);
  __syncthreads();

  const float4 vv = make_float4(vs[4 * c4], vs[4 * c4 + 1], vs[4 * c4 + 2], vs[4 * c4 + 3]);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float dacc = 0.0f;
  float4* Hn = reinterpret_cast<float4*>(H + (size_t)n * D * DV);
  float* sn = s + (size_t)n * D;
#pragma unroll 4
  for (int f = rg; f < D; f += R) {
    const uint16_t ab = tab[f];
    const float pk = phi_of(ks, ab);
    const float pq = phi_of(qs, ab);
    float4 h = Hn[(size_t)f * C4 + c4];
    h.x += pk * vv.x;
    h.y += pk * vv.y;
    h.z += pk * vv.z;
    h.w += pk * vv.w;
    Hn[(size_t)f * C4 + c4] = h;
    acc.x += pq * h.x;
    acc.y += pq * h.y;
    acc.z += pq * h.z;
    acc.w += pq * h.w;
    if (c4 == 0) {
      const float sv = sn[f] + pk;
      sn[f] = sv;
      dacc += pq * sv;
    }
  }
  red[rg][4 * c4] = acc.x;
  red[rg][4 * c4 + 1] = acc.y;
  red[rg][4 * c4 + 2] = acc.z;
  red[rg][4 * c4 + 3] = acc.w;
  dacc = wave_sum(dacc);
  if ((tid & 63) == 0) rden[tid >> 6] = dacc;
  __syncthreads();
  if (tid < DV) {
    float num = 0.0f;
    for (int r = 0; r < R; ++r) num += red[r][tid];
    float den = eps;
    for (int w = 0; w < W; ++w) den += rden[w];
    Elem<Tout>::store(o, (size_t)n * DV + tid, den != 0.0f ? num / den : 0.0f);
  }
}

// Scores of up to 64 candidates per block: grid (ceil(n_cand / 64), N).
template <int DQK, int DV>
__global__ __launch_bounds__(kThreads) void sre_kernel(const float* __restrict__ H,
                                                       const float* __restrict__ s,
                                                       const float* __restrict__ ck,
                                                       const float* __restrict__ cv, int n_cand,
                                                       float* __restrict__ scores, float eps) {
  constexpr int D = phi_dim(DQK);
  __shared__ SreShared<DQK, DV> sh;
  const int n = blockIdx.y;
  const int cbase = blockIdx.x * 64;
  const float* ckn = ck + (size_t)n * n_cand * DQK;
  const float* cvn = cv + (size_t)n * n_cand * DV;
  auto load_k = [&](int c, int d) { return ckn[(size_t)c * DQK + d]; };
  auto load_v = [&](int c, int d) { return cvn[(size_t)c * DV + d]; };
  sre_block<DQK, DV>(sh, H + (size_t)n * D * DV, s + (size_t)n * D, cbase, n_cand, load_k, load_v,
                     scores + (size_t)n * n_cand, eps);
}

// Top-k of n_cand scores per head (one block per head), optional gather.
__global__ __launch_bounds__(kThreads) void topk_kernel(const float* __restrict__ scores,
                                                        int n_cand, int top_k, int npow2,
                                                        int32_t* __restrict__ sel,
                                                        const float* __restrict__ ck,
                                                        const float* __restrict__ cv,
                                                        float* __restrict__ sel_k,
                                                        float* __restrict__ sel_v,
                                                        int sel_stride, int dqk, int dv) {
  __shared__ uint64_t keys[256];
  const int n = blockIdx.x;
  for (int i = threadIdx.x; i < npow2; i += blockDim.x)
    keys[i] = i < n_cand ? topk_key(scores[(size_t)n * n_cand + i], (uint32_t)i) : 0ull;
  bitonic_sort_desc(keys, npow2);
  for (int i = threadIdx.x; i < top_k; i += blockDim.x)
    sel[(size_t)n * top_k + i] = (int32_t)topk_index(keys[i]);
  if (sel_k) {
    for (int i = threadIdx.x; i < top_k * dqk; i += blockDim.x) {
      const int j = i / dqk, d = i % dqk;
      const uint32_t c = topk_index(keys[j]);
      sel_k[((size_t)n * sel_stride + j) * dqk + d] = ck[((size_t)n * n_cand + c) * dqk + d];
    }
    for (int i = threadIdx.x; i < top_k * dv; i += blockDim.x) {
      const int j = i / dv, d = i % dv;
      const uint32_t c = topk_index(keys[j]);
      sel_v[((size_t)n * sel_stride + j) * dv + d] = cv[((size_t)n * n_cand + c) * dv + d];
    }
  }
}

int pow2_at_least(int x) {
  int p = 64;
  while (p < x) p <<= 1;
  return p;
}

template <int DQK, int DV, typename Tin, typename Tout>
hipError_t decode_typed(const DecodeArgs& a, hipStream_t st) {
  prof_begin(st);
  hipLaunchKernelGGL((decode_kernel<DQK, DV, Tin, Tout>), dim3(a.N), dim3(kThreads), 0, st, a.H,
                     a.s, static_cast<const Tin*>(a.q), static_cast<const Tin*>(a.k),
                     static_cast<const Tin*>(a.v), static_cast<Tout*>(a.o), a.eps);
  prof_end(st);
  return hipGetLastError();
}

template <int DQK, int DV>
hipError_t decode_dt(const DecodeArgs& a, hipStream_t st) {
  if (a.in_bf16)
    return a.out_bf16 ? decode_typed<DQK, DV, uint16_t, uint16_t>(a, st)
                      : decode_typed<DQK, DV, uint16_t, float>(a, st);
  return a.out_bf16 ? decode_typed<DQK, DV, float, uint16_t>(a, st)
                    : decode_typed<DQK, DV, float, float>(a, st);
}

template <int DQK, int DV>
hipError_t sre_typed(int N, float eps, const float* H, const float* s, const SreArgs& sre,
                     float* scores, hipStream_t st) {
  hipLaunchKernelGGL((sre_kernel<DQK, DV>), dim3((sre.n_cand + 63) / 64, N), dim3(kThreads), 0, st,
                     H, s, sre.cand_k, sre.cand_v, sre.n_cand, scores, eps);
  return hipGetLastError();
}

template <typename F>
hipError_t dispatch_dd(int dqk, int dv, F&& f) {
#define KLA_CASE(A, B) \
  if (dqk == A && dv == B) return f(std::integral_constant<int, A>(), std::integral_constant<int, B>());
  KLA_CASE(16, 16) KLA_CASE(16, 32) KLA_CASE(16, 64)
  KLA_CASE(32, 16) KLA_CASE(32, 32) KLA_CASE(32, 64)
  KLA_CASE(64, 16) KLA_CASE(64, 32) KLA_CASE(64, 64)
#undef KLA_CASE
  return hipErrorInvalidValue;
}

hipError_t score_and_select(int N, int dqk, int dv, float eps, const float* H, const float* s,
                            const SreArgs& sre, void* ws, hipStream_t st, bool timed) {
  float* scores = sre.scores ? sre.scores : static_cast<float*>(ws);
  if (timed) prof_begin(st);
  hipError_t e = dispatch_dd(dqk, dv, [&](auto A, auto B) {
    return sre_typed<decltype(A)::value, decltype(B)::value>(N, eps, H, s, sre, scores, st);
  });
  if (timed) prof_end(st);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(topk_kernel, dim3(N), dim3(kThreads), 0, st, scores, sre.n_cand, sre.top_k,
                     pow2_at_least(sre.n_cand), sre.sel, sre.cand_k, sre.cand_v, sre.sel_k,
                     sre.sel_v, sre.sel_stride, dqk, dv);
  return hipGetLastError();
}

}  // namespace

size_t sre_workspace(int N, int dqk, int dv, const SreArgs& s) {
  if (decode_fused_supported(dqk, dv, s)) return 0;
  return s.scores ? 0 : align_up((size_t)N * s.n_cand * sizeof(float));
}

hipError_t sre_launch(int N, int dqk, int dv, float eps, const float* H, const float* s,
                      const SreArgs& sre, void* ws, hipStream_t st) {
  if (decode_fused_supported(dqk, dv, sre)) return sre_fused_launch(N, eps, H, s, sre, st);
  return score_and_select(N, dqk, dv, eps, H, s, sre, ws, st, true);
}

size_t decode_workspace(const DecodeArgs& a, const SreArgs* sre) {
  return sre ? sre_workspace(a.N, a.dqk, a.dv, *sre) : 0;
}

hipError_t decode_launch(const DecodeArgs& a, const SreArgs* sre, void* ws, hipStream_t st) {
  if (sre && decode_fused_supported(a.dqk, a.dv, *sre)) return decode_fused_launch(a, *sre, st);
  hipError_t e = dispatch_dd(a.dqk, a.dv, [&](auto A, auto B) {
    return decode_dt<decltype(A)::value, decltype(B)::value>(a, st);
  });
  if (e != hipSuccess || !sre) return e;
  return score_and_select(a.N, a.dqk, a.dv, a.eps, a.H, a.s, *sre, ws, st, false);
}

}  // namespace kla
