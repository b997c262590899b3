// Internal host-side interface between the C ABI (kla_api.hip) and the
// kernel translation units. Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "kla.h"

namespace kla {

// Timing hooks around a call's dominant kernel (no-ops unless enabled).
void prof_begin(hipStream_t st);
void prof_end(hipStream_t st);

// Workspace carving: every region is 256-byte aligned.
inline size_t align_up(size_t x, size_t a = 256) { return (x + a - 1) / a * a; }

// ---------------------------------------------------------------- prefill

struct PrefillArgs {
  int N, T, dqk, dv, chunk;
  bool in_bf16, out_bf16;
  float eps;
  const void* q;
  const void* k;
  const void* v;
  void* o;  // NULL = state only
  const float* H0;
  const float* s0;
  float* HT;
  float* sT;
  float* den;  // quadratic form only: row denominators [N, T], or NULL
  // multi-factor lift, kind 0 concatenated (KATA-Mg), 1 summed
  // (KATA-Sigma-g: quadratic form and float32 vector path), over `factors`
  // equal slices (1: rank-one lift)
  int factor_kind = 0;
  int factors = 1;
};

// Generic float32-arithmetic path (VALU): any supported shape, either dtype.
size_t prefill_valu_workspace(const PrefillArgs& a);
hipError_t prefill_valu_launch(const PrefillArgs& a, void* ws, hipStream_t st);

// bf16 matrix-core path for d_qk = d_v = 64; returns false from *_supported
// when the shape is outside what it handles.
bool prefill_mfma_supported(const PrefillArgs& a);
size_t prefill_mfma_workspace(const PrefillArgs& a);
hipError_t prefill_mfma_launch(const PrefillArgs& a, void* ws, hipStream_t st);

// Quadratic (O(T^2)) form, d_qk = d_v = 64 and bf16 inputs; no workspace.
bool prefill_quad_supported(const PrefillArgs& a);
hipError_t prefill_quad_launch(const PrefillArgs& a, hipStream_t st);

// Its backward: dq, dk, dv from q, k, v (bf16), do (out dtype) and the
// forward's row denominators.
struct QuadBwdArgs {
  int N, T;
  bool out_bf16;
  const void* q;
  const void* k;
  const void* v;
  const float* den;
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
};
size_t prefill_quad_bwd_workspace(const QuadBwdArgs& a);
hipError_t prefill_quad_bwd_launch(const QuadBwdArgs& a, void* ws, hipStream_t st);

// ---------------------------------------------------------------- decode / SRE

struct SreArgs {
  int n_cand, top_k;
  const float* cand_k;
  const float* cand_v;
  float* scores;
  int32_t* sel;
  float* sel_k;
  float* sel_v;
  int sel_stride;  // rows between heads in sel_k / sel_v (>= top_k)
};

struct DecodeArgs {
  int N, dqk, dv;
  float eps;
  float* H;
  float* s;
  const void* q;
  const void* k;
  const void* v;
  bool in_bf16;
  void* o;
  bool out_bf16;
};

size_t decode_workspace(const DecodeArgs& a, const SreArgs* sre);
hipError_t decode_launch(const DecodeArgs& a, const SreArgs* sre, void* ws, hipStream_t st);

// Fused decode + scoring + selection on the matrix cores (d_qk = d_v = 64,
// n_cand <= 64); no workspace.
bool decode_fused_supported(int dqk, int dv, const SreArgs& sre);
hipError_t decode_fused_launch(const DecodeArgs& a, const SreArgs& sre, hipStream_t st);
hipError_t sre_fused_launch(int N, float eps, const float* H, const float* s, const SreArgs& sre,
                            hipStream_t st);
// The same step with deferred folds (d_qk = d_v = 64; sre NULL or n_cand <=
// 64): pend_k / pend_v hold decode_pending_slots() pairs per head-state, the
// first n_pend in use; n_pend = decode_pending_slots() - 1 folds them and the
// step's token, fewer only read the state and store the token in slot n_pend.
int decode_pending_slots();
hipError_t decode_deferred_launch(const DecodeArgs& a, const SreArgs* sre, float* pend_k, float* pend_v,
                                  int n_pend, hipStream_t st);
hipError_t decode_flush_launch(int N, float* H, float* s, const float* pend_k, const float* pend_v, int n_pend,
                               hipStream_t st);

size_t sre_workspace(int N, int dqk, int dv, const SreArgs& s);
hipError_t sre_launch(int N, int dqk, int dv, float eps, const float* H, const float* s,
                      const SreArgs& sre, void* ws, hipStream_t st);

// ---------------------------------------------------------------- hybrid

struct HybridArgs {
  int N, T, dqk, dv;
  bool in_bf16, out_bf16;
  float eps;
  int window, cache_size, refresh;
  float scale;
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* HT;
  float* sT;
  int32_t* cache_T;
  int32_t* trace;
};

size_t hybrid_workspace(const HybridArgs& a);
// aux: a second stream of the caller's for the batch work of the matrix-core
// path (folds, state sums, readouts), or NULL to run everything on `st`.
hipError_t hybrid_launch(const HybridArgs& a, void* ws, hipStream_t st, hipStream_t aux);
// The matrix-core form (d_qk = d_v = 64, bf16 inputs).
bool hybrid_mfma_supported(const HybridArgs& a);
size_t hybrid_mfma_workspace(const HybridArgs& a);
hipError_t hybrid_mfma_launch(const HybridArgs& a, void* ws, hipStream_t st, hipStream_t aux);

// Token-by-token hybrid: one token for every head-state.
struct HybridDecodeArgs {
  int N, dqk, dv;
  bool in_bf16, out_bf16;
  float eps;
  int window, cache_size;
  float scale;
  int t;  // tokens each head-state has seen before this one
  float* H;
  float* s;
  void* win_k;  // window and cache rows, in the input type (in_bf16)
  void* win_v;
  void* cache_k;
  void* cache_v;
  int32_t* cache_ids;
  float* pend_k;  // [N][KLA_HYBRID_PENDING][dqk]: rejected pairs whose folds are deferred
  float* pend_v;
  float* cache_sums;  // [N][cache_size][dv + 4]: the cached pairs' sums against H + the pending slots
  const void* q;
  const void* k;
  const void* v;
  void* o;
  int32_t* rejected;
};

size_t hybrid_decode_workspace(const HybridDecodeArgs& a);
hipError_t hybrid_decode_launch(const HybridDecodeArgs& a, void* ws, hipStream_t st);
// Folds the pending slots into (H, s) and clears them (uses N, dqk, dv, H, s, pend_k, pend_v).
hipError_t hybrid_decode_flush_launch(const HybridDecodeArgs& a, hipStream_t st);
// Computes cache_sums for the cached rows of step t from H, s and the pending slots.
hipError_t hybrid_decode_prime_launch(const HybridDecodeArgs& a, hipStream_t st);

// Size of the library's static scratch for the allocation-free hybrid decode
// step, and its device address on the current device (looked up once per
// device).
constexpr size_t kHybridDecodeStaticScratch = size_t(16) << 20;
hipError_t hybrid_decode_static_scratch(void** out);

}  // namespace kla
