// C ABI of libkla: host-side argument checks, workspace sizing and dispatch.
// Every check runs before anything is enqueued, so a call that fails one
// writes nothing. No exception leaves this file.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <initializer_list>
#include <string>
#include <utility>
#include <vector>

#include "kla_internal.hpp"

namespace {

thread_local std::string g_last_error;

kla_status_t fail(kla_status_t st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

kla_status_t ok() {
  g_last_error.clear();
  return KLA_OK;
}

kla_status_t hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(KLA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool dim_ok(int d) { return d == 16 || d == 32 || d == 64; }
bool dtype_ok(kla_dtype_t t) { return t == KLA_F32 || t == KLA_BF16; }

// Grid dimensions y/z are limited to 65535 on this target.
constexpr int kMaxHeads = 65535;

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const char* pa = static_cast<const char*>(a);
  const char* pb = static_cast<const char*>(b);
  return pa < pb + nb && pb < pa + na;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Every device pointer of a call must be 16-byte aligned: the kernels move
// rows with 16-byte vector accesses. NULL (an absent optional argument)
// passes.
struct NamedPtr {
  const char* name;
  const void* p;
};
kla_status_t check_align(const char* fn, std::initializer_list<NamedPtr> ptrs) {
  for (const NamedPtr& x : ptrs)
    if (x.p && !aligned16(x.p))
      return fail(KLA_ERR_INVALID_ARGUMENT, "%s: %s must be 16-byte aligned (got %p)", fn, x.name, x.p);
  return KLA_OK;
}

kla_status_t check_shape(const kla_shape_t* shp, const char* fn) {
  if (!shp) return fail(KLA_ERR_INVALID_ARGUMENT, "%s: shape is NULL", fn);
  if (shp->B < 1 || shp->H < 1 || shp->T < 1)
    return fail(KLA_ERR_INVALID_ARGUMENT, "%s: B, H, T must be >= 1 (got %d, %d, %d)", fn, shp->B,
                shp->H, shp->T);
  if (shp->d_qk < 1 || shp->d_v < 1)
    return fail(KLA_ERR_INVALID_ARGUMENT, "%s: d_qk, d_v must be >= 1", fn);
  if (!dim_ok(shp->d_qk) || !dim_ok(shp->d_v))
    return fail(KLA_ERR_UNSUPPORTED, "%s: d_qk, d_v must be 16, 32 or 64 (got %d, %d)", fn,
                shp->d_qk, shp->d_v);
  if (!dtype_ok(shp->in_dtype) || !dtype_ok(shp->out_dtype))
    return fail(KLA_ERR_UNSUPPORTED, "%s: unknown dtype", fn);
  if (!std::isfinite(shp->eps) || shp->eps < 0.0f)
    return fail(KLA_ERR_INVALID_ARGUMENT, "%s: eps must be finite and >= 0", fn);
  const long long N = (long long)shp->B * shp->H;
  if (N > kMaxHeads) return fail(KLA_ERR_UNSUPPORTED, "%s: B*H = %lld exceeds %d", fn, N, kMaxHeads);
  if ((long long)shp->T * 256 > 0x7FFFFFFFLL)
    return fail(KLA_ERR_UNSUPPORTED, "%s: T = %d too large", fn, shp->T);
  return KLA_OK;
}

kla_status_t check_ws(size_t need, const void* ws, size_t ws_bytes, const char* fn) {
  if (need == 0) return KLA_OK;
  if (!ws) return fail(KLA_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, ws is NULL", fn, need);
  if (ws_bytes < need)
    return fail(KLA_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need, ws_bytes);
  return KLA_OK;
}

kla::PrefillArgs make_prefill(const kla_shape_t* shp, int chunk) {
  kla::PrefillArgs a{};
  a.N = shp->B * shp->H;
  a.T = shp->T;
  a.dqk = shp->d_qk;
  a.dv = shp->d_v;
  a.chunk = chunk;
  a.in_bf16 = shp->in_dtype == KLA_BF16;
  a.out_bf16 = shp->out_dtype == KLA_BF16;
  a.eps = shp->eps;
  return a;
}

size_t prefill_ws(const kla::PrefillArgs& a) {
  if (kla::prefill_mfma_supported(a)) return kla::prefill_mfma_workspace(a);
  return kla::prefill_valu_workspace(a);
}

kla_status_t check_sre(int N, int dqk, int dv, const kla_sre_args_t* sre, const char* fn) {
  if (!sre) return fail(KLA_ERR_INVALID_ARGUMENT, "%s: sre arguments are NULL", fn);
  if (sre->n_cand < 1 || sre->top_k < 1 || sre->top_k > sre->n_cand)
    return fail(KLA_ERR_INVALID_ARGUMENT, "%s: need 1 <= top_k <= n_cand (got %d, %d)", fn,
                sre->top_k, sre->n_cand);
  if (sre->n_cand > 256)
    return fail(KLA_ERR_UNSUPPORTED, "%s: n_cand = %d exceeds 256", fn, sre->n_cand);
  if (!sre->cand_k || !sre->cand_v || !sre->sel)
    return fail(KLA_ERR_INVALID_ARGUMENT, "%s: cand_k, cand_v and sel are required", fn);
  if ((sre->sel_k == nullptr) != (sre->sel_v == nullptr))
    return fail(KLA_ERR_INVALID_ARGUMENT, "%s: give both sel_k and sel_v or neither", fn);
  const size_t nck = (size_t)N * sre->n_cand * dqk * sizeof(float);
  const size_t ncv = (size_t)N * sre->n_cand * dv * sizeof(float);
  if (sre->sel_stride != 0 && sre->sel_stride < sre->top_k)
    return fail(KLA_ERR_INVALID_ARGUMENT, "%s: sel_stride must be 0 or >= top_k", fn);
  const size_t stride = sre->sel_stride ? (size_t)sre->sel_stride : (size_t)sre->top_k;
  // extent of the gathered rows (rows between heads are not written)
  const size_t rows = (size_t)(N - 1) * stride + sre->top_k;
  const size_t nsk = rows * dqk * sizeof(float);
  const size_t nsv = rows * dv * sizeof(float);
  if (overlaps(sre->sel_k, nsk, sre->cand_k, nck) || overlaps(sre->sel_k, nsk, sre->cand_v, ncv) ||
      overlaps(sre->sel_v, nsv, sre->cand_k, nck) || overlaps(sre->sel_v, nsv, sre->cand_v, ncv))
    return fail(KLA_ERR_INVALID_ARGUMENT, "%s: sel_k / sel_v overlap the candidates", fn);
  return check_align(fn, {{"cand_k", sre->cand_k}, {"cand_v", sre->cand_v}, {"scores", sre->scores},
                          {"sel", sre->sel}, {"sel_k", sre->sel_k}, {"sel_v", sre->sel_v}});
}

kla::SreArgs make_sre(const kla_sre_args_t* s) {
  kla::SreArgs a{};
  a.n_cand = s->n_cand;
  a.top_k = s->top_k;
  a.cand_k = s->cand_k;
  a.cand_v = s->cand_v;
  a.scores = s->scores;
  a.sel = s->sel;
  a.sel_k = s->sel_k;
  a.sel_v = s->sel_v;
  a.sel_stride = s->sel_stride ? s->sel_stride : s->top_k;
  return a;
}

kla_status_t check_hybrid(const kla_shape_t* shp, const kla_hybrid_cfg_t* cfg, const char* fn) {
  kla_status_t st = check_shape(shp, fn);
  if (st != KLA_OK) return st;
  if (!cfg) return fail(KLA_ERR_INVALID_ARGUMENT, "%s: cfg is NULL", fn);
  if (cfg->refresh < 1 || cfg->window < 0 || cfg->cache_size < 0)
    return fail(KLA_ERR_INVALID_ARGUMENT, "%s: need refresh >= 1, window >= 0, cache_size >= 0", fn);
  if (!std::isfinite(cfg->softmax_scale))
    return fail(KLA_ERR_INVALID_ARGUMENT, "%s: softmax_scale must be finite", fn);
  if (cfg->refresh > 128 || cfg->cache_size + cfg->refresh > 256)
    return fail(KLA_ERR_UNSUPPORTED, "%s: need refresh <= 128 and cache_size + refresh <= 256", fn);
  return KLA_OK;
}

kla::HybridArgs make_hybrid(const kla_shape_t* shp, const kla_hybrid_cfg_t* cfg) {
  kla::HybridArgs a{};
  a.N = shp->B * shp->H;
  a.T = shp->T;
  a.dqk = shp->d_qk;
  a.dv = shp->d_v;
  a.in_bf16 = shp->in_dtype == KLA_BF16;
  a.out_bf16 = shp->out_dtype == KLA_BF16;
  a.eps = shp->eps;
  a.window = cfg->window;
  a.cache_size = cfg->cache_size;
  a.refresh = cfg->refresh;
  a.scale = cfg->softmax_scale;
  return a;
}

struct ProfState {
  bool on = false;
  std::vector<std::pair<hipEvent_t, hipEvent_t>> pool;
  size_t used = 0;
  int dropped = 0;
  bool open = false;
  ~ProfState() {
    for (auto& e : pool) {
      (void)hipEventDestroy(e.first);
      (void)hipEventDestroy(e.second);
    }
  }
};
thread_local ProfState g_prof;
constexpr size_t kProfMax = 65536;

}  // namespace

namespace kla {

void prof_begin(hipStream_t st) {
  ProfState& p = g_prof;
  if (!p.on) return;
  if (p.used >= kProfMax) {
    ++p.dropped;
    return;
  }
  if (p.used == p.pool.size()) {
    hipEvent_t a = nullptr, b = nullptr;
    if (hipEventCreate(&a) != hipSuccess || hipEventCreate(&b) != hipSuccess) {
      ++p.dropped;
      return;
    }
    p.pool.emplace_back(a, b);
  }
  (void)hipEventRecord(p.pool[p.used].first, st);
  p.open = true;
}

void prof_end(hipStream_t st) {
  ProfState& p = g_prof;
  if (!p.on || !p.open) return;
  (void)hipEventRecord(p.pool[p.used].second, st);
  ++p.used;
  p.open = false;
}

}  // namespace kla

extern "C" {

kla_status_t kla_profile_enable(int on) {
  g_prof.on = on != 0;
  g_prof.open = false;
  return ok();
}

kla_status_t kla_profile_read(double* total_ms, int* kernels, int* dropped) {
  const char* fn = "kla_profile_read";
  if (!total_ms || !kernels) return fail(KLA_ERR_INVALID_ARGUMENT, "%s: NULL output", fn);
  ProfState& p = g_prof;
  double sum = 0.0;
  if (p.used > 0) {
    hipError_t e = hipEventSynchronize(p.pool[p.used - 1].second);
    if (e != hipSuccess) return hip_status(e, fn);
    for (size_t i = 0; i < p.used; ++i) {
      float ms = 0.0f;
      e = hipEventElapsedTime(&ms, p.pool[i].first, p.pool[i].second);
      if (e != hipSuccess) return hip_status(e, fn);
      sum += ms;
    }
  }
  *total_ms = sum;
  *kernels = (int)p.used;
  if (dropped) *dropped = p.dropped;
  p.used = 0;
  p.dropped = 0;
  return ok();
}

int kla_abi_version(void) { return KLA_ABI_VERSION; }

int kla_phi_dim(int d_qk) { return d_qk < 1 ? -1 : d_qk * (d_qk + 1) / 2; }

const char* kla_status_string(kla_status_t s) {
  switch (s) {
    case KLA_OK: return "ok";
    case KLA_ERR_INVALID_ARGUMENT: return "invalid argument";
    case KLA_ERR_UNSUPPORTED: return "unsupported";
    case KLA_ERR_WORKSPACE: return "workspace too small";
    case KLA_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

const char* kla_last_error(void) { return g_last_error.c_str(); }

// ---------------------------------------------------------------- prefill

int kla_prefill_matrix_path(const kla_shape_t* shp, int chunk) {
  if (check_shape(shp, "kla_prefill_matrix_path") != KLA_OK) return -1;
  if (chunk != 32 && chunk != 64 && chunk != 128) return -1;
  kla::PrefillArgs a = make_prefill(shp, chunk);
  a.o = reinterpret_cast<void*>(1);
  return kla::prefill_mfma_supported(a) ? 1 : 0;
}

kla_status_t kla_prefill_workspace_size(const kla_shape_t* shp, int chunk, int with_output,
                                        size_t* bytes) {
  const char* fn = "kla_prefill_workspace_size";
  if (!bytes) return fail(KLA_ERR_INVALID_ARGUMENT, "%s: bytes is NULL", fn);
  *bytes = 0;
  kla_status_t st = check_shape(shp, fn);
  if (st != KLA_OK) return st;
  if (chunk != 32 && chunk != 64 && chunk != 128)
    return fail(KLA_ERR_UNSUPPORTED, "%s: chunk must be 32, 64 or 128 (got %d)", fn, chunk);
  kla::PrefillArgs a = make_prefill(shp, chunk);
  a.o = with_output ? reinterpret_cast<void*>(1) : nullptr;
  *bytes = prefill_ws(a);
  return ok();
}

namespace {

kla_status_t prefill_call(const char* fn, const kla_shape_t* shp, int chunk, int factors, int kind, const void* q,
                          const void* k, const void* v, void* o, const float* H0, const float* s0, float* H_T,
                          float* s_T, void* ws, size_t ws_bytes, kla_stream_t stream) {
  kla_status_t st = check_shape(shp, fn);
  if (st != KLA_OK) return st;
  if (chunk != 32 && chunk != 64 && chunk != 128)
    return fail(KLA_ERR_UNSUPPORTED, "%s: chunk must be 32, 64 or 128 (got %d)", fn, chunk);
  if (!q || !k || !v) return fail(KLA_ERR_INVALID_ARGUMENT, "%s: q, k, v are required", fn);
  if ((H0 == nullptr) != (s0 == nullptr))
    return fail(KLA_ERR_INVALID_ARGUMENT, "%s: give both H0 and s0 or neither", fn);
  if ((H_T == nullptr) != (s_T == nullptr))
    return fail(KLA_ERR_INVALID_ARGUMENT, "%s: give both H_T and s_T or neither", fn);
  if (!o && !H_T)
    return fail(KLA_ERR_INVALID_ARGUMENT, "%s: o may be NULL only when H_T and s_T are given", fn);
  st = check_align(fn, {{"q", q}, {"k", k}, {"v", v}, {"o", o}, {"H0", H0}, {"s0", s0}, {"H_T", H_T},
                        {"s_T", s_T}, {"ws", ws}});
  if (st != KLA_OK) return st;
  kla::PrefillArgs a = make_prefill(shp, chunk);
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.H0 = H0;
  a.s0 = s0;
  a.HT = H_T;
  a.sT = s_T;
  a.factors = factors;
  a.factor_kind = factors > 1 ? kind : 0;  // with one factor both lifts are the rank-one lift
  const size_t need = prefill_ws(a);
  st = check_ws(need, ws, ws_bytes, fn);
  if (st != KLA_OK) return st;
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  if (kla::prefill_mfma_supported(a)) return hip_status(kla::prefill_mfma_launch(a, ws, hs), fn);
  return hip_status(kla::prefill_valu_launch(a, ws, hs), fn);
}

}  // namespace

kla_status_t kla_prefill(const kla_shape_t* shp, int chunk, const void* q, const void* k,
                         const void* v, void* o, const float* H0, const float* s0, float* H_T,
                         float* s_T, void* ws, size_t ws_bytes, kla_stream_t stream) {
  return prefill_call("kla_prefill", shp, chunk, 1, KLA_FACTORS_CONCAT, q, k, v, o, H0, s0, H_T, s_T, ws, ws_bytes,
                      stream);
}

kla_status_t kla_prefill_factors(const kla_shape_t* shp, int chunk, int kind, int factors, const void* q,
                                 const void* k, const void* v, void* o, const float* H0, const float* s0,
                                 float* H_T, float* s_T, void* ws, size_t ws_bytes, kla_stream_t stream) {
  const char* fn = "kla_prefill_factors";
  if (kind != KLA_FACTORS_CONCAT && kind != KLA_FACTORS_SUM)
    return fail(KLA_ERR_INVALID_ARGUMENT, "%s: kind %d is neither KLA_FACTORS_CONCAT nor KLA_FACTORS_SUM", fn, kind);
  if (factors != 1 && factors != 2 && factors != 4)
    return fail(KLA_ERR_INVALID_ARGUMENT, "%s: factors = %d (1, 2 or 4 supported)", fn, factors);
  return prefill_call(fn, shp, chunk, factors, kind, q, k, v, o, H0, s0, H_T, s_T, ws, ws_bytes, stream);
}

kla_status_t kla_prefill_factors_workspace_size(const kla_shape_t* shp, int chunk, int kind, int factors,
                                                int with_output, size_t* bytes) {
  const char* fn = "kla_prefill_factors_workspace_size";
  if (!bytes) return fail(KLA_ERR_INVALID_ARGUMENT, "%s: bytes is NULL", fn);
  *bytes = 0;
  kla_status_t st = check_shape(shp, fn);
  if (st != KLA_OK) return st;
  if (chunk != 32 && chunk != 64 && chunk != 128)
    return fail(KLA_ERR_UNSUPPORTED, "%s: chunk must be 32, 64 or 128 (got %d)", fn, chunk);
  if (kind != KLA_FACTORS_CONCAT && kind != KLA_FACTORS_SUM)
    return fail(KLA_ERR_INVALID_ARGUMENT, "%s: kind %d is neither KLA_FACTORS_CONCAT nor KLA_FACTORS_SUM", fn, kind);
  if (factors != 1 && factors != 2 && factors != 4)
    return fail(KLA_ERR_INVALID_ARGUMENT, "%s: factors = %d (1, 2 or 4 supported)", fn, factors);
  kla::PrefillArgs a = make_prefill(shp, chunk);
  a.o = with_output ? reinterpret_cast<void*>(1) : nullptr;
  a.factors = factors;
  a.factor_kind = factors > 1 ? kind : 0;
  *bytes = prefill_ws(a);
  return ok();
}

kla_status_t kla_prefill_quadratic(const kla_shape_t* shp, const void* q, const void* k, const void* v,
                                   void* o, float* den, kla_stream_t stream) {
  const char* fn = "kla_prefill_quadratic";
  kla_status_t st = check_shape(shp, fn);
  if (st != KLA_OK) return st;
  if (!q || !k || !v || !o) return fail(KLA_ERR_INVALID_ARGUMENT, "%s: q, k, v and o are required", fn);
  st = check_align(fn, {{"q", q}, {"k", k}, {"v", v}, {"o", o}, {"den", den}});
  if (st != KLA_OK) return st;
  kla::PrefillArgs a = make_prefill(shp, 64);
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.den = den;
  if (!kla::prefill_quad_supported(a))
    return fail(KLA_ERR_UNSUPPORTED, "%s: needs d_qk = d_v = 64 and bf16 inputs", fn);
  return hip_status(kla::prefill_quad_launch(a, reinterpret_cast<hipStream_t>(stream)), fn);
}

kla_status_t kla_prefill_quadratic_factors(const kla_shape_t* shp, int kind, int factors, const void* q,
                                           const void* k, const void* v, void* o, float* den, kla_stream_t stream) {
  const char* fn = "kla_prefill_quadratic_factors";
  kla_status_t st = check_shape(shp, fn);
  if (st != KLA_OK) return st;
  if (!q || !k || !v || !o) return fail(KLA_ERR_INVALID_ARGUMENT, "%s: q, k, v and o are required", fn);
  if (kind != KLA_FACTORS_CONCAT && kind != KLA_FACTORS_SUM)
    return fail(KLA_ERR_INVALID_ARGUMENT, "%s: kind %d is neither KLA_FACTORS_CONCAT nor KLA_FACTORS_SUM", fn, kind);
  if (factors != 1 && factors != 2 && factors != 4)
    return fail(KLA_ERR_INVALID_ARGUMENT, "%s: factors = %d (1, 2 or 4 supported)", fn, factors);
  st = check_align(fn, {{"q", q}, {"k", k}, {"v", v}, {"o", o}, {"den", den}});
  if (st != KLA_OK) return st;
  kla::PrefillArgs a = make_prefill(shp, 64);
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.den = den;
  a.factor_kind = kind;
  a.factors = factors;
  if (!kla::prefill_quad_supported(a))
    return fail(KLA_ERR_UNSUPPORTED, "%s: needs d_qk = d_v = 64 and bf16 inputs", fn);
  return hip_status(kla::prefill_quad_launch(a, reinterpret_cast<hipStream_t>(stream)), fn);
}

kla_status_t kla_prefill_quadratic_backward_workspace_size(const kla_shape_t* shp, size_t* bytes) {
  const char* fn = "kla_prefill_quadratic_backward_workspace_size";
  if (!bytes) return fail(KLA_ERR_INVALID_ARGUMENT, "%s: bytes is NULL", fn);
  *bytes = 0;
  kla_status_t st = check_shape(shp, fn);
  if (st != KLA_OK) return st;
  kla::QuadBwdArgs a{};
  a.N = shp->B * shp->H;
  a.T = shp->T;
  *bytes = kla::prefill_quad_bwd_workspace(a);
  return ok();
}

kla_status_t kla_prefill_quadratic_backward(const kla_shape_t* shp, const void* q, const void* k, const void* v,
                                            const float* den, const void* dout, void* dq, void* dk, void* dv,
                                            void* ws, size_t ws_bytes, kla_stream_t stream) {
  const char* fn = "kla_prefill_quadratic_backward";
  kla_status_t st = check_shape(shp, fn);
  if (st != KLA_OK) return st;
  if (!q || !k || !v || !den || !dout || !dq || !dk || !dv)
    return fail(KLA_ERR_INVALID_ARGUMENT, "%s: q, k, v, den, dout, dq, dk and dv are required", fn);
  if (shp->in_dtype != KLA_BF16 || shp->d_qk != 64 || shp->d_v != 64)
    return fail(KLA_ERR_UNSUPPORTED, "%s: needs d_qk = d_v = 64 and bf16 inputs", fn);
  st = check_align(fn, {{"q", q}, {"k", k}, {"v", v}, {"den", den}, {"dout", dout}, {"dq", dq}, {"dk", dk},
                        {"dv", dv}, {"ws", ws}});
  if (st != KLA_OK) return st;
  kla::QuadBwdArgs a{};
  a.N = shp->B * shp->H;
  a.T = shp->T;
  a.out_bf16 = shp->out_dtype == KLA_BF16;
  a.q = q;
  a.k = k;
  a.v = v;
  a.den = den;
  a.dout = dout;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  st = check_ws(kla::prefill_quad_bwd_workspace(a), ws, ws_bytes, fn);
  if (st != KLA_OK) return st;
  return hip_status(kla::prefill_quad_bwd_launch(a, ws, reinterpret_cast<hipStream_t>(stream)), fn);
}

// ---------------------------------------------------------------- decode / SRE

kla_status_t kla_decode_workspace_size(int N, int d_qk, int d_v, const kla_sre_args_t* sre,
                                       size_t* bytes) {
  const char* fn = "kla_decode_workspace_size";
  if (!bytes) return fail(KLA_ERR_INVALID_ARGUMENT, "%s: bytes is NULL", fn);
  *bytes = 0;
  if (N < 1) return fail(KLA_ERR_INVALID_ARGUMENT, "%s: N must be >= 1", fn);
  if (!dim_ok(d_qk) || !dim_ok(d_v))
    return fail(KLA_ERR_UNSUPPORTED, "%s: d_qk, d_v must be 16, 32 or 64", fn);
  kla::DecodeArgs a{};
  a.N = N;
  a.dqk = d_qk;
  a.dv = d_v;
  kla::SreArgs s{};
  if (sre) {
    if (sre->n_cand < 1 || sre->n_cand > 256)
      return fail(KLA_ERR_UNSUPPORTED, "%s: n_cand must be in [1, 256]", fn);
    s = make_sre(sre);
  }
  *bytes = kla::decode_workspace(a, sre ? &s : nullptr);
  return ok();
}

kla_status_t kla_decode_step(int N, int d_qk, int d_v, float eps, float* H, float* s,
                             const void* q, const void* k, const void* v, kla_dtype_t in_dtype,
                             void* o, kla_dtype_t out_dtype, const kla_sre_args_t* sre, void* ws,
                             size_t ws_bytes, kla_stream_t stream) {
  const char* fn = "kla_decode_step";
  if (N < 1) return fail(KLA_ERR_INVALID_ARGUMENT, "%s: N must be >= 1", fn);
  if (!dim_ok(d_qk) || !dim_ok(d_v))
    return fail(KLA_ERR_UNSUPPORTED, "%s: d_qk, d_v must be 16, 32 or 64 (got %d, %d)", fn, d_qk, d_v);
  if (!dtype_ok(in_dtype) || !dtype_ok(out_dtype))
    return fail(KLA_ERR_UNSUPPORTED, "%s: unknown dtype", fn);
  if (!std::isfinite(eps) || eps < 0.0f)
    return fail(KLA_ERR_INVALID_ARGUMENT, "%s: eps must be finite and >= 0", fn);
  if (!H || !s || !q || !k || !v || !o)
    return fail(KLA_ERR_INVALID_ARGUMENT, "%s: H, s, q, k, v, o are required", fn);
  if (N > kMaxHeads) return fail(KLA_ERR_UNSUPPORTED, "%s: N = %d exceeds %d", fn, N, kMaxHeads);
  kla_status_t st = check_align(fn, {{"H", H}, {"s", s}, {"q", q}, {"k", k}, {"v", v}, {"o", o}, {"ws", ws}});
  if (st != KLA_OK) return st;
  kla::SreArgs sa{};
  if (sre) {
    st = check_sre(N, d_qk, d_v, sre, fn);
    if (st != KLA_OK) return st;
    sa = make_sre(sre);
  }
  kla::DecodeArgs a{};
  a.N = N;
  a.dqk = d_qk;
  a.dv = d_v;
  a.eps = eps;
  a.H = H;
  a.s = s;
  a.q = q;
  a.k = k;
  a.v = v;
  a.in_bf16 = in_dtype == KLA_BF16;
  a.o = o;
  a.out_bf16 = out_dtype == KLA_BF16;
  st = check_ws(kla::decode_workspace(a, sre ? &sa : nullptr), ws, ws_bytes, fn);
  if (st != KLA_OK) return st;
  return hip_status(kla::decode_launch(a, sre ? &sa : nullptr, ws, reinterpret_cast<hipStream_t>(stream)),
                    fn);
}

int kla_decode_pending_period(void) { return KLA_DECODE_PENDING; }

namespace {

kla_status_t check_pending(const char* fn, int N, const float* H, const float* s, const float* pend_k,
                           const float* pend_v, int n_pend) {
  if (n_pend < 0 || n_pend > KLA_DECODE_PENDING - 1)
    return fail(KLA_ERR_INVALID_ARGUMENT, "%s: n_pend must be in [0, %d] (got %d)", fn, KLA_DECODE_PENDING - 1,
                n_pend);
  if (!pend_k || !pend_v) return fail(KLA_ERR_INVALID_ARGUMENT, "%s: pend_k and pend_v are required", fn);
  const size_t np = (size_t)N * KLA_DECODE_PENDING * 64 * sizeof(float);
  const size_t nH = (size_t)N * kla_phi_dim(64) * 64 * sizeof(float);
  const size_t ns = (size_t)N * kla_phi_dim(64) * sizeof(float);
  if (overlaps(pend_k, np, pend_v, np) || overlaps(pend_k, np, H, nH) || overlaps(pend_k, np, s, ns) ||
      overlaps(pend_v, np, H, nH) || overlaps(pend_v, np, s, ns))
    return fail(KLA_ERR_INVALID_ARGUMENT, "%s: pend_k, pend_v, H and s must not overlap", fn);
  return KLA_OK;
}

}  // namespace

kla_status_t kla_decode_step_deferred(int N, int d_qk, int d_v, float eps, float* H, float* s, float* pend_k,
                                      float* pend_v, int n_pend, const void* q, const void* k, const void* v,
                                      kla_dtype_t in_dtype, void* o, kla_dtype_t out_dtype,
                                      const kla_sre_args_t* sre, kla_stream_t stream) {
  const char* fn = "kla_decode_step_deferred";
  if (N < 1) return fail(KLA_ERR_INVALID_ARGUMENT, "%s: N must be >= 1", fn);
  if (d_qk != 64 || d_v != 64)
    return fail(KLA_ERR_UNSUPPORTED, "%s: needs d_qk = d_v = 64 (got %d, %d)", fn, d_qk, d_v);
  if (!dtype_ok(in_dtype) || !dtype_ok(out_dtype)) return fail(KLA_ERR_UNSUPPORTED, "%s: unknown dtype", fn);
  if (!std::isfinite(eps) || eps < 0.0f)
    return fail(KLA_ERR_INVALID_ARGUMENT, "%s: eps must be finite and >= 0", fn);
  if (!H || !s || !q || !k || !v || !o)
    return fail(KLA_ERR_INVALID_ARGUMENT, "%s: H, s, q, k, v, o are required", fn);
  if (N > kMaxHeads) return fail(KLA_ERR_UNSUPPORTED, "%s: N = %d exceeds %d", fn, N, kMaxHeads);
  kla_status_t st = check_pending(fn, N, H, s, pend_k, pend_v, n_pend);
  if (st != KLA_OK) return st;
  st = check_align(fn, {{"H", H}, {"s", s}, {"pend_k", pend_k}, {"pend_v", pend_v}, {"q", q}, {"k", k},
                        {"v", v}, {"o", o}});
  if (st != KLA_OK) return st;
  kla::SreArgs sa{};
  if (sre) {
    st = check_sre(N, d_qk, d_v, sre, fn);
    if (st != KLA_OK) return st;
    sa = make_sre(sre);
    if (!kla::decode_fused_supported(d_qk, d_v, sa))
      return fail(KLA_ERR_UNSUPPORTED, "%s: n_cand = %d exceeds 64", fn, sre->n_cand);
  }
  kla::DecodeArgs a{};
  a.N = N;
  a.dqk = d_qk;
  a.dv = d_v;
  a.eps = eps;
  a.H = H;
  a.s = s;
  a.q = q;
  a.k = k;
  a.v = v;
  a.in_bf16 = in_dtype == KLA_BF16;
  a.o = o;
  a.out_bf16 = out_dtype == KLA_BF16;
  return hip_status(kla::decode_deferred_launch(a, sre ? &sa : nullptr, pend_k, pend_v, n_pend,
                                                reinterpret_cast<hipStream_t>(stream)),
                    fn);
}

kla_status_t kla_decode_flush(int N, int d_qk, int d_v, float* H, float* s, const float* pend_k,
                              const float* pend_v, int n_pend, kla_stream_t stream) {
  const char* fn = "kla_decode_flush";
  if (N < 1) return fail(KLA_ERR_INVALID_ARGUMENT, "%s: N must be >= 1", fn);
  if (d_qk != 64 || d_v != 64)
    return fail(KLA_ERR_UNSUPPORTED, "%s: needs d_qk = d_v = 64 (got %d, %d)", fn, d_qk, d_v);
  if (!H || !s) return fail(KLA_ERR_INVALID_ARGUMENT, "%s: H and s are required", fn);
  if (N > kMaxHeads) return fail(KLA_ERR_UNSUPPORTED, "%s: N = %d exceeds %d", fn, N, kMaxHeads);
  kla_status_t st = check_pending(fn, N, H, s, pend_k, pend_v, n_pend);
  if (st != KLA_OK) return st;
  st = check_align(fn, {{"H", H}, {"s", s}, {"pend_k", pend_k}, {"pend_v", pend_v}});
  if (st != KLA_OK) return st;
  return hip_status(kla::decode_flush_launch(N, H, s, pend_k, pend_v, n_pend, reinterpret_cast<hipStream_t>(stream)),
                    fn);
}

kla_status_t kla_sre_workspace_size(int N, int d_qk, int d_v, const kla_sre_args_t* sre,
                                    size_t* bytes) {
  const char* fn = "kla_sre_workspace_size";
  if (!bytes) return fail(KLA_ERR_INVALID_ARGUMENT, "%s: bytes is NULL", fn);
  *bytes = 0;
  if (N < 1) return fail(KLA_ERR_INVALID_ARGUMENT, "%s: N must be >= 1", fn);
  if (!dim_ok(d_qk) || !dim_ok(d_v))
    return fail(KLA_ERR_UNSUPPORTED, "%s: d_qk, d_v must be 16, 32 or 64", fn);
  if (!sre) return fail(KLA_ERR_INVALID_ARGUMENT, "%s: sre arguments are NULL", fn);
  if (sre->n_cand < 1 || sre->n_cand > 256)
    return fail(KLA_ERR_UNSUPPORTED, "%s: n_cand must be in [1, 256]", fn);
  *bytes = kla::sre_workspace(N, d_qk, d_v, make_sre(sre));
  return ok();
}

kla_status_t kla_sre_select(int N, int d_qk, int d_v, float eps, const float* H, const float* s,
                            const kla_sre_args_t* sre, void* ws, size_t ws_bytes,
                            kla_stream_t stream) {
  const char* fn = "kla_sre_select";
  if (N < 1) return fail(KLA_ERR_INVALID_ARGUMENT, "%s: N must be >= 1", fn);
  if (!dim_ok(d_qk) || !dim_ok(d_v))
    return fail(KLA_ERR_UNSUPPORTED, "%s: d_qk, d_v must be 16, 32 or 64 (got %d, %d)", fn, d_qk, d_v);
  if (!std::isfinite(eps) || eps < 0.0f)
    return fail(KLA_ERR_INVALID_ARGUMENT, "%s: eps must be finite and >= 0", fn);
  if (!H || !s) return fail(KLA_ERR_INVALID_ARGUMENT, "%s: H and s are required", fn);
  if (N > kMaxHeads) return fail(KLA_ERR_UNSUPPORTED, "%s: N = %d exceeds %d", fn, N, kMaxHeads);
  kla_status_t st = check_sre(N, d_qk, d_v, sre, fn);
  if (st != KLA_OK) return st;
  st = check_align(fn, {{"H", H}, {"s", s}, {"ws", ws}});
  if (st != KLA_OK) return st;
  const kla::SreArgs sa = make_sre(sre);
  st = check_ws(kla::sre_workspace(N, d_qk, d_v, sa), ws, ws_bytes, fn);
  if (st != KLA_OK) return st;
  return hip_status(kla::sre_launch(N, d_qk, d_v, eps, H, s, sa, ws, reinterpret_cast<hipStream_t>(stream)),
                    fn);
}

// ---------------------------------------------------------------- hybrid

kla_status_t kla_hybrid_workspace_size(const kla_shape_t* shp, const kla_hybrid_cfg_t* cfg,
                                       size_t* bytes) {
  const char* fn = "kla_hybrid_workspace_size";
  if (!bytes) return fail(KLA_ERR_INVALID_ARGUMENT, "%s: bytes is NULL", fn);
  *bytes = 0;
  kla_status_t st = check_hybrid(shp, cfg, fn);
  if (st != KLA_OK) return st;
  *bytes = kla::hybrid_workspace(make_hybrid(shp, cfg));
  return ok();
}

kla_status_t kla_hybrid_prefill_streams(const kla_shape_t* shp, const kla_hybrid_cfg_t* cfg, const void* q,
                                        const void* k, const void* v, void* o, float* H_T, float* s_T,
                                        int32_t* cache_tokens_T, int32_t* sel_trace, void* ws, size_t ws_bytes,
                                        kla_stream_t stream, kla_stream_t aux_stream) {
  const char* fn = "kla_hybrid_prefill";
  kla_status_t st = check_hybrid(shp, cfg, fn);
  if (st != KLA_OK) return st;
  if (!q || !k || !v || !o) return fail(KLA_ERR_INVALID_ARGUMENT, "%s: q, k, v, o are required", fn);
  if ((H_T == nullptr) != (s_T == nullptr))
    return fail(KLA_ERR_INVALID_ARGUMENT, "%s: give both H_T and s_T or neither", fn);
  st = check_align(fn, {{"q", q}, {"k", k}, {"v", v}, {"o", o}, {"H_T", H_T}, {"s_T", s_T},
                        {"cache_tokens_T", cache_tokens_T}, {"sel_trace", sel_trace}, {"ws", ws}});
  if (st != KLA_OK) return st;
  kla::HybridArgs a = make_hybrid(shp, cfg);
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.HT = H_T;
  a.sT = s_T;
  a.cache_T = cache_tokens_T;
  a.trace = sel_trace;
  // the workspace size depends on which state outputs the caller provides
  st = check_ws(kla::hybrid_workspace(a), ws, ws_bytes, fn);
  if (st != KLA_OK) return st;
  return hip_status(kla::hybrid_launch(a, ws, reinterpret_cast<hipStream_t>(stream),
                                       reinterpret_cast<hipStream_t>(aux_stream)),
                    fn);
}

kla_status_t kla_hybrid_prefill(const kla_shape_t* shp, const kla_hybrid_cfg_t* cfg,
                                const void* q, const void* k, const void* v, void* o, float* H_T,
                                float* s_T, int32_t* cache_tokens_T, int32_t* sel_trace,
                                void* ws, size_t ws_bytes, kla_stream_t stream) {
  return kla_hybrid_prefill_streams(shp, cfg, q, k, v, o, H_T, s_T, cache_tokens_T, sel_trace, ws, ws_bytes,
                                    stream, nullptr);
}

// ---------------------------------------------------------------- hybrid decode

}  // extern "C"

namespace {

kla_status_t check_hybrid_decode(int N, int d_qk, int d_v, const kla_hybrid_cfg_t* cfg, const char* fn) {
  if (N < 1) return fail(KLA_ERR_INVALID_ARGUMENT, "%s: N must be >= 1", fn);
  if (!dim_ok(d_qk) || !dim_ok(d_v))
    return fail(KLA_ERR_UNSUPPORTED, "%s: d_qk, d_v must be 16, 32 or 64 (got %d, %d)", fn, d_qk, d_v);
  if (N > kMaxHeads) return fail(KLA_ERR_UNSUPPORTED, "%s: N = %d exceeds %d", fn, N, kMaxHeads);
  if (!cfg) return fail(KLA_ERR_INVALID_ARGUMENT, "%s: cfg is NULL", fn);
  if (cfg->window < 0 || cfg->cache_size < 0)
    return fail(KLA_ERR_INVALID_ARGUMENT, "%s: need window >= 0, cache_size >= 0", fn);
  if (cfg->refresh != 1)
    return fail(KLA_ERR_UNSUPPORTED, "%s: token-by-token decode needs refresh = 1 (got %d)", fn, cfg->refresh);
  if (cfg->cache_size > 255)
    return fail(KLA_ERR_UNSUPPORTED, "%s: cache_size = %d exceeds 255", fn, cfg->cache_size);
  if (cfg->window > (1 << 24))
    return fail(KLA_ERR_UNSUPPORTED, "%s: window = %d too large", fn, cfg->window);
  if (!std::isfinite(cfg->softmax_scale))
    return fail(KLA_ERR_INVALID_ARGUMENT, "%s: softmax_scale must be finite", fn);
  return KLA_OK;
}

}  // namespace

extern "C" {

kla_status_t kla_hybrid_decode_workspace_size(int N, int d_qk, int d_v, const kla_hybrid_cfg_t* cfg,
                                              size_t* bytes) {
  const char* fn = "kla_hybrid_decode_workspace_size";
  if (!bytes) return fail(KLA_ERR_INVALID_ARGUMENT, "%s: bytes is NULL", fn);
  *bytes = 0;
  kla_status_t st = check_hybrid_decode(N, d_qk, d_v, cfg, fn);
  if (st != KLA_OK) return st;
  kla::HybridDecodeArgs a{};
  a.N = N;
  a.dqk = d_qk;
  a.dv = d_v;
  a.window = cfg->window;
  a.cache_size = cfg->cache_size;
  *bytes = kla::hybrid_decode_workspace(a);
  return ok();
}

}  // extern "C"

namespace {

// Checks and argument packing shared by the two hybrid decode entry points;
// `ws` may be NULL here (the static variant brings its own scratch).
kla_status_t hybrid_decode_args(const char* fn, int N, int d_qk, int d_v, float eps, const kla_hybrid_cfg_t* cfg,
                                int t, const kla_hybrid_state_t* state, const void* q, const void* k, const void* v,
                                kla_dtype_t in_dtype, void* o, kla_dtype_t out_dtype, int32_t* rejected,
                                const void* ws, kla::HybridDecodeArgs* out) {
  kla_status_t st = check_hybrid_decode(N, d_qk, d_v, cfg, fn);
  if (st != KLA_OK) return st;
  if (!dtype_ok(in_dtype) || !dtype_ok(out_dtype)) return fail(KLA_ERR_UNSUPPORTED, "%s: unknown dtype", fn);
  if (!std::isfinite(eps) || eps < 0.0f)
    return fail(KLA_ERR_INVALID_ARGUMENT, "%s: eps must be finite and >= 0", fn);
  if (t < 0) return fail(KLA_ERR_INVALID_ARGUMENT, "%s: t must be >= 0 (got %d)", fn, t);
  if (!state) return fail(KLA_ERR_INVALID_ARGUMENT, "%s: state is NULL", fn);
  if (!q || !k || !v || !o) return fail(KLA_ERR_INVALID_ARGUMENT, "%s: q, k, v, o are required", fn);
  const kla_hybrid_state_t& S = *state;
  if (!S.H || !S.s || !S.win_k || !S.win_v || !S.pend_k || !S.pend_v)
    return fail(KLA_ERR_INVALID_ARGUMENT, "%s: state H, s, win_k, win_v, pend_k, pend_v are required", fn);
  if (cfg->cache_size > 0 && (!S.cache_k || !S.cache_v || !S.cache_ids || !S.cache_sums))
    return fail(KLA_ERR_INVALID_ARGUMENT,
                "%s: cache_k, cache_v, cache_ids, cache_sums are required when cache_size > 0", fn);
  if (!aligned16(S.H) || !aligned16(S.s) || !aligned16(S.win_k) || !aligned16(S.win_v) ||
      !aligned16(S.cache_k) || !aligned16(S.cache_v) || !aligned16(S.cache_ids) || !aligned16(S.pend_k) ||
      !aligned16(S.pend_v) || !aligned16(S.cache_sums))
    return fail(KLA_ERR_INVALID_ARGUMENT, "%s: state pointers must be 16-byte aligned", fn);
  if (S.row_dtype != in_dtype)
    return fail(KLA_ERR_INVALID_ARGUMENT, "%s: the state's row_dtype (%d) must be the step's in_dtype (%d)", fn,
                (int)S.row_dtype, (int)in_dtype);
  st = check_align(fn, {{"q", q}, {"k", k}, {"v", v}, {"o", o}, {"rejected", rejected}, {"ws", ws}});
  if (st != KLA_OK) return st;
  kla::HybridDecodeArgs& a = *out;
  a = kla::HybridDecodeArgs{};
  a.N = N;
  a.dqk = d_qk;
  a.dv = d_v;
  a.in_bf16 = in_dtype == KLA_BF16;
  a.out_bf16 = out_dtype == KLA_BF16;
  a.eps = eps;
  a.window = cfg->window;
  a.cache_size = cfg->cache_size;
  a.scale = cfg->softmax_scale;
  a.t = t;
  a.H = S.H;
  a.s = S.s;
  a.win_k = S.win_k;
  a.win_v = S.win_v;
  a.cache_k = S.cache_k;
  a.cache_v = S.cache_v;
  a.cache_ids = S.cache_ids;
  a.pend_k = S.pend_k;
  a.pend_v = S.pend_v;
  a.cache_sums = S.cache_sums;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.rejected = rejected;
  return KLA_OK;
}

}  // namespace

extern "C" {

kla_status_t kla_hybrid_decode_step(int N, int d_qk, int d_v, float eps, const kla_hybrid_cfg_t* cfg, int t,
                                    const kla_hybrid_state_t* state, const void* q, const void* k,
                                    const void* v, kla_dtype_t in_dtype, void* o, kla_dtype_t out_dtype,
                                    int32_t* rejected, void* ws, size_t ws_bytes, kla_stream_t stream) {
  const char* fn = "kla_hybrid_decode_step";
  kla::HybridDecodeArgs a;
  kla_status_t st = hybrid_decode_args(fn, N, d_qk, d_v, eps, cfg, t, state, q, k, v, in_dtype, o, out_dtype,
                                       rejected, ws, &a);
  if (st != KLA_OK) return st;
  st = check_ws(kla::hybrid_decode_workspace(a), ws, ws_bytes, fn);
  if (st != KLA_OK) return st;
  return hip_status(kla::hybrid_decode_launch(a, ws, reinterpret_cast<hipStream_t>(stream)), fn);
}

size_t kla_hybrid_decode_static_limit(void) { return kla::kHybridDecodeStaticScratch; }
int kla_hybrid_decode_pending_slots(void) { return KLA_HYBRID_PENDING; }

kla_status_t kla_hybrid_decode_step_static(int N, int d_qk, int d_v, float eps, const kla_hybrid_cfg_t* cfg, int t,
                                           const kla_hybrid_state_t* state, const void* q, const void* k,
                                           const void* v, kla_dtype_t in_dtype, void* o, kla_dtype_t out_dtype,
                                           int32_t* rejected, kla_stream_t stream) {
  const char* fn = "kla_hybrid_decode_step_static";
  kla::HybridDecodeArgs a;
  kla_status_t st = hybrid_decode_args(fn, N, d_qk, d_v, eps, cfg, t, state, q, k, v, in_dtype, o, out_dtype,
                                       rejected, nullptr, &a);
  if (st != KLA_OK) return st;
  const size_t need = kla::hybrid_decode_workspace(a);
  if (need > kla::kHybridDecodeStaticScratch)
    return fail(KLA_ERR_UNSUPPORTED,
                "%s: this call needs %zu bytes of scratch, more than the library's static %zu "
                "(use kla_hybrid_decode_step with a workspace)",
                fn, need, (size_t)kla::kHybridDecodeStaticScratch);
  void* scratch = nullptr;
  const hipError_t e = kla::hybrid_decode_static_scratch(&scratch);
  if (e != hipSuccess) return hip_status(e, fn);
  return hip_status(kla::hybrid_decode_launch(a, scratch, reinterpret_cast<hipStream_t>(stream)), fn);
}

kla_status_t kla_hybrid_decode_flush(int N, int d_qk, int d_v, const kla_hybrid_state_t* state,
                                     kla_stream_t stream) {
  const char* fn = "kla_hybrid_decode_flush";
  if (N < 1) return fail(KLA_ERR_INVALID_ARGUMENT, "%s: N must be >= 1", fn);
  if (!dim_ok(d_qk) || !dim_ok(d_v))
    return fail(KLA_ERR_UNSUPPORTED, "%s: d_qk, d_v must be 16, 32 or 64 (got %d, %d)", fn, d_qk, d_v);
  if (N > kMaxHeads) return fail(KLA_ERR_UNSUPPORTED, "%s: N = %d exceeds %d", fn, N, kMaxHeads);
  if (!state || !state->H || !state->s || !state->pend_k || !state->pend_v)
    return fail(KLA_ERR_INVALID_ARGUMENT, "%s: state H, s, pend_k, pend_v are required", fn);
  kla_status_t st = check_align(fn, {{"H", state->H}, {"s", state->s}, {"pend_k", state->pend_k},
                                     {"pend_v", state->pend_v}});
  if (st != KLA_OK) return st;
  kla::HybridDecodeArgs a{};
  a.N = N;
  a.dqk = d_qk;
  a.dv = d_v;
  a.H = state->H;
  a.s = state->s;
  a.pend_k = state->pend_k;
  a.pend_v = state->pend_v;
  return hip_status(kla::hybrid_decode_flush_launch(a, reinterpret_cast<hipStream_t>(stream)), fn);
}

kla_status_t kla_hybrid_decode_prime(int N, int d_qk, int d_v, const kla_hybrid_cfg_t* cfg, int t,
                                     const kla_hybrid_state_t* state, kla_stream_t stream) {
  const char* fn = "kla_hybrid_decode_prime";
  kla_status_t st = check_hybrid_decode(N, d_qk, d_v, cfg, fn);
  if (st != KLA_OK) return st;
  if (t < 0) return fail(KLA_ERR_INVALID_ARGUMENT, "%s: t must be >= 0 (got %d)", fn, t);
  if (!state || !state->H || !state->s || !state->pend_k || !state->pend_v)
    return fail(KLA_ERR_INVALID_ARGUMENT, "%s: state H, s, pend_k, pend_v are required", fn);
  if (cfg->cache_size > 0 && (!state->cache_k || !state->cache_sums))
    return fail(KLA_ERR_INVALID_ARGUMENT, "%s: cache_k, cache_sums are required when cache_size > 0", fn);
  if (!dtype_ok(state->row_dtype)) return fail(KLA_ERR_UNSUPPORTED, "%s: unknown row_dtype", fn);
  st = check_align(fn, {{"H", state->H}, {"s", state->s}, {"pend_k", state->pend_k}, {"pend_v", state->pend_v},
                        {"cache_k", state->cache_k}, {"cache_sums", state->cache_sums}});
  if (st != KLA_OK) return st;
  kla::HybridDecodeArgs a{};
  a.N = N;
  a.dqk = d_qk;
  a.dv = d_v;
  a.window = cfg->window;
  a.cache_size = cfg->cache_size;
  a.t = t;
  a.in_bf16 = state->row_dtype == KLA_BF16;
  a.H = state->H;
  a.s = state->s;
  a.pend_k = state->pend_k;
  a.pend_v = state->pend_v;
  a.cache_k = state->cache_k;
  a.cache_sums = state->cache_sums;
  return hip_status(kla::hybrid_decode_prime_launch(a, reinterpret_cast<hipStream_t>(stream)), fn);
}

}  // extern "C"
