/*
 * kla.h - C ABI of libkla: causal kernelized linear attention on AMD MI355X
 * (gfx950).
 *
 * Pages cited:
 *   KATA = "Kernelized Linear Attention: Breaking the Capacity Wall with
 *          Symmetric Cones" (gist.science/pt/paper/2607.17419);
 *   LoLA = "LoLA: Low-Rank Linear Attention with Sparse Caching", Portuguese
 *          technical summary (gist.science/pt/paper/2505.23666).
 *
 * What is computed (per attention head, tokens t = 0..T-1):
 *   o_t = phi(q_t)^T H_t / (phi(q_t)^T s_t + eps),
 *   H_t = sum_{i<=t} phi(k_i) v_i^T,   s_t = sum_{i<=t} phi(k_i)
 * with the rank-one PSD lift of KATA §2.2, psi(u) = u u^T, vectorised as
 *   phi(x)_f = x_i^2 (i == j),  sqrt(2) x_i x_j (i < j),
 *   f(i, j) = i*d - i*(i-1)/2 + (j - i),  D = d(d+1)/2,
 * so that phi(q) . phi(k) = (q . k)^2. KATA §1 states the problem (normalised
 * linear attention over a fixed-size state); KATA §2.3 gives the chunked
 * form with a cross-chunk prefix of the state; LoLA ("Metodologia") names the
 * state (H_t, s_t) and defines the self-recall error and the three-memory
 * hybrid ("Estratégia de Inferência").
 *
 * Conventions shared by every call:
 *   - Memory: every tensor pointer is a device pointer owned by the caller.
 *     The library never allocates or frees device memory and keeps no
 *     state between calls; scratch memory comes from the caller through
 *     `ws`, sized by the matching *_workspace_size query (the one exception,
 *     kla_hybrid_decode_step_static, uses an array of the library's own,
 *     described there). Every device
 *     pointer (tensors and `ws`) must be 16-byte aligned: the kernels move
 *     rows with 16-byte vector accesses. A misaligned pointer is rejected
 *     with KLA_ERR_INVALID_ARGUMENT.
 *   - Layout: tensors are dense row-major (C order), shapes given below.
 *     N = B*H heads, ordered (b, h). The state is H [N, D, d_v] and
 *     s [N, D], float32, in the coordinate order and sqrt(2) scaling above.
 *   - Execution: every call enqueues its kernels on `stream` (a hipStream_t;
 *     NULL is the null stream) and returns without synchronising; it
 *     launches on no other stream unless the caller passes one
 *     (kla_hybrid_prefill_streams). Device faults surface at the caller's
 *     next synchronisation.
 *   - Errors: every argument is checked on the host before anything is
 *     enqueued; a call that fails a check returns its status, enqueues
 *     nothing and writes no output. A failed launch returns KLA_ERR_HIP.
 *     kla_last_error() gives a text for the last failure on this thread.
 *     No C++ exception crosses this interface.
 *   - Data: inputs must be finite; values are not checked.
 *   - Supported now: d_qk, d_v in {16, 32, 64}; chunk in {32, 64, 128};
 *     any T >= 1 (the last chunk may be partial). Other shapes return
 *     KLA_ERR_UNSUPPORTED.
 */
#ifndef KLA_H
#define KLA_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define KLA_API __attribute__((visibility("default")))
#else
#define KLA_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

/* Same type as hipStream_t, declared here so that C callers need no HIP header. */
struct ihipStream_t;
typedef struct ihipStream_t* kla_stream_t;

typedef enum {
  KLA_OK = 0,
  KLA_ERR_INVALID_ARGUMENT = 1, /* NULL required pointer, bad size, aliasing */
  KLA_ERR_UNSUPPORTED = 2,      /* shape or dtype outside the supported set */
  KLA_ERR_WORKSPACE = 3,        /* ws too small or NULL when needed */
  KLA_ERR_HIP = 4               /* a HIP runtime call or kernel launch failed */
} kla_status_t;

typedef enum { KLA_F32 = 0, KLA_BF16 = 1 } kla_dtype_t;

/* ABI version of this header (bumped on any incompatible change). */
#define KLA_ABI_VERSION 9
KLA_API int kla_abi_version(void);

/* D = d_qk (d_qk + 1) / 2, or -1 when d_qk < 1. */
KLA_API int kla_phi_dim(int d_qk);

/* Static text for a status code. */
KLA_API const char* kla_status_string(kla_status_t s);

/* Text describing the last failed call on the calling thread ("" if none). */
KLA_API const char* kla_last_error(void);

/* Shapes of a prefill-type call. q, k: [B, H, T, d_qk]; v, o: [B, H, T, d_v].
 * in_dtype applies to q, k and v; out_dtype to o. eps is added to every
 * denominator; a denominator of exactly 0 gives o = 0. */
typedef struct {
  int B, H, T, d_qk, d_v;
  kla_dtype_t in_dtype, out_dtype;
  float eps;
} kla_shape_t;

/* ------------------------------------------------------------------------
 * kla_prefill - chunked causal prefill (KATA §2.3, "Paralelismo por Blocos"
 * and the linear chunked-state operating point).
 *
 * Splits each head's tokens into chunks of `chunk`. Within a chunk the
 * masked (Q K^T)∘(Q K^T) scores multiply [V | 1]; across chunks the float32
 * state (H, s) is carried as a running prefix sum and read out by phi(Q).
 * Results equal the causal definition above up to rounding for every
 * supported chunk length.
 *
 *   q, k, v : inputs, in_dtype, shapes above (required).
 *   o       : output [B, H, T, d_v], out_dtype. May be NULL only when H_T and
 *             s_T are given (state-only mode: no outputs are computed).
 *   H0, s0  : initial state [N, D, d_v] and [N, D] float32, or both NULL for
 *             a zero state (resuming a previous call).
 *   H_T,s_T : final state, or both NULL to skip writing it. May alias H0/s0.
 *   ws      : workspace of at least kla_prefill_workspace_size() bytes
 *             (may be NULL when that size is 0).
 * ------------------------------------------------------------------------ */
/* 1 when kla_prefill serves this shape with the bf16 matrix-core kernel,
 * 0 when it uses the float32 vector-ALU kernel, -1 for an invalid shape. */
KLA_API int kla_prefill_matrix_path(const kla_shape_t* shp, int chunk);

KLA_API kla_status_t kla_prefill_workspace_size(const kla_shape_t* shp, int chunk, int with_output,
                                        size_t* bytes);
KLA_API kla_status_t kla_prefill(const kla_shape_t* shp, int chunk, const void* q, const void* k,
                         const void* v, void* o, const float* H0, const float* s0, float* H_T,
                         float* s_T, void* ws, size_t ws_bytes, kla_stream_t stream);

/* Multi-factor lifts (KATA-Mg, KATA-Sigma-g); see kla_prefill_factors and
 * kla_prefill_quadratic_factors. */
#define KLA_FACTORS_CONCAT 0
#define KLA_FACTORS_SUM 1

/* ------------------------------------------------------------------------
 * kla_prefill_factors - kla_prefill with a multi-factor lift (KATA §2.3,
 * "Variantes"; the factors read as g equal slices of p = d_qk / g of the
 * d_qk dimensions, see kla_prefill_quadratic_factors below):
 *   KLA_FACTORS_CONCAT (KATA-Mg): the factors' rank-one lifts concatenated,
 *     D_g = g p (p + 1) / 2 features (2080, 1056, 544 for d_qk = 64 and
 *     g = 1, 2, 4), laid out factor by factor, each block in the vec_sym
 *     order of kla_prefill (upper triangle row-major, sqrt(2) off the
 *     diagonal) over its p dimensions. bf16 inputs with d_qk = d_v = 64 run
 *     on the matrix path, the rest on the float32 vector path (1e-4).
 *   KLA_FACTORS_SUM (KATA-Sigma-g): the lift of sum_i x_i x_i^T,
 *     D = p (p + 1) / 2 features (2080, 528, 136), in the vec_sym order over
 *     p dimensions, feature (a, b) = sum_i x_i,a x_i,b (times sqrt(2) for
 *     a < b). bf16 inputs with d_qk = d_v = 64 run on the matrix path (bf16
 *     accuracy, 2e-2), the rest on the float32 vector path (float32
 *     arithmetic, 1e-4 relative; bf16 inputs are read exactly).
 * H0/s0/H_T/s_T are [N, D, d_v] and [N, D] float32 in that layout. The
 * outputs are those of kla_prefill_quadratic_factors with the same kind.
 *
 *   kind    : KLA_FACTORS_CONCAT or KLA_FACTORS_SUM.
 *   factors : 1, 2 or 4 (1 is kla_prefill, for either kind).
 *   ws      : at least kla_prefill_factors_workspace_size(shp, chunk, kind,
 *             factors, o != NULL) bytes (for KLA_FACTORS_CONCAT,
 *             kla_prefill_workspace_size of the same shape and chunk is
 *             enough too).
 *   other arguments: as for kla_prefill.
 * Every shape kla_prefill supports.
 * ------------------------------------------------------------------------ */
KLA_API kla_status_t kla_prefill_factors(const kla_shape_t* shp, int chunk, int kind, int factors,
                                         const void* q, const void* k, const void* v, void* o,
                                         const float* H0, const float* s0, float* H_T, float* s_T,
                                         void* ws, size_t ws_bytes, kla_stream_t stream);
/* Workspace bytes of kla_prefill_factors for this shape, chunk, kind and
 * number of factors, with (with_output != 0) or without outputs. */
KLA_API kla_status_t kla_prefill_factors_workspace_size(const kla_shape_t* shp, int chunk, int kind,
                                                        int factors, int with_output, size_t* bytes);

/* ------------------------------------------------------------------------
 * kla_prefill_quadratic - the same causal outputs in the quadratic form
 * (KATA §2.3, the first of its two operating points: a FlashAttention-style
 * forward that never forms the state). Since phi(q) . phi(k) = (q . k)^2,
 *   num_t = sum_{i<=t} (q_t . k_i)^2 v_i,  den_t = sum_{i<=t} (q_t . k_i)^2,
 *   o_t = num_t / (den_t + eps)  (0 when that denominator is 0),
 * equal to kla_prefill's outputs up to rounding. Work grows as T^2 (against
 * T D for the state form); the two are about equal at T of about
 * 4 D d_v / (d_qk + d_v) tokens. No state is produced and no workspace is
 * needed.
 *
 *   q, k, v : [B, H, T, 64] bf16 (required);  o : [B, H, T, 64], out_dtype
 *             (required).
 *   den     : [B, H, T] float32, or NULL: den_t + eps, the row denominators
 *             kla_prefill_quadratic_backward needs.
 * Supported: d_qk = d_v = 64, in_dtype bf16, out_dtype bf16 or float32;
 * other shapes return KLA_ERR_UNSUPPORTED.
 * ------------------------------------------------------------------------ */
KLA_API kla_status_t kla_prefill_quadratic(const kla_shape_t* shp, const void* q, const void* k,
                                   const void* v, void* o, float* den, kla_stream_t stream);

/* ------------------------------------------------------------------------
 * kla_prefill_quadratic_factors - kla_prefill_quadratic with a multi-factor
 * PSD lift (KATA §2.3, "Variantes": KATA-Mg, several PSD factors, and
 * KATA-Sigma-g, summed PSD factors). The page names the variants but not how
 * the factors are formed; this library reads them as g equal slices of the
 * d = 64 dimensions, q = (q_1, ..., q_g), k = (k_1, ..., k_g):
 *   kind KLA_FACTORS_CONCAT (KATA-Mg): the factors' rank-one lifts are
 *       concatenated (g p(p+1)/2 features, p = 64 / g), so the weight is
 *       w(q, k) = sum_i (q_i . k_i)^2;
 *   kind KLA_FACTORS_SUM (KATA-Sigma-g): the lift of sum_i x_i x_i^T
 *       (p(p+1)/2 features), so w(q, k) = sum_{i,j} (q_i . k_j)^2;
 * and o_t = sum_{i<=t} w(q_t, k_i) v_i / (sum_{i<=t} w(q_t, k_i) + eps).
 * factors = 1 is the rank-one lift of kla_prefill_quadratic (either kind).
 *
 *   kind    : KLA_FACTORS_CONCAT or KLA_FACTORS_SUM.
 *   factors : 1, 2 or 4.
 *   q, k, v, o, den : as for kla_prefill_quadratic (den holds the variant's
 *             denominators).
 * Supported: d_qk = d_v = 64, in_dtype bf16, out_dtype bf16 or float32;
 * another kind or factor count returns KLA_ERR_INVALID_ARGUMENT, other shapes
 * KLA_ERR_UNSUPPORTED.
 * ------------------------------------------------------------------------ */
KLA_API kla_status_t kla_prefill_quadratic_factors(const kla_shape_t* shp, int kind, int factors,
                                                   const void* q, const void* k, const void* v, void* o,
                                                   float* den, kla_stream_t stream);

/* ------------------------------------------------------------------------
 * kla_prefill_quadratic_backward - gradients of the causal prefill (the
 * function of kla_prefill and kla_prefill_quadratic) for training. With
 * s_ti = q_t . k_i, w_ti = s_ti^2 (i <= t), D_t = sum_i w_ti + eps and a
 * loss gradient g_t = dL/do_t, c_t = g_t . o_t = sum_i (w_ti / D_t) g_t . v_i:
 *   dv_i = sum_{t>=i} (w_ti / D_t) g_t,
 *   ds_ti = 2 s_ti (g_t . v_i - c_t) / D_t,
 *   dq_t = sum_{i<=t} ds_ti k_i,   dk_i = sum_{t>=i} ds_ti q_t
 * (the chain rule on the outputs of KATA §1 with the lift of §2.2). Rows
 * whose D_t is 0 pass no gradient. Computed in the quadratic form on the
 * bf16 matrix cores (float32 sums); c_t is recomputed from the same products
 * the gradients use, so the forward's output is not an input.
 *
 *   q, k, v     : [B, H, T, 64] bf16, the forward's inputs.
 *   den         : [B, H, T] float32 from kla_prefill_quadratic.
 *   dout        : [B, H, T, 64] out_dtype, dL/do.
 *   dq, dk, dv  : [B, H, T, 64] out_dtype outputs.
 *   ws          : kla_prefill_quadratic_backward_workspace_size bytes.
 * Supported: d_qk = d_v = 64, in_dtype bf16, out_dtype bf16 or float32.
 * ------------------------------------------------------------------------ */
KLA_API kla_status_t kla_prefill_quadratic_backward_workspace_size(const kla_shape_t* shp, size_t* bytes);
KLA_API kla_status_t kla_prefill_quadratic_backward(const kla_shape_t* shp, const void* q, const void* k,
                                            const void* v, const float* den, const void* dout, void* dq,
                                            void* dk, void* dv, void* ws, size_t ws_bytes,
                                            kla_stream_t stream);

/* ------------------------------------------------------------------------
 * Self-recall error and selection (LoLA, the self-recall-error section and
 * "Estratégia de Inferência" item 2).
 *
 * For candidate c of head n: pred = phi(k_c)^T H / (phi(k_c)^T s + eps)
 * (pred = 0 when that denominator is 0) and score = ||pred - v_c||^2.
 * The top_k candidates by (score descending, candidate index ascending) are
 * selected; `sel` lists them in that order.
 *
 *   cand_k : [N, n_cand, d_qk] float32;  cand_v : [N, n_cand, d_v] float32.
 *   scores : [N, n_cand] float32 output, or NULL.
 *   sel    : [N, top_k] int32 output (required).
 *   sel_k, sel_v : optional gather of the selected pairs, both or neither:
 *            head n's j-th selected pair goes to row n * sel_stride + j of
 *            sel_k ([., d_qk]) and sel_v ([., d_v]), float32. sel_stride = 0
 *            means top_k (dense [N, top_k, d]); a larger stride lets the gather
 *            fill the first top_k rows of a following call's candidate array.
 *            The gathered rows must not overlap cand_k / cand_v.
 * Supported: 1 <= top_k <= n_cand <= 256; sel_stride = 0 or >= top_k.
 * ------------------------------------------------------------------------ */
typedef struct {
  int n_cand, top_k;
  const float* cand_k;
  const float* cand_v;
  float* scores;
  int32_t* sel;
  float* sel_k;
  float* sel_v;
  int sel_stride;
} kla_sre_args_t;

/* ------------------------------------------------------------------------
 * kla_decode_step - one recurrent token for N independent head-states
 * (KATA §1, constant-time recurrent inference; LoLA "Estratégia de
 * Inferência", token-by-token mode).
 *
 * For every head n: s += phi(k); H += phi(k) v^T (the update comes first,
 * since H_t sums i <= t); o = phi(q)^T H / (phi(q)^T s + eps).
 * If `sre` is not NULL, the candidates are then scored and selected as in
 * kla_sre_select, against the UPDATED state, in the same call.
 *
 *   H, s : [N, D, d_v], [N, D] float32, updated in place.
 *   q, k : [N, d_qk]; v : [N, d_v]; in_dtype.   o : [N, d_v], out_dtype.
 * ------------------------------------------------------------------------ */
KLA_API kla_status_t kla_decode_workspace_size(int N, int d_qk, int d_v, const kla_sre_args_t* sre,
                                       size_t* bytes);
KLA_API kla_status_t kla_decode_step(int N, int d_qk, int d_v, float eps, float* H, float* s,
                             const void* q, const void* k, const void* v, kla_dtype_t in_dtype,
                             void* o, kla_dtype_t out_dtype, const kla_sre_args_t* sre, void* ws,
                             size_t ws_bytes, kla_stream_t stream);

/* ------------------------------------------------------------------------
 * kla_decode_step_deferred - kla_decode_step with deferred folds (the same
 * passages; KATA §2.2 for the closed form below).
 *
 * A head-state is (H, s) plus the pairs waiting in its pending slots:
 *   H' = H + sum_{j < n_pend} phi(pend_k_j) pend_v_j^T,
 *   s' = s + sum_{j < n_pend} phi(pend_k_j).
 * The lift gives phi(x) . phi(y) = (x . y)^2, so a readout or a score over
 * H' is the one over H plus sum_j (x . pend_k_j)^2 [pend_v_j | 1]: H and s
 * need not be written at every token. The call stores the token's (k, v)
 * in slot n_pend, reads H and s (writing neither), and reads out and scores
 * against H' with the token added. The caller then holds n_pend + 1 pending
 * pairs, except when that fills the slots (n_pend = KLA_DECODE_PENDING - 1):
 * the call then adds all KLA_DECODE_PENDING of them to H and s in a second
 * pass over the state, and the caller holds 0. H is read once per token and
 * read and written once more per KLA_DECODE_PENDING tokens. o, the scores and
 * the selection are those of kla_decode_step on the same sequence of tokens
 * (the same values up to float32 rounding order).
 *
 *   H, s   : [N, D, d_v], [N, D] float32.
 *   pend_k, pend_v : [N, KLA_DECODE_PENDING, d_qk] / [.., d_v] float32;
 *            slots n_pend and above are ignored and may hold anything.
 *   n_pend : 0 .. KLA_DECODE_PENDING - 1, the same for every head-state.
 *   q, k, v, o, sre : as kla_decode_step; sre may be NULL.
 * Errors: n_pend out of range, overlapping pend_k / pend_v / H / s, or a
 * pointer not 16-byte aligned is KLA_ERR_INVALID_ARGUMENT.
 * Supported: d_qk = d_v = 64; sre NULL or n_cand <= 64. No workspace.
 *
 * kla_decode_flush adds the first n_pend slots to H and s (n_pend = 0 does
 * nothing; 0 <= n_pend < KLA_DECODE_PENDING); afterwards the caller holds 0
 * pending pairs. kla_decode_pending_period returns KLA_DECODE_PENDING.
 * ------------------------------------------------------------------------ */
#define KLA_DECODE_PENDING 8
KLA_API int kla_decode_pending_period(void);
KLA_API kla_status_t kla_decode_step_deferred(int N, int d_qk, int d_v, float eps, float* H, float* s,
                                              float* pend_k, float* pend_v, int n_pend, const void* q,
                                              const void* k, const void* v, kla_dtype_t in_dtype, void* o,
                                              kla_dtype_t out_dtype, const kla_sre_args_t* sre,
                                              kla_stream_t stream);
KLA_API kla_status_t kla_decode_flush(int N, int d_qk, int d_v, float* H, float* s, const float* pend_k,
                                      const float* pend_v, int n_pend, kla_stream_t stream);

/* kla_sre_select - scoring and selection only; H and s are read, not written. */
KLA_API kla_status_t kla_sre_workspace_size(int N, int d_qk, int d_v, const kla_sre_args_t* sre,
                                    size_t* bytes);
KLA_API kla_status_t kla_sre_select(int N, int d_qk, int d_v, float eps, const float* H, const float* s,
                            const kla_sre_args_t* sre, void* ws, size_t ws_bytes,
                            kla_stream_t stream);

/* ------------------------------------------------------------------------
 * kla_hybrid_prefill - LoLA's three memories over a prefill (LoLA
 * "Metodologia" items 1-3, "Estratégia de Inferência" items 1-4).
 *
 * Tokens are processed in blocks of `refresh`. At the start of block b the
 * eviction frontier is f = max(0, b*refresh - window); tokens that cross it
 * join the candidate set together with the current sparse cache. When the
 * candidates exceed cache_size, each is scored by the self-recall error
 * against the current linear state (before this refresh's fold); the
 * cache_size highest (score desc, token id asc) stay in the cache and all
 * others are folded into (H, s) by outer products. Each query t of the
 * block then reads one jointly normalised mixture:
 *   num = sum_{i in [f, t]} e^{a q.k_i} v_i + sum_{j in cache} e^{a q.k_j} v_j
 *         + phi(q)^T H,
 *   den = the same sums without v + phi(q)^T s + eps,   o_t = num / den,
 * with a = softmax_scale.
 *
 *   q, k : [B, H, T, d_qk]; v, o : [B, H, T, d_v]  (in_dtype / out_dtype).
 *   H_T, s_T        : final linear state, or both NULL.
 *   cache_tokens_T  : [N, cache_size] int32 final cache token ids ascending,
 *                     -1 for empty slots, or NULL.
 *   sel_trace       : [N, ceil(T/refresh), cache_size] int32, or NULL. Row b
 *                     holds the ids kept by block b's scored refresh
 *                     (ascending); rows of blocks without one are all -1.
 * Supported: d_qk, d_v in {16, 32, 64}; 1 <= refresh <= 128; window >= 0;
 * 0 <= cache_size and cache_size + refresh <= 256; softmax_scale finite.
 *
 * Every kernel runs on `stream`, in order.
 * ------------------------------------------------------------------------ */
typedef struct {
  int window, cache_size, refresh;
  float softmax_scale;
} kla_hybrid_cfg_t;

KLA_API kla_status_t kla_hybrid_workspace_size(const kla_shape_t* shp, const kla_hybrid_cfg_t* cfg,
                                       size_t* bytes);
KLA_API kla_status_t kla_hybrid_prefill(const kla_shape_t* shp, const kla_hybrid_cfg_t* cfg,
                                const void* q, const void* k, const void* v, void* o, float* H_T,
                                float* s_T, int32_t* cache_tokens_T, int32_t* sel_trace,
                                void* ws, size_t ws_bytes, kla_stream_t stream);

/* kla_hybrid_prefill with a second stream of the caller's (same results,
 * same passages). With d_qk = d_v = 64 and bf16 inputs, each block's
 * readout runs on `aux_stream` so that it overlaps the next refresh; the
 * call forks `aux_stream` from `stream` at its start and joins it back
 * before returning, so work queued afterwards on `stream` is ordered after
 * every kernel of the call, and work queued on `aux_stream` afterwards is
 * ordered after the call's readouts. The fork and join events are created
 * and released by the call itself. aux_stream = NULL (or = stream) runs
 * everything on `stream`. Two calls must not share one aux_stream
 * concurrently from different host threads. */
KLA_API kla_status_t kla_hybrid_prefill_streams(const kla_shape_t* shp, const kla_hybrid_cfg_t* cfg,
                                                const void* q, const void* k, const void* v, void* o,
                                                float* H_T, float* s_T, int32_t* cache_tokens_T,
                                                int32_t* sel_trace, void* ws, size_t ws_bytes,
                                                kla_stream_t stream, kla_stream_t aux_stream);

/* ------------------------------------------------------------------------
 * kla_hybrid_decode_step - LoLA's three memories token by token (LoLA
 * "Estratégia de Inferência", the token-by-token mode of items 1-4;
 * "Metodologia" items 1-3). One call advances every head-state by one token
 * and gives the same outputs as kla_hybrid_prefill with refresh = 1.
 *
 * `t` is the number of tokens each head-state has already seen (the new
 * token's id). With W = window and lambda = cache_size:
 *   1. when t > W, token e = t - W - 1 leaves the window. If the cache holds
 *      fewer than lambda pairs, e is added to it. Otherwise the lambda cached
 *      pairs and e are scored by the self-recall error against the linear
 *      state as it is before this call; the lambda highest (score desc,
 *      token id asc) stay in the cache and the remaining one, r, is folded
 *      into the state: H += phi(k_r) v_r^T, s += phi(k_r);
 *   2. the new token's query reads one jointly normalised mixture of the
 *      window [max(0, t - W), t] (the new token included), the cache and the
 *      linear state after the fold, with the weights of kla_hybrid_prefill;
 *   3. the new token's (k, v) enters the window.
 *
 * Deferred folds: the call does not add r's fold to H and s itself. It
 * stores r in pending slot t mod P of the state (P = KLA_HYBRID_PENDING),
 * and every call with t mod P = 0 folds all P slots into H and s in its own
 * pass over H and clears them; the calls between only read H. H is then
 * read once per token and written once per P tokens. The linear state is
 * always
 *   H' = H + sum_j phi(pend_k_j) pend_v_j^T,  s' = s + sum_j phi(pend_k_j),
 * over the P slots; a zero slot holds nothing (phi(0) = 0), and a slot is
 * written only by the call t = j (mod P) after the fold that cleared it.
 * kla_hybrid_decode_flush folds every slot into H and s and zeroes them.
 *
 * State (device memory owned by the caller, updated in place; float32 but
 * for the window and cache rows, which hold the tokens in row_dtype, the
 * step's in_dtype: bf16 tokens are kept as they are, at half the bytes):
 *   H, s       : [N, D, d_v], [N, D] (zero before the first token).
 *   pend_k/pend_v : [N, P, d_qk] / [N, P, d_v] (zero before the first
 *                token).
 *   win_k/win_v: [N, W + 1, d_qk] / [N, W + 1, d_v] (row_dtype); token i
 *                is kept in row i mod (W + 1) while it is in the window.
 *   cache_k/cache_v/cache_ids : [N, lambda, d_qk] / [N, lambda, d_v]
 *                (row_dtype) / [N, lambda] int32. Rows 0 .. n-1 hold the
 *                cached pairs and their token ids, in no particular order, with
 *                n = min(lambda, max(0, t - W - 1)) before the call and
 *                min(lambda, max(0, t - W)) after it; other rows are unused.
 *                May be NULL when lambda = 0.
 *   cache_sums : [N, lambda, d_v + 4]: for cached row i, the sums of its key
 *                against the linear state (pending slots included),
 *                (phi(k_i)^T H', phi(k_i)^T s'), in columns 0 .. d_v - 1 and
 *                d_v (the last three of a row are padding, for 16-byte
 *                rows). Each call keeps them: a
 *                fold of pair r adds (k_i . k_r)^2 [v_r | 1] (KATA page §2.2:
 *                phi(x) . phi(y) = (x . y)^2), and a pair entering the cache
 *                takes its sums from the call's pass over H. The refresh
 *                scores candidates from them. Zero for a zero state; may be
 *                NULL when lambda = 0.
 *   row_dtype  : KLA_F32 or KLA_BF16, equal to the step's in_dtype.
 * To continue from a prefill of t tokens, the caller fills the window rows of
 * tokens max(0, t - W - 1) .. t - 1, the cache rows and the state the prefill
 * left, with zero pending slots, then calls kla_hybrid_decode_prime to
 * compute cache_sums.
 *
 *   q, k : [N, d_qk]; v : [N, d_v]; in_dtype.   o : [N, d_v], out_dtype.
 *   rejected : [N] int32, or NULL: the token id folded by this call (now
 *              in pending slot t mod P), -1 when there was none.
 *   ws : workspace of kla_hybrid_decode_workspace_size bytes (per
 *        head-state, the linear readouts of the query and of the evicted
 *        key).
 * Every state pointer must be 16-byte aligned. A row_dtype other than
 * in_dtype is KLA_ERR_INVALID_ARGUMENT.
 * Supported: d_qk, d_v in {16, 32, 64}; refresh = 1; window >= 0;
 * 0 <= cache_size <= 255; t >= 0; softmax_scale finite.
 * ------------------------------------------------------------------------ */
/* Pending slots of a token-by-token hybrid state (P above). */
#define KLA_HYBRID_PENDING 8
KLA_API int kla_hybrid_decode_pending_slots(void);

typedef struct {
  float* H;
  float* s;
  void* win_k;
  void* win_v;
  void* cache_k;
  void* cache_v;
  int32_t* cache_ids;
  float* pend_k;
  float* pend_v;
  float* cache_sums;
  kla_dtype_t row_dtype; /* element type of win_k, win_v, cache_k, cache_v */
} kla_hybrid_state_t;

KLA_API kla_status_t kla_hybrid_decode_workspace_size(int N, int d_qk, int d_v,
                                              const kla_hybrid_cfg_t* cfg, size_t* bytes);
KLA_API kla_status_t kla_hybrid_decode_step(int N, int d_qk, int d_v, float eps,
                                    const kla_hybrid_cfg_t* cfg, int t,
                                    const kla_hybrid_state_t* state, const void* q,
                                    const void* k, const void* v, kla_dtype_t in_dtype, void* o,
                                    kla_dtype_t out_dtype, int32_t* rejected, void* ws,
                                    size_t ws_bytes, kla_stream_t stream);
/* kla_hybrid_decode_step_static - the same step for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation). Arguments, results and errors are those
 * of kla_hybrid_decode_step, without `ws`: the scratch lives in a static
 * device array inside the library, kla_hybrid_decode_static_limit() bytes
 * (16 MiB) on each device, looked up once per device on the first call made
 * with that device current. A call whose kla_hybrid_decode_workspace_size
 * exceeds that limit returns KLA_ERR_UNSUPPORTED and enqueues nothing. The
 * call allocates and frees nothing. Every call on one device shares that
 * device's array: calls that overlap on one device (other streams, other
 * threads) race and must be ordered by the caller. Nothing in the array has
 * to be cleared between calls. */
KLA_API size_t kla_hybrid_decode_static_limit(void);
KLA_API kla_status_t kla_hybrid_decode_step_static(int N, int d_qk, int d_v, float eps,
                                           const kla_hybrid_cfg_t* cfg, int t,
                                           const kla_hybrid_state_t* state, const void* q,
                                           const void* k, const void* v, kla_dtype_t in_dtype,
                                           void* o, kla_dtype_t out_dtype, int32_t* rejected,
                                           kla_stream_t stream);
/* Folds every pending slot into (H, s) and zeroes the slots (H, s, pend_k,
 * pend_v of `state` are used). The linear state H' does not change, so
 * cache_sums stay valid. */
KLA_API kla_status_t kla_hybrid_decode_flush(int N, int d_qk, int d_v, const kla_hybrid_state_t* state,
                                     kla_stream_t stream);
/* kla_hybrid_decode_prime - computes cache_sums for the cached rows
 * 0 .. min(lambda, max(0, t - W - 1)) - 1 of a state about to take token t
 * (H, s, pend_k, pend_v, cache_k and cache_sums of `state` are used), in
 * float32: sum_f phi_f(k_i) H_f + sum_j (k_i . pend_k_j)^2 pend_v_j and the
 * same for s.
 * For a state filled from elsewhere (a prefill); a state that only ever went
 * through kla_hybrid_decode_step keeps its sums itself. */
KLA_API kla_status_t kla_hybrid_decode_prime(int N, int d_qk, int d_v, const kla_hybrid_cfg_t* cfg, int t,
                                     const kla_hybrid_state_t* state, kla_stream_t stream);

/* ------------------------------------------------------------------------
 * Kernel timing without a profiler. While enabled on the calling thread,
 * every call records a pair of HIP events on its stream around its dominant
 * kernel: the state/readout kernel of kla_prefill, the state-streaming
 * kernel of kla_decode_step, the scoring kernel of kla_sre_select, each
 * scoring kernel of kla_hybrid_prefill, every kernel of a
 * kla_hybrid_decode_step (one span), the kernel of kla_prefill_quadratic and
 * the two kernels of kla_prefill_quadratic_backward (one span). kla_profile_read waits for the last
 * recorded event, returns the summed elapsed milliseconds and the number of
 * recorded kernels, and clears the record. Events come from a pool owned by
 * the thread; up to 65536 pairs are kept per read (later ones are counted in
 * `dropped`).
 * ------------------------------------------------------------------------ */
KLA_API kla_status_t kla_profile_enable(int on);
KLA_API kla_status_t kla_profile_read(double* total_ms, int* kernels, int* dropped);

#ifdef __cplusplus
}
#endif

#endif /* KLA_H */
