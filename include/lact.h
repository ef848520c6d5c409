/*
 * lact.h - C ABI of the MI355X (gfx950) LaCT fast-weight chunk layer.
 *
 * The layer is the chunk-wise SwiGLU fast-weight layer of "Test-Time Training
 * Done Right" (LaCT).  Each (batch, head) holds three matrices
 *     W1, W3 : [dh, d]   (gate and up)      W2 : [d, dh]   (down)
 * and the fast-weight function f_W(x) = W2 (silu(W1 x) * (W3 x)), no biases
 * (OpenReview rebuttal page, Python pseudocode, docstring of
 * block_causal_lact_swiglu; summary page section 3.2, Eq. 6).
 *
 * Conventions shared by every call:
 *  - All pointers are DEVICE pointers unless stated otherwise.  The caller
 *    owns every buffer; the library allocates nothing and keeps no state
 *    between calls.
 *  - Every call is asynchronous on `stream` (a hipStream_t; NULL = the null
 *    stream) and never synchronises.  Argument checks run on the host before
 *    anything is enqueued: on any error nothing is enqueued and the state is
 *    untouched.  A HIP launch error returns LACT_ERR_HIP and
 *    lact_last_hip_error() gives the hipError_t.
 *  - Activations (q, k, v, o) are element arrays with the head dim contiguous;
 *    token t of head b starts at element  b * stride_bh + t * stride_tok.
 *    Both [BH, T, d] and [B, T, H, d] layouts are expressible.  Their element
 *    type is shape.dtype (fp32 or bf16); base pointers must be 16-byte
 *    aligned and stride_tok * elemsize a multiple of 16 bytes.
 *  - Per-token learning rates eta1, eta3, eta2 (for W1, W3, W2) and momentum
 *    coefficients are fp32 arrays [bh, *] with row stride `eta_stride_bh`
 *    elements; the three eta pointers may alias.
 *
 * Supported shapes: d in {64, 128, 256}; dh a multiple of 64 with
 * d <= dh <= 4096; bh >= 1; with LACT_F32 activations d <= 128.  Anything
 * else returns LACT_ERR_UNSUPPORTED.
 */
#ifndef LACT_H
#define LACT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LACT_OK = 0,
  LACT_ERR_INVALID_ARG = 1,  /* null pointer, negative size, bad enum       */
  LACT_ERR_UNSUPPORTED = 2,  /* shape outside the supported set            */
  LACT_ERR_ALIGNMENT = 3,    /* pointer or stride not 16-byte aligned      */
  LACT_ERR_WORKSPACE = 4,    /* workspace NULL or smaller than required    */
  LACT_ERR_HIP = 5           /* a HIP call failed (see lact_last_hip_error) */
} lact_status;

typedef enum { LACT_F32 = 0, LACT_BF16 = 1 } lact_dtype;

/* Update/apply ordering of one chunk (summary page, section 3.1 / Fig. 3).
 * APPLY_THEN_UPDATE: read the chunk with W_c, then write it -> W_{c+1}
 *   (shifted block-causal mask; causal LM, and AR video with a subset).
 * UPDATE_THEN_APPLY: write the chunk, then read it with the result
 *   (bidirectional; NVS with one chunk = the whole sequence). */
typedef enum { LACT_APPLY_THEN_UPDATE = 0, LACT_UPDATE_THEN_APPLY = 1 } lact_order;

typedef struct {
  int32_t bh;     /* independent (batch, head) states                        */
  int32_t d;      /* head dim (dk = dv)                                      */
  int32_t dh;     /* SwiGLU hidden dim                                       */
  int32_t dtype;  /* lact_dtype of activations and of the MFMA operands      */
} lact_shape;

/* Fast-weight state of all bh heads.  Masters are fp32, row-major:
 *   w1, w3 : [bh, dh, d]      w2 : [bh, d, dh]
 *   n1, n3 : [bh, dh]         n2 : [bh, d]     row norms at sequence start
 *   m1, m3, m2 : [bh, d, dh]  momentum buffers in the wide orientation
 *                             (m1, m3 hold the transposes of the W1/W3
 *                             momentum); NULL when momentum is never used
 *   shadow : lact_shadow_bytes() bytes; operand copies of the weights in
 *            shape.dtype, rewritten by every call that changes w.          */
typedef struct {
  float *w1, *w3, *w2;
  float *n1, *n3, *n2;
  float *m1, *m3, *m2;
  void *shadow;
} lact_state;

typedef struct {
  int64_t stride_bh;   /* elements between heads                 */
  int64_t stride_tok;  /* elements between consecutive tokens    */
} lact_layout;

typedef struct {
  int32_t use_muon;      /* orthogonalise the step with Newton-Schulz-5      */
  int32_t use_momentum;  /* G <- G + beta M, M <- G (beta = mean coefficient) */
  int32_t renorm;        /* rescale rows to their sequence-start norms       */
  float renorm_eps;      /* added to the row norm (page: 1e-5)               */
  float ns_eps;          /* added to the Frobenius norm (page: 1e-7)         */
  int32_t ns_fp32;       /* 0: Newton-Schulz products on bf16 operands, as
                            the page (X stays fp32 between steps);
                            1: fp32 operands (slower, for precision)         */
} lact_update_opts;

/* Bytes of lact_state.shadow for this shape. */
size_t lact_shadow_bytes(const lact_shape* shape);

/* Bytes of device workspace needed by lact_update / lact_chunk_step /
 * lact_sequence for writes of at most `max_update_tokens` tokens. */
size_t lact_workspace_bytes(const lact_shape* shape, int64_t max_update_tokens,
                            const lact_update_opts* opts);

/* Sequence start: n* <- row norms of w*, m* <- 0 (when non-NULL), shadow <-
 * operand copies of w*.  (Rebuttal page: the norms are taken once, before
 * the chunk loop; the momentum buffers start at zero.) */
lact_status lact_init_state(const lact_shape* shape, const lact_state* state,
                            void* stream);

/* Read (apply) on n_tok tokens: o_t = W2 (silu(W1 q_t) * (W3 q_t)), with the
 * current weights, for every head.  State unchanged.  o may not alias q.
 * (Rebuttal page, apply step of both pseudocode functions.) */
lact_status lact_apply(const lact_shape* shape, const lact_state* state,
                       const void* q, lact_layout q_layout,
                       void* o, lact_layout o_layout,
                       int64_t n_tok, void* stream);

/* Chunk gradient (descent direction) of L_j = -sum_t eta_j,t <f_W(k_t), v_t>
 * over n_tok tokens, written in the wide orientation, fp32:
 *   g1 <- G1^T, g3 <- G3^T, g2 <- G2, each [bh, d, dh].
 * State unchanged.  (Rebuttal page, "compute the gradient" block; summary
 * page section 3.2, Eq. 4-5.) */
lact_status lact_gradient(const lact_shape* shape, const lact_state* state,
                          const void* k, lact_layout k_layout,
                          const void* v, lact_layout v_layout,
                          const float* eta1, const float* eta3, const float* eta2,
                          int64_t eta_stride_bh, int64_t n_tok,
                          float* g1, float* g3, float* g2,
                          void* workspace, size_t workspace_bytes, void* stream);

/* Newton-Schulz-5 on `count` matrices [rows, cols] (rows <= cols), fp32 in,
 * fp32 out (in == out allowed): X = G / (||G||_F + eps), then five quintic
 * steps A = X X^T, B = b A + c A A, X = a X + B X with the page's
 * coefficients.  MFMA operands are rounded to `dtype` (bf16, as the page
 * does; or fp32).  (Rebuttal page, zeropower_via_newtonschulz5; summary page
 * section 3.2, Eq. 9-10.)  Workspace: lact_ns_workspace_bytes(). */
size_t lact_ns_workspace_bytes(int32_t count, int32_t rows, int32_t cols);
lact_status lact_newton_schulz(int32_t count, int32_t rows, int32_t cols,
                               int32_t dtype, const float* g, float* u, float eps,
                               void* workspace, size_t workspace_bytes,
                               void* stream);

/* Weight step: W <- W + U, then (opts->renorm) every row rescaled to
 * n0 / (||row|| + renorm_eps); shadow rewritten.  u1, u3, u2 are the steps in
 * the wide orientation [bh, d, dh] (u1 = U1^T, u3 = U3^T, u2 = U2).
 * Workspace: at least lact_workspace_bytes(shape, 0, opts) bytes.
 * (Rebuttal page, end of the chunk loop; summary page section 3.2, Eq. 8.) */
lact_status lact_step_renorm(const lact_shape* shape, const lact_state* state,
                             const float* u1, const float* u3, const float* u2,
                             const lact_update_opts* opts,
                             void* workspace, size_t workspace_bytes, void* stream);

/* One write on n_tok tokens: gradient -> momentum (beta = mean of mom over
 * the n_tok tokens; mom may be NULL when momentum is off) -> Newton-Schulz
 * -> step + renorm.  State updated in place.  n_tok = 0 writes nothing. */
lact_status lact_update(const lact_shape* shape, const lact_state* state,
                        const void* k, lact_layout k_layout,
                        const void* v, lact_layout v_layout,
                        const float* eta1, const float* eta3, const float* eta2,
                        const float* mom, int64_t eta_stride_bh, int64_t n_tok,
                        const lact_update_opts* opts,
                        void* workspace, size_t workspace_bytes, void* stream);

/* One causal chunk: read q with W_c into o, then write (k, v) -> W_{c+1}. */
lact_status lact_chunk_step(const lact_shape* shape, const lact_state* state,
                            const void* q, lact_layout q_layout,
                            const void* k, lact_layout k_layout,
                            const void* v, lact_layout v_layout,
                            void* o, lact_layout o_layout,
                            const float* eta1, const float* eta3, const float* eta2,
                            const float* mom, int64_t eta_stride_bh, int64_t n_tok,
                            const lact_update_opts* opts,
                            void* workspace, size_t workspace_bytes, void* stream);

/* Whole sequence of T tokens in chunks of `chunk` (the last may be short),
 * starting at token 0 of every array:
 *  - APPLY_THEN_UPDATE: each chunk is read with the current weights and then
 *    written; the chunk that ends at T is read only unless update_last.
 *  - UPDATE_THEN_APPLY: each chunk is written, then read.
 * Writes use the tokens [s + subset_offset, s + subset_offset + subset_len)
 * of each chunk [s, e) (clipped to the chunk); subset_len < 0 = whole chunk.
 * The state must have been initialised (lact_init_state) at sequence start;
 * passing the state of an earlier call continues that sequence.
 * Workspace: lact_workspace_bytes(shape, min(chunk, subset), opts). */
lact_status lact_sequence(const lact_shape* shape, const lact_state* state,
                          const void* q, lact_layout q_layout,
                          const void* k, lact_layout k_layout,
                          const void* v, lact_layout v_layout,
                          void* o, lact_layout o_layout,
                          const float* eta1, const float* eta3, const float* eta2,
                          const float* mom, int64_t eta_stride_bh,
                          int64_t T, int64_t chunk, int32_t order,
                          int64_t subset_offset, int64_t subset_len,
                          int32_t update_last, const lact_update_opts* opts,
                          void* workspace, size_t workspace_bytes, void* stream);

/* Kernel timing for benchmarks.  lact_prof_begin(kind, max_launches)
 * creates 2 * max_launches HIP events; until lact_prof_end, every launch of
 * the kernel `kind` made by the calls above is bracketed by events recorded
 * on the stream it runs on (at most max_launches).  lact_prof_end waits for
 * the events, returns the number of bracketed launches and the total, min and
 * max duration in milliseconds, and destroys the events.  Not for use under
 * graph capture; one profiling window per process at a time.
 * kinds: 1 apply (k_apply), 2 gradient (k_grad), 3 split reduction,
 *        4 Newton-Schulz (whole iteration per write), 5 step + renorm. */
enum { LACT_PROF_APPLY = 1, LACT_PROF_GRAD = 2, LACT_PROF_REDUCE = 3, LACT_PROF_NS = 4,
       LACT_PROF_STEP = 5 };
lact_status lact_prof_begin(int32_t kind, int32_t max_launches);
lact_status lact_prof_end(int32_t* launches, float* total_ms, float* min_ms, float* max_ms);

const char* lact_status_string(lact_status status);

/* hipError_t of the last failed HIP call on this thread (0 if none). */
int lact_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* LACT_H */
