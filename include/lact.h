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
 *    owns every buffer; the library allocates no device memory and keeps no
 *    device state between calls.  Its process-wide state is the
 *    kernel-timing window (lact_prof_begin / lact_prof_end), a record of
 *    which kernels have had their LDS limit raised on which device, and
 *    (lact_sequence and lact_chunk_step with d = 256 and Muon) one HIP
 *    stream and two events per device, created on first use and kept until
 *    the process ends: the read of a chunk runs there beside the write's
 *    Newton-Schulz, forked from and joined back into `stream` within the
 *    call, so the call stays ordered on `stream` as one unit (and can be
 *    captured into a graph; a first call made under capture uses `stream`
 *    alone).  That stream is shared by every caller on a device, so reads
 *    of calls made on different streams may wait for one another; results
 *    do not depend on it.
 *  - Every call is asynchronous on `stream` (a hipStream_t; NULL = the null
 *    stream) and never synchronises, except lact_check_finite and
 *    lact_prof_end, which exist to wait.  Argument checks run on the host
 *    before anything is enqueued: on an argument error nothing is enqueued
 *    and the state is untouched.
 *  - A HIP launch error returns LACT_ERR_HIP and lact_last_hip_error() gives
 *    the hipError_t.  A call that enqueues several kernels (a write, a chunk
 *    step, a sequence) may fail after some of them were enqueued: the state
 *    is then partly updated and must be re-initialised.
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
  LACT_ERR_HIP = 5,          /* a HIP call failed (see lact_last_hip_error) */
  LACT_ERR_NONFINITE = 6     /* lact_check_finite: a write produced a
                                weight row that is NaN or infinite          */
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

/* Precision of the Newton-Schulz products for bf16 shapes (fp32 shapes
 * always use fp32 operands).  In every mode the iterate X stays fp32
 * between the five steps and every product accumulates in fp32.
 *  LACT_NS_BF16_SHIFTED (default): bf16 operands; the last three steps,
 *    where A = X X^T is near the identity, store A - I and form
 *    B - (b + c) I from it, and take X <- (a + b + c) X + (B - (b + c) I) X.
 *    The same polynomial in exact arithmetic; the identity parts stay in
 *    fp32, so the rounded operands are small and the step is about as
 *    accurate as fp32 operands at the cost of bf16 ones.
 *  LACT_NS_BF16: bf16 operands in every step, as the rebuttal page's
 *    zeropower_via_newtonschulz5 (which casts the iterate to bf16).
 *  LACT_NS_F32: fp32 operands (fp32 MFMA; slow, for reference runs).     */
typedef enum { LACT_NS_BF16_SHIFTED = 0, LACT_NS_BF16 = 1, LACT_NS_F32 = 2 } lact_ns_prec;

typedef struct {
  int32_t use_muon;      /* orthogonalise the step with Newton-Schulz-5      */
  int32_t use_momentum;  /* G <- G + beta M, M <- G (beta = mean coefficient) */
  int32_t renorm;        /* 0: no renorm; 1: every row of W + U rescaled to
                            its sequence-start norm (the rebuttal page's
                            loop); 2: master variant (uTTT page section
                            C.1): w* accumulate W + U unscaled and only the
                            operand copies, which every read and gradient
                            uses, hold the rescaled rows                  */
  float renorm_eps;      /* added to the row norm (page: 1e-5)               */
  float ns_eps;          /* added to the Frobenius norm (page: 1e-7)         */
  int32_t ns_prec;       /* lact_ns_prec                                     */
  int32_t* nonfinite;    /* NULL, or a device int32 that the caller zeroes:
                            every write then ORs 1 into it when a row of the
                            new weights has a sum of squares that is not a
                            finite fp32 number (NaN or Inf anywhere in the
                            row).  Nothing waits for it; read it with
                            lact_check_finite or a copy of your own.       */
  int32_t eta_per_channel; /* 0: eta1, eta3, eta2 hold one rate per token;
                            1: per channel (the rebuttal page's learning-rate
                            tensors of shape [b, l, d]): eta1, eta3 are
                            [bh, *, d] and scale k channel by channel, eta2
                            is [bh, *, dh] and scales the hidden units;
                            eta_stride_bh still counts tokens.  Shapes with
                            d <= 128 (else LACT_ERR_UNSUPPORTED); the
                            gradient then runs on the generic kernel.      */
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

/* Streaming decode read: the read of lact_apply for 1 <= n_tok <=
 * LACT_DECODE_MAX_TOKENS tokens per head (e.g. the newest token of each of
 * bh streams), as a weight-streaming matrix-vector kernel: each hidden unit's
 * rows of the operand copies are read once for all n_tok tokens, so the
 * call is bound by reading 3 d dh operand values per head (plus a second,
 * small launch that adds the hidden blocks' partial outputs).  A stream
 * reads every token this way and writes (lact_update) only when a chunk of
 * keys and values has filled (uTTT page section 2; rebuttal page, the causal
 * function's chunk loop).  Fp32 sums in a fixed order; o in shape.dtype.
 * n_tok = 0 does nothing.  Workspace: lact_decode_workspace_bytes(). */
#define LACT_DECODE_MAX_TOKENS 8
size_t lact_decode_workspace_bytes(const lact_shape* shape, int64_t n_tok);
lact_status lact_decode_apply(const lact_shape* shape, const lact_state* state,
                              const void* q, lact_layout q_layout,
                              void* o, lact_layout o_layout, int64_t n_tok,
                              void* workspace, size_t workspace_bytes, void* stream);

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

/* Newton-Schulz-5 on `count` matrices [rows, cols] (rows <= cols, both
 * multiples of 64), fp32 in, fp32 out (in == out allowed): X = G /
 * (||G||_F + eps), then five quintic steps A = X X^T, B = b A + c A A,
 * X = a X + B X with the page's coefficients.  `prec` is a lact_ns_prec.
 * (Rebuttal page, zeropower_via_newtonschulz5; summary page section 3.2,
 * Eq. 9-10.)  Workspace: lact_ns_workspace_bytes(). */
size_t lact_ns_workspace_bytes(int32_t count, int32_t rows, int32_t cols);
lact_status lact_newton_schulz(int32_t count, int32_t rows, int32_t cols,
                               int32_t prec, const float* g, float* u, float eps,
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

/* One write on n_tok tokens, as the body of the chunk loop of the rebuttal
 * page's block_causal_lact_swiglu after its read: chunk gradient ->
 * momentum (beta = mean of mom over the n_tok tokens; mom may be NULL when
 * momentum is off; the buffer keeps the pre-Newton-Schulz sum) ->
 * Newton-Schulz -> W <- W + step -> row renorm to the sequence-start norms
 * (summary page section 3.2, Eq. 4-5, 8-10).  State updated in place.
 * n_tok = 0 writes nothing. */
lact_status lact_update(const lact_shape* shape, const lact_state* state,
                        const void* k, lact_layout k_layout,
                        const void* v, lact_layout v_layout,
                        const float* eta1, const float* eta3, const float* eta2,
                        const float* mom, int64_t eta_stride_bh, int64_t n_tok,
                        const lact_update_opts* opts,
                        void* workspace, size_t workspace_bytes, void* stream);

/* One causal chunk, one iteration of the chunk loop of the rebuttal page's
 * block_causal_lact_swiglu (apply then update, summary page section 3.1 /
 * Fig. 3): read q with W_c into o, then write (k, v) -> W_{c+1} as
 * lact_update.  The read may run inside the write's Newton-Schulz launch
 * (it only needs W_c). */
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
 * starting at token 0 of every array: the update/apply orderings of the
 * summary page (section 3.1, Fig. 3) as the rebuttal page's two functions
 * run them (block_causal_lact_swiglu: chunks starting before T - chunk are
 * read then written, the rest read only; bidirectional_lact_swiglu: one
 * write, then the read):
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

/* lact_sequence for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same arguments without the workspace, which is instead a device array
 * of LACT_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it runs
 * on, from the first call on that GPU until the process ends.  The call
 * allocates nothing and runs every kernel on `stream`.  A sequence whose writes need more workspace than that
 * (lact_workspace_bytes) returns LACT_ERR_WORKSPACE.  Every call on one GPU
 * shares the array: calls that may overlap on one GPU (different streams or
 * threads without ordering between them) race and must not be made; calls
 * on one stream are ordered and safe.  The array keeps the last call's
 * contents; nothing in it needs to start at zero. */
#define LACT_NOALLOC_SCRATCH_BYTES (160u * 1024u * 1024u)
lact_status lact_sequence_noalloc(const lact_shape* shape, const lact_state* state,
                                  const void* q, lact_layout q_layout,
                                  const void* k, lact_layout k_layout,
                                  const void* v, lact_layout v_layout,
                                  void* o, lact_layout o_layout,
                                  const float* eta1, const float* eta3, const float* eta2,
                                  const float* mom, int64_t eta_stride_bh,
                                  int64_t T, int64_t chunk, int32_t order,
                                  int64_t subset_offset, int64_t subset_len,
                                  int32_t update_last, const lact_update_opts* opts,
                                  void* stream);

/* Linear fast-weight variant (the rebuttal page's comparison of fast-weight
 * networks, Fig. 8(a)): one d x d matrix per head, f_W(x) = W x.  A write's
 * descent direction of -sum_t eta_t <W k_t, v_t> is G = sum_t eta_t v_t k_t^T
 * (one rate per token); momentum, Newton-Schulz (opts->ns_prec, on the
 * square matrix), the step and the renorm modes are those of lact_update.
 * shape.dh must equal shape.d (d in {64, 128, 256}, bf16 or fp32).
 *   w : [bh, d, d] fp32 (row-major)   n : [bh, d] sequence-start row norms
 *   m : [bh, d, d] momentum (NULL without momentum)
 *   shadow : lact_linear_shadow_bytes() operand copy.
 * lact_linear_sequence has the arguments and orderings of lact_sequence with
 * one learning-rate array; workspace: lact_linear_workspace_bytes(). */
typedef struct {
  float* w;
  float* n;
  float* m;
  void* shadow;
} lact_linear_state;
size_t lact_linear_shadow_bytes(const lact_shape* shape);
size_t lact_linear_workspace_bytes(const lact_shape* shape, const lact_update_opts* opts);
lact_status lact_linear_init_state(const lact_shape* shape, const lact_linear_state* state,
                                   void* stream);
lact_status lact_linear_sequence(const lact_shape* shape, const lact_linear_state* state,
                                 const void* q, lact_layout q_layout,
                                 const void* k, lact_layout k_layout,
                                 const void* v, lact_layout v_layout,
                                 void* o, lact_layout o_layout,
                                 const float* eta, const float* mom, int64_t eta_stride_bh,
                                 int64_t T, int64_t chunk, int32_t order,
                                 int64_t subset_offset, int64_t subset_len,
                                 int32_t update_last, const lact_update_opts* opts,
                                 void* workspace, size_t workspace_bytes, void* stream);

/* Outer-loop backward (how the layer is trained: task-loss gradients flow
 * back through the earlier writes, uTTT page section 2): the
 * vector-Jacobian product of lact_sequence.  Given dout = dL/do for the
 * outputs o of lact_sequence run from the initial weights (w1, w3, w2) with
 * the same arguments, it writes dL/dq, dL/dk, dL/dv, dL/deta1..3, dL/dmom
 * and dL/dW0 (through the weights and through the renorm targets, the row
 * norms of W0).  The forward is recomputed in fp32 (the state before every
 * chunk kept in the workspace) and the chain rule taken step by step:
 * read, chunk gradient (with silu''), momentum (beta = mean coefficient),
 * Newton-Schulz (the five quintic steps as matrix products, whatever
 * opts->ns_prec), step + row renorm.  renorm 2 and per-channel rates are
 * not supported (LACT_ERR_UNSUPPORTED); nonfinite is ignored.  fp32
 * activations are accepted at every supported d (256 included).
 *   w1, w3 : [bh, dh, d] fp32, w2 : [bh, d, dh] fp32 (W0, natural layout)
 *   q, k, v : activations of shape.dtype with their layouts
 *   dout    : [bh, T, d] fp32, contiguous
 *   eta1, eta3, eta2, mom : [bh, *] fp32 (row stride eta_stride_bh >= T)
 * Every output is written in full (the call zeroes them first):
 *   dq, dk, dv : [bh, T, d] fp32 contiguous
 *   deta1, deta3, deta2, dmom : [bh, eta_stride_bh] fp32 (dmom NULL
 *       without momentum; the deta pointers may alias, the terms then add)
 *   dw1, dw3, dw2 : like w1, w3, w2.
 * Workspace: lact_backward_workspace_bytes(shape, T, chunk, opts) (it holds
 * one fp32 state per chunk). */
typedef struct {
  float* dq;
  float* dk;
  float* dv;
  float* deta1;
  float* deta3;
  float* deta2;
  float* dmom;
  float* dw1;
  float* dw3;
  float* dw2;
} lact_grads;
size_t lact_backward_workspace_bytes(const lact_shape* shape, int64_t T, int64_t chunk,
                                     const lact_update_opts* opts);
lact_status lact_sequence_backward(const lact_shape* shape, const float* w1, const float* w3,
                                   const float* w2, const void* q, lact_layout q_layout,
                                   const void* k, lact_layout k_layout, const void* v,
                                   lact_layout v_layout, const float* dout, const float* eta1,
                                   const float* eta3, const float* eta2, const float* mom,
                                   int64_t eta_stride_bh, int64_t T, int64_t chunk, int32_t order,
                                   int64_t subset_offset, int64_t subset_len, int32_t update_last,
                                   const lact_update_opts* opts, const lact_grads* grads,
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

/* Waits for `stream`, then returns LACT_ERR_NONFINITE if the device int32
 * `flag` (lact_update_opts.nonfinite) is non-zero, else LACT_OK.  The flag
 * is left as it is. */
lact_status lact_check_finite(const int32_t* flag, void* stream);

const char* lact_status_string(lact_status status);

/* hipError_t of the last failed HIP call on this thread (0 if none). */
int lact_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* LACT_H */
