// Internal launch interface between the C ABI driver and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace lact {

// Operand copies of the weights, per head, in the MFMA operand type:
//   w1s, w3s : [dh][d]   w2s : [d][dh]   w2ts : [dh][d] (W2 transposed)
struct Shadow {
  void* base;
  int64_t per_head;  // elements per head (4 d dh)
  int64_t off_w1, off_w3, off_w2, off_w2t;
};
Shadow make_shadow(void* base, int d, int dh);

struct ApplyArgs {
  const void* q; int64_t q_sbh, q_st;
  void* o; int64_t o_sbh, o_st;
  Shadow sh;
  int bh, d, dh;
  int64_t n_tok;
};

// Read of 1..8 tokens per head (k_decode.hip): q, o as for ApplyArgs; part:
// [bh][nblk][n][d] fp32 partial outputs of the hidden blocks.
struct DecodeArgs {
  const void* q; int64_t q_sbh, q_st;
  void* o; int64_t o_sbh, o_st;
  Shadow sh;
  int bh, d, dh, n;
  int nblk;
  float* part;
};

// Linear fast-weight variant (k_linear.hip): one d x d matrix per head.
struct LinArgs {
  const void* q; int64_t q_sbh, q_st;
  void* o; int64_t o_sbh, o_st;
  const void* k; int64_t k_sbh, k_st;
  const void* v; int64_t v_sbh, v_st;
  const float* eta; int64_t eta_sbh;   // one rate per token
  const float* mom; int64_t mom_sbh;   // momentum coefficients (with m)
  float* w; float* n; float* m;        // [bh][d][d], [bh][d], [bh][d][d] or NULL
  void* shadow;                        // [bh][d][d] operand copy
  float* g;                            // [bh][d][d] gradient (+ momentum)
  int bh, d;
  int64_t n_tok;
  int renorm; float eps;
  int* nonfinite;
};
hipError_t launch_linear(int dtype, int what, const LinArgs& a, const float* U, hipStream_t s);

struct GradArgs {
  const void* k; int64_t k_sbh, k_st;
  const void* v; int64_t v_sbh, v_st;
  const float* eta1; const float* eta3; const float* eta2; int64_t eta_sbh;
  // 0: one learning rate per token; 1: per channel (eta1, eta3 [bh][*][d],
  // eta2 [bh][*][dh]; eta_sbh counts tokens)
  int eta_per_channel;
  Shadow sh;
  int bh, d, dh;
  int64_t n_tok;
  int nsplit;
  int64_t split_len;
  float* partial;  // [nsplit][bh][3][dh][d] fp32
  // momentum (else mom = NULL): one workgroup per head writes beta[head], the
  // mean of the head's per-token coefficients mom[head * mom_sbh + t], t < n_tok
  const float* mom; int64_t mom_sbh; float* beta;
  // old momentum M1, M3, M2 (wide [bh][d][dh]) to fold in, or NULL: the
  // workgroups of split 0 start from beta M instead of zero (bf16 d <= 128),
  // so that the split sum is G + beta M
  const float* mo1; const float* mo3; const float* mo2;
};

// Sum of split partials, transpose to the wide orientation, momentum.
struct ReduceArgs {
  const float* partial;  // [nsplit][bh][3][dh][d]
  int nsplit;
  int bh, d, dh;
  float* out1; float* out3; float* out2;  // [bh][d][dh] each (NULL: only M holds the result)
  float* m1; float* m3; float* m2;        // momentum (NULL = off)
  const float* beta;                      // [bh] coefficient of M (from the gradient launch)
  // NULL, or [3 bh][tiles]: sum of squares of each 64 x 64 tile of the
  // result, matrix mat bh + head (the Newton-Schulz input order), tiles in
  // launch order (the first pass of the Frobenius normalisation)
  float* ss_part;
};


// Batched C = alpha * A B + beta * Dm, fp32 storage, MFMA operands in T.
// A is [M][K] (K contiguous).  B is [N][K] (b_kn = 0) or [K][N] (b_kn = 1).
struct GemmArgs {
  const float* A; int64_t a_bs;
  const float* B; int64_t b_bs; int b_kn;
  const float* Dm; int64_t d_bs;
  float* C; int64_t c_bs;
  int M, N, K, batch;
  float alpha, beta;
};

// bf16-operand GEMM of the large-matrix Newton-Schulz path (k_gemm.hip).
struct NsGemmArgs {
  const __bf16* A; int64_t a_bs; int lda;
  const __bf16* B; int64_t b_bs; int ldb;
  const float* D; int64_t d_bs;
  float* C; __bf16* Ch; int64_t c_bs;
  int M, N, K;
  float alpha, beta;
  // Shifted Newton-Schulz steps: mu = (sum of mu_part[batch][0 .. mu_np)) /
  // mu_div (0 when mu_part is NULL); the D coefficient is then beta +
  // beta_mu mu + beta_mu2 mu^2 and diag_mu mu is added to the diagonal.
  const float* mu_part; int mu_np; float mu_div;
  float beta_mu, beta_mu2, diag_mu;
  // NULL, or [batch][tiles]: sum of squares of each 64 x 64 tile of the fp32
  // result, in tile order (the next step's mu)
  float* ss_part;
  // 1: the product is symmetric (M == N; A B^T with B = A, or a product of
  // commuting symmetric factors): only the tiles on and above the diagonal
  // are computed, each written also transposed below it (D, if any, must be
  // symmetric too; ss_part must be NULL)
  int sym;
  // the first c_tall matrices of the batch get C written transposed ([N][M],
  // row pitch M, in the same c_bs slot; not with sym, Ch or ss_part)
  int c_tall;
};

// Input matrices of a Newton-Schulz batch: matrix m is p[m / per] +
// (m % per) * size (three separately allocated blocks, e.g. the momentum
// buffers of W1, W3, W2, or one contiguous block with per = count).
struct NsIn {
  const float* p[3];
  int per;
  __host__ __device__ const float* at(int m, int64_t size) const {
    return p[m / per] + (int64_t)(m % per) * size;
  }
};

struct NsNormArgs {
  NsIn g; float* x; int64_t count, n; float eps;
};

// Step: W <- W + U (wide U), per-row partial sums of squares.
struct StepArgs {
  float* w1; float* w3; float* w2;
  const float* u1; const float* u3; const float* u2;  // wide [bh][d][dh]; NULL = no add
  int u13_tall;  // 1: u1, u3 are [bh][dh][d] (the layout of w1, w3)
  float* n1; float* n3; float* n2;                    // renorm targets
  Shadow sh;
  int bh, d, dh;
  int renorm;  // 0: factor 1 (copies only), 1: n0 / (||row|| + eps), 2: the
               // rescaled rows go to the copies only, W keeps W + U
  float eps;
  // sequence start (init = 1, with renorm = 0 and no U): the row norms are
  // written to n1, n3, n2 and the momentum buffers (non-NULL ones) zeroed
  int init;
  float* mz1; float* mz3; float* mz2;
  int* nonfinite;  // NULL, or set to 1 when a row's sum of squares is not finite
};

// Raises a kernel's dynamic LDS limit to `bytes`, once per (kernel, device);
// safe to call from several threads.
hipError_t allow_dynamic_lds(const void* kernel, int bytes);

// max_blocks > 0: at most that many workgroups (d = 256 only; the tiles are
// then dealt to them by XCD), else one per tile.
hipError_t launch_apply(int dtype, const ApplyArgs& a, hipStream_t s, int max_blocks = 0);
hipError_t launch_grad(int dtype, const GradArgs& a, hipStream_t s);
int decode_blocks(int dtype, int bh, int d, int dh);
hipError_t launch_decode(int dtype, const DecodeArgs& a, hipStream_t s);
// Hidden units per workgroup of the gradient launch (generic: the kernel
// that fp32 shapes and per-channel learning rates use).
int grad_hidden_per_block(int dtype, int d, bool generic);
hipError_t launch_reduce(const ReduceArgs& a, hipStream_t s);
hipError_t launch_gemm(int dtype, const GemmArgs& a, hipStream_t s);
// Newton-Schulz in one workgroup per matrix (bf16 operands; steps from
// shift_from on are shifted, see k_ns.hip); hipErrorNotSupported for shapes
// without such a kernel.
hipError_t launch_ns_fused(int count, int rows, int cols, NsIn g, float* u, float eps,
                           int shift_from, hipStream_t s);
// Weight step done by the Newton-Schulz workgroups themselves: matrix
// m = mat * bh + head (mat 0: W1, 1: W3, 2: W2) adds its result U (wide
// orientation) to W, rescales the rows (renorm) and writes the operand copies
// into `sh`, which may differ from the shadow a read in the same launch uses.
struct NsStep {
  float* w1; float* w3; float* w2;
  const float* n1; const float* n3; const float* n2;
  Shadow sh;
  int bh;
  int renorm;      // as StepArgs::renorm
  float eps;
  int* nonfinite;  // NULL, or set to 1 when a row's sum of squares is not finite
};
// Input of a Newton-Schulz launch that also finishes the gradient: matrix
// m = mat * bh + head starts from G = the sum over splits s (in split order)
// of partial[s][head][mat]^T (with momentum, split 0 already holds beta M_old:
// GradArgs::mo*), and M <- G when m[mat] != NULL.
struct NsGrad {
  const float* partial;  // [nsplit][bh][3][dh][d]
  int nsplit, bh;
  float* m[3];           // wide [bh][d][dh] each, or NULL
};
// Gradient reduction + Newton-Schulz + step (bf16, 128 rows, 256 or 512
// columns), with the tiles of a d = 128 bf16 read (a.n_tok > 0) in the same
// launch; hipErrorNotSupported for other shapes.
hipError_t launch_ns_step_apply(int count, int rows, int cols, const NsGrad& gr, float eps,
                                int shift_from, const NsStep& st, const ApplyArgs& a,
                                hipStream_t s);
// Device copy of `bytes` (a multiple of 16, 16-byte aligned pointers).
hipError_t launch_copy16(void* dst, const void* src, int64_t bytes, hipStream_t s);
hipError_t launch_ns_norm(const NsNormArgs& a, hipStream_t s);
hipError_t launch_nsgemm(bool b_kn, const NsGemmArgs& a, int batch, hipStream_t s);
// pre_np > 0: part already holds pre_np partial sums of squares per matrix
// (written by the split sum), so only the scaling pass runs.
hipError_t launch_nsn(NsIn g, float* part, float* x, __bf16* xh, int count, int64_t n, float eps,
                      hipStream_t s, int pre_np = 0);
hipError_t launch_step(int dtype, const StepArgs& a, hipStream_t s);


// ------------------------------------------------ outer-loop backward --
// Batched fp32 GEMM with strides (k_backward.hip): for b < batch,
//   C(m, n) = alpha * sum_k A(m, k) B(k, n) + beta * D(m, n)
//   A(m, k) = A[b a_bs + m a_sm + k a_sk]  (bf16 when a_bf16)
//   B(k, n) = B[b b_bs + k b_sk + n b_sn]  (bf16 when b_bf16)
//   D(m, n) = D[b d_bs + m d_sm + n] (D may be C or NULL), C(m, n) =
//   C[b c_bs + m c_sm + n].
struct BGemm {
  const void* A; int a_bf16; int64_t a_bs, a_sm, a_sk;
  const void* B; int b_bf16; int64_t b_bs, b_sk, b_sn;
  const float* D; int64_t d_bs, d_sm;
  float* C; int64_t c_bs, c_sm;
  int M, N, K, batch;
  float alpha, beta;
};
// partial: NULL, or a scratch of partial_floats floats for split-K
// partial sums (used when the tiles alone would leave the GPU idle).
hipError_t launch_bgemm(const BGemm& g, hipStream_t s, float* partial = nullptr,
                        int64_t partial_floats = 0);
hipError_t bw_read(float* g, float* u, float* dh, int64_t n, hipStream_t s);
hipError_t bw_grad_fwd(const float* g, const float* u, const float* e, float* o1, float* o3, float* o2,
                       const float* e1, const float* e3, const float* e2, int64_t esbh, int64_t t0, int n,
                       int dh, int bh, hipStream_t s);
hipError_t bw_grad_bwd(float* g, float* u, float* e, float* p1, float* p3, float* p2, float* r1, float* r3,
                       float* r2, const float* e1, const float* e3, const float* e2, int64_t esbh,
                       int64_t t0, int n, int dh, int bh, hipStream_t s);
hipError_t bw_rowsum(const float* x, float* out, int64_t osbh, int64_t t0, int n, int dh, int bh,
                     hipStream_t s);
hipError_t bw_dot(const float* x, const float* y, float* out, int64_t size, int count, hipStream_t s);
hipError_t bw_axpby(float* y, const float* x, const float* z, const float* am, float a, const float* bm,
                    float b, int64_t size, int count, hipStream_t s);
hipError_t bw_transpose(const float* in, float* out, int rows, int cols, int count, hipStream_t s);
hipError_t bw_symm(const float* a, float* out, int n, int count, hipStream_t s);
hipError_t bw_step(float* w, const float* u, const float* n0, int64_t rows, int L, int renorm, float eps,
                   hipStream_t s);
hipError_t bw_rownorm(const float* w, float* n, int64_t rows, int L, hipStream_t s);
hipError_t bw_step_vjp(const float* w, const float* u, const float* n0, const float* dwn, float* dr,
                       float* dn0, int64_t rows, int L, int renorm, float eps, hipStream_t s);
hipError_t bw_w0(const float* w0, const float* dw, const float* dn0, float* out, int64_t rows, int L,
                 hipStream_t s);
hipError_t bw_beta(const float* mom, int64_t sbh, int64_t t0, int n, float* beta, int bh, hipStream_t s);
hipError_t bw_dmom(const float* dbeta, float* dmom, int64_t sbh, int64_t t0, int n, int bh, hipStream_t s);
hipError_t bw_gather(const void* x, int bf, int64_t sbh, int64_t st, int64_t t0, int n, int d, int bh,
                     float* out, hipStream_t s);
hipError_t bw_scatter_add(const float* x, int64_t sbh, int64_t st, int64_t t0, int n, int d, int bh,
                          float* out, hipStream_t s);
hipError_t bw_fill(float* p, float v, int64_t n, hipStream_t s);
hipError_t bw_nscoef(const float* ss, const float* dot, float* c1, float* c2, int count, float eps,
                     hipStream_t s);

}  // namespace lact
