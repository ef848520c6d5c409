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

struct GradArgs {
  const void* k; int64_t k_sbh, k_st;
  const void* v; int64_t v_sbh, v_st;
  const float* eta1; const float* eta3; const float* eta2; int64_t eta_sbh;
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
  float* n1; float* n3; float* n2;                    // renorm targets
  Shadow sh;
  int bh, d, dh;
  int renorm;  // 0: factor 1 (copies only), 1: n0 / (||row|| + eps)
  float eps;
  // sequence start (init = 1, with renorm = 0 and no U): the row norms are
  // written to n1, n3, n2 and the momentum buffers (non-NULL ones) zeroed
  int init;
  float* mz1; float* mz3; float* mz2;
};

hipError_t launch_apply(int dtype, const ApplyArgs& a, hipStream_t s);
hipError_t launch_grad(int dtype, const GradArgs& a, hipStream_t s);
int grad_hidden_per_block(int dtype, int d);
hipError_t launch_reduce(const ReduceArgs& a, hipStream_t s);
hipError_t launch_gemm(int dtype, const GemmArgs& a, hipStream_t s);
hipError_t launch_ns_fused(int dtype, int count, int rows, int cols, NsIn g, float* u,
                           float eps, hipStream_t s);
// Weight step done by the Newton-Schulz workgroups themselves: matrix
// m = mat * bh + head (mat 0: W1, 1: W3, 2: W2) adds its result U (wide
// orientation) to W, rescales the rows (renorm) and writes the operand copies
// into `sh`, which may differ from the shadow a read in the same launch uses.
struct NsStep {
  float* w1; float* w3; float* w2;
  const float* n1; const float* n3; const float* n2;
  Shadow sh;
  int bh;
  int renorm;
  float eps;
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
                                const NsStep& st, const ApplyArgs& a, hipStream_t s);
// Device copy of `bytes` (a multiple of 16, 16-byte aligned pointers).
hipError_t launch_copy16(void* dst, const void* src, int64_t bytes, hipStream_t s);
hipError_t launch_ns_norm(const NsNormArgs& a, hipStream_t s);
hipError_t launch_nsgemm(bool b_kn, const NsGemmArgs& a, int batch, hipStream_t s);
hipError_t launch_nsn(NsIn g, float* part, float* x, __bf16* xh, int count, int64_t n, float eps,
                      hipStream_t s);
hipError_t launch_step(int dtype, const StepArgs& a, hipStream_t s);

}  // namespace lact
