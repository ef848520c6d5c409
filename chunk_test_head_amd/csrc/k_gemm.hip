// Batched small GEMM for the Newton-Schulz iteration (LaCT rebuttal page,
// zeropower_via_newtonschulz5; summary page section 3.2, Eq. 9-10):
//   C = alpha * A B + beta * Dm     (fp32 storage, MFMA operands in T)
// A is [M][K] with K contiguous; B is [N][K] (b_kn = 0) or [K][N] (b_kn = 1).
// One workgroup = one 64 x 64 tile of C; K is walked in slabs of 32 staged
// through LDS in the operand type.
#include "lact_internal.hpp"
#include "mfma.hpp"

namespace lact {

template <class T>
__global__ __launch_bounds__(256) void k_gemm(GemmArgs a) {
  constexpr int BM = 64, BN = 64, BK = 32;
  constexpr int PA = BK + 16 / sizeof(T);
  __shared__ __attribute__((aligned(16))) T sA[BM * PA];
  __shared__ __attribute__((aligned(16))) T sB[BN * PA];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = lane & 15, g = lane >> 4;
  const int wm = wave >> 1, wn = wave & 1;
  const int tn = a.N / BN;
  const int tile = blockIdx.x, b = blockIdx.y;
  const int m0 = (tile / tn) * BM, n0 = (tile % tn) * BN;
  const float* A = a.A + (int64_t)b * a.a_bs;
  const float* B = a.B + (int64_t)b * a.b_bs;

  f32x4 acc[2][2];
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y) acc[x][y] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int k0 = 0; k0 < a.K; k0 += BK) {
    // A tile 64 x 32: 512 float4, 2 per thread
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const int vi = tid + 256 * x;
      const int r = vi >> 3, cc = (vi & 7) * 4;
      const f32x4 v = *reinterpret_cast<const f32x4*>(A + (int64_t)(m0 + r) * a.K + k0 + cc);
      T* d = sA + r * PA + cc;
      d[0] = to_t<T>(v[0]); d[1] = to_t<T>(v[1]); d[2] = to_t<T>(v[2]); d[3] = to_t<T>(v[3]);
    }
    if (a.b_kn == 0) {
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const int vi = tid + 256 * x;
        const int r = vi >> 3, cc = (vi & 7) * 4;
        const f32x4 v = *reinterpret_cast<const f32x4*>(B + (int64_t)(n0 + r) * a.K + k0 + cc);
        T* d = sB + r * PA + cc;
        d[0] = to_t<T>(v[0]); d[1] = to_t<T>(v[1]); d[2] = to_t<T>(v[2]); d[3] = to_t<T>(v[3]);
      }
    } else {
      // B [K][N]: 32 rows of k x 64 n -> transposed into sB[n][k]
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const int vi = tid + 256 * x;
        const int kr = vi >> 4, nc = (vi & 15) * 4;
        const f32x4 v = *reinterpret_cast<const f32x4*>(B + (int64_t)(k0 + kr) * a.N + n0 + nc);
        sB[(nc + 0) * PA + kr] = to_t<T>(v[0]);
        sB[(nc + 1) * PA + kr] = to_t<T>(v[1]);
        sB[(nc + 2) * PA + kr] = to_t<T>(v[2]);
        sB[(nc + 3) * PA + kr] = to_t<T>(v[3]);
      }
    }
    __syncthreads();
    frag_t<T> fa[2], fb[2];
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      fa[x] = ld8(sA + (32 * wm + 16 * x + c) * PA + 8 * g);
      fb[x] = ld8(sB + (32 * wn + 16 * x + c) * PA + 8 * g);
    }
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int y = 0; y < 2; ++y) mma(acc[x][y], fa[x], fb[y]);
    __syncthreads();
  }

  float* C = a.C + (int64_t)b * a.c_bs;
  const float* Dm = a.Dm ? a.Dm + (int64_t)b * a.d_bs : nullptr;
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = m0 + 32 * wm + 16 * x + 4 * g + i;
        const int col = n0 + 32 * wn + 16 * y + c;
        float v = a.alpha * acc[x][y][i];
        if (Dm) v += a.beta * Dm[(int64_t)r * a.N + col];
        C[(int64_t)r * a.N + col] = v;
      }
}

hipError_t launch_gemm(int dtype, const GemmArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)((a.M / 64) * (a.N / 64)), (unsigned)a.batch);
  if (dtype == 1)
    hipLaunchKernelGGL(k_gemm<bf16>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(k_gemm<float>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace lact
