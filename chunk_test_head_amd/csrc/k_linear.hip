// Linear fast-weight variant (LaCT rebuttal page, the comparison of
// fast-weight networks, Fig. 8(a)): one d x d matrix per head,
//   read   o_t = W q_t,
//   write  G = sum_t eta_t v_t k_t^T   (descent direction of
//          -sum_t eta_t <W k_t, v_t>; it does not depend on W),
// then the momentum, Newton-Schulz, step and row renorm of the SwiGLU layer.
// Plain GEMM-shaped work on bf16 (or fp32) MFMA operands with fp32 sums:
//   k_lin_apply: 64 tokens per workgroup, a wave per 16 tokens, all d
//     outputs; q and W fragments straight from global memory (16-byte rows);
//   k_lin_grad:  one 64 x 64 tile of G per workgroup over all the write's
//     tokens, 32-token slabs of eta v and k staged row-major in LDS and read
//     as K-per-lane fragments (LDS transpose reads); momentum in the epilogue;
//   k_lin_step:  one wave per row: W <- W + U, rescale (or keep a master),
//     operand copy.
#include "lact_internal.hpp"
#include "mfma.hpp"

namespace lact {

template <class T, int D>
__global__ __launch_bounds__(256) void k_lin_apply(LinArgs a) {
  constexpr int IT = D / 16, KS = D / 32;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = lane & 15, g = lane >> 4;
  const int tiles = (int)((a.n_tok + 63) / 64);
  const int head = blockIdx.x / tiles;
  const int64_t t0 = (int64_t)(blockIdx.x % tiles) * 64 + 16 * wave;
  const T* q = reinterpret_cast<const T*>(a.q) + (int64_t)head * a.q_sbh;
  const T* W = reinterpret_cast<const T*>(a.shadow) + (int64_t)head * D * D;
  f32x4 acc[IT];
#pragma unroll
  for (int it = 0; it < IT; ++it) acc[it] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int64_t tr = t0 + c;  // this lane's token row of the A fragment
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    frag_t<T> fa;
    if (tr < a.n_tok) {
      fa = ld8(q + tr * a.q_st + 32 * ks + 8 * g);
    } else {
#pragma unroll
      for (int m = 0; m < 8; ++m) fa[m] = to_t<T>(0.f);
    }
#pragma unroll
    for (int it = 0; it < IT; ++it) mma(acc[it], fa, ld8(W + (int64_t)(16 * it + c) * D + 32 * ks + 8 * g));
  }
  T* o = reinterpret_cast<T*>(a.o) + (int64_t)head * a.o_sbh;
#pragma unroll
  for (int it = 0; it < IT; ++it)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t t = t0 + 4 * g + i;
      if (t < a.n_tok) o[t * a.o_st + 16 * it + c] = to_t<T>(acc[it][i]);
    }
}

// A K-per-lane fragment (lane (c, g): rows 8 g .. 8 g + 7 of column col0 + c)
// of a row-major [32][pitch] LDS tile.
__device__ __forceinline__ bf16x8 col_frag(const bf16* s, int pitch, int col0, int c, int g) {
  const bf16* p = s + (8 * g + (c >> 2)) * pitch + col0 + 4 * (c & 3);
  return cat8(ld_tr4(p), ld_tr4(p + 4 * pitch));
}
__device__ __forceinline__ f32x8 col_frag(const float* s, int pitch, int col0, int c, int g) {
  f32x8 r;
#pragma unroll
  for (int m = 0; m < 8; ++m) r[m] = s[(8 * g + m) * pitch + col0 + c];
  return r;
}

template <class T, int D>
__global__ __launch_bounds__(256) void k_lin_grad(LinArgs a) {
  constexpr int NT = 32, P = 64 + 16 / (int)sizeof(T) * 2;  // padded pitch
  constexpr int TPR = D / 64;                                // tiles per row of G
  __shared__ __attribute__((aligned(16))) T sV[NT * P];
  __shared__ __attribute__((aligned(16))) T sK[NT * P];
  __shared__ float red[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = lane & 15, g = lane >> 4;
  const int head = blockIdx.x / (TPR * TPR);
  const int ti = (blockIdx.x / TPR) % TPR, tj = blockIdx.x % TPR;
  const int i0 = 64 * ti, j0 = 64 * tj;
  const T* kp = reinterpret_cast<const T*>(a.k) + (int64_t)head * a.k_sbh;
  const T* vp = reinterpret_cast<const T*>(a.v) + (int64_t)head * a.v_sbh;
  const float* ep = a.eta + (int64_t)head * a.eta_sbh;
  constexpr int V = 16 / sizeof(T);  // elements per 16-byte vector
  f32x4 acc[4];
#pragma unroll
  for (int jt = 0; jt < 4; ++jt) acc[jt] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int64_t t0 = 0; t0 < a.n_tok; t0 += NT) {
    __syncthreads();  // the previous slab is fully read
    // 32 tokens x 64 features of eta v (columns i0..) and k (columns j0..)
    for (int x = tid; x < NT * 64 / V; x += 256) {
      const int r = x / (64 / V), cv = (x % (64 / V)) * V;
      const int64_t t = t0 + r;
      if (t < a.n_tok) {
        const float e = ep[t];
        const T* vr = vp + t * a.v_st + i0 + cv;
        const T* kr = kp + t * a.k_st + j0 + cv;
#pragma unroll
        for (int u = 0; u < V; ++u) {
          sV[r * P + cv + u] = to_t<T>(e * to_f(vr[u]));
          sK[r * P + cv + u] = kr[u];
        }
      } else {
#pragma unroll
        for (int u = 0; u < V; ++u) {
          sV[r * P + cv + u] = to_t<T>(0.f);
          sK[r * P + cv + u] = to_t<T>(0.f);
        }
      }
    }
    __syncthreads();
    const frag_t<T> fa = col_frag(sV, P, 16 * wave, c, g);
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) mma(acc[jt], fa, col_frag(sK, P, 16 * jt, c, g));
  }
  // momentum: beta = mean of the write's coefficients; G~ = G + beta M, M <- G~
  float beta = 0.f;
  if (a.m != nullptr) {
    const float* mp = a.mom + (int64_t)head * a.mom_sbh;
    float s = 0.f;
    for (int64_t t = tid; t < a.n_tok; t += 256) s += mp[t];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
    if (lane == 0) red[wave] = s;
    __syncthreads();
    beta = a.n_tok > 0 ? ((red[0] + red[1]) + (red[2] + red[3])) / (float)a.n_tok : 0.f;
  }
  float* G = a.g + (int64_t)head * D * D;
  float* M = a.m != nullptr ? a.m + (int64_t)head * D * D : nullptr;
#pragma unroll
  for (int jt = 0; jt < 4; ++jt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t off = (int64_t)(i0 + 16 * wave + 4 * g + i) * D + j0 + 16 * jt + c;
      float x = acc[jt][i];
      if (M != nullptr) {
        x += beta * M[off];
        M[off] = x;
      }
      G[off] = x;
    }
}

// One wave per row of W: W <- W + U (U NULL: sequence start, which takes the
// row norms and zeroes the momentum), then the row rescaled to n0 / (||row||
// + eps) (renorm 1) or kept unscaled with a rescaled operand copy (renorm 2).
template <class T, int D>
__global__ __launch_bounds__(256) void k_lin_step(LinArgs a, const float* U, int init) {
  constexpr int PL = D / 64;  // values per lane
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= (int64_t)a.bh * D) return;
  float* w = a.w + row * D;
  T* sh = reinterpret_cast<T*>(a.shadow) + row * D;
  float x[PL];
  float ss = 0.f;
#pragma unroll
  for (int p = 0; p < PL; ++p) {
    x[p] = w[64 * p + lane] + (U != nullptr ? U[row * D + 64 * p + lane] : 0.f);
    ss += x[p] * x[p];
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
  if (a.nonfinite != nullptr && lane == 0 && !(ss <= 3.402823466e38f)) atomicOr(a.nonfinite, 1);
  float f = 1.f;
  if (init) {
    if (lane == 0) a.n[row] = sqrtf(ss);
    if (a.m != nullptr) {
#pragma unroll
      for (int p = 0; p < PL; ++p) a.m[row * D + 64 * p + lane] = 0.f;
    }
  } else if (a.renorm) {
    f = a.n[row] / (sqrtf(ss) + a.eps);
  }
#pragma unroll
  for (int p = 0; p < PL; ++p) {
    const float y = x[p] * f;
    if (!init) w[64 * p + lane] = a.renorm == 2 ? x[p] : y;
    sh[64 * p + lane] = to_t<T>(y);
  }
}

template <class T, int D>
static hipError_t run_lin(int what, const LinArgs& a, const float* U, hipStream_t s) {
  if (what == 0) {
    const int64_t blocks = (int64_t)a.bh * ((a.n_tok + 63) / 64);
    if (blocks > 0) hipLaunchKernelGGL((k_lin_apply<T, D>), dim3((unsigned)blocks), dim3(256), 0, s, a);
  } else if (what == 1) {
    hipLaunchKernelGGL((k_lin_grad<T, D>), dim3((unsigned)(a.bh * (D / 64) * (D / 64))), dim3(256), 0, s, a);
  } else {
    const int64_t rows = (int64_t)a.bh * D;
    hipLaunchKernelGGL((k_lin_step<T, D>), dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, a, U,
                       what == 3 ? 1 : 0);
  }
  return hipGetLastError();
}

// what: 0 read, 1 gradient (+ momentum) into a.g, 2 step with U, 3 sequence
// start (norms, momentum zeroed, operand copy).
hipError_t launch_linear(int dtype, int what, const LinArgs& a, const float* U, hipStream_t s) {
  if (dtype == 1) {
    switch (a.d) {
      case 64: return run_lin<bf16, 64>(what, a, U, s);
      case 128: return run_lin<bf16, 128>(what, a, U, s);
      case 256: return run_lin<bf16, 256>(what, a, U, s);
    }
  } else {
    switch (a.d) {
      case 64: return run_lin<float, 64>(what, a, U, s);
      case 128: return run_lin<float, 128>(what, a, U, s);
      case 256: return run_lin<float, 256>(what, a, U, s);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace lact
