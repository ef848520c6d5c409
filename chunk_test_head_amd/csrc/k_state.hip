// State kernels: split reduction + momentum, momentum coefficient, Frobenius
// normalisation, weight step + row renorm + operand copies, fill.
//
// Momentum (LaCT rebuttal page, momentum block of block_causal_lact_swiglu):
//   beta = mean over the written tokens of the per-token momentum,
//   G <- G + beta M,  M <- G   (before Muon).
// Step + renorm (same page, end of the chunk loop; summary page section 3.2
// Eq. 8):  W <- W + U,  row <- row / (||row|| + eps) * n0[row], with n0 the
// row norms at sequence start.
#include "lact_internal.hpp"
#include "mfma.hpp"

namespace lact {

// ------------------------------------------------------------ reduce ----
// Tile of 64 (hidden j) x 64 (feature i) of one matrix of one head: sum the
// split partials [j][i] in split order, transpose through LDS, add momentum
// and write the wide [i][j] result.
__global__ __launch_bounds__(256) void k_reduce(ReduceArgs a) {
  __shared__ float tile[64][65];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int jt = a.dh / 64, itn = a.d / 64;
  int id = blockIdx.x;
  const int ti = id % itn; id /= itn;
  const int tj = id % jt; id /= jt;
  const int mat = id % 3;
  const int head = id / 3;
  const int64_t msz = (int64_t)a.d * a.dh;
  const int64_t pstride = (int64_t)a.bh * 3 * msz;  // between splits
  const float* p = a.partial + ((int64_t)head * 3 + mat) * msz;
  const int j0 = tj * 64, i0 = ti * 64;
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    const int j = ty + 16 * rr;
    const int64_t off = (int64_t)(j0 + j) * a.d + i0 + 4 * tx;
    f32x4 s = *reinterpret_cast<const f32x4*>(p + off);
    for (int sp = 1; sp < a.nsplit; ++sp) s += *reinterpret_cast<const f32x4*>(p + sp * pstride + off);
    tile[j][4 * tx + 0] = s[0];
    tile[j][4 * tx + 1] = s[1];
    tile[j][4 * tx + 2] = s[2];
    tile[j][4 * tx + 3] = s[3];
  }
  __syncthreads();
  float* out = (mat == 0 ? a.out1 : mat == 1 ? a.out3 : a.out2) + (int64_t)head * msz;
  float* m = (mat == 0 ? a.m1 : mat == 1 ? a.m3 : a.m2);
  const float beta = (m != nullptr) ? a.beta[head] : 0.f;
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    const int i = ty + 16 * rr;
    const int64_t off = (int64_t)(i0 + i) * a.dh + j0 + 4 * tx;
    f32x4 v;
    v[0] = tile[4 * tx + 0][i];
    v[1] = tile[4 * tx + 1][i];
    v[2] = tile[4 * tx + 2][i];
    v[3] = tile[4 * tx + 3][i];
    if (m != nullptr) {
      float* mp = m + (int64_t)head * msz + off;
      const f32x4 mo = *reinterpret_cast<const f32x4*>(mp);
      v = v + beta * mo;
      *reinterpret_cast<f32x4*>(mp) = v;
    }
    *reinterpret_cast<f32x4*>(out + off) = v;
  }
}

hipError_t launch_reduce(const ReduceArgs& a, hipStream_t s) {
  const int64_t blocks = (int64_t)a.bh * 3 * (a.dh / 64) * (a.d / 64);
  hipLaunchKernelGGL(k_reduce, dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

// ------------------------------------------------------------- beta -----
__global__ __launch_bounds__(256) void k_beta(BetaArgs a) {
  __shared__ float red[256];
  const int head = blockIdx.x, tid = threadIdx.x;
  const float* m = a.mom + (int64_t)head * a.sbh;
  float s = 0.f;
  for (int64_t t = tid; t < a.n_tok; t += 256) s += m[t];
  red[tid] = s;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (tid < w) red[tid] += red[tid + w];
    __syncthreads();
  }
  if (tid == 0) a.beta[head] = a.n_tok > 0 ? red[0] / (float)a.n_tok : 0.f;
}

hipError_t launch_beta(const BetaArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_beta, dim3(a.bh), dim3(256), 0, s, a);
  return hipGetLastError();
}

// ---------------------------------------------------- ns normalisation --
// X = G / (||G||_F + eps), one workgroup per matrix, fixed reduction order.
__global__ __launch_bounds__(256) void k_ns_norm(NsNormArgs a) {
  __shared__ float red[256];
  const int tid = threadIdx.x;
  const float* g = a.g + (int64_t)blockIdx.x * a.n;
  float* x = a.x + (int64_t)blockIdx.x * a.n;
  float s = 0.f;
  for (int64_t e = (int64_t)tid * 4; e < a.n; e += 1024) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(g + e);
    s += v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3];
  }
  red[tid] = s;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (tid < w) red[tid] += red[tid + w];
    __syncthreads();
  }
  const float scale = 1.0f / (sqrtf(red[0]) + a.eps);
  for (int64_t e = (int64_t)tid * 4; e < a.n; e += 1024) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(g + e);
    *reinterpret_cast<f32x4*>(x + e) = v * scale;
  }
}

hipError_t launch_ns_norm(const NsNormArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_ns_norm, dim3((unsigned)a.count), dim3(256), 0, s, a);
  return hipGetLastError();
}

// ------------------------------------------------------------- step -----
// Tiles of 64 x 64 over the natural layout of each matrix:
//   mat 0, 1 (W1, W3): rows = hidden j (dh), cols = feature i (d)
//   mat 2    (W2)    : rows = feature i (d), cols = hidden j (dh)
// U is wide ([i][j]) for all three, so W1/W3 tiles read it transposed.
// Row partial sums of squares go to rowpart[head][mat][coltile][row].
int64_t step_rowpart_elems(int bh, int d, int dh) {
  // per head: W1, W3: (d/64) x dh ; W2: (dh/64) x d
  return (int64_t)bh * (2 * (int64_t)(d / 64) * dh + (int64_t)(dh / 64) * d);
}

struct TileInfo {
  int head, mat, tr, tc;  // tile row / col index in the natural layout
  int rows, cols;         // natural dims of the matrix
  int64_t rp_off;         // rowpart offset of this matrix for this head
};

__device__ __forceinline__ TileInfo tile_info(int id, int d, int dh) {
  TileInfo t;
  const int per = (dh / 64) * (d / 64);
  t.head = id / (3 * per);
  id -= t.head * 3 * per;
  t.mat = id / per;
  id -= t.mat * per;
  if (t.mat < 2) { t.rows = dh; t.cols = d; } else { t.rows = d; t.cols = dh; }
  const int ctn = t.cols / 64;
  t.tr = id / ctn;
  t.tc = id % ctn;
  const int64_t per_head = 2 * (int64_t)(d / 64) * dh + (int64_t)(dh / 64) * d;
  t.rp_off = (int64_t)t.head * per_head + (t.mat == 0 ? 0 : t.mat == 1 ? (int64_t)(d / 64) * dh : 2 * (int64_t)(d / 64) * dh);
  return t;
}

// Pass 1: W <- W + U (written back when U is given), row partial sums.
__global__ __launch_bounds__(256) void k_step_add(StepArgs a) {
  __shared__ float tile[64][65];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const TileInfo t = tile_info(blockIdx.x, a.d, a.dh);
  const int64_t msz = (int64_t)a.d * a.dh;
  float* W = (t.mat == 0 ? a.w1 : t.mat == 1 ? a.w3 : a.w2) + (int64_t)t.head * msz;
  const float* U = (t.mat == 0 ? a.u1 : t.mat == 1 ? a.u3 : a.u2);
  const int r0 = t.tr * 64, c0 = t.tc * 64;
  if (U != nullptr) {
    U += (int64_t)t.head * msz;
    if (t.mat < 2) {
      // U wide [i][j]: tile rows j (r0..), cols i (c0..) -> read U[c0 + .][r0 + .]
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int i = ty + 16 * rr;
        const f32x4 v = *reinterpret_cast<const f32x4*>(U + (int64_t)(c0 + i) * a.dh + r0 + 4 * tx);
        tile[4 * tx + 0][i] = v[0];
        tile[4 * tx + 1][i] = v[1];
        tile[4 * tx + 2][i] = v[2];
        tile[4 * tx + 3][i] = v[3];
      }
    } else {
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int r = ty + 16 * rr;
        const f32x4 v = *reinterpret_cast<const f32x4*>(U + (int64_t)(r0 + r) * a.dh + c0 + 4 * tx);
        tile[r][4 * tx + 0] = v[0];
        tile[r][4 * tx + 1] = v[1];
        tile[r][4 * tx + 2] = v[2];
        tile[r][4 * tx + 3] = v[3];
      }
    }
    __syncthreads();
  }
  __shared__ float part[64][17];
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    const int r = ty + 16 * rr;
    float* wp = W + (int64_t)(r0 + r) * t.cols + c0 + 4 * tx;
    f32x4 w = *reinterpret_cast<const f32x4*>(wp);
    if (U != nullptr) {
      w[0] += tile[r][4 * tx + 0];
      w[1] += tile[r][4 * tx + 1];
      w[2] += tile[r][4 * tx + 2];
      w[3] += tile[r][4 * tx + 3];
      if (a.write_w) *reinterpret_cast<f32x4*>(wp) = w;
    }
    part[r][tx] = w[0] * w[0] + w[1] * w[1] + w[2] * w[2] + w[3] * w[3];
  }
  __syncthreads();
  if (tid < 64) {
    float s = 0.f;
#pragma unroll
    for (int x = 0; x < 16; ++x) s += part[tid][x];
    a.rowpart[t.rp_off + (int64_t)t.tc * t.rows + r0 + tid] = s;
  }
}

// Pass 2: per-row factor, W <- W * factor, operand copies.
template <class T>
__global__ __launch_bounds__(256) void k_step_scale(StepArgs a) {
  __shared__ float fac[64];
  __shared__ float tile[64][65];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const TileInfo t = tile_info(blockIdx.x, a.d, a.dh);
  const int64_t msz = (int64_t)a.d * a.dh;
  float* W = (t.mat == 0 ? a.w1 : t.mat == 1 ? a.w3 : a.w2) + (int64_t)t.head * msz;
  float* N0 = (t.mat == 0 ? a.n1 : t.mat == 1 ? a.n3 : a.n2) + (int64_t)t.head * t.rows;
  const int r0 = t.tr * 64, c0 = t.tc * 64;
  if (tid < 64) {
    float f = 1.f;
    if (a.renorm) {
      const int ctn = t.cols / 64;
      float sq = 0.f;
      for (int x = 0; x < ctn; ++x) sq += a.rowpart[t.rp_off + (int64_t)x * t.rows + r0 + tid];
      f = N0[r0 + tid] / (sqrtf(sq) + a.eps);
    }
    fac[tid] = f;
  }
  __syncthreads();
  T* sb = reinterpret_cast<T*>(a.sh.base) + (int64_t)t.head * a.sh.per_head;
  T* S = sb + (t.mat == 0 ? a.sh.off_w1 : t.mat == 1 ? a.sh.off_w3 : a.sh.off_w2);
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    const int r = ty + 16 * rr;
    float* wp = W + (int64_t)(r0 + r) * t.cols + c0 + 4 * tx;
    f32x4 w = *reinterpret_cast<const f32x4*>(wp);
    w = w * fac[r];
    if (a.renorm) *reinterpret_cast<f32x4*>(wp) = w;
    st4(S + (int64_t)(r0 + r) * t.cols + c0 + 4 * tx, w[0], w[1], w[2], w[3]);
    if (t.mat == 2) {
      tile[r][4 * tx + 0] = w[0];
      tile[r][4 * tx + 1] = w[1];
      tile[r][4 * tx + 2] = w[2];
      tile[r][4 * tx + 3] = w[3];
    }
  }
  if (t.mat == 2) {
    // W2^T copy: [dh][d]; tile rows i (r0..), cols j (c0..)
    __syncthreads();
    T* St = sb + a.sh.off_w2t;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int j = ty + 16 * rr;
      st4(St + (int64_t)(c0 + j) * a.d + r0 + 4 * tx, tile[4 * tx + 0][j], tile[4 * tx + 1][j],
          tile[4 * tx + 2][j], tile[4 * tx + 3][j]);
    }
  }
}

hipError_t launch_step(int dtype, const StepArgs& a, hipStream_t s) {
  const int64_t blocks = (int64_t)a.bh * 3 * (a.dh / 64) * (a.d / 64);
  if (a.u1 != nullptr || a.renorm) {
    hipLaunchKernelGGL(k_step_add, dim3((unsigned)blocks), dim3(256), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (dtype == 1)
    hipLaunchKernelGGL(k_step_scale<bf16>, dim3((unsigned)blocks), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(k_step_scale<float>, dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

// -------------------------------------------------------- row norms -----
// n0 <- L2 norm of every row, one wave per row (rows of W1, W3: d; W2: dh).
__global__ __launch_bounds__(256) void k_row_norms(StepArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t per_head = 2 * (int64_t)a.dh + a.d;
  if (row >= per_head * a.bh) return;
  const int head = (int)(row / per_head);
  int64_t r = row % per_head;
  const int64_t msz = (int64_t)a.d * a.dh;
  const float* W;
  float* N;
  int len;
  if (r < a.dh) { W = a.w1 + head * msz + r * a.d; N = a.n1 + (int64_t)head * a.dh + r; len = a.d; }
  else if (r < 2 * a.dh) { r -= a.dh; W = a.w3 + head * msz + r * a.d; N = a.n3 + (int64_t)head * a.dh + r; len = a.d; }
  else { r -= 2 * a.dh; W = a.w2 + head * msz + r * a.dh; N = a.n2 + (int64_t)head * a.d + r; len = a.dh; }
  float s = 0.f;
  for (int x = lane; x < len; x += 64) s += W[x] * W[x];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
  if (lane == 0) *N = sqrtf(s);
}

hipError_t launch_row_norms(const StepArgs& a, hipStream_t s) {
  const int64_t rows = (int64_t)a.bh * (2 * (int64_t)a.dh + a.d);
  hipLaunchKernelGGL(k_row_norms, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, a);
  return hipGetLastError();
}

// ------------------------------------------------------------- fill -----
__global__ void k_fill(float* p, int64_t n, float v) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

hipError_t launch_fill(float* p, int64_t n, float v, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_fill, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, n, v);
  return hipGetLastError();
}

}  // namespace lact
