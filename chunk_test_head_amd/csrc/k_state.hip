// State kernels: split reduction + momentum, Frobenius normalisation, weight
// step + row renorm + operand copies, fill.
//
// Momentum (LaCT rebuttal page, momentum block of block_causal_lact_swiglu):
//   beta = mean over the written tokens of the per-token momentum,
//   G <- G + beta M,  M <- G   (before Muon).
// Step + renorm (same page, end of the chunk loop; summary page section 3.2
// Eq. 8):  W <- W + U,  row <- row / (||row|| + eps) * n0[row], with n0 the
// row norms at sequence start.  Master variant (uTTT page section C.1,
// renorm = 2): the fp32 state keeps W + U unscaled and only the operand
// copies, which reads and gradients use, hold the rescaled rows.
#include "lact_internal.hpp"
#include "mfma.hpp"

namespace lact {

// ------------------------------------------------------------ reduce ----
// Tile of 64 (hidden j) x 64 (feature i) of one matrix of one head: sum the
// split partials [j][i] in split order, transpose through LDS, add momentum
// and write the wide [i][j] result.
__global__ __launch_bounds__(256) void k_reduce(ReduceArgs a) {
  __shared__ float tile[64][65];
  __shared__ float red[4];
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
  float* out = mat == 0 ? a.out1 : mat == 1 ? a.out3 : a.out2;
  if (out != nullptr) out += (int64_t)head * msz;
  float* m = (mat == 0 ? a.m1 : mat == 1 ? a.m3 : a.m2);
  if (m != nullptr) m += (int64_t)head * msz;
  // the old momentum rows first (independent of the sum)
  f32x4 mo[4];
  if (m != nullptr) {
#pragma unroll
    for (int rr = 0; rr < 4; ++rr)
      mo[rr] = *reinterpret_cast<const f32x4*>(m + (int64_t)(i0 + ty + 16 * rr) * a.dh + j0 + 4 * tx);
  }
  // split partials, up to four splits' loads in flight per row, summed in
  // split order
  f32x4 acc[4];
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) acc[rr] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int sp0 = 0; sp0 < a.nsplit; sp0 += 4) {
    f32x4 v[4][4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int64_t off = (int64_t)(j0 + ty + 16 * rr) * a.d + i0 + 4 * tx;
        v[q][rr] = sp0 + q < a.nsplit ? *reinterpret_cast<const f32x4*>(p + (sp0 + q) * pstride + off)
                                      : f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr)
        if (sp0 + q < a.nsplit) acc[rr] = (sp0 + q == 0) ? v[q][rr] : acc[rr] + v[q][rr];
  }
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    const int j = ty + 16 * rr;
    tile[j][4 * tx + 0] = acc[rr][0];
    tile[j][4 * tx + 1] = acc[rr][1];
    tile[j][4 * tx + 2] = acc[rr][2];
    tile[j][4 * tx + 3] = acc[rr][3];
  }
  __syncthreads();
  const float beta = m != nullptr ? a.beta[head] : 0.f;
  float ss = 0.f;
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
      v = v + beta * mo[rr];
      *reinterpret_cast<f32x4*>(m + off) = v;
    }
    if (out != nullptr) *reinterpret_cast<f32x4*>(out + off) = v;
    ss += v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3];
  }
  if (a.ss_part != nullptr) {
    // the tile's sum of squares, waves in index order
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
    if ((tid & 63) == 0) red[tid >> 6] = ss;
    __syncthreads();
    if (tid == 0)
      a.ss_part[((int64_t)mat * a.bh + head) * (jt * itn) + tj * itn + ti] = (red[0] + red[1]) + (red[2] + red[3]);
  }
}

hipError_t launch_reduce(const ReduceArgs& a, hipStream_t s) {
  const int64_t blocks = (int64_t)a.bh * 3 * (a.dh / 64) * (a.d / 64);
  hipLaunchKernelGGL(k_reduce, dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

// ---------------------------------------------------- ns normalisation --
// X = G / (||G||_F + eps), one workgroup per matrix, fixed reduction order.
__global__ __launch_bounds__(256) void k_ns_norm(NsNormArgs a) {
  __shared__ float red[256];
  const int tid = threadIdx.x;
  const float* g = a.g.at(blockIdx.x, a.n);
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
// One pass per matrix: W <- W + U, row <- row * n0[row] / (||row|| + eps),
// operand copies.  Every workgroup owns whole rows, so the row norms need no
// second pass over W.
//   W1, W3 ([dh][d], rows = hidden j): 32 rows per workgroup; U is wide
//     ([d][dh]), so its 32-column block is transposed through LDS first.
//   W2 ([d][dh], rows = feature i): 8 rows per workgroup (two per wave);
//     the W2^T copy ([dh][d]) is written from an LDS tile, 8 features of a
//     hidden unit per 16-byte store.
template <class T>
__device__ __forceinline__ void step_w13(const StepArgs& a, int blk, float* ut) {
  constexpr int RB = 16;  // rows per workgroup (16: two workgroups per CU); ut: [RB][d + 1]
  const int tid = threadIdx.x;
  const int d = a.d, dh = a.dh, pt = d + 1;
  const int nb = dh / RB;
  const int jb = blk % nb, mat = (blk / nb) % 2, head = blk / (2 * nb);
  const int64_t msz = (int64_t)d * dh;
  const int j0 = RB * jb;
  float* W = (mat == 0 ? a.w1 : a.w3) + (int64_t)head * msz + (int64_t)j0 * d;
  const float* U = mat == 0 ? a.u1 : a.u3;
  // The RB x d block of W is contiguous: thread tid takes float4 number
  // tid + 256 k (row (tid + 256 k) / (d/4)); the d/4 threads of a row are
  // consecutive lanes and combine their sums of squares by shuffles.  W is
  // requested first so that its loads overlap the transpose of U (wide U);
  // with u13_tall the update arrives in W's own layout and is added row for
  // row, without the transpose.
  const int q4 = d / 4, nk = RB * q4 / 256, rstep = 256 / q4;
  const int r0 = tid / q4, c4 = 4 * (tid % q4);
  constexpr int KMAX = RB / 4;  // d <= 256
  f32x4 w[KMAX];
#pragma unroll
  for (int k = 0; k < KMAX; ++k)
    if (k < nk) w[k] = *reinterpret_cast<const f32x4*>(W + (int64_t)(r0 + rstep * k) * d + c4);
  const bool add_u = U != nullptr;
  if (U != nullptr && a.u13_tall) {
    // U in the layout of W: the same rows, read like W
    const float* Ut = U + (int64_t)head * msz + (int64_t)j0 * d;
    f32x4 uv[KMAX];
#pragma unroll
    for (int k = 0; k < KMAX; ++k)
      if (k < nk) uv[k] = *reinterpret_cast<const f32x4*>(Ut + (int64_t)(r0 + rstep * k) * d + c4);
#pragma unroll
    for (int k = 0; k < KMAX; ++k)
      if (k < nk) w[k] += uv[k];
    U = nullptr;  // (added)
  }
  if (U != nullptr) {
    U += (int64_t)head * msz + j0;
    // U[i][j0 + 4q .. +3] -> ut[4q .. 4q+3][i]: every load of the thread is
    // issued before the first store (one memory latency, not one per vector)
    constexpr int UMAX = 256 * (RB / 4) / 256;  // vectors per thread, d <= 256
    f32x4 uv[UMAX];
#pragma unroll
    for (int k = 0; k < UMAX; ++k) {
      const int e = tid + 256 * k;
      if (e < d * (RB / 4))
        uv[k] = *reinterpret_cast<const f32x4*>(U + (int64_t)(e / (RB / 4)) * dh + 4 * (e % (RB / 4)));
    }
#pragma unroll
    for (int k = 0; k < UMAX; ++k) {
      const int e = tid + 256 * k;
      if (e < d * (RB / 4)) {
        const int i = e / (RB / 4), q = e % (RB / 4);
        ut[(4 * q + 0) * pt + i] = uv[k][0];
        ut[(4 * q + 1) * pt + i] = uv[k][1];
        ut[(4 * q + 2) * pt + i] = uv[k][2];
        ut[(4 * q + 3) * pt + i] = uv[k][3];
      }
    }
    __syncthreads();
  }
  float ss[KMAX];
#pragma unroll
  for (int k = 0; k < KMAX; ++k) {
    if (k < nk) {
      const int r = r0 + rstep * k;
      if (U != nullptr) {
#pragma unroll
        for (int x = 0; x < 4; ++x) w[k][x] += ut[r * pt + c4 + x];
      }
      ss[k] = w[k][0] * w[k][0] + w[k][1] * w[k][1] + w[k][2] * w[k][2] + w[k][3] * w[k][3];
      for (int o = 1; o < q4; o <<= 1) ss[k] += __shfl_xor(ss[k], o);
      if (a.nonfinite != nullptr && c4 == 0 && !(ss[k] <= 3.402823466e38f)) atomicOr(a.nonfinite, 1);
    }
  }
  const bool write_w = add_u || a.renorm;
  float* N0 = (mat == 0 ? a.n1 : a.n3) + (int64_t)head * dh + j0;
  T* S = reinterpret_cast<T*>(a.sh.base) + (int64_t)head * a.sh.per_head +
         (mat == 0 ? a.sh.off_w1 : a.sh.off_w3) + (int64_t)j0 * d;
#pragma unroll
  for (int k = 0; k < KMAX; ++k) {
    if (k < nk) {
      const int r = r0 + rstep * k;
      const float f = a.renorm ? N0[r] / (sqrtf(ss[k]) + a.eps) : 1.f;
      if (a.init && c4 == 0) N0[r] = sqrtf(ss[k]);  // sequence-start norm
      const f32x4 v = w[k] * f;
      if (write_w) *reinterpret_cast<f32x4*>(W + (int64_t)r * d + c4) = a.renorm == 2 ? w[k] : v;
      st4(S + (int64_t)r * d + c4, v[0], v[1], v[2], v[3]);
    }
  }
}

template <class T, int KMAX>
__device__ __forceinline__ void step_w2(const StepArgs& a, int blk, T* tl) {
  // tl: [8][dh] operand values of the 8 rows
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int d = a.d, dh = a.dh;
  const int nb = d / 8;
  const int ib = blk % nb, head = blk / nb;
  const int64_t msz = (int64_t)d * dh;
  const int i0 = 8 * ib;
  const bool write_w = a.u2 != nullptr || a.renorm;
  T* sb = reinterpret_cast<T*>(a.sh.base) + (int64_t)head * a.sh.per_head;
  // float4 columns 4 lane + 256 k, k <= KMAX (dh <= 256 (KMAX + 1)); the
  // wave's two rows (wave, wave + 4) are loaded before anything is stored
  const int nk = dh / 256, rem = dh % 256;
  f32x4 w[2][KMAX + 1];
#pragma unroll
  for (int rr = 0; rr < 2; ++rr) {
    const int row = wave + 4 * rr;  // 0..7
    const float* W = a.w2 + (int64_t)head * msz + (int64_t)(i0 + row) * dh;
    const float* U = a.u2 != nullptr ? a.u2 + (int64_t)head * msz + (int64_t)(i0 + row) * dh : nullptr;
#pragma unroll
    for (int k = 0; k <= KMAX; ++k) {
      const int col = 4 * lane + 256 * k;
      if (k < nk || (k == nk && 4 * lane < rem)) {
        w[rr][k] = *reinterpret_cast<const f32x4*>(W + col);
        if (U != nullptr) w[rr][k] += *reinterpret_cast<const f32x4*>(U + col);
      }
    }
  }
#pragma unroll
  for (int rr = 0; rr < 2; ++rr) {
    const int row = wave + 4 * rr;  // 0..7
    float* W = a.w2 + (int64_t)head * msz + (int64_t)(i0 + row) * dh;
    float ss = 0.f;
#pragma unroll
    for (int k = 0; k <= KMAX; ++k) {
      const int col = 4 * lane + 256 * k;
      if (k < nk || (k == nk && 4 * lane < rem))
        ss += w[rr][k][0] * w[rr][k][0] + w[rr][k][1] * w[rr][k][1] + w[rr][k][2] * w[rr][k][2] +
              w[rr][k][3] * w[rr][k][3];
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
    if (a.nonfinite != nullptr && lane == 0 && !(ss <= 3.402823466e38f)) atomicOr(a.nonfinite, 1);
    float f = 1.f;
    if (a.renorm) f = a.n2[(int64_t)head * d + i0 + row] / (sqrtf(ss) + a.eps);
    if (a.init && lane == 0) a.n2[(int64_t)head * d + i0 + row] = sqrtf(ss);  // sequence-start norm
    T* S = sb + a.sh.off_w2 + (int64_t)(i0 + row) * dh;
#pragma unroll
    for (int k = 0; k <= KMAX; ++k) {
      const int col = 4 * lane + 256 * k;
      if (k < nk || (k == nk && 4 * lane < rem)) {
        const f32x4 v = w[rr][k] * f;
        if (write_w) *reinterpret_cast<f32x4*>(W + col) = a.renorm == 2 ? w[rr][k] : v;
        st4(S + col, v[0], v[1], v[2], v[3]);
        st4(tl + row * dh + col, v[0], v[1], v[2], v[3]);
      }
    }
  }
  __syncthreads();
  // W2^T[j][i0 .. i0 + 7]
  T* St = sb + a.sh.off_w2t;
  for (int j = tid; j < dh; j += 256) {
    T* dst = St + (int64_t)j * d + i0;
    st4(dst, (float)tl[0 * dh + j], (float)tl[1 * dh + j], (float)tl[2 * dh + j], (float)tl[3 * dh + j]);
    st4(dst + 4, (float)tl[4 * dh + j], (float)tl[5 * dh + j], (float)tl[6 * dh + j], (float)tl[7 * dh + j]);
  }
}

// Sequence start: workgroup blk of nblk zeroes its share of the momentum
// buffers (as one concatenation of m1, m3, m2; NULL buffers skipped).
__device__ __forceinline__ void zero_share(const StepArgs& a, int blk, int nblk) {
  const int64_t per = (int64_t)a.bh * a.d * a.dh / 4;  // float4 per buffer
  const int64_t tot = 3 * per, q = (tot + nblk - 1) / nblk;
  const int64_t end = (int64_t)(blk + 1) * q < tot ? (int64_t)(blk + 1) * q : tot;
  for (int64_t i = (int64_t)blk * q + threadIdx.x; i < end; i += 256) {
    const int mb = (int)(i / per);
    float* m = mb == 0 ? a.mz1 : (mb == 1 ? a.mz3 : a.mz2);
    if (m != nullptr) reinterpret_cast<f32x4*>(m)[i - mb * per] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
}

// One launch for all three matrices: workgroups [0, n13) take W1 / W3 row
// blocks, the rest W2 row blocks.
template <class T, int KMAX>
__global__ __launch_bounds__(256) void k_step(StepArgs a, int n13) {
  extern __shared__ __attribute__((aligned(16))) float step_lds[];
  if (a.init) zero_share(a, blockIdx.x, gridDim.x);
  if ((int)blockIdx.x < n13) step_w13<T>(a, blockIdx.x, step_lds);
  else step_w2<T, KMAX>(a, blockIdx.x - n13, reinterpret_cast<T*>(step_lds));
}

template <class T, int KMAX>
static hipError_t run_step(const StepArgs& a, hipStream_t s) {
  const size_t l13 = (size_t)16 * (a.d + 1) * sizeof(float);
  const size_t l2 = (size_t)8 * a.dh * sizeof(T);
  const size_t lds = l13 > l2 ? l13 : l2;
  hipError_t e = allow_dynamic_lds(reinterpret_cast<const void*>(&k_step<T, KMAX>),
                                   (int)(8 * 4096 * sizeof(T)));
  if (e != hipSuccess) return e;
  const int n13 = a.bh * 2 * (a.dh / 16), n2 = a.bh * (a.d / 8);
  hipLaunchKernelGGL((k_step<T, KMAX>), dim3((unsigned)(n13 + n2)), dim3(256), lds, s, a, n13);
  return hipGetLastError();
}

hipError_t launch_step(int dtype, const StepArgs& a, hipStream_t s) {
  if (dtype == 1) return a.dh <= 1024 ? run_step<bf16, 3>(a, s) : run_step<bf16, 15>(a, s);
  return a.dh <= 1024 ? run_step<float, 3>(a, s) : run_step<float, 15>(a, s);
}

}  // namespace lact
