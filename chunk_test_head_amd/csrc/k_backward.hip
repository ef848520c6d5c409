// Kernels of the outer-loop backward: the vector-Jacobian product of a whole
// sequence of the fast-weight layer with respect to q, k, v, the learning
// rates, the momentum coefficients and the initial weights (the layer is
// trained through its writes; uTTT page section 2).  The chain rule is taken
// step by step through the forward of the LaCT rebuttal page's chunk loop:
// read (apply step), chunk gradient (its derivative needs silu''), momentum,
// Newton-Schulz (the five quintic steps as matrix products; summary page
// section 3.2, Eq. 9-10), step and row renorm (Eq. 8).
//
// Everything here is fp32 (the backward recomputes the forward in fp32 and
// differentiates that):
//   * k_bgemm: batched C = alpha op(A) op(B) + beta D with arbitrary strides
//     (transposes are strides), bounds-checked 64 x 64 tiles, K in slabs of
//     32 staged through LDS, v_mfma_f32_16x16x4f32;
//   * elementwise passes over [bh][n][dh] activations (SwiGLU and its first
//     and second derivatives), row reductions for the learning-rate
//     gradients, row passes for the step + renorm and its VJP, per-matrix
//     reductions (Frobenius norms, momentum dots) in a fixed order.
#include "lact_internal.hpp"
#include "mfma.hpp"

namespace lact {

// ------------------------------------------------------------- GEMM ----
__device__ __forceinline__ float ldx(const void* p, int64_t i, int bf) {
  return bf ? (float)reinterpret_cast<const bf16*>(p)[i] : reinterpret_cast<const float*>(p)[i];
}
template <bool BF>
__device__ __forceinline__ float ldt(const void* p, int64_t i) {
  if constexpr (BF) return (float)reinterpret_cast<const bf16*>(p)[i];
  else return reinterpret_cast<const float*>(p)[i];
}

// One 64 x 64 tile of C over the K range [kb, ke) of matrix b: the next K
// slab of 32 is loaded into registers while the current one is contracted
// from LDS (two LDS buffers, one barrier per slab).  With P (split-K) the
// raw sum goes to P[z][b][m][n] instead of the epilogue.
template <bool ABF, bool BBF>
__global__ __launch_bounds__(256) void k_bgemm(BGemm g, int kchunk, float* P) {
  constexpr int T = 64, KS = 32, PD = T + 4, V = T * KS / 256;
  __shared__ float sA[2][KS][PD];  // [k][m]
  __shared__ float sB[2][KS][PD];  // [k][n]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = lane & 15, q = lane >> 4;
  const int wm = wave >> 1, wn = wave & 1;
  const int tn = (g.N + T - 1) / T;
  const int m0 = (blockIdx.x / tn) * T, n0 = (blockIdx.x % tn) * T;
  const int64_t b = blockIdx.y;
  const int kb = blockIdx.z * kchunk, ke = min(g.K, kb + kchunk);
  const void* A = reinterpret_cast<const char*>(g.A) + b * g.a_bs * (ABF ? 2 : 4);
  const void* B = reinterpret_cast<const char*>(g.B) + b * g.b_bs * (BBF ? 2 : 4);
  const bool a_kfast = g.a_sk == 1, b_nfast = g.b_sn == 1;
  // this thread's elements of a slab: A (m, k) and B (k, n), following the
  // unit stride so that a wave's loads are contiguous
  int am[V], ak[V], bn[V], bk[V];
#pragma unroll
  for (int i = 0; i < V; ++i) {
    const int e = tid + 256 * i;
    am[i] = a_kfast ? e / KS : e % T;
    ak[i] = a_kfast ? e % KS : e / T;
    bn[i] = b_nfast ? e % T : e / KS;
    bk[i] = b_nfast ? e / T : e % KS;
  }
  float ra[V], rb[V];
  auto load = [&](int k0) {
#pragma unroll
    for (int i = 0; i < V; ++i) {
      const int m = m0 + am[i], k = k0 + ak[i];
      ra[i] = (m < g.M && k < ke) ? ldt<ABF>(A, (int64_t)m * g.a_sm + (int64_t)k * g.a_sk) : 0.f;
      const int n = n0 + bn[i], kk = k0 + bk[i];
      rb[i] = (n < g.N && kk < ke) ? ldt<BBF>(B, (int64_t)kk * g.b_sk + (int64_t)n * g.b_sn) : 0.f;
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < V; ++i) {
      sA[buf][ak[i]][am[i]] = ra[i];
      sB[buf][bk[i]][bn[i]] = rb[i];
    }
  };
  f32x4 acc[2][2];
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y) acc[x][y] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int nslab = ke > kb ? (ke - kb + KS - 1) / KS : 0;
  if (nslab > 0) {
    load(kb);
    store(0);
  }
  __syncthreads();
  for (int j = 0; j < nslab; ++j) {
    const int buf = j & 1;
    if (j + 1 < nslab) load(kb + (j + 1) * KS);
#pragma unroll
    for (int s = 0; s < KS / 4; ++s) {
      float fa[2], fb[2];
#pragma unroll
      for (int x = 0; x < 2; ++x) fa[x] = sA[buf][4 * s + q][32 * wm + 16 * x + c];
#pragma unroll
      for (int y = 0; y < 2; ++y) fb[y] = sB[buf][4 * s + q][32 * wn + 16 * y + c];
#pragma unroll
      for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int y = 0; y < 2; ++y)
          acc[x][y] = __builtin_amdgcn_mfma_f32_16x16x4f32(fa[x], fb[y], acc[x][y], 0, 0, 0);
    }
    // buffer buf ^ 1 was last read in slab j - 1, before the previous barrier
    if (j + 1 < nslab) store(buf ^ 1);
    __syncthreads();
  }
  if (P != nullptr) {
    float* out = P + ((int64_t)blockIdx.z * gridDim.y + b) * g.M * g.N;
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int y = 0; y < 2; ++y)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int m = m0 + 32 * wm + 16 * x + 4 * q + i, n = n0 + 32 * wn + 16 * y + c;
          if (m < g.M && n < g.N) out[(int64_t)m * g.N + n] = acc[x][y][i];
        }
    return;
  }
  const float* D = g.D ? g.D + b * g.d_bs : nullptr;
  float* C = g.C + b * g.c_bs;
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = m0 + 32 * wm + 16 * x + 4 * q + i, n = n0 + 32 * wn + 16 * y + c;
        if (m < g.M && n < g.N) {
          float v = g.alpha * acc[x][y][i];
          if (D) v += g.beta * D[(int64_t)m * g.d_sm + n];
          C[(int64_t)m * g.c_sm + n] = v;
        }
      }
}

// One 128 x 128 tile of C over [kb, ke) of matrix b, for the large
// products: four waves of 64 x 64 (4 x 4 MFMA tiles each), K slabs of KS
// through two LDS buffers.  A slab's rows are stored permuted, row 16 x + c
// of each 64-row half at position 4 c + x, so that the values a lane needs
// for its four row tiles are one 16-byte read.  Each thread moves runs of 4
// elements along the operand's unit stride: as one 16-byte load for a slab
// inside the matrix when the operand is 16-byte aligned (vec_*), else
// element by element with bounds checks.  Logical workgroup ids are dealt
// by XCD: neighbouring tiles of one matrix share an L2.
template <bool ABF, bool BBF, int KS>
__global__ __launch_bounds__(256) void k_bgemm128(BGemm g, int kchunk, float* P, int vec_a, int vec_b,
                                                 int ntile) {
  constexpr int T = 128, PD = T + 4;
  constexpr int NQ = T * KS / 1024;  // runs of 4 per thread per operand per slab
  __shared__ __attribute__((aligned(16))) float sA[2][KS][PD];  // [k][permuted m]
  __shared__ __attribute__((aligned(16))) float sB[2][KS][PD];  // [k][permuted n]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = lane & 15, q = lane >> 4;
  const int wm = wave >> 1, wn = wave & 1;
  const int lid = xcd_logical_id(blockIdx.x, gridDim.x);
  const int tile = lid % ntile, rest = lid / ntile;
  const int64_t b = rest % g.batch;
  const int z = rest / g.batch;
  const int tn = (g.N + T - 1) / T;
  const int m0 = (tile / tn) * T, n0 = (tile % tn) * T;
  const int kb = z * kchunk, ke = min(g.K, kb + kchunk);
  const void* A = reinterpret_cast<const char*>(g.A) + b * g.a_bs * (ABF ? 2 : 4);
  const void* B = reinterpret_cast<const char*>(g.B) + b * g.b_bs * (BBF ? 2 : 4);
  const bool a_kfast = g.a_sk == 1, b_nfast = g.b_sn == 1;
  const bool a_full = vec_a && m0 + T <= g.M, b_full = vec_b && n0 + T <= g.N;
  // this thread's runs: (row, k) of the first element and the run direction
  // (along k for a k-contiguous operand, along rows otherwise)
  int ar[NQ], ak[NQ], br[NQ], bk[NQ];
#pragma unroll
  for (int i = 0; i < NQ; ++i) {
    const int x = tid + 256 * i;
    ar[i] = a_kfast ? x / (KS / 4) : 4 * (x % (T / 4));
    ak[i] = a_kfast ? 4 * (x % (KS / 4)) : x / (T / 4);
    br[i] = b_nfast ? 4 * (x % (T / 4)) : x / (KS / 4);
    bk[i] = b_nfast ? x / (T / 4) : 4 * (x % (KS / 4));
  }
  f32x4 ra[NQ], rb[NQ];
  auto load = [&](int k0) {
    const bool in_k = k0 + KS <= ke;
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
      const int m = m0 + ar[i], k = k0 + ak[i];
      if (!ABF && a_full && in_k) {
        ra[i] = *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(A) + (int64_t)m * g.a_sm +
                                                 (int64_t)k * g.a_sk);
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int mj = a_kfast ? m : m + j, kj = a_kfast ? k + j : k;
          ra[i][j] = (mj < g.M && kj < ke) ? ldt<ABF>(A, (int64_t)mj * g.a_sm + (int64_t)kj * g.a_sk) : 0.f;
        }
      }
      const int n = n0 + br[i], kk = k0 + bk[i];
      if (!BBF && b_full && in_k) {
        rb[i] = *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(B) + (int64_t)kk * g.b_sk +
                                                 (int64_t)n * g.b_sn);
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int nj = b_nfast ? n + j : n, kj = b_nfast ? kk : kk + j;
          rb[i][j] = (nj < g.N && kj < ke) ? ldt<BBF>(B, (int64_t)kj * g.b_sk + (int64_t)nj * g.b_sn) : 0.f;
        }
      }
    }
  };
  auto pos = [](int r) { return (r & 64) + 4 * (r & 15) + ((r >> 4) & 3); };
  auto store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (a_kfast) sA[buf][ak[i] + j][pos(ar[i])] = ra[i][j];
        else sA[buf][ak[i]][pos(ar[i]) + 4 * j] = ra[i][j];  // rows ar .. ar + 3: one 16-row group
        if (b_nfast) sB[buf][bk[i]][pos(br[i]) + 4 * j] = rb[i][j];
        else sB[buf][bk[i] + j][pos(br[i])] = rb[i][j];
      }
    }
  };
  f32x4 acc[4][4];
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int y = 0; y < 4; ++y) acc[x][y] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int nslab = ke > kb ? (ke - kb + KS - 1) / KS : 0;
  if (nslab > 0) {
    load(kb);
    store(0);
  }
  __syncthreads();
  for (int j = 0; j < nslab; ++j) {
    const int buf = j & 1;
    if (j + 1 < nslab) load(kb + (j + 1) * KS);
#pragma unroll
    for (int st = 0; st < KS / 4; ++st) {
      const f32x4 fa = *reinterpret_cast<const f32x4*>(&sA[buf][4 * st + q][64 * wm + 4 * c]);
      const f32x4 fb = *reinterpret_cast<const f32x4*>(&sB[buf][4 * st + q][64 * wn + 4 * c]);
#pragma unroll
      for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int y = 0; y < 4; ++y)
          acc[x][y] = __builtin_amdgcn_mfma_f32_16x16x4f32(fa[x], fb[y], acc[x][y], 0, 0, 0);
    }
    // buffer buf ^ 1 was last read in slab j - 1, before the previous barrier
    if (j + 1 < nslab) store(buf ^ 1);
    __syncthreads();
  }
  if (P != nullptr) {
    float* out = P + ((int64_t)z * g.batch + b) * g.M * g.N;
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
      for (int y = 0; y < 4; ++y)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int m = m0 + 64 * wm + 16 * x + 4 * q + i, n = n0 + 64 * wn + 16 * y + c;
          if (m < g.M && n < g.N) out[(int64_t)m * g.N + n] = acc[x][y][i];
        }
    return;
  }
  const float* D = g.D ? g.D + b * g.d_bs : nullptr;
  float* C = g.C + b * g.c_bs;
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int y = 0; y < 4; ++y)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = m0 + 64 * wm + 16 * x + 4 * q + i, n = n0 + 64 * wn + 16 * y + c;
        if (m < g.M && n < g.N) {
          float v = g.alpha * acc[x][y][i];
          if (D) v += g.beta * D[(int64_t)m * g.d_sm + n];
          C[(int64_t)m * g.c_sm + n] = v;
        }
      }
}

// Split-K epilogue: C = alpha * (sum over the splits in order of P) + beta D.
__global__ void k_bgemm_sum(BGemm g, const float* P, int nsplit) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t mn = (int64_t)g.M * g.N;
  if (i >= mn * g.batch) return;
  const int64_t b = i / mn, r = i % mn;
  const int m = (int)(r / g.N), n = (int)(r % g.N);
  float acc = 0.f;
  for (int z = 0; z < nsplit; ++z) acc += P[((int64_t)z * g.batch + b) * mn + r];
  float v = g.alpha * acc;
  if (g.D) v += g.beta * g.D[b * g.d_bs + (int64_t)m * g.d_sm + n];
  g.C[b * g.c_bs + (int64_t)m * g.c_sm + n] = v;
}

// Split count for a contraction: about two workgroups per CU over all
// tiles, each split at least 512 deep, at most `max_split` (the partial
// buffer's capacity in M x N x batch units).
static int bgemm_splits(const BGemm& g, int max_split) {
  const int64_t tiles = (int64_t)((g.M + 63) / 64) * ((g.N + 63) / 64) * g.batch;
  int ns = 1;
  while (ns < max_split && tiles * ns * 2 <= 512 && g.K / (2 * ns) >= 512) ns *= 2;
  return ns;
}

// 16-byte loads of an operand need its base, batch stride and the stride
// of its non-contiguous dimension to be multiples of 4 floats.
static bool vec_ok(const void* p, int bf, int64_t bs, int64_t s_row, int64_t s_k, bool kfast) {
  return !bf && ((uintptr_t)p & 15u) == 0 && bs % 4 == 0 && (kfast ? s_row : s_k) % 4 == 0;
}

// The 128 x 128 kernel for products with at least 128 rows and columns and
// enough tiles (after splitting K) to give every CU two workgroups (fewer
// leave CUs idle: the 64 x 64 kernel is then faster);
// its split count: the smallest power of two reaching 512 workgroups with
// slabs of at least 256, at most max_split.
static int bgemm128_splits(const BGemm& g, int max_split) {
  if (g.M < 128 || g.N < 128 || (g.a_sk != 1 && g.a_sm != 1) || (g.b_sn != 1 && g.b_sk != 1)) return 0;
  const int64_t tiles = (int64_t)((g.M + 127) / 128) * ((g.N + 127) / 128) * g.batch;
  int ns = 1;
  while (ns < max_split && tiles * ns < 512 && g.K / (2 * ns) >= 256) ns *= 2;
  return tiles * ns >= 512 ? ns : 0;
}

hipError_t launch_bgemm(const BGemm& g, hipStream_t s, float* partial, int64_t partial_floats) {
  if (g.M <= 0 || g.N <= 0 || g.batch <= 0) return hipSuccess;
  const int64_t mnb = (int64_t)g.M * g.N * g.batch;
  int cap = 1;
  if (partial != nullptr && mnb > 0) {
    const int64_t c = partial_floats / mnb;
    cap = (int)(c < 64 ? (c > 1 ? c : 1) : 64);
  }
  const int ns128 = bgemm128_splits(g, cap);
  int ns = ns128 > 0 ? ns128 : (cap > 1 ? bgemm_splits(g, cap) : 1);
  const int kchunk = ns > 1 ? ((g.K + ns - 1) / ns + 31) / 32 * 32 : (g.K > 0 ? g.K : 1);
  float* P = ns > 1 ? partial : nullptr;
  // 16-byte runs only along a unit stride
  const int va = vec_ok(g.A, g.a_bf16, g.a_bs, g.a_sm, g.a_sk, g.a_sk == 1) && (g.a_sk == 1 || g.a_sm == 1);
  const int vb = vec_ok(g.B, g.b_bf16, g.b_bs, g.b_sn, g.b_sk, g.b_sk == 1) && (g.b_sk == 1 || g.b_sn == 1);
  if (ns128 > 0) {
    const int ntile = ((g.M + 127) / 128) * ((g.N + 127) / 128);
    const dim3 grid((unsigned)((int64_t)ntile * g.batch * ns));
    if (g.a_bf16 && g.b_bf16) hipLaunchKernelGGL((k_bgemm128<true, true, 16>), grid, dim3(256), 0, s, g, kchunk, P, va, vb, ntile);
    else if (g.a_bf16) hipLaunchKernelGGL((k_bgemm128<true, false, 16>), grid, dim3(256), 0, s, g, kchunk, P, va, vb, ntile);
    else if (g.b_bf16) hipLaunchKernelGGL((k_bgemm128<false, true, 16>), grid, dim3(256), 0, s, g, kchunk, P, va, vb, ntile);
    else hipLaunchKernelGGL((k_bgemm128<false, false, 16>), grid, dim3(256), 0, s, g, kchunk, P, va, vb, ntile);
  } else {
    const dim3 grid((unsigned)(((g.M + 63) / 64) * ((g.N + 63) / 64)), (unsigned)g.batch, (unsigned)ns);
    if (g.a_bf16 && g.b_bf16) hipLaunchKernelGGL((k_bgemm<true, true>), grid, dim3(256), 0, s, g, kchunk, P);
    else if (g.a_bf16) hipLaunchKernelGGL((k_bgemm<true, false>), grid, dim3(256), 0, s, g, kchunk, P);
    else if (g.b_bf16) hipLaunchKernelGGL((k_bgemm<false, true>), grid, dim3(256), 0, s, g, kchunk, P);
    else hipLaunchKernelGGL((k_bgemm<false, false>), grid, dim3(256), 0, s, g, kchunk, P);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || ns == 1) return e;
  hipLaunchKernelGGL(k_bgemm_sum, dim3((unsigned)((mnb + 255) / 256)), dim3(256), 0, s, g, P, ns);
  return hipGetLastError();
}

// ------------------------------------------------------- elementwise ----
__device__ __forceinline__ float sig(float x) { return 1.0f / (1.0f + expf(-x)); }

// Read: from g = x W1^T, u = x W3^T, dh = dO W2 (each [n][dh] per head):
//   h = silu(g) u,  du = dh silu(g),  dg = dh u silu'(g)   (in place: g <- dg,
//   u <- du, dh <- h).
__global__ void k_bw_read(float* g, float* u, float* dh, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const float x = g[i], uu = u[i], d = dh[i];
  const float s = sig(x), sl = x * s, s1 = s * (1.f + x * (1.f - s));
  g[i] = d * uu * s1;
  u[i] = d * sl;
  dh[i] = sl * uu;
}

// Chunk gradient, forward: from g = k W1^T, u = k W3^T, e = v W2 and the
// per-token rates, the factors of the three token contractions:
// o1 = eta1 e u silu'(g), o3 = eta3 e silu(g), o2 = eta2 silu(g) u  (rows t
// of head b use eta[b * esbh + t0 + t]).
__global__ void k_bw_grad_fwd(const float* g, const float* u, const float* e, float* o1, float* o3,
                              float* o2, const float* e1, const float* e3, const float* e2, int64_t esbh,
                              int64_t t0, int n, int dh, int bh) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)bh * n * dh) return;
  const int64_t row = i / dh;
  const int t = (int)(row % n), b = (int)(row / n);
  const int64_t ei = (int64_t)b * esbh + t0 + t;
  const float x = g[i], uu = u[i], ee = e[i];
  const float s = sig(x), sl = x * s, s1 = s * (1.f + x * (1.f - s));
  o1[i] = e1[ei] * ee * uu * s1;
  o3[i] = e3[ei] * ee * sl;
  o2[i] = e2[ei] * sl * uu;
}

// Chunk gradient, backward.  In: g, u, e (forward products), p1 = k dG1^T,
// p3 = k dG3^T, p2 = v dG2 ([n][dh] per head).  Out (in place):
//   g  <- dg (cotangent of g),   u <- du,   e <- dE,
//   p1 <- eta1 b,  p3 <- eta3 a,  p2 <- eta2 h   (the scaled forward
//   factors that the dK / dV contractions need),
// and r1 = b p1, r3 = a p3, r2 = h p2, whose row sums (k_bw_rowsum) are
// the per-token rate gradients.
// With s = silu(g), s1 = silu'(g), s2 = silu''(g): h = s u, a = e s,
// b = e u s1; dh = eta2 p2, da = eta3 p3, db = eta1 p1.
__global__ void k_bw_grad_bwd(float* g, float* u, float* e, float* p1, float* p3, float* p2,
                              float* r1, float* r3, float* r2, const float* e1, const float* e3,
                              const float* e2, int64_t esbh, int64_t t0, int n, int dh, int bh) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)bh * n * dh) return;
  const int64_t row = i / dh;
  const int t = (int)(row % n), b = (int)(row / n);
  const int64_t ei = (int64_t)b * esbh + t0 + t;
  const float x = g[i], uu = u[i], ee = e[i];
  const float s = sig(x), sl = x * s, s1 = s * (1.f + x * (1.f - s));
  const float s2 = s * (1.f - s) * (2.f + x * (1.f - 2.f * s));
  const float h = sl * uu, a = ee * sl, bb = ee * uu * s1;
  const float q1 = p1[i], q3 = p3[i], q2 = p2[i];
  const float et1 = e1[ei], et3 = e3[ei], et2 = e2[ei];
  const float dh_ = et2 * q2, da = et3 * q3, db = et1 * q1;
  const float ds = dh_ * uu + da * ee;
  g[i] = ds * s1 + db * ee * uu * s2;
  u[i] = dh_ * sl + db * ee * s1;
  e[i] = da * sl + db * uu * s1;
  // the rate gradients' terms (summed over the row by k_bw_rowdot)
  r1[i] = bb * q1;
  r3[i] = a * q3;
  r2[i] = h * q2;
  p1[i] = et1 * bb;
  p3[i] = et3 * a;
  p2[i] = et2 * h;
}

// out[b * osbh + t0 + t] += sum_j x[(b n + t) dh + j], one wave per row, a
// fixed order (lane-strided 16-byte partial sums, then a butterfly; dh is a
// multiple of 64 and the rows are 16-byte aligned).
__global__ void k_bw_rowsum(const float* x, float* out, int64_t osbh, int64_t t0, int n, int dh,
                            int bh) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= (int64_t)bh * n) return;
  const f32x4* p = reinterpret_cast<const f32x4*>(x + row * dh);
  float s = 0.f;
  for (int j = lane; j < dh / 4; j += 64) {
    const f32x4 v = p[j];
    s += (v[0] + v[1]) + (v[2] + v[3]);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
  if (lane == 0) {
    const int t = (int)(row % n), b = (int)(row / n);
    out[(int64_t)b * osbh + t0 + t] += s;
  }
}

// ---------------------------------------------------- per-matrix sums ----
// out[m] = sum over the matrix m (size elements) of x[i] * y[i] (y NULL:
// x[i]^2), one workgroup of 1024 threads per matrix, fixed order: each
// thread sums its 16-byte vectors (VEC: size % 4 == 0, aligned operands) or
// elements, strided by the workgroup, then the 16 waves in index order.
template <bool VEC>
__global__ __launch_bounds__(1024) void k_bw_dot(const float* x, const float* y, float* out, int64_t size) {
  __shared__ float red[16];
  const float* px = x + (int64_t)blockIdx.x * size;
  const float* py = y ? y + (int64_t)blockIdx.x * size : px;
  float s = 0.f;
  if constexpr (VEC) {
    const f32x4* vx = reinterpret_cast<const f32x4*>(px);
    const f32x4* vy = reinterpret_cast<const f32x4*>(py);
#pragma unroll 4
    for (int64_t i = threadIdx.x; i < size / 4; i += 1024) {
      const f32x4 a = vx[i], b = vy[i];
      s += (a[0] * b[0] + a[1] * b[1]) + (a[2] * b[2] + a[3] * b[3]);
    }
  } else {
#pragma unroll 4
    for (int64_t i = threadIdx.x; i < size; i += 1024) s += px[i] * py[i];
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    float t = 0.f;
#pragma unroll
    for (int w = 0; w < 16; ++w) t += red[w];
    out[blockIdx.x] = t;
  }
}

// y[m] = alpha[m] x[m] + beta[m] z[m] over matrices of `size` elements, with
// per-matrix coefficients from arrays (NULL: the scalar a / b).
__global__ void k_bw_axpby(float* y, const float* x, const float* z, const float* am, float a,
                           const float* bm, float b, int64_t size, int64_t total) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= total) return;
  const int64_t m = i / size;
  const float ca = am ? am[m] : a, cb = bm ? bm[m] : b;
  float v = ca * x[i];
  if (z) v += cb * z[i];
  y[i] = v;
}

// Batched transpose: out[m][j][i] = in[m][i][j], in [rows][cols].
__global__ void k_bw_transpose(const float* in, float* out, int rows, int cols, int count) {
  __shared__ float t[32][33];
  const int m = blockIdx.z;
  const int i0 = blockIdx.y * 32, j0 = blockIdx.x * 32;
  const float* pi = in + (int64_t)m * rows * cols;
  float* po = out + (int64_t)m * rows * cols;
  for (int r = threadIdx.y; r < 32; r += 8) {
    const int i = i0 + r, j = j0 + threadIdx.x;
    if (i < rows && j < cols) t[r][threadIdx.x] = pi[(int64_t)i * cols + j];
  }
  __syncthreads();
  for (int r = threadIdx.y; r < 32; r += 8) {
    const int j = j0 + r, i = i0 + threadIdx.x;
    if (i < rows && j < cols) po[(int64_t)j * rows + i] = t[threadIdx.x][r];
  }
}

// out = A + A^T for square [n][n] matrices (batched).
__global__ void k_bw_symm(const float* a, float* out, int n, int count) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)count * n * n) return;
  const int64_t m = i / ((int64_t)n * n);
  const int r = (int)((i / n) % n), c = (int)(i % n);
  const float* p = a + m * n * n;
  out[i] = p[(int64_t)r * n + c] + p[(int64_t)c * n + r];
}

// ------------------------------------------------------ step + renorm ----
// Rows of length L: W <- (W + U) rescaled to n0 / (||W + U|| + eps) (renorm)
// or W + U; one wave per row.
__global__ void k_bw_step(float* w, const float* u, const float* n0, int64_t rows, int L, int renorm,
                          float eps) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  float* pw = w + row * L;
  const float* pu = u + row * L;
  float ss = 0.f;
  for (int j = lane; j < L; j += 64) {
    const float r = pw[j] + pu[j];
    ss += r * r;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
  const float f = renorm ? n0[row] / (sqrtf(ss) + eps) : 1.f;
  for (int j = lane; j < L; j += 64) pw[j] = (pw[j] + pu[j]) * f;
}

// Row norms: n[row] = ||w[row]||.
__global__ void k_bw_rownorm(const float* w, float* n, int64_t rows, int L) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  float ss = 0.f;
  for (int j = lane; j < L; j += 64) ss += w[row * L + j] * w[row * L + j];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
  if (lane == 0) n[row] = sqrtf(ss);
}

// VJP of the step + renorm row by row.  R = W + U (W, U given), dWn the
// cotangent of the new row:  dR = f dWn - n0 / (r + eps)^2 / r (dWn . R) R,
// f = n0 / (r + eps);  dn0 += (dWn . R) / (r + eps).  Without renorm dR =
// dWn.  dR is written to dr (the cotangent of both W and U).
__global__ void k_bw_step_vjp(const float* w, const float* u, const float* n0, const float* dwn,
                              float* dr, float* dn0, int64_t rows, int L, int renorm, float eps) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  const float* pw = w + row * L;
  const float* pu = u + row * L;
  const float* pd = dwn + row * L;
  float* po = dr + row * L;
  if (!renorm) {
    for (int j = lane; j < L; j += 64) po[j] = pd[j];
    return;
  }
  float ss = 0.f, pr = 0.f;
  for (int j = lane; j < L; j += 64) {
    const float r = pw[j] + pu[j];
    ss += r * r;
    pr += pd[j] * r;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    ss += __shfl_xor(ss, o);
    pr += __shfl_xor(pr, o);
  }
  const float r = sqrtf(ss), re = r + eps, nn = n0[row];
  const float f = nn / re;
  const float k = r > 0.f ? nn / (re * re) / r * pr : 0.f;
  for (int j = lane; j < L; j += 64) po[j] = f * pd[j] - k * (pw[j] + pu[j]);
  if (lane == 0) dn0[row] += pr / re;
}

// dW0 = dW + (dn0 / ||row of W0||) W0, rows of length L.
__global__ void k_bw_w0(const float* w0, const float* dw, const float* dn0, float* out, int64_t rows,
                        int L) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  float ss = 0.f;
  for (int j = lane; j < L; j += 64) ss += w0[row * L + j] * w0[row * L + j];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
  const float r = sqrtf(ss);
  const float k = r > 0.f ? dn0[row] / r : 0.f;
  for (int j = lane; j < L; j += 64) out[row * L + j] = dw[row * L + j] + k * w0[row * L + j];
}

// Momentum coefficient per head: beta[b] = mean of mom[b * sbh + t0 ..
// t0 + n) (0 when n = 0); one wave per head.
__global__ void k_bw_beta(const float* mom, int64_t sbh, int64_t t0, int n, float* beta, int bh) {
  const int b = blockIdx.x;
  const int lane = threadIdx.x;
  float s = 0.f;
  for (int t = lane; t < n; t += 64) s += mom[(int64_t)b * sbh + t0 + t];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
  if (lane == 0) beta[b] = n > 0 ? s / (float)n : 0.f;
}

// dmom[b * sbh + t0 + t] += (dbeta[b] + dbeta[bh + b] + dbeta[2 bh + b]) / n
// (the three matrices' momentum dots of head b, in that order).
__global__ void k_bw_dmom(const float* dbeta, float* dmom, int64_t sbh, int64_t t0, int n, int bh) {
  const int b = blockIdx.y;
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= n) return;
  const float db = (dbeta[b] + dbeta[bh + b]) + dbeta[2 * bh + b];
  dmom[(int64_t)b * sbh + t0 + t] += db / (float)n;
}

// Activations to fp32 (rows of d of a [bh][T][*] array with the layout's
// strides): out[(b n + t) d + i] = x[b sbh + (t0 + t) st + i].
// Four consecutive features per thread (d % 4 == 0; the token rows 8-byte
// (bf16) or 16-byte (fp32) aligned): one load, one 16-byte store.
template <bool BF>
__global__ void k_bw_gather4(const void* x, int64_t sbh, int64_t st, int64_t t0, int n, int d4, int bh,
                             float* out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)bh * n * d4) return;
  const int64_t row = i / d4;
  const int c = 4 * (int)(i - row * d4);
  const int t = (int)(row % n), b = (int)(row / n);
  const int64_t src = (int64_t)b * sbh + (t0 + t) * st + c;
  f32x4 v;
  if constexpr (BF) {
    const bf16x4 h = *reinterpret_cast<const bf16x4*>(reinterpret_cast<const bf16*>(x) + src);
    v = f32x4{(float)h[0], (float)h[1], (float)h[2], (float)h[3]};
  } else {
    v = *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(x) + src);
  }
  *reinterpret_cast<f32x4*>(out + 4 * i) = v;
}
__global__ void k_bw_gather(const void* x, int bf, int64_t sbh, int64_t st, int64_t t0, int n, int d,
                            int bh, float* out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)bh * n * d) return;
  const int64_t row = i / d;
  const int t = (int)(row % n), b = (int)(row / n), c = (int)(i % d);
  out[i] = ldx(x, (int64_t)b * sbh + (t0 + t) * st + c, bf);
}

// out[b sbh + (t0 + t) st + i] += x[(b n + t) d + i]
__global__ void k_bw_scatter_add4(const float* x, int64_t sbh, int64_t st, int64_t t0, int n, int d4,
                                  int bh, float* out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)bh * n * d4) return;
  const int64_t row = i / d4;
  const int c = 4 * (int)(i - row * d4);
  const int t = (int)(row % n), b = (int)(row / n);
  f32x4* o = reinterpret_cast<f32x4*>(out + (int64_t)b * sbh + (t0 + t) * st + c);
  const f32x4 a = *reinterpret_cast<const f32x4*>(x + 4 * i);
  f32x4 v = *o;
  v[0] += a[0]; v[1] += a[1]; v[2] += a[2]; v[3] += a[3];
  *o = v;
}
__global__ void k_bw_scatter_add(const float* x, int64_t sbh, int64_t st, int64_t t0, int n, int d,
                                 int bh, float* out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)bh * n * d) return;
  const int64_t row = i / d;
  const int t = (int)(row % n), b = (int)(row / n), c = (int)(i % d);
  out[(int64_t)b * sbh + (t0 + t) * st + c] += x[i];
}

// p[0 .. n) = v
__global__ void k_bw_fill(float* p, float v, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

// Frobenius normalisation of Newton-Schulz and its VJP, per matrix m with
// sum of squares ss[m]: c1[m] = 1 / (r + eps), r = sqrt(ss[m]); with dot
// (= sum dX * G): c2[m] = -dot[m] / ((r + eps)^2 r) (0 when r = 0), so that
// dG = c1 dX + c2 G.
__global__ void k_bw_nscoef(const float* ss, const float* dot, float* c1, float* c2, int count, float eps) {
  const int m = blockIdx.x * blockDim.x + threadIdx.x;
  if (m >= count) return;
  const float r = sqrtf(ss[m]), re = r + eps;
  c1[m] = 1.0f / re;
  if (dot != nullptr) c2[m] = r > 0.f ? -dot[m] / (re * re * r) : 0.f;
}

// ------------------------------------------------------------ launches ----
hipError_t bw_fill(float* p, float v, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_bw_fill, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, v, n);
  return hipGetLastError();
}
hipError_t bw_nscoef(const float* ss, const float* dot, float* c1, float* c2, int count, float eps,
                     hipStream_t s) {
  if (count <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_bw_nscoef, dim3((unsigned)((count + 63) / 64)), dim3(64), 0, s, ss, dot, c1, c2, count,
                     eps);
  return hipGetLastError();
}
static dim3 g1(int64_t n, int tpb = 256) { return dim3((unsigned)((n + tpb - 1) / tpb)); }
static dim3 grows(int64_t rows) { return dim3((unsigned)((rows + 3) / 4)); }

hipError_t bw_read(float* g, float* u, float* dh, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_bw_read, g1(n), dim3(256), 0, s, g, u, dh, n);
  return hipGetLastError();
}
hipError_t bw_grad_fwd(const float* g, const float* u, const float* e, float* o1, float* o3, float* o2,
                       const float* e1, const float* e3, const float* e2, int64_t esbh, int64_t t0, int n,
                       int dh, int bh, hipStream_t s) {
  const int64_t tot = (int64_t)bh * n * dh;
  if (tot <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_bw_grad_fwd, g1(tot), dim3(256), 0, s, g, u, e, o1, o3, o2, e1, e3, e2, esbh, t0, n,
                     dh, bh);
  return hipGetLastError();
}
hipError_t bw_grad_bwd(float* g, float* u, float* e, float* p1, float* p3, float* p2, float* r1, float* r3,
                       float* r2, const float* e1, const float* e3, const float* e2, int64_t esbh,
                       int64_t t0, int n, int dh, int bh, hipStream_t s) {
  const int64_t tot = (int64_t)bh * n * dh;
  if (tot <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_bw_grad_bwd, g1(tot), dim3(256), 0, s, g, u, e, p1, p3, p2, r1, r3, r2, e1, e3, e2,
                     esbh, t0, n, dh, bh);
  return hipGetLastError();
}
hipError_t bw_rowsum(const float* x, float* out, int64_t osbh, int64_t t0, int n, int dh, int bh,
                     hipStream_t s) {
  const int64_t rows = (int64_t)bh * n;
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_bw_rowsum, grows(rows), dim3(256), 0, s, x, out, osbh, t0, n, dh, bh);
  return hipGetLastError();
}
static bool al16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
hipError_t bw_dot(const float* x, const float* y, float* out, int64_t size, int count, hipStream_t s) {
  if (count <= 0) return hipSuccess;
  if (size % 4 == 0 && al16(x) && (y == nullptr || al16(y)))
    hipLaunchKernelGGL(k_bw_dot<true>, dim3((unsigned)count), dim3(1024), 0, s, x, y, out, size);
  else
    hipLaunchKernelGGL(k_bw_dot<false>, dim3((unsigned)count), dim3(1024), 0, s, x, y, out, size);
  return hipGetLastError();
}
hipError_t bw_axpby(float* y, const float* x, const float* z, const float* am, float a, const float* bm,
                    float b, int64_t size, int count, hipStream_t s) {
  const int64_t tot = size * count;
  if (tot <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_bw_axpby, g1(tot), dim3(256), 0, s, y, x, z, am, a, bm, b, size, tot);
  return hipGetLastError();
}
hipError_t bw_transpose(const float* in, float* out, int rows, int cols, int count, hipStream_t s) {
  if (count <= 0) return hipSuccess;
  const dim3 grid((unsigned)((cols + 31) / 32), (unsigned)((rows + 31) / 32), (unsigned)count);
  hipLaunchKernelGGL(k_bw_transpose, grid, dim3(32, 8), 0, s, in, out, rows, cols, count);
  return hipGetLastError();
}
hipError_t bw_symm(const float* a, float* out, int n, int count, hipStream_t s) {
  const int64_t tot = (int64_t)count * n * n;
  if (tot <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_bw_symm, g1(tot), dim3(256), 0, s, a, out, n, count);
  return hipGetLastError();
}
hipError_t bw_step(float* w, const float* u, const float* n0, int64_t rows, int L, int renorm, float eps,
                   hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_bw_step, grows(rows), dim3(256), 0, s, w, u, n0, rows, L, renorm, eps);
  return hipGetLastError();
}
hipError_t bw_rownorm(const float* w, float* n, int64_t rows, int L, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_bw_rownorm, grows(rows), dim3(256), 0, s, w, n, rows, L);
  return hipGetLastError();
}
hipError_t bw_step_vjp(const float* w, const float* u, const float* n0, const float* dwn, float* dr,
                       float* dn0, int64_t rows, int L, int renorm, float eps, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_bw_step_vjp, grows(rows), dim3(256), 0, s, w, u, n0, dwn, dr, dn0, rows, L, renorm,
                     eps);
  return hipGetLastError();
}
hipError_t bw_w0(const float* w0, const float* dw, const float* dn0, float* out, int64_t rows, int L,
                 hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_bw_w0, grows(rows), dim3(256), 0, s, w0, dw, dn0, out, rows, L);
  return hipGetLastError();
}
hipError_t bw_beta(const float* mom, int64_t sbh, int64_t t0, int n, float* beta, int bh, hipStream_t s) {
  if (bh <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_bw_beta, dim3((unsigned)bh), dim3(64), 0, s, mom, sbh, t0, n, beta, bh);
  return hipGetLastError();
}
hipError_t bw_dmom(const float* dbeta, float* dmom, int64_t sbh, int64_t t0, int n, int bh, hipStream_t s) {
  if (n <= 0 || bh <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_bw_dmom, dim3((unsigned)((n + 255) / 256), (unsigned)bh), dim3(256), 0, s, dbeta,
                     dmom, sbh, t0, n, bh);
  return hipGetLastError();
}
hipError_t bw_gather(const void* x, int bf, int64_t sbh, int64_t st, int64_t t0, int n, int d, int bh,
                     float* out, hipStream_t s) {
  const int64_t tot = (int64_t)bh * n * d;
  if (tot <= 0) return hipSuccess;
  // runs of 4 features as one load each when every run is aligned
  if (d % 4 == 0 && sbh % 4 == 0 && st % 4 == 0 && ((uintptr_t)x & (bf ? 7u : 15u)) == 0 && al16(out)) {
    const int64_t nv = tot / 4;
    if (bf)
      hipLaunchKernelGGL(k_bw_gather4<true>, g1(nv), dim3(256), 0, s, x, sbh, st, t0, n, d / 4, bh, out);
    else
      hipLaunchKernelGGL(k_bw_gather4<false>, g1(nv), dim3(256), 0, s, x, sbh, st, t0, n, d / 4, bh, out);
  } else {
    hipLaunchKernelGGL(k_bw_gather, g1(tot), dim3(256), 0, s, x, bf, sbh, st, t0, n, d, bh, out);
  }
  return hipGetLastError();
}
hipError_t bw_scatter_add(const float* x, int64_t sbh, int64_t st, int64_t t0, int n, int d, int bh,
                          float* out, hipStream_t s) {
  const int64_t tot = (int64_t)bh * n * d;
  if (tot <= 0) return hipSuccess;
  if (d % 4 == 0 && sbh % 4 == 0 && st % 4 == 0 && al16(out) && al16(x))
    hipLaunchKernelGGL(k_bw_scatter_add4, g1(tot / 4), dim3(256), 0, s, x, sbh, st, t0, n, d / 4, bh, out);
  else
    hipLaunchKernelGGL(k_bw_scatter_add, g1(tot), dim3(256), 0, s, x, sbh, st, t0, n, d, bh, out);
  return hipGetLastError();
}

}  // namespace lact
