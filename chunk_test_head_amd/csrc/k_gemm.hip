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

// ---------------------------------------------------------------------------
// bf16 path for matrices too large for one workgroup (d = 256): the iterate
// X stays fp32 in global memory (for the exact a X term) and a bf16 copy is
// the MFMA operand of the next products.
//
//   C = alpha A B + beta' D + diag' I, A bf16 [M][K] (row pitch lda), B bf16 [N][K]
//   (BKN = false, pitch ldb) or [K][N] (BKN = true); D fp32 [M][N]; outputs
//   fp32 C and / or bf16 Ch, [M][N].
// One workgroup = one 64 x 64 tile, 4 waves of 32 x 32; K in slabs of 64,
// double buffered through LDS (rows padded by 16 elements: conflict-free
// fragment and transpose reads); with BKN the B fragments (K per lane) are
// transpose reads of the [k][n] tile.  The result tile goes through LDS so
// that D, C and Ch move as whole 16-byte row pieces.  beta' and diag' take
// the step's shift mu into account (NsGemmArgs), and the launch can leave the
// sum of squares of every result tile for the next step's mu.  The loop is
// bound by the latency of the slabs' loads (a slab is only 8 MFMAs per
// wave), so four slabs are in flight in registers ahead of the LDS stores,
// and the epilogue's D tile is loaded before the loop; the small slabs keep
// the LDS at 40 KiB.
namespace {
constexpr int NSG_T = 64, NSG_K = 64;
constexpr int NSG_PA = NSG_K + 16;                    // [m][k] / [n][k] tiles
constexpr int NSG_PB = NSG_T + 16;                    // [k][n] tile
constexpr int NSG_VA = NSG_T * NSG_K / 8 / 256;       // 16-byte vectors per thread and operand
constexpr int NSG_RA = NSG_K / 8;                     // vectors per [m][k] row
constexpr int NSG_SA = NSG_T * NSG_PA;                // elements per A stage
constexpr int NSG_SB = NSG_T * NSG_PA > NSG_K * NSG_PB ? NSG_T * NSG_PA : NSG_K * NSG_PB;
constexpr int NSG_PC = NSG_T + 4;                     // fp32 result tile pitch
constexpr int NSG_PD = 4;                             // K slabs in flight
// slab j sits in register slot j % NSG_PD and LDS buffer slot % 2: with an
// even slot count the two buffers alternate from slab to slab
static_assert(NSG_PD % 2 == 0, "the LDS buffers alternate by slot parity");
}

template <bool BKN>
__global__ __launch_bounds__(256) void k_nsgemm(NsGemmArgs a) {
  __shared__ __attribute__((aligned(16))) bf16 lds_g[2 * NSG_SA + 2 * NSG_SB];
  static_assert(NSG_T * NSG_PC * 4 <= (2 * NSG_SA + 2 * NSG_SB) * 2, "result tile");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = lane & 15, g = lane >> 4;
  const int wm = wave >> 1, wn = wave & 1;
  const int tn = a.N / NSG_T;
  // one launch-wide id per (matrix, tile), dealt so that the tiles of a
  // matrix run on one or two XCDs and share their L2's copy of the operands;
  // a symmetric product has tn (tn + 1) / 2 tiles (tm <= tn) per matrix
  const int ntile = a.sym ? tn * (tn + 1) / 2 : (a.M / NSG_T) * tn;
  const int lid = xcd_logical_id(blockIdx.x, gridDim.x);
  const int tile = lid % ntile;
  int tmi = tile / tn, tni = tile % tn;
  if (a.sym) {
    // row tm holds tiles tm .. tn - 1: walk the rows
    int t = tile;
    tmi = 0;
    while (t >= tn - tmi) t -= tn - tmi++;
    tni = tmi + t;
  }
  const int m0 = tmi * NSG_T, n0 = tni * NSG_T;
  const bool mirror = a.sym && tmi != tni;
  const int64_t bidx = lid / ntile;
  const bf16* A = a.A + bidx * a.a_bs;
  const bf16* B = a.B + bidx * a.b_bs;

  // staging: 16-byte vectors vi = tid + 256 x; A: row vi / 16, chunk vi % 16
  // ([m][k]); B: [n][k] likewise, or ([k][n]) row vi / 8, chunk vi % 8.
  // NSG_PD slabs are in flight in registers (the loop is bound by load
  // latency, not by the few MFMAs per slab): slab j sits in slot j % NSG_PD
  // until it is stored to LDS buffer j % 2, and its slot is then refilled
  // with slab j + NSG_PD.
  constexpr int PD = NSG_PD;
  bf16x8 ra[PD][NSG_VA], rb[PD][NSG_VA];
  const int nslab = a.K / NSG_K;  // (K is a multiple of 64)
#define LACT_NSG_GLOAD(P, K0)                                                                \
  {                                                                                          \
    _Pragma("unroll") for (int x = 0; x < NSG_VA; ++x) {                                     \
      const int vi = tid + 256 * x;                                                          \
      const int ka = (K0) + 8 * (vi % NSG_RA), kb = BKN ? (K0) + (vi >> 3) : ka;             \
      ra[P][x] = ld8(A + (int64_t)(m0 + vi / NSG_RA) * a.lda + ka);                           \
      rb[P][x] = BKN ? ld8(B + (int64_t)kb * a.ldb + n0 + 8 * (vi & 7))                        \
                     : ld8(B + (int64_t)(n0 + vi / NSG_RA) * a.ldb + kb);                      \
    }                                                                                        \
  }
#define LACT_NSG_LSTORE(P, BUF)                                                              \
  {                                                                                          \
    bf16* sa_ = lds_g + (BUF) * NSG_SA;                                                      \
    bf16* sb_ = lds_g + 2 * NSG_SA + (BUF) * NSG_SB;                                         \
    _Pragma("unroll") for (int x = 0; x < NSG_VA; ++x) {                                     \
      const int vi = tid + 256 * x;                                                          \
      *reinterpret_cast<bf16x8*>(sa_ + (vi / NSG_RA) * NSG_PA + 8 * (vi % NSG_RA)) = ra[P][x]; \
      if (BKN) *reinterpret_cast<bf16x8*>(sb_ + (vi >> 3) * NSG_PB + 8 * (vi & 7)) = rb[P][x]; \
      else *reinterpret_cast<bf16x8*>(sb_ + (vi / NSG_RA) * NSG_PA + 8 * (vi % NSG_RA)) = rb[P][x]; \
    }                                                                                        \
  }
  // the epilogue's own loads go out first: the D tile and the shift's partials
  const float* D = a.D ? a.D + bidx * a.d_bs : nullptr;
  f32x4 dv[4], dt[4];
  if (D) {
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const int vi = tid + 256 * x, r = vi >> 4, c4 = 4 * (vi & 15);
      dv[x] = *reinterpret_cast<const f32x4*>(D + (int64_t)(m0 + r) * a.N + n0 + c4);
      if (mirror) dt[x] = *reinterpret_cast<const f32x4*>(D + (int64_t)(n0 + r) * a.N + m0 + c4);
    }
  }
  float mu_t = 0.f;
  if (a.mu_part != nullptr) {
    const float* mp = a.mu_part + bidx * a.mu_np;
    for (int q = lane; q < a.mu_np; q += 64) mu_t += mp[q];
  }
  f32x4 acc[2][2];
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y) acc[x][y] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int p = 0; p < PD; ++p)
    if (p < nslab) LACT_NSG_GLOAD(p, p * NSG_K);
  for (int j0 = 0; j0 < nslab; j0 += PD) {
#pragma unroll
    for (int p = 0; p < PD; ++p) {
      const int j = j0 + p;
      if (j < nslab) {
        // one barrier per slab: every thread is past its reads of buffer
        // p % 2 from slab j - 2 (done before its store of slab j - 1)
        LACT_NSG_LSTORE(p, p & 1);
        __syncthreads();
        if (j + PD < nslab) LACT_NSG_GLOAD(p, (j + PD) * NSG_K);
        const bf16* sa = lds_g + (p & 1) * NSG_SA;
        const bf16* sb = lds_g + 2 * NSG_SA + (p & 1) * NSG_SB;
#pragma unroll
        for (int s = 0; s < NSG_K / 32; ++s) {
          bf16x8 fa[2], fb[2];
#pragma unroll
          for (int x = 0; x < 2; ++x) fa[x] = ld8(sa + (32 * wm + 16 * x + c) * NSG_PA + 32 * s + 8 * g);
#pragma unroll
          for (int y = 0; y < 2; ++y) {
            if constexpr (BKN) {
              const bf16* q = sb + (32 * s + 8 * g + (c >> 2)) * NSG_PB + 32 * wn + 16 * y + 4 * (c & 3);
              fb[y] = cat8(ld_tr4(q), ld_tr4(q + 4 * NSG_PB));
            } else {
              fb[y] = ld8(sb + (32 * wn + 16 * y + c) * NSG_PA + 32 * s + 8 * g);
            }
          }
#pragma unroll
          for (int x = 0; x < 2; ++x)
#pragma unroll
            for (int y = 0; y < 2; ++y) mma(acc[x][y], fa[x], fb[y]);
        }
      }
    }
  }
#undef LACT_NSG_GLOAD
#undef LACT_NSG_LSTORE
  __syncthreads();  // every read of the operand tiles is done
  // result tile through LDS
  float* sc = reinterpret_cast<float*>(lds_g);
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        sc[(32 * wm + 16 * x + 4 * g + i) * NSG_PC + 32 * wn + 16 * y + c] = acc[x][y][i];
  __syncthreads();
  float* C = a.C ? a.C + bidx * a.c_bs : nullptr;
  bf16* Ch = a.Ch ? a.Ch + bidx * a.c_bs : nullptr;
  // shift of this step (the same mu in every workgroup of the matrix: the
  // partial sums are added in a fixed order)
  float mu = 0.f;
  if (a.mu_part != nullptr) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) mu_t += __shfl_xor(mu_t, o);
    mu = mu_t / a.mu_div;
  }
  const float be = a.beta + (a.beta_mu + a.beta_mu2 * mu) * mu;
  const float dg = a.diag_mu * mu;
  float ss = 0.f;
  f32x4 ctv[4];  // (c_tall: the tile's values, written transposed below)
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    const int vi = tid + 256 * x, r = vi >> 4, c4 = 4 * (vi & 15);
    const int64_t o = (int64_t)(m0 + r) * a.N + n0 + c4;
    f32x4 v = *reinterpret_cast<const f32x4*>(sc + r * NSG_PC + c4) * a.alpha;
    if (D) v += dv[x] * be;
    if (dg != 0.f) {
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] += (m0 + r == n0 + c4 + j) ? dg : 0.f;
    }
    ss += v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3];
    if ((int)bidx < a.c_tall) ctv[x] = v;
    else if (C) *reinterpret_cast<f32x4*>(C + o) = v;
    if (Ch) st4(Ch + o, v[0], v[1], v[2], v[3]);
  }
  if ((int)bidx < a.c_tall) {
    // C transposed: the finished tile back into LDS, then its columns out as
    // rows of C^T (16-byte pieces of row n0 + r)
    __syncthreads();  // every read of the result tile done
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const int vi = tid + 256 * x, r = vi >> 4, c4 = 4 * (vi & 15);
      *reinterpret_cast<f32x4*>(sc + r * NSG_PC + c4) = ctv[x];
    }
    __syncthreads();
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const int vi = tid + 256 * x, r = vi >> 4, c4 = 4 * (vi & 15);
      f32x4 v;
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = sc[(c4 + j) * NSG_PC + r];
      *reinterpret_cast<f32x4*>(C + (int64_t)(n0 + r) * a.M + m0 + c4) = v;
    }
  }
  if (mirror) {
    // the transposed tile at (tn, tm): row r of it is column r of the result
    // tile (off the diagonal: no diagonal term)
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const int vi = tid + 256 * x, r = vi >> 4, c4 = 4 * (vi & 15);
      const int64_t o = (int64_t)(n0 + r) * a.N + m0 + c4;
      f32x4 v;
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = sc[(c4 + j) * NSG_PC + r] * a.alpha;
      if (D) v += dt[x] * be;
      if (C) *reinterpret_cast<f32x4*>(C + o) = v;
      if (Ch) st4(Ch + o, v[0], v[1], v[2], v[3]);
    }
  }
  if (a.ss_part != nullptr) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
    __syncthreads();  // every read of the result tile done
    if (lane == 0) sc[wave] = ss;
    __syncthreads();
    if (tid == 0)
      a.ss_part[bidx * ntile + tile] = (sc[0] + sc[1]) + (sc[2] + sc[3]);
  }
}

hipError_t launch_nsgemm(bool b_kn, const NsGemmArgs& a, int batch, hipStream_t s) {
  const int tm = a.M / NSG_T, tn = a.N / NSG_T;
  if (a.sym && (a.M != a.N || a.ss_part != nullptr)) return hipErrorInvalidValue;
  if (a.c_tall > 0 && (a.sym || a.Ch != nullptr || a.ss_part != nullptr || a.C == nullptr))
    return hipErrorInvalidValue;
  const dim3 grid((unsigned)((a.sym ? tn * (tn + 1) / 2 : tm * tn) * batch));
  if (b_kn)
    hipLaunchKernelGGL(k_nsgemm<true>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(k_nsgemm<false>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

// Frobenius normalisation in two deterministic passes over NSN_B blocks per
// matrix: partial sums of squares, then X = G / (||G|| + eps) as fp32 and bf16.
namespace {
constexpr int NSN_B = 32;
}

__global__ __launch_bounds__(256) void k_nsn_part(NsIn g, float* part, int64_t n) {
  __shared__ float red[4];
  const int tid = threadIdx.x;
  const int64_t per = n / NSN_B;
  const float* p = g.at(blockIdx.y, n) + (int64_t)blockIdx.x * per;
  float s = 0.f;
  // unrolled so that the loads are in flight together (the sum keeps its order)
#pragma unroll 8
  for (int64_t e = 4 * tid; e < per; e += 1024) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(p + e);
    s += v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3];
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
  if ((tid & 63) == 0) red[tid >> 6] = s;
  __syncthreads();
  if (tid == 0) part[blockIdx.y * NSN_B + blockIdx.x] = (red[0] + red[1]) + (red[2] + red[3]);
}

__global__ __launch_bounds__(256) void k_nsn_scale(NsIn g, const float* part, int np, float* x,
                                                   bf16* xh, int64_t n, float eps) {
  const int tid = threadIdx.x;
  float tot = 0.f;
  for (int b = 0; b < np; ++b) tot += part[blockIdx.y * np + b];
  const float scale = 1.0f / (sqrtf(tot) + eps);
  const int64_t per = n / NSN_B;
  const int64_t base = (int64_t)blockIdx.y * n + (int64_t)blockIdx.x * per;
  const float* gp = g.at(blockIdx.y, n) + (int64_t)blockIdx.x * per;
#pragma unroll 8
  for (int64_t e = 4 * tid; e < per; e += 1024) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(gp + e) * scale;
    *reinterpret_cast<f32x4*>(x + base + e) = v;
    st4(xh + base + e, v[0], v[1], v[2], v[3]);
  }
}

hipError_t launch_nsn(NsIn g, float* part, float* x, bf16* xh, int count, int64_t n, float eps,
                      hipStream_t s, int pre_np) {
  if (n % (4 * NSN_B) != 0) return hipErrorInvalidValue;
  const dim3 grid(NSN_B, (unsigned)count);
  if (pre_np <= 0) {
    hipLaunchKernelGGL(k_nsn_part, grid, dim3(256), 0, s, g, part, n);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(k_nsn_scale, grid, dim3(256), 0, s, g, part, pre_np > 0 ? pre_np : NSN_B, x, xh, n,
                     eps);
  return hipGetLastError();
}

}  // namespace lact
