// Fused Newton-Schulz-5 (LaCT rebuttal page, zeropower_via_newtonschulz5;
// summary page section 3.2, Eq. 9-10) for matrices that fit one CU:
// one workgroup of 16 waves per matrix X [ROWS][COLS] (wide orientation),
// all five quintic steps in one launch.
//
//   X = G / (||G||_F + eps);  5 x { A = X X^T; B = b A + c A A; X = a X + B X }
//
// Each wave owns COLS/NW columns of X for the whole iteration, held in fp32
// registers in the MFMA accumulator layout; products take bf16 operands and
// accumulate in fp32 (X itself stays fp32: rounding it to bf16 between steps
// loses the small singular directions that the iteration amplifies).  Per
// step:
//   1. X is written to LDS column-major (8-byte stores straight from the
//      accumulator layout); A = X X^T, each wave one block of A, with the
//      row fragments of X read by LDS transpose reads.
//   2. A goes to LDS (bf16); A A is formed the same way; B = b A + c A A,
//      B goes to LDS (bf16).  A and B are symmetric, so each wave stores the
//      transpose of its tiles, again as 8-byte stores.
//   3. each wave computes its columns of B X from bf16 fragments of its own
//      X (B operand, K = rows) and rows of B from LDS; X = a X + B X in fp32.
#include "lact_internal.hpp"
#include "mfma.hpp"

namespace lact {

static __constant__ float kNsCoef[5][3] = {
    {4.0848f, -6.8946f, 2.9270f}, {3.9505f, -6.3029f, 2.6377f}, {3.7418f, -5.5913f, 2.3037f},
    {2.8769f, -3.1427f, 1.2046f}, {2.8366f, -3.0525f, 1.2012f}};

// LDS elements: column-major X, or A and B side by side (they alias X).
constexpr int ns_lds_elems(int rows, int cols) {
  return cols * (rows + 8) > 2 * rows * (rows + 8) ? cols * (rows + 8) : 2 * rows * (rows + 8);
}

// XG: keep the fp32 iterate in the output buffer (each wave reads and writes
// only its own columns, L2-resident) instead of in registers, for shapes
// whose register copy would not fit.
template <int ROWS, int COLS, int NW, bool XG>
__global__ __launch_bounds__(NW * 64) void k_ns_fused(const float* g, float* u, float eps) {
  constexpr int NRT = ROWS / 16;          // row tiles of X
  constexpr int CW = COLS / NW;           // columns per wave
  constexpr int NCT = CW / 16;            // column tiles per wave
  constexpr int NKS = ROWS / 32;          // K slabs over rows (B X)
  constexpr int PX = ROWS + 8;            // LDS pitch of column-major X (bf16)
  constexpr int PA = ROWS + 8;            // LDS pitch of A / B (bf16)
  constexpr int WN = NW / 4;              // waves over A: 4 x WN
  constexpr int BMS = ROWS / 4, BNS = ROWS / WN;  // A block per wave
  constexpr int BTM = BMS / 16, BTN = BNS / 16;
  static_assert(CW % 16 == 0 && ROWS % 32 == 0, "shape");
  static_assert(ns_lds_elems(ROWS, COLS) * 2 <= 160 * 1024, "lds");

  // LDS: sX = COLS x PX column-major X; sA, sB = ROWS x PA each (alias sX)
  extern __shared__ __attribute__((aligned(16))) bf16 lds_ns[];
  __shared__ float red[NW];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int c = lane & 15, gq = lane >> 4;
  const int col0 = w * CW;
  const float* G = g + (int64_t)blockIdx.x * ROWS * COLS;
  float* Uo = u + (int64_t)blockIdx.x * ROWS * COLS;

  // ---- Frobenius norm (fixed order), then this wave's columns (C layout) ----
  float ss = 0.f;
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float v = G[(int64_t)(16 * rt + 4 * gq + i) * COLS + col0 + 16 * ct + c];
        ss += v * v;
      }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
  if (lane == 0) red[w] = ss;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int x = 0; x < NW; ++x) tot += red[x];
  const float scale = 1.0f / (sqrtf(tot) + eps);

  // X in the accumulator layout: xv[rt][ct][i] = X[16 rt + 4 g + i][col0 + 16 ct + c]
  // (XG: the same values live in Uo and xv is only a staging copy)
  f32x4 xv[NRT][NCT];
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        xv[rt][ct][i] = G[(int64_t)(16 * rt + 4 * gq + i) * COLS + col0 + 16 * ct + c] * scale;
  if constexpr (XG) {
    __syncthreads();  // every read of G (possibly == Uo) is done
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          Uo[(int64_t)(16 * rt + 4 * gq + i) * COLS + col0 + 16 * ct + c] = xv[rt][ct][i];
  }
  float* Xg = Uo + (int64_t)(4 * gq) * COLS + col0 + c;  // lane base of its X elements

  const int bm = w / WN, bn = w % WN;  // A block of this wave
  auto step = [&](const int it, const bool last) {
    // Per-lane LDS bases, re-derived every step so the compiler does not keep
    // one address register per access alive across the iteration loop.
    int lb = 0;
    asm volatile("" : "+v"(lb));
    lb &= 0xff;  // known small and non-negative: offsets fold into ds_* immediates
    bf16* sX = lds_ns + lb;
    bf16* sA = lds_ns + lb;
    bf16* sB = lds_ns + lb + ROWS * PA;
    const float ca = kNsCoef[it][0], cb = kNsCoef[it][1], cc = kNsCoef[it][2];
    // ---- 1. X -> LDS row-major; A = X X^T ----
    __syncthreads();  // previous step's readers of sB are done
    // X^T row-major: lane (c, g) stores rows 4g .. 4g+3 of column col as 8 bytes
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      bf16* xc = sX + (col0 + 16 * ct + c) * PX + 4 * gq;
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) {
        if constexpr (XG) {
#pragma unroll
          for (int i = 0; i < 4; ++i) xv[rt][ct][i] = Xg[(16 * rt + i) * COLS + 16 * ct];
        }
        bf16x4 v;
        v[0] = (bf16)xv[rt][ct][0]; v[1] = (bf16)xv[rt][ct][1];
        v[2] = (bf16)xv[rt][ct][2]; v[3] = (bf16)xv[rt][ct][3];
        *reinterpret_cast<bf16x4*>(xc + 16 * rt) = v;
      }
    }
    __syncthreads();
    // A block in column halves of BTH tiles to bound live accumulators; each
    // half is stored to LDS (transposed tiles, A symmetric) straight away.
    constexpr int BTH = BTN > 2 ? BTN / 2 : BTN;
    // Row fragments of X (K = columns) by transpose reads of X^T: lane j of
    // each 16-lane group points at column k + 8g + j/4 (+4), rows 4 (j%4).
    const bf16* xa = sX + (8 * gq + (c >> 2)) * PX + BMS * bm + 4 * (c & 3);
    const bf16* xbn = sX + (8 * gq + (c >> 2)) * PX + BNS * bn + 4 * (c & 3);
    f32x4 acc[BTM][BTN];
#pragma unroll
    for (int y0 = 0; y0 < BTN; y0 += BTH) {
#pragma unroll
      for (int x = 0; x < BTM; ++x)
#pragma unroll
        for (int y = 0; y < BTH; ++y) acc[x][y0 + y] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
      for (int k = 0; k < COLS; k += 32) {
        bf16x8 fa[BTM], fb[BTH];
#pragma unroll
        for (int x = 0; x < BTM; ++x)
          fa[x] = cat8(ld_tr4(xa + k * PX + 16 * x), ld_tr4(xa + (k + 4) * PX + 16 * x));
#pragma unroll
        for (int y = 0; y < BTH; ++y)
          fb[y] = cat8(ld_tr4(xbn + k * PX + 16 * (y0 + y)), ld_tr4(xbn + (k + 4) * PX + 16 * (y0 + y)));
#pragma unroll
        for (int x = 0; x < BTM; ++x)
#pragma unroll
          for (int y = 0; y < BTH; ++y) mma(acc[x][y0 + y], fa[x], fb[y]);
      }
    }
    __syncthreads();  // all reads of sX done before A overwrites it
    // ---- 2. A -> LDS; A A; B = b A + c A A -> LDS ----
    // A symmetric: store the transposed tile, row (col of the tile) gets 4
    // consecutive elements
#pragma unroll
    for (int x = 0; x < BTM; ++x)
#pragma unroll
      for (int y = 0; y < BTN; ++y) {
        bf16x4 v;
        v[0] = (bf16)acc[x][y][0]; v[1] = (bf16)acc[x][y][1];
        v[2] = (bf16)acc[x][y][2]; v[3] = (bf16)acc[x][y][3];
        *reinterpret_cast<bf16x4*>(sA + (BNS * bn + 16 * y + c) * PA + BMS * bm + 16 * x + 4 * gq) = v;
      }
    __syncthreads();
#pragma unroll
    for (int y0 = 0; y0 < BTN; y0 += BTH) {
      f32x4 a2[BTM][BTH];
#pragma unroll
      for (int x = 0; x < BTM; ++x)
#pragma unroll
        for (int y = 0; y < BTH; ++y) a2[x][y] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < ROWS; k += 32) {
        bf16x8 fa[BTM], fb[BTH];
#pragma unroll
        for (int x = 0; x < BTM; ++x) fa[x] = ld8(sA + (BMS * bm + 16 * x + c) * PA + k + 8 * gq);
#pragma unroll
        for (int y = 0; y < BTH; ++y)
          fb[y] = ld8(sA + (BNS * bn + 16 * (y0 + y) + c) * PA + k + 8 * gq);  // A symmetric
#pragma unroll
        for (int x = 0; x < BTM; ++x)
#pragma unroll
          for (int y = 0; y < BTH; ++y) mma(a2[x][y], fa[x], fb[y]);
      }
      // B = b A + c A A (symmetric): transposed tile, 8-byte stores; b A uses
      // the bf16 A in LDS (its accumulators are dead by now)
#pragma unroll
      for (int x = 0; x < BTM; ++x)
#pragma unroll
        for (int y = 0; y < BTH; ++y) {
          const int o = (BNS * bn + 16 * (y0 + y) + c) * PA + BMS * bm + 16 * x + 4 * gq;
          const bf16x4 av = *reinterpret_cast<const bf16x4*>(sA + o);
          bf16x4 v;
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] = (bf16)(cb * (float)av[i] + cc * a2[x][y][i]);
          *reinterpret_cast<bf16x4*>(sB + o) = v;
        }
    }
    __syncthreads();
    // ---- 3. X = a X + B X on this wave's columns, one column tile at a
    // time (columns of B X only depend on the same columns of X) ----
    // (opaque to the optimiser: the bf16 copies made for step 1 must not be
    // kept alive until here)
    if constexpr (!XG) {
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) asm volatile("" : "+v"(xv[rt][ct]));
    }
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      if constexpr (XG) {
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
          for (int i = 0; i < 4; ++i) xv[rt][ct][i] = Xg[(16 * rt + i) * COLS + 16 * ct];
      }
      // bf16 fragments of X (B operand, K = rows): slab ks, slot m <-> row
      // 32 ks + kappa(g, m), i.e. tiles 2 ks and 2 ks + 1 of the accumulator layout
      bf16x8 xf[NKS];
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          xf[ks][i] = (bf16)xv[2 * ks][ct][i];
          xf[ks][4 + i] = (bf16)xv[2 * ks + 1][ct][i];
        }
      // rows in halves: xf holds the old X of this column tile, so the
      // first half can be updated in place before the second is computed
      constexpr int RH = NRT > 4 ? NRT / 2 : NRT;
#pragma unroll
      for (int r0 = 0; r0 < NRT; r0 += RH) {
        f32x4 xo[RH];
#pragma unroll
        for (int rr = 0; rr < RH; ++rr) xo[rr] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
          for (int rr = 0; rr < RH; ++rr) {
            const bf16* br = sB + (16 * (r0 + rr) + c) * PA + 32 * ks;
            mma(xo[rr], ld4x2(br + 4 * gq, br + 16 + 4 * gq), xf[ks]);
          }
#pragma unroll
        for (int rr = 0; rr < RH; ++rr) xv[r0 + rr][ct] = ca * xv[r0 + rr][ct] + xo[rr];
        if (last || XG) {
#pragma unroll
          for (int rr = 0; rr < RH; ++rr)
#pragma unroll
            for (int i = 0; i < 4; ++i) Xg[(16 * (r0 + rr) + i) * COLS + 16 * ct] = xv[r0 + rr][ct][i];
        }
      }
    }
  };
#pragma unroll 1
  for (int it = 0; it < 4; ++it) step(it, false);
  step(4, true);
}

template <int ROWS, int COLS, int NW, bool XG>
static hipError_t run_ns_fused(int count, const float* g, float* u, float eps, hipStream_t s) {
  const size_t lds = (size_t)ns_lds_elems(ROWS, COLS) * sizeof(bf16);
  static bool attr = false;
  if (!attr) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_ns_fused<ROWS, COLS, NW, XG>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr = true;
  }
  hipLaunchKernelGGL((k_ns_fused<ROWS, COLS, NW, XG>), dim3(count), dim3(NW * 64), lds, s, g, u, eps);
  return hipGetLastError();
}

// Returns hipErrorNotSupported when no fused variant covers the shape.
hipError_t launch_ns_fused(int dtype, int count, int rows, int cols, const float* g, float* u,
                           float eps, hipStream_t s) {
  if (dtype != 1) return hipErrorNotSupported;
  if (rows == 128 && cols == 512) return run_ns_fused<128, 512, 8, false>(count, g, u, eps, s);
  if (rows == 128 && cols == 256) return run_ns_fused<128, 256, 16, false>(count, g, u, eps, s);
  if (rows == 64 && cols == 256) return run_ns_fused<64, 256, 16, false>(count, g, u, eps, s);
  if (rows == 64 && cols == 512) return run_ns_fused<64, 512, 16, true>(count, g, u, eps, s);
  return hipErrorNotSupported;
}

}  // namespace lact
