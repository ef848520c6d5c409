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
//
// Shifted steps (every step from `shift_from` on): once most singular values
// are near one, A is near a multiple mu I of the identity and B near
// (b mu + c mu^2) I, so rounding A, B and the X operand of B X to bf16 costs
// about 2^-9 of X per step.  Those steps take mu = trace(A) / rows, store
// A_s = A - mu I instead and form
//   B_s = (b + 2 c mu) A_s + c A_s A_s      (= B - (b mu + c mu^2) I),
//   X  <- (a + b mu + c mu^2) X + B_s X      (the same step in real numbers),
// so the multiples of the identity stay in fp32 and only the remainders are
// rounded.  mu is the mean eigenvalue of A, so a spectrum that has not yet
// gathered near one is shifted by little.
#include "lact_internal.hpp"
#include "mfma.hpp"
#include "k_apply.hpp"

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
__global__ __launch_bounds__(NW * 64) void k_ns_fused(NsIn g, float* u, float eps, int shift_from) {
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
  const float* G = g.at(blockIdx.x, (int64_t)ROWS * COLS);
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
    const bool shf = it >= shift_from;
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
    // consecutive elements (shifted step: A - mu I, mu = trace(A) / ROWS,
    // from the waves' partial traces in a fixed order)
    float mu = 0.f;
    if (shf) {
      float pt = 0.f;
#pragma unroll
      for (int x = 0; x < BTM; ++x)
#pragma unroll
        for (int y = 0; y < BTN; ++y)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (BMS * bm + 16 * x + 4 * gq + i == BNS * bn + 16 * y + c) pt += acc[x][y][i];
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) pt += __shfl_xor(pt, o);
      if (lane == 0) red[w] = pt;
      __syncthreads();
      float tr = 0.f;
#pragma unroll
      for (int x = 0; x < NW; ++x) tr += red[x];
      mu = tr * (1.0f / ROWS);
      __syncthreads();  // every read of red done before the next step writes it
#pragma unroll
      for (int x = 0; x < BTM; ++x)
#pragma unroll
        for (int y = 0; y < BTN; ++y)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (BMS * bm + 16 * x + 4 * gq + i == BNS * bn + 16 * y + c) acc[x][y][i] -= mu;
    }
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
      // the bf16 A in LDS (its accumulators are dead by now); shifted step:
      // B_s = (b + 2 c mu) A_s + c A_s A_s
      const float cbs = cb + 2.f * cc * mu;
#pragma unroll
      for (int x = 0; x < BTM; ++x)
#pragma unroll
        for (int y = 0; y < BTH; ++y) {
          const int o = (BNS * bn + 16 * (y0 + y) + c) * PA + BMS * bm + 16 * x + 4 * gq;
          const bf16x4 av = *reinterpret_cast<const bf16x4*>(sA + o);
          bf16x4 v;
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] = (bf16)(cbs * (float)av[i] + cc * a2[x][y][i]);
          *reinterpret_cast<bf16x4*>(sB + o) = v;
        }
    }
    __syncthreads();
    // ---- 3. X = a X + B X on this wave's columns, one column tile at a
    // time (columns of B X only depend on the same columns of X); shifted
    // step: X = (a + b mu + c mu^2) X + B_s X ----
    const float cas = ca + cb * mu + cc * mu * mu;
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
        for (int rr = 0; rr < RH; ++rr) xv[r0 + rr][ct] = cas * xv[r0 + rr][ct] + xo[rr];
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

// ---------------------------------------------------------------------------
// Newton-Schulz-5 for 128-row matrices (d = 128): one workgroup of 8 waves per
// matrix, the fp32 iterate in registers, everything else in LDS:
//   sX [128][COLS] bf16  operand copy of the iterate (row-major)
//   sA [128][128]  bf16  A = X X^T, then B (in place)
// i.e. 160 KiB for COLS = 512.
//
// The iterate is kept rescaled, Y_k = X_k / P_k with P_k = a_0 ... a_{k-1}:
//   A_k = P_k^2 Y Y^T,  B'_k = (b A_k + c A_k A_k) / a_k,  Y <- Y + B'_k Y
// which is the same quintic step (X_{k+1} = a X + B X = P_{k+1} Y_{k+1})
// with the fp32 term a X kept exact and no rescaling of the registers;
// X_5 = P_5 Y_5 on the way out.  Products take bf16 operands and accumulate
// in fp32.
//
// Per step:
//   1. A (symmetric, 8 x 8 tiles of 16 x 16): every wave forms a set of
//      tiles on or above the diagonal (NsrSet): each diagonal 4 x 4 block
//      is split into two sets of 5 tiles that share their operand reads (4
//      and 3 row tiles per K slab), the block of row tiles 0-3 by column
//      tiles 4-7 into four 2 x 2 blocks.  Wave w runs on SIMD w mod 4, so
//      every SIMD forms 9 tiles and has two waves whose LDS reads and MFMAs
//      interleave; fragment reads per K slab total 30 row tiles.  (Blocks of
//      4 x 2 tiles with two of them skipped left two SIMDs with 16 tiles;
//      unequal blocks left single waves on a SIMD waiting on their reads.)
//      Every tile is stored transposed (8-byte stores), which for a
//      symmetric result is the tile at the mirrored position; tiles off the
//      diagonal also in place (8-byte stores after a transpose within lane
//      quads), so all of A is written.
//   2. A A the same way, then (after every read of A) B' = p A + q A A over
//      A, with A read back from the wave's own transposed tiles.
//   3. Y <- Y + B' Y: wave w owns columns [w COLS/8, (w+1) COLS/8) and forms
//      their tiles of (B' Y)^T = Y^T B' (B' symmetric): lane (c, g) holds
//      Y[16 nt + c][col0 + 16 mt + 4 g + i], four consecutive columns of one
//      row, so global loads/stores and the bf16 copy to sX are 16 / 8-byte
//      vectors.  The Y^T fragments are transpose reads of sX.
// LDS rows are split into 16-byte chunks whose index is XORed with a linear
// function of the row bits r0..r3, chosen with the measured gfx950 bank
// model (16-byte reads in 16-lane passes by lane-quad parity, 8-byte reads
// in 32-lane passes, 8-byte writes in 16-lane passes over 128 bytes):
//   sX (rows of COLS):  s(r) = 2 r0 ^ 4 r1 ^ 9 r3 - fragment reads (16 rows,
//     one chunk column) and transpose reads (rows 8 g + 0..3) conflict-free,
//     operand-copy stores (16 rows, one column) two-way, the least possible;
//   sA (rows of 128):   s(r) = r mod 16 - fragment reads and the 8-byte reads
//     of B' conflict-free, transposed tile stores two-way.
template <int W>
__device__ __forceinline__ int nsr_swz(int r) {
  if constexpr (W == 128) return r & 15;
  return ((r & 1) << 1) ^ (((r >> 1) & 1) << 2) ^ (((r >> 3) & 1) * 9);
}
template <int W>
__device__ __forceinline__ int nsr_off(int r, int col) {
  return r * W + ((((col >> 3) ^ nsr_swz<W>(r))) << 3) + (col & 7);
}

// An opaque copy of a lane index: address arithmetic derived from it is
// redone where it is used instead of being hoisted out of the step loop and
// kept alive (one register per distinct swizzled address) across all steps.
__device__ __forceinline__ int nsr_opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// Tile sets of a symmetric 128 x 128 product (8 x 8 tiles of 16 x 16), one
// set per wave.  A set reads NF row tiles of the operand per K slab (row
// tile nsr_row<SH>(f, a, b) for f < NF) and forms the NT tiles (row tile of
// TI[t], row tile of TJ[t]), each on or above the diagonal.
template <int SH> struct NsrSet;
template <> struct NsrSet<0> {  // rows a..a+3: (a,a) (a,a+1) (a,a+2) (a,a+3) (a+1,a+1)
  static constexpr int NF = 4, NT = 5;
  static constexpr int TI[NT] = {0, 0, 0, 0, 1}, TJ[NT] = {0, 1, 2, 3, 1};
};
template <> struct NsrSet<1> {  // rows a..a+2: (a,a+1) (a,a+2) (a+1,a+1) (a+1,a+2) (a+2,a+2)
  static constexpr int NF = 3, NT = 5;
  static constexpr int TI[NT] = {0, 0, 1, 1, 2}, TJ[NT] = {1, 2, 1, 2, 2};
};
template <> struct NsrSet<2> {  // rows a, a+1 by rows b, b+1
  static constexpr int NF = 4, NT = 4;
  static constexpr int TI[NT] = {0, 0, 1, 1}, TJ[NT] = {2, 3, 2, 3};
};
template <int SH>
__device__ __forceinline__ int nsr_row(int f, int a, int b) {
  return SH == 2 ? (f < 2 ? a + f : b + f - 2) : a + f;
}

// acc[t] = sum over k < K of M[16 x + .][k] M[16 y + .][k] for the tiles
// (x, y) of set SH of the row-major array s [.][W].
template <int W, int K, int SH>
__device__ __forceinline__ void nsr_gram(const bf16* s, int a, int b, int c, int gq, f32x4 (&acc)[8]) {
  using S = NsrSet<SH>;
#pragma unroll
  for (int t = 0; t < S::NT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  const bf16* ba = s + (16 * a + c) * W;
  const bf16* bb = s + (16 * b + c) * W;
  const int sw = nsr_swz<W>(c);
  bf16x8 fr[S::NF];
#define LACT_NSR_LOAD(K0, FR)                                                        \
  {                                                                                  \
    const int ch = ((((K0) >> 3) + gq) ^ sw) << 3;                                   \
    _Pragma("unroll") for (int f = 0; f < S::NF; ++f)                                \
      FR[f] = ld8((SH == 2 && f >= 2 ? bb + 16 * (f - 2) * W : ba + 16 * f * W) + ch); \
  }
  LACT_NSR_LOAD(0, fr);
#pragma unroll 1
  for (int k = 0; k < K; k += 32) {
    bf16x8 nf[S::NF];
    const int kn = k + 32 < K ? k + 32 : k;  // last slab: harmless re-read
    LACT_NSR_LOAD(kn, nf);
#pragma unroll
    for (int t = 0; t < S::NT; ++t) mma(acc[t], fr[S::TI[t]], fr[S::TJ[t]]);
#pragma unroll
    for (int f = 0; f < S::NF; ++f) fr[f] = nf[f];
  }
#undef LACT_NSR_LOAD
}

// 4 x 4 transpose of 16-bit values over the four lanes of a quad (lanes
// 4k .. 4k + 3): value i of lane j becomes value j of lane i.  p[0] holds
// values 0, 1 and p[1] values 2, 3 (lower half first).  Lane j first swaps a
// dword with lane j ^ 2 (the one the partner needs), then each dword's
// halves with lane j ^ 1 (DPP quad permutations and a byte permute; no LDS).
__device__ __forceinline__ void quad_transpose16(uint32_t (&p)[2], int j) {
  const bool b1 = (j & 2) != 0, b0 = (j & 1) != 0;
  const uint32_t send = b1 ? p[0] : p[1];
  const uint32_t recv = (uint32_t)__builtin_amdgcn_mov_dpp((int)send, 0x4E, 0xF, 0xF, true);  // j ^ 2
  p[0] = b1 ? recv : p[0];
  p[1] = b1 ? p[1] : recv;
  // even lane: (own low half, partner's low half); odd: (partner's high, own high)
  const uint32_t sel = b0 ? 0x03020706u : 0x05040100u;
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    const uint32_t r = (uint32_t)__builtin_amdgcn_mov_dpp((int)p[x], 0xB1, 0xF, 0xF, true);  // j ^ 1
    p[x] = __builtin_amdgcn_perm(r, p[x], sel);
  }
}

// Stores the set's tiles v[t] (values of M[16 x + 4 g + i][16 y + c] of a
// symmetric 128 x 128 matrix) transposed, which for a symmetric result is
// the tile at the mirrored position (y, x), and, off the diagonal, also in
// place (x, y): after a transpose within lane quads, lane (c, g) holds row
// 16 x + 4 g + c % 4, columns 16 y + 4 (c / 4) + 0..3 (8-byte stores).
template <int SH>
__device__ __forceinline__ void nsr_store(bf16* s, int a, int b, int c, int gq, const f32x4 (&v)[8]) {
  using S = NsrSet<SH>;
#pragma unroll
  for (int t = 0; t < S::NT; ++t) {
    const int tx = nsr_row<SH>(S::TI[t], a, b), ty = nsr_row<SH>(S::TJ[t], a, b);
    bf16x4 q;
    q[0] = (bf16)v[t][0]; q[1] = (bf16)v[t][1];
    q[2] = (bf16)v[t][2]; q[3] = (bf16)v[t][3];
    *reinterpret_cast<bf16x4*>(s + nsr_off<128>(16 * ty + c, 16 * tx + 4 * gq)) = q;
    if (S::TI[t] != S::TJ[t]) {
      uint32_t p[2];
      __builtin_memcpy(p, &q, sizeof(p));
      quad_transpose16(p, c & 3);
      *reinterpret_cast<uint2*>(s + nsr_off<128>(16 * tx + 4 * gq + (c & 3), 16 * ty + 4 * (c >> 2))) =
          make_uint2(p[0], p[1]);
    }
  }
}

template <int COLS, int NMT, int NRT>
__device__ __forceinline__ void ns_step_epilogue(const f32x4 (&yv)[NMT][NRT], float P, int m,
                                                 const NsStep& st, float* stg);

template <int COLS, int NMT, int NRT>
__device__ __forceinline__ void ns_load_grad(f32x4 (&yv)[NMT][NRT], int m, const NsGrad& gr,
                                             float* stg);

// STEP: G from the split partials (ns_load_grad) instead of g, and instead of
// writing U, add it to the weights (ns_step_epilogue).
template <int COLS, bool STEP>
__device__ __forceinline__ void ns_r128_block(const NsIn& g, const NsGrad& gr, float* u, float eps,
                                              int shift_from, int m, bf16* lds_r, const NsStep& st) {
  constexpr int R = 128, NW = 8;
  constexpr int CW = COLS / NW;  // columns per wave
  constexpr int NMT = CW / 16;   // column tiles per wave
  constexpr int NRT = R / 16;    // row tiles
  static_assert(CW % 16 == 0, "shape");
  bf16* sX = lds_r;
  bf16* sA = lds_r + R * COLS;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int c = lane & 15, gq = lane >> 4;
  const int col0 = w * CW;
  // this wave's tile set of A and A A (NsrSet): the diagonal 4 x 4 blocks
  // are split into sets 0 and 1 (waves 0, 1: rows 0-3; waves 2, 3: rows
  // 4-7), the block of row tiles 0-3 by column tiles 4-7 into four 2 x 2
  // sets (waves 4-7)
  const int sh = w < 4 ? (w & 1) : 2;
  const int sa = w < 4 ? 4 * (w >> 1) + (w & 1) : 2 * ((w - 4) >> 1);
  const int sb = w < 4 ? 0 : 4 + 2 * (w & 1);
  // ---- load G: whole rows, coalesced, staged through LDS (fp32, 16-byte
  // chunks XORed with the row) into the accumulator layout ----
  // rows per staging pass: fp32 rows must fit the LDS allocation (sX + sA)
  constexpr int LDSB = (R * COLS + R * R) * 2;
  constexpr int SR = R * COLS * 4 <= LDSB ? R : 64 * COLS * 4 <= LDSB ? 64 : 32;
  static_assert(SR * COLS * 4 <= LDSB && (SR * COLS / 4) % (NW * 64) == 0, "staging");
  constexpr int SV = SR * COLS / 4 / (NW * 64);           // float4 per thread per pass
  float* stg = reinterpret_cast<float*>(lds_r);
  auto soff = [](int r, int col) { return r * COLS + ((((col >> 2) ^ (r & 15))) << 2) + (col & 3); };
  f32x4 yv[NMT][NRT];
  if constexpr (STEP) ns_load_grad<COLS>(yv, m, gr, stg);
  else {
  const float* G = g.at(m, (int64_t)R * COLS);
#pragma unroll
  for (int p0 = 0; p0 < R; p0 += SR) {
    if (p0) __syncthreads();  // previous pass fully read
#pragma unroll
    for (int v = 0; v < SV; ++v) {
      const int q = tid + v * NW * 64, r = q / (COLS / 4), cq = 4 * (q % (COLS / 4));
      *reinterpret_cast<f32x4*>(stg + soff(r, cq)) =
          *reinterpret_cast<const f32x4*>(G + (int64_t)(p0 + r) * COLS + cq);
    }
    __syncthreads();
#pragma unroll
    for (int nt = p0 / 16; nt < (p0 + SR) / 16; ++nt)
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt)
        yv[mt][nt] = *reinterpret_cast<const f32x4*>(stg + soff(16 * nt + c - p0, col0 + 16 * mt + 4 * gq));
  }
  }
  // Frobenius norm (fixed order)
  float ss = 0.f;
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NRT; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) ss += yv[mt][nt][i] * yv[mt][nt][i];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
  __syncthreads();  // staging fully read
  float* red = reinterpret_cast<float*>(sA);
  if (lane == 0) red[w] = ss;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int x = 0; x < NW; ++x) tot += red[x];
  const float scale = 1.0f / (sqrtf(tot) + eps);
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NRT; ++nt) yv[mt][nt] = yv[mt][nt] * scale;

  // operand copy: lane (c, g) writes 4 consecutive columns of row 16 nt + c
#define LACT_NSR_PUT_X()                                                                 \
  {                                                                                      \
    const int c_ = nsr_opaque(c), g_ = nsr_opaque(gq);                                   \
    _Pragma("unroll") for (int mt = 0; mt < NMT; ++mt)                                   \
    _Pragma("unroll") for (int nt = 0; nt < NRT; ++nt)                                   \
      st4(sX + nsr_off<COLS>(16 * nt + c_, col0 + 16 * mt + 4 * g_), yv[mt][nt][0],      \
          yv[mt][nt][1], yv[mt][nt][2], yv[mt][nt][3]);                                  \
  }
  LACT_NSR_PUT_X();

  float P = 1.0f;
#pragma unroll 1
  for (int it = 0; it < 5; ++it) {
    const float ca = kNsCoef[it][0], cb = kNsCoef[it][1], cc = kNsCoef[it][2];
    const bool shf = it >= shift_from;
    __syncthreads();  // sX complete; last step's reads of sA done
    // ---- 1. A = P^2 Y Y^T (shifted step: A - mu I, mu = trace(A) / 128) ----
    // (one instantiation per tile set; the branch is uniform per wave)
    float mu = 0.f;
    {
      const int c = nsr_opaque(lane & 15), gq = nsr_opaque(lane >> 4);
      f32x4 ta[8];
      if (sh == 0) nsr_gram<COLS, COLS, 0>(sX, sa, sb, c, gq, ta);
      else if (sh == 1) nsr_gram<COLS, COLS, 1>(sX, sa, sb, c, gq, ta);
      else nsr_gram<COLS, COLS, 2>(sX, sa, sb, c, gq, ta);
      const float s2 = P * P;
#pragma unroll
      for (int x = 0; x < 5; ++x) ta[x] = ta[x] * s2;
      if (shf) {
        // the diagonal tiles: set 0 holds (a, a) and (a+1, a+1) as tiles 0
        // and 4, set 1 (a+1, a+1) and (a+2, a+2) as tiles 2 and 4; lane
        // (c, g) holds element i of row 4 g + i, column c of a tile
        const int x0 = sh == 0 ? 0 : 2;
        float pt = 0.f;
        if (sh < 2) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (4 * gq + i == c) pt += ta[x0][i] + ta[4][i];
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) pt += __shfl_xor(pt, o);
        // sA is free until the stores below: exchange the four partial traces
        float* red = reinterpret_cast<float*>(sA);
        if (lane == 0 && w < 4) red[w] = pt;
        __syncthreads();
        mu = ((red[0] + red[1]) + (red[2] + red[3])) * (1.0f / 128.0f);
        __syncthreads();  // every read of red done before A overwrites it
        if (sh < 2) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (4 * gq + i == c) {
              ta[x0][i] -= mu;
              ta[4][i] -= mu;
            }
        }
      }
      if (sh == 0) nsr_store<0>(sA, sa, sb, c, gq, ta);
      else if (sh == 1) nsr_store<1>(sA, sa, sb, c, gq, ta);
      else nsr_store<2>(sA, sa, sb, c, gq, ta);
    }
    __syncthreads();
    // ---- 2. B' = (b A + c A A) / a, over A (shifted step: B'_s = ((b +
    // 2 c mu) A_s + c A_s A_s) / a = B' - (b mu + c mu^2) / a I) ----
    f32x4 t[8];
    if (sh == 0) nsr_gram<128, 128, 0>(sA, sa, sb, nsr_opaque(c), nsr_opaque(gq), t);
    else if (sh == 1) nsr_gram<128, 128, 1>(sA, sa, sb, nsr_opaque(c), nsr_opaque(gq), t);
    else nsr_gram<128, 128, 2>(sA, sa, sb, nsr_opaque(c), nsr_opaque(gq), t);
    __syncthreads();  // every read of A as an operand is done
#define LACT_NSR_B(SH)                                                                   \
  {                                                                                      \
    const int c = nsr_opaque(lane & 15), gq = nsr_opaque(lane >> 4);                     \
    const float p = (cb + 2.f * cc * mu) / ca, q = cc / ca;                              \
    _Pragma("unroll") for (int x = 0; x < NsrSet<SH>::NT; ++x) {                         \
      const int tx = nsr_row<SH>(NsrSet<SH>::TI[x], sa, sb);                             \
      const int ty = nsr_row<SH>(NsrSet<SH>::TJ[x], sa, sb);                             \
      const bf16x4 a = *reinterpret_cast<const bf16x4*>(                                 \
          sA + nsr_off<128>(16 * ty + c, 16 * tx + 4 * gq));                             \
      _Pragma("unroll") for (int i = 0; i < 4; ++i) t[x][i] = p * (float)a[i] + q * t[x][i]; \
    }                                                                                    \
    nsr_store<SH>(sA, sa, sb, c, gq, t);                                                 \
  }
    if (sh == 0) LACT_NSR_B(0) else if (sh == 1) LACT_NSR_B(1) else LACT_NSR_B(2)
#undef LACT_NSR_B
    __syncthreads();  // B' complete
    // ---- 3. Y <- Y + B' Y on this wave's columns: (Y^T B') tiles (shifted
    // step: Y <- (1 + (b mu + c mu^2) / a) Y + B'_s Y) ----
    if (shf) {
      const float f = 1.f + (cb * mu + cc * mu * mu) / ca;
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NRT; ++nt) yv[mt][nt] = yv[mt][nt] * f;
    }
    {
      const int c = nsr_opaque(lane & 15), gq = nsr_opaque(lane >> 4);
#pragma unroll 1
      for (int ks = 0; ks < R / 32; ++ks) {
        bf16x8 bf[NRT], af[NMT];
#pragma unroll
        for (int nt = 0; nt < NRT; ++nt) bf[nt] = ld8(sA + nsr_off<128>(16 * nt + c, 32 * ks + 8 * gq));
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt) {
          // lane (c, g): Y[32 ks + 8 g + 0..7][col0 + 16 mt + c]
          const int r0 = 32 * ks + 8 * gq + (c >> 2), cl = col0 + 16 * mt + 4 * (c & 3);
          af[mt] = cat8(ld_tr4(sX + nsr_off<COLS>(r0, cl)), ld_tr4(sX + nsr_off<COLS>(r0 + 4, cl)));
        }
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
          for (int nt = 0; nt < NRT; ++nt) mma(yv[mt][nt], af[mt], bf[nt]);
      }
    }
    P *= ca;
    // own columns only: no other wave reads them before the next barrier
    if (it < 4) LACT_NSR_PUT_X();
  }
#undef LACT_NSR_PUT_X
  if constexpr (STEP) {
    ns_step_epilogue<COLS>(yv, P, m, st, stg);
    return;
  }
  float* U = u + (int64_t)m * R * COLS;
  // ---- X_5 = P_5 Y_5, staged through LDS into whole rows ----
#pragma unroll
  for (int p0 = 0; p0 < R; p0 += SR) {
    __syncthreads();  // every read of sX / sA (or of the previous pass) done
    const int cf = nsr_opaque(c), gf = nsr_opaque(gq);
#pragma unroll
    for (int nt = p0 / 16; nt < (p0 + SR) / 16; ++nt)
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt)
        *reinterpret_cast<f32x4*>(stg + soff(16 * nt + cf - p0, col0 + 16 * mt + 4 * gf)) = yv[mt][nt] * P;
    __syncthreads();
    const int tf = nsr_opaque(tid);
#pragma unroll
    for (int v = 0; v < SV; ++v) {
      const int q = tf + v * NW * 64, r = q / (COLS / 4), cq = 4 * (q % (COLS / 4));
      *reinterpret_cast<f32x4*>(U + (int64_t)(p0 + r) * COLS + cq) =
          *reinterpret_cast<const f32x4*>(stg + soff(r, cq));
    }
  }
}

template <int COLS>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void k_ns_r128(NsIn g, float* u, float eps, int shift_from) {
  extern __shared__ __attribute__((aligned(16))) bf16 lds_r[];
  ns_r128_block<COLS, false>(g, NsGrad{}, u, eps, shift_from, blockIdx.x, lds_r, NsStep{});
}

// ---- gradient prologue ----
// G in the accumulator layout (lane (c, g): row 16 nt + c, columns col0 +
// 16 mt + 4 g .. + 3) from the split partials, which hold G^T ([dh][128]):
// every wave sums the partial rows of its own columns, 32 per pass, 8 lanes
// per row (128-byte segments), in split order, stores the sums in its own
// 16 KiB of LDS and reads them back transposed.  With momentum the gradient
// launch has already put beta M_old into split 0, so the sum is the new M:
// M <- G (stored from the accumulator layout, 16 bytes per lane).  The LDS
// key is the one of the W1 step below (every store and read on 64 distinct
// banks); no barrier: each wave touches only its own block.
template <int COLS, int NMT, int NRT>
__device__ __forceinline__ void ns_load_grad(f32x4 (&yv)[NMT][NRT], int m, const NsGrad& gr,
                                             float* stg) {
  constexpr int CW = COLS / 8;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int col0 = w * CW;
  const int mat = m / gr.bh, head = m - mat * gr.bh;
  const int64_t msz = (int64_t)128 * COLS;
  const float* P0 = gr.partial + ((int64_t)head * 3 + mat) * msz;
  const int64_t pstr = (int64_t)gr.bh * 3 * msz;  // between splits
  float* M = gr.m[mat] != nullptr ? gr.m[mat] + head * msz : nullptr;
  float* ws = stg + w * 32 * 128;
  auto off = [](int t, int i) {
    return t * 128 + (((i >> 2) ^ (4 * (((t >> 2) ^ t) & 3))) << 2) + (i & 3);
  };
#pragma unroll
  for (int p = 0; p < NMT / 2; ++p) {
    asm volatile("" ::: "memory");  // no load of this pass above the last one (registers)
    const int c = opaque(lane & 15), gq = opaque(lane >> 4);
    const int lr = opaque(lane >> 3), lk = lane & 7;
    // partial rows col0 + 32 p + 8 v + lr, features 4 (lk + 8 kk) .. + 3
    const float* pp = P0 + (int64_t)(col0 + 32 * p + lr) * 128 + 4 * lk;
    f32x4 x[4][4];
#pragma unroll
    for (int v = 0; v < 4; ++v)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) x[v][kk] = *reinterpret_cast<const f32x4*>(pp + 8 * v * 128 + 32 * kk);
    for (int sp = 1; sp < gr.nsplit; ++sp) {
      const float* q = pp + sp * pstr;
      f32x4 y[4][4];
#pragma unroll
      for (int v = 0; v < 4; ++v)
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) y[v][kk] = *reinterpret_cast<const f32x4*>(q + 8 * v * 128 + 32 * kk);
#pragma unroll
      for (int v = 0; v < 4; ++v)
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) x[v][kk] += y[v][kk];
    }
#pragma unroll
    for (int v = 0; v < 4; ++v)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        *reinterpret_cast<f32x4*>(ws + off(8 * v + lr, 4 * (lk + 8 * kk))) = x[v][kk];
    // transposed read-back: G[16 nt + c][col0 + 16 (2p + mh) + 4 gq + e]
#pragma unroll
    for (int mh = 0; mh < 2; ++mh)
#pragma unroll
      for (int nt = 0; nt < NRT; ++nt)
#pragma unroll
        for (int e = 0; e < 4; ++e) yv[2 * p + mh][nt][e] = ws[off(16 * mh + 4 * gq + e, 16 * nt + c)];
    if (M != nullptr) {
      float* mrow = M + (int64_t)c * COLS + col0 + 32 * p + 4 * gq;
#pragma unroll
      for (int mh = 0; mh < 2; ++mh)
#pragma unroll
        for (int nt = 0; nt < NRT; ++nt)
          *reinterpret_cast<f32x4*>(mrow + (int64_t)16 * nt * COLS + 16 * mh) = yv[2 * p + mh][nt];
    }
  }
}

// ---- step epilogue ----
// The result X5 = P Y (this wave's columns col0 .. col0 + COLS / 8 of the
// 128 x COLS wide matrix, accumulator layout) is added to the fp32 weights,
// each row rescaled to n0 / (||row|| + eps) (renorm; else left as is), and
// the weights and their bf16 operand copies written (master variant: the
// weights keep the unscaled sum, the copies the rescaled rows).  Part of X5 at a time is
// staged in LDS (fp32) and each W row goes to 8 consecutive lanes (128-byte
// segments, 16 float4 per lane), so a row norm is three shuffles.  W loads
// are issued after the staging stores, when those registers of X5 are free.
//   W1, W3 ([COLS][128], row j = column j of X5): every wave steps the rows of
//     its own columns, 32 per pass, through its own 16 KiB of LDS (no
//     barrier after the first).
//   W2 ([128][COLS], the orientation of X5): 64 (COLS 512) or 128 (COLS 256)
//     rows per pass, staged by all waves; the final rows go back into the
//     tile, whose columns then give the W2^T copy (8 features of a hidden unit
//     per 16-byte store).
// LDS keys (measured bank model: 16-byte reads in 16-lane passes by lane-quad
// parity, 16-byte writes in 8-lane passes): every staging store and every
// read below touches 64 distinct banks.
template <int COLS, int NMT, int NRT>
__device__ __forceinline__ void ns_step_epilogue(const f32x4 (&yv)[NMT][NRT], float P, int m,
                                                 const NsStep& st, float* stg) {
  constexpr int CW = COLS / 8;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int col0 = w * CW;
  const int mat = m / st.bh, head = m - mat * st.bh;
  const int64_t msz = (int64_t)128 * COLS;
  bf16* sb = reinterpret_cast<bf16*>(st.sh.base) + (int64_t)head * st.sh.per_head;
  __syncthreads();  // every Newton-Schulz read of LDS done
  if (mat < 2) {
    float* W = (mat == 0 ? st.w1 : st.w3) + head * msz;
    const float* N0 = (mat == 0 ? st.n1 : st.n3) + (int64_t)head * COLS;
    bf16* S = sb + (mat == 0 ? st.sh.off_w1 : st.sh.off_w3);
    float* ws = stg + w * 32 * 128;  // this wave's [32][128] block
    // element (row t, feature i) of the block
    auto off = [](int t, int i) {
      return t * 128 + (((i >> 2) ^ (4 * (((t >> 2) ^ t) & 3))) << 2) + (i & 3);
    };
#pragma unroll
    for (int p = 0; p < NMT / 2; ++p) {
      // rows col0 + 32 p + 8 v + lr, features 4 (lk + 8 kk) .. + 3; lane
      // indices laundered per pass so that no address outlives its pass
      const int c = opaque(lane & 15), gq = opaque(lane >> 4);
      const int lr = opaque(lane >> 3), lk = lane & 7;
#pragma unroll
      for (int mh = 0; mh < 2; ++mh)
#pragma unroll
        for (int nt = 0; nt < NRT; ++nt)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            ws[off(16 * mh + 4 * gq + e, 16 * nt + c)] = yv[2 * p + mh][nt][e] * P;
      asm volatile("" ::: "memory");  // loads stay after the stores (register pressure)
      f32x4 x[4][4];
      float n0[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int j = col0 + 32 * p + 8 * v + lr;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
          x[v][kk] = *reinterpret_cast<const f32x4*>(W + (int64_t)j * 128 + 4 * (lk + 8 * kk));
        n0[v] = st.renorm ? N0[j] : 1.f;
      }
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int t = 8 * v + lr;
        float ss = 0.f;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          x[v][kk] += *reinterpret_cast<const f32x4*>(ws + off(t, 4 * (lk + 8 * kk)));
          ss += x[v][kk][0] * x[v][kk][0] + x[v][kk][1] * x[v][kk][1] +
                x[v][kk][2] * x[v][kk][2] + x[v][kk][3] * x[v][kk][3];
        }
        ss += __shfl_xor(ss, 1);
        ss += __shfl_xor(ss, 2);
        ss += __shfl_xor(ss, 4);
        if (st.nonfinite != nullptr && lk == 0 && !(ss <= 3.402823466e38f)) atomicOr(st.nonfinite, 1);
        const float f = st.renorm ? n0[v] / (sqrtf(ss) + st.eps) : 1.f;
        const int64_t row = (int64_t)(col0 + 32 * p + t) * 128;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const f32x4 y = x[v][kk] * f;
          *reinterpret_cast<f32x4*>(W + row + 4 * (lk + 8 * kk)) = st.renorm == 2 ? x[v][kk] : y;
          st4(S + row + 4 * (lk + 8 * kk), y[0], y[1], y[2], y[3]);
        }
      }
    }
  } else {
    constexpr int KK = COLS / 32;  // float4 per lane per row
    constexpr int V = 16 / KK;     // rows per lane per pass
    constexpr int SR = 64 * V;     // rows per pass
    float* W = st.w2 + head * msz;
    const float* N0 = st.n2 + (int64_t)head * 128;
    bf16* S = sb + st.sh.off_w2;
    bf16* St = sb + st.sh.off_w2t;
    auto off = [](int r, int j) {
      return r * COLS + (((j >> 2) ^ ((4 * (r & 3)) | ((r >> 2) & 1))) << 2) + (j & 3);
    };
#pragma unroll
    for (int p0 = 0; p0 < 128; p0 += SR) {
      if (p0) __syncthreads();  // the previous pass's tile fully read
      const int c = opaque(lane & 15), gq = opaque(lane >> 4);
      const int lr = opaque(lane >> 3), lk = lane & 7;
#pragma unroll
      for (int nt = p0 / 16; nt < (p0 + SR) / 16; ++nt)
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt)
          *reinterpret_cast<f32x4*>(stg + off(16 * nt + c - p0, col0 + 16 * mt + 4 * gq)) = yv[mt][nt] * P;
      asm volatile("" ::: "memory");  // loads stay after the stores (register pressure)
      f32x4 x[V][KK];
      float n0[V];
#pragma unroll
      for (int v = 0; v < V; ++v) {
        const int r = 64 * v + 8 * w + lr;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk)
          x[v][kk] = *reinterpret_cast<const f32x4*>(W + (int64_t)(p0 + r) * COLS + 4 * (lk + 8 * kk));
        n0[v] = st.renorm ? N0[p0 + r] : 1.f;
      }
      __syncthreads();
#pragma unroll
      for (int v = 0; v < V; ++v) {
        const int r = 64 * v + 8 * w + lr;
        float ss = 0.f;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          x[v][kk] += *reinterpret_cast<const f32x4*>(stg + off(r, 4 * (lk + 8 * kk)));
          ss += x[v][kk][0] * x[v][kk][0] + x[v][kk][1] * x[v][kk][1] +
                x[v][kk][2] * x[v][kk][2] + x[v][kk][3] * x[v][kk][3];
        }
        ss += __shfl_xor(ss, 1);
        ss += __shfl_xor(ss, 2);
        ss += __shfl_xor(ss, 4);
        if (st.nonfinite != nullptr && lk == 0 && !(ss <= 3.402823466e38f)) atomicOr(st.nonfinite, 1);
        const float f = st.renorm ? n0[v] / (sqrtf(ss) + st.eps) : 1.f;
        const int64_t row = (int64_t)(p0 + r) * COLS;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          const f32x4 y = x[v][kk] * f;
          *reinterpret_cast<f32x4*>(W + row + 4 * (lk + 8 * kk)) = st.renorm == 2 ? x[v][kk] : y;
          st4(S + row + 4 * (lk + 8 * kk), y[0], y[1], y[2], y[3]);
          *reinterpret_cast<f32x4*>(stg + off(r, 4 * (lk + 8 * kk))) = y;  // own slot
        }
      }
      __syncthreads();
      // W2^T[j][p0 + 8 s .. + 7]: eight 16-byte stores per thread
      const int j = opaque(tid) % COLS, s0 = (tid / COLS) * 8;
#pragma unroll 1
      for (int q = 0; q < 8; ++q) {
        const int r0 = 8 * (s0 + q);
        bf16x8 b;
#pragma unroll
        for (int x8 = 0; x8 < 8; ++x8) b[x8] = (bf16)stg[off(r0 + x8, j)];
        *reinterpret_cast<bf16x8*>(St + (int64_t)j * 128 + p0 + r0) = b;
      }
    }
  }
}

// Newton-Schulz of the write and a read that uses the weights this write
// replaces, in one launch: workgroups [0, count) run the matrices, the rest
// the read's tiles (d = 128).  Workgroups start in index order, so the
// matrices get their compute units first and the read fills the others -
// the Newton-Schulz launch alone holds one workgroup per matrix and leaves
// most compute units idle.
template <int COLS>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void k_ns_apply(NsGrad gr, float eps, int shift_from, int count, NsStep st, ApplyArgs a) {
  extern __shared__ __attribute__((aligned(16))) bf16 lds_f[];
  const int b = blockIdx.x;
  if (b < count) ns_r128_block<COLS, true>(NsIn{}, gr, nullptr, eps, shift_from, b, lds_f, st);
  else apply_block<bf16, 128, 32, 8>(a, xcd_logical_id(b - count, (int)gridDim.x - count), lds_f);
}

// Dynamic LDS of the fused launch: the Newton-Schulz block (X copy + A),
// the staging of its gradient prologue and step epilogue (8 waves x [32][128]
// fp32), and the read's tiles - whichever is largest.
template <int COLS>
constexpr size_t ns_apply_lds() {
  constexpr size_t lns = (size_t)(128 * COLS + 128 * 128) * sizeof(bf16);
  constexpr size_t lstep = (size_t)8 * 32 * 128 * sizeof(float);
  constexpr size_t lap = (size_t)ApplyLds<bf16, 128>::ELEMS * sizeof(bf16);
  constexpr size_t m = lns > lstep ? lns : lstep;
  return m > lap ? m : lap;
}
static_assert(ns_apply_lds<512>() <= 160 * 1024 && ns_apply_lds<256>() <= 160 * 1024, "LDS");
// the W2 step of the epilogue stages up to 128 rows of COLS fp32
static_assert((size_t)64 * 512 * 4 <= ns_apply_lds<512>() && (size_t)128 * 256 * 4 <= ns_apply_lds<256>(),
              "W2 staging");

template <int COLS>
static hipError_t run_ns_apply(int count, const NsGrad& g, float eps, int shift_from,
                               const NsStep& st, const ApplyArgs& a, hipStream_t s) {
  constexpr size_t lds = ns_apply_lds<COLS>();
  hipError_t e = allow_dynamic_lds(reinterpret_cast<const void*>(&k_ns_apply<COLS>), (int)lds);
  if (e != hipSuccess) return e;
  const int64_t napply = a.n_tok > 0 ? (a.n_tok + 255) / 256 * a.bh : 0;
  hipLaunchKernelGGL((k_ns_apply<COLS>), dim3((unsigned)(count + napply)), dim3(512), lds, s, g,
                     eps, shift_from, count, st, a);
  return hipGetLastError();
}

template <int COLS>
static hipError_t run_ns_r128(int count, NsIn g, float* u, float eps, int shift_from,
                              hipStream_t s) {
  const size_t lds = (size_t)(128 * COLS + 128 * 128) * sizeof(bf16);
  hipError_t e = allow_dynamic_lds(reinterpret_cast<const void*>(&k_ns_r128<COLS>), (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_ns_r128<COLS>), dim3(count), dim3(512), lds, s, g, u, eps, shift_from);
  return hipGetLastError();
}

template <int ROWS, int COLS, int NW, bool XG>
static hipError_t run_ns_fused(int count, NsIn g, float* u, float eps, int shift_from,
                               hipStream_t s) {
  const size_t lds = (size_t)ns_lds_elems(ROWS, COLS) * sizeof(bf16);
  hipError_t e = allow_dynamic_lds(reinterpret_cast<const void*>(&k_ns_fused<ROWS, COLS, NW, XG>),
                                   (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_ns_fused<ROWS, COLS, NW, XG>), dim3(count), dim3(NW * 64), lds, s, g, u, eps,
                     shift_from);
  return hipGetLastError();
}

// Returns hipErrorNotSupported when no fused variant covers the shape.
hipError_t launch_ns_step_apply(int count, int rows, int cols, const NsGrad& g, float eps,
                                int shift_from, const NsStep& st, const ApplyArgs& a,
                                hipStream_t s) {
  if (rows != 128 || (a.n_tok > 0 && a.d != 128) || count != 3 * st.bh || g.bh != st.bh ||
      g.nsplit < 1)
    return hipErrorNotSupported;
  if (cols == 512) return run_ns_apply<512>(count, g, eps, shift_from, st, a, s);
  if (cols == 256) return run_ns_apply<256>(count, g, eps, shift_from, st, a, s);
  return hipErrorNotSupported;
}

__global__ void k_copy16(f32x4* __restrict__ dst, const f32x4* __restrict__ src, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = src[i];
}

hipError_t launch_copy16(void* dst, const void* src, int64_t bytes, hipStream_t s) {
  const int64_t n = bytes / 16;
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_copy16, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                     reinterpret_cast<f32x4*>(dst), reinterpret_cast<const f32x4*>(src), n);
  return hipGetLastError();
}

hipError_t launch_ns_fused(int count, int rows, int cols, NsIn g, float* u, float eps,
                           int shift_from, hipStream_t s) {
  if (rows == 128 && cols == 512) return run_ns_r128<512>(count, g, u, eps, shift_from, s);
  if (rows == 128 && cols == 256) return run_ns_r128<256>(count, g, u, eps, shift_from, s);
  if (rows == 64 && cols == 256) return run_ns_fused<64, 256, 16, false>(count, g, u, eps, shift_from, s);
  if (rows == 64 && cols == 512) return run_ns_fused<64, 512, 16, true>(count, g, u, eps, shift_from, s);
  return hipErrorNotSupported;
}

}  // namespace lact
