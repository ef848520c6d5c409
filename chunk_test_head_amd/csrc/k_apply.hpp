// Read (apply) workgroup body and the LDS layouts of the MFMA operand tiles.
//
// Read (LaCT rebuttal page, apply step of both pseudocode functions):
//   o_t = W2 (silu(W1 q_t) * (W3 q_t)).
#pragma once
#include "lact_internal.hpp"
#include "mfma.hpp"

namespace lact {

// ------------------------------------------------------------ LDS layout --
// gfx950 LDS banks, as measured with the bank-conflict counter: the banks
// repeat every 256 bytes for reads; a 16-byte read (ds_read_b128) is served
// in four passes of 16 lanes, lanes 32 h + 4 j .. +3 (j = 0..7) going to pass
// (h, parity of j); an 8-byte read (plain or transposing) in two passes of 32
// lanes; a 16-byte write in eight passes of 8 lanes over 128 bytes.  A pass
// is conflict-free when its lanes touch distinct bank words.
//
// Token (or weight) rows of D bf16 are stored unpadded with the 16-byte chunk
// q of row r at chunk q ^ s(r):
//   D >= 128:  s(r) = 2 (r % 8)        D = 64:  s(r) = 2 ((r / 2) % 4).
// With it the three access patterns of the MFMA operands are conflict-free:
// 16-byte row reads (lane (c, g) = (lane % 16, lane / 16) reads row c, chunk
// 4 ks + g), 8-byte transposing reads (row 4 g + c / 4, columns
// 16 it + 4 (c % 4) ..) and 16-byte staging writes of consecutive chunks.
template <int D>
__device__ __forceinline__ int swz_key(int r) {
  return D >= 128 ? (r & 7) << 1 : ((r >> 1) & 3) << 1;
}
template <int D>
__device__ __forceinline__ int swz(int r, int col) {
  return r * D + (((col >> 3) ^ swz_key<D>(r)) << 3) + (col & 7);
}
// Padded alternative for token tiles: rows of D bf16 stored at a pitch of
// D + 16 elements (32 bytes of padding) are conflict-free for the same three
// patterns, and every fragment address is a per-lane base plus a
// compile-time offset (no per-fragment XOR, no address registers per tile).
template <int D>
__device__ __forceinline__ int tpad(int r, int col) {
  return r * (D + 16) + col;
}
// Rows of 32 bf16 (64 bytes: a W2 block row, the block's hidden units in the
// kappa run order): the 8-byte slot k stored at chunk (k / 2) ^ t(r), half
// k % 2, with t(r) = (r / 2) % 2 + 2 ((r / 8) % 2) - conflict-free for the
// 16-byte A-fragment reads (lane (c, g): row c, slots 2g, 2g+1) and for the
// 8-byte staging writes (4 lanes per row).
__device__ __forceinline__ int swz32(int r, int k) {
  return r * 32 + ((((k >> 1) ^ (((r >> 1) & 1) | (((r >> 3) & 1) << 1)))) << 3) + 4 * (k & 1);
}

// ----------------------------------------------------------------- apply --
// One workgroup = WAVES waves x NTW tokens of one head.  The hidden dim is
// streamed in blocks of 32 rows: W1/W3 rows and W2 columns of the block are
// staged in LDS (double buffered) and shared by all waves; each wave keeps its
// q fragments and its output accumulators (o^T, d x NTW) in registers.
template <class T, int D>
struct ApplyLds {
  static constexpr int HB = 32, V = 16 / sizeof(T);
  static constexpr bool BF = sizeof(T) == 2;
  static constexpr int P1 = BF ? D + 16 : D + V, P2 = BF ? HB : HB + 4;
  static constexpr int STAGE = 2 * HB * P1 + D * P2;
  static constexpr int SUB = (BF && D <= 128) ? 2 : 1;
  // three stage buffers where the waves of a SIMD run out of phase (the W2
  // block of a deferred product must outlive the next stage's staging)
  static constexpr int NBUF = (BF && D == 128) ? 3 : 2;
  static constexpr int ELEMS = NBUF * SUB * STAGE;
};

// Body of one workgroup: logical block lid (head-major tiles), LDS of
// ApplyLds<T, D>::ELEMS elements.
template <class T, int D, int NTW, int WAVES>
__device__ __forceinline__ void apply_block(const ApplyArgs& a, int lid, T* lds) {
  constexpr int NTH = WAVES * 64;
  constexpr int HB = 32;                 // hidden rows per stage
  constexpr int NT = NTW / 16;           // 16-token tiles per wave
  constexpr int KS = D / 32;             // K slabs over d
  constexpr int IT = D / 16;             // output feature tiles
  constexpr int V = 16 / sizeof(T);      // elements per 16-byte vector
  // W1/W3 block rows at a padded pitch (bf16: tpad, conflict-free)
  constexpr bool BF = sizeof(T) == 2;
  constexpr int P1 = BF ? D + 16 : D + V;  // LDS pitch of W1/W3 block rows
  // W2 block rows: the 32 hidden values of a row stored in kappa order (runs
  // of four: 0-3, 16-19, 4-7, 20-23, ...), so that the A fragment of lane
  // group g (hidden 4g..4g+3, 16+4g..16+4g+3) is one 16-byte read (bf16:
  // swz32 rows; fp32: padded rows)
  constexpr int P2 = BF ? HB : HB + 4;
  constexpr int STAGE = 2 * HB * P1 + D * P2;
  constexpr int NV1 = HB * D / V / NTH;  // 16-byte vectors per thread (W1 / W3)
  constexpr int NV2 = D * HB / V / NTH;  // (W2)
  static_assert(NV1 * V * NTH == HB * D && NV2 * V * NTH == D * HB, "stage split");

  // SUB hidden blocks per barrier (bf16, d <= 128: LDS allows two), double
  // buffered: slots (stage % 2) SUB + sub
  constexpr int SUB = ApplyLds<T, D>::SUB;
  static_assert(ApplyLds<T, D>::STAGE == STAGE, "layout");

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = lane & 15, g = lane >> 4;
  const int tiles = (int)((a.n_tok + (int64_t)WAVES * NTW - 1) / ((int64_t)WAVES * NTW));
  const int head = lid / tiles, tile = lid % tiles;
  if (head >= a.bh) return;
  const int dh = a.dh;
  const int64_t tok0 = (int64_t)tile * WAVES * NTW + (int64_t)wave * NTW;

  const T* q = reinterpret_cast<const T*>(a.q) + (int64_t)head * a.q_sbh;
  T* o = reinterpret_cast<T*>(a.o) + (int64_t)head * a.o_sbh;
  const T* sb = reinterpret_cast<const T*>(a.sh.base) + (int64_t)head * a.sh.per_head;
  const T* w1 = sb + a.sh.off_w1;
  const T* w3 = sb + a.sh.off_w3;
  const T* w2 = sb + a.sh.off_w2;

  // q^T fragments (B operand, K = d): lane holds q[token 16tt + c][32ks + 8g ..]
  frag_t<T> qf[NT][KS];
#pragma unroll
  for (int tt = 0; tt < NT; ++tt) {
    const int64_t t = tok0 + 16 * tt + c;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (t < a.n_tok) {
        qf[tt][ks] = ld8(q + t * a.q_st + 32 * ks + 8 * g);
      } else {
#pragma unroll
        for (int m = 0; m < 8; ++m) qf[tt][ks][m] = to_t<T>(0.f);
      }
    }
  }

  f32x4 acc[IT][NT];
#pragma unroll
  for (int it = 0; it < IT; ++it)
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) acc[it][tt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // 16-byte staging vectors as native vector types (register-allocated;
  // a struct type would be copied through a stack slot)
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
  u32x4 r1[NV1], r3[NV1], r2[NV2];
  // stage jb: W1 / W3 rows [jb HB, +HB) (contiguous) and W2 columns (rows of
  // HB elements at pitch dh), as 16-byte vectors
#define LACT_APPLY_GLOAD(JB)                                                        \
  {                                                                                 \
    _Pragma("unroll") for (int x = 0; x < NV1; ++x) {                               \
      const int vi = tid + x * NTH;                                                 \
      r1[x] = *reinterpret_cast<const u32x4*>(w1 + (int64_t)(JB) * HB * D + (int64_t)vi * V); \
      r3[x] = *reinterpret_cast<const u32x4*>(w3 + (int64_t)(JB) * HB * D + (int64_t)vi * V); \
    }                                                                               \
    _Pragma("unroll") for (int x = 0; x < NV2; ++x) {                               \
      const int vi = tid + x * NTH;                                                 \
      r2[x] = *reinterpret_cast<const u32x4*>(w2 + (int64_t)(vi / (HB / V)) * dh + (JB) * HB + (vi % (HB / V)) * V); \
    }                                                                               \
  }
#define LACT_APPLY_LSTORE(BUF)                                                      \
  {                                                                                 \
    T* s1_ = lds + (BUF) * STAGE;                                                   \
    T* s3_ = s1_ + HB * P1;                                                         \
    T* s2_ = s3_ + HB * P1;                                                         \
    _Pragma("unroll") for (int x = 0; x < NV1; ++x) {                               \
      const int vi = tid + x * NTH;                                                 \
      const int row = vi / (D / V), col = (vi % (D / V)) * V;                       \
      const int o_ = row * P1 + col;                                                \
      *reinterpret_cast<u32x4*>(s1_ + o_) = r1[x];                                  \
      *reinterpret_cast<u32x4*>(s3_ + o_) = r3[x];                                  \
    }                                                                               \
    _Pragma("unroll") for (int x = 0; x < NV2; ++x) {                               \
      const int vi = tid + x * NTH;                                                 \
      const int row = vi / (HB / V), col = (vi % (HB / V)) * V;                     \
      if constexpr (sizeof(T) == 2) {                                               \
        /* hidden col..col+7 = runs 2q, 2q+1 (q = col / 8) -> slots kpos */         \
        const int r0_ = col >> 2, r1_ = r0_ + 1;                                    \
        const int k0_ = 2 * (r0_ & 3) + (r0_ >> 2), k1_ = 2 * (r1_ & 3) + (r1_ >> 2); \
        *reinterpret_cast<u32x2*>(s2_ + swz32(row, k0_)) = r2[x].xy;                  \
        *reinterpret_cast<u32x2*>(s2_ + swz32(row, k1_)) = r2[x].zw;                  \
      } else {                                                                      \
        *reinterpret_cast<u32x4*>(s2_ + row * P2 + col) = r2[x];                    \
      }                                                                             \
    }                                                                               \
  }

  // Three stage buffers (d = 128, 8 waves): waves WAVES/2.. (sharing their
  // SIMDs with waves 0..WAVES/2-1) run the output product of a stage's second
  // block at the start of the next stage, so the two waves of a SIMD are out
  // of phase (one's SiLU, VALU, overlaps the other's MFMA phases).
  constexpr int NBUF = ApplyLds<T, D>::NBUF;
  constexpr bool SKEW = NBUF == 3 && SUB == 2 && WAVES == 8;
  const bool late = SKEW && wave >= WAVES / 2;
  const int NB = dh / HB;
  const int nst = (NB + SUB - 1) / SUB;
  frag_t<T> hf[NT];
  // o^T[feature][token] += W2[:, block] h^T, W2 block of slot BUF
#define LACT_APPLY_OPROD(BUF)                                                       \
  {                                                                                 \
    const T* s2_ = lds + (BUF) * STAGE + 2 * HB * P1;                               \
    _Pragma("unroll") for (int it = 0; it < IT; ++it) {                             \
      frag_t<T> a2;                                                                 \
      if constexpr (BF) {                                                           \
        a2 = ld8(s2_ + swz32(16 * it + c, 2 * g));                                  \
      } else {                                                                      \
        const T* row = s2_ + (16 * it + c) * P2;                                    \
        a2 = ld4x2(row + 4 * g, row + 16 + 4 * g);                                  \
      }                                                                             \
      _Pragma("unroll") for (int tt = 0; tt < NT; ++tt) mma(acc[it][tt], a2, hf[tt]); \
    }                                                                               \
  }
#pragma unroll
  for (int sb = 0; sb < SUB; ++sb)
    if (sb < NB) {
      LACT_APPLY_GLOAD(sb);
      LACT_APPLY_LSTORE(sb);
    }
  wait_global_loads();  // the q fragments: complete before the loop
  __syncthreads();
  for (int st = 0; st < nst; ++st) {
    if (late && st > 0) LACT_APPLY_OPROD(((st + NBUF - 1) % NBUF) * SUB + SUB - 1);  // deferred
#pragma unroll
    for (int sb = 0; sb < SUB; ++sb) {
      const int jb = st * SUB + sb, jn = jb + SUB;
      const int buf = (st % NBUF) * SUB + sb, nbuf = ((st + 1) % NBUF) * SUB + sb;
      if (jn < NB) LACT_APPLY_GLOAD(jn);
      if (jb < NB) {
        const T* s1 = lds + buf * STAGE;
        const T* s3 = s1 + HB * P1;
        // gate / up pre-activations, transposed: P^T[hidden][token]
        f32x4 P[2][NT], U[2][NT];
#pragma unroll
        for (int jt = 0; jt < 2; ++jt)
#pragma unroll
          for (int tt = 0; tt < NT; ++tt) {
            P[jt][tt] = f32x4{0.f, 0.f, 0.f, 0.f};
            U[jt][tt] = f32x4{0.f, 0.f, 0.f, 0.f};
          }
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
          for (int jt = 0; jt < 2; ++jt) {
            const int o1 = (16 * jt + c) * P1 + 32 * ks + 8 * g;
            const frag_t<T> a1 = ld8(s1 + o1);
            const frag_t<T> a3 = ld8(s3 + o1);
#pragma unroll
            for (int tt = 0; tt < NT; ++tt) {
              mma(P[jt][tt], a1, qf[tt][ks]);
              mma(U[jt][tt], a3, qf[tt][ks]);
            }
          }
        }
        // h = silu(P) * U, packed as the B operand (K = the 32 hidden rows).
#pragma unroll
        for (int tt = 0; tt < NT; ++tt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float p0 = P[0][tt][i], p1 = P[1][tt][i];
            hf[tt][i] = to_t<T>(p0 * sigmoid_fast(p0) * U[0][tt][i]);
            hf[tt][4 + i] = to_t<T>(p1 * sigmoid_fast(p1) * U[1][tt][i]);
          }
        if (!(late && sb == SUB - 1)) LACT_APPLY_OPROD(buf);
      }
      if (jn < NB) LACT_APPLY_LSTORE(nbuf);
    }
    __syncthreads();
  }
  // the last stage's second block (late waves), if it exists
  if (late && nst > 0 && (nst - 1) * SUB + SUB - 1 < NB) LACT_APPLY_OPROD(((nst - 1) % NBUF) * SUB + SUB - 1);
#undef LACT_APPLY_OPROD
#undef LACT_APPLY_GLOAD
#undef LACT_APPLY_LSTORE

#pragma unroll
  for (int tt = 0; tt < NT; ++tt) {
    const int64_t t = tok0 + 16 * tt + c;
    if (t < a.n_tok) {
#pragma unroll
      for (int it = 0; it < IT; ++it)
        st4(o + t * a.o_st + 16 * it + 4 * g, acc[it][tt][0], acc[it][tt][1], acc[it][tt][2],
            acc[it][tt][3]);
    }
  }
}

// ------------------------------------------------ apply, d = 256, solo --
// One wave per SIMD holding 32 tokens over all D features: q fragments
// (D / 4 VGPRs) and the o^T accumulators (D / 2, in AGPRs) - no partial
// exchange and no duplicated silu(g) u as when two waves per SIMD split the
// features (measured 14-16 % slower).  4 waves = 128 tokens per workgroup.
// The hidden dim is streamed in blocks of 32 through two LDS stages of the
// W1 / W3 block rows (padded pitch tpad<D>) and two of the W2 block (swz32),
// 100 KiB, staged by buffer loads (uniform descriptors, per-lane 32-bit
// offsets) so that neither the loads nor the LDS stores and fragment reads
// spend per-lane address arithmetic inside the loop; software-pipelined:
// iteration jb runs the gate / up contractions of block jb + 1 with
// h = silu(g) u of block jb between them, then o^T += W2[:, block jb] h^T
// with the staging stores (W1 / W3 of block jb + 2, W2 of block jb + 1)
// between those; fragment reads two steps ahead, the order held by
// scheduling fences.  (Three stages of both, 150 KiB, measured 1 % slower
// on 8 heads x 49152 tokens.)
template <int D>
struct ApplySoloLds {
  static constexpr int HB = 32;
  static constexpr int S13 = 2 * HB * (D + 16), S2 = D * HB;
  static constexpr int ELEMS = 2 * (S13 + S2);
  // stage b (0, 1) of the W1 / W3 rows and of the W2 block (elements)
  static constexpr int w13(int b) { return b * S13; }
  static constexpr int w2(int b) { return 2 * S13 + b * S2; }
};

// Body of one workgroup (256 threads, one wave per SIMD): logical block lid
// (head-major tiles of 128 tokens), LDS of ApplySoloLds<D>::ELEMS elements.
template <int D>
__device__ __forceinline__ void apply_solo_block(const ApplyArgs& a, int lid, bf16* lds) {
  constexpr int NTH = 256, HB = 32;
  constexpr int KS = D / 32;     // K slabs of the gate / up contractions
  constexpr int IT = D / 16;     // output feature tiles
  constexpr int G1 = HB * D;     // one W1 / W3 block in memory, [HB][D]
  constexpr int S1 = HB * (D + 16);  // the same in LDS (tpad)
  constexpr int S2 = D * HB;     // W2 block, [D][HB] (kappa slot order)
  constexpr int NV1 = G1 / 8 / NTH, NV2 = S2 / 8 / NTH;
  constexpr int NST = 2 * KS;    // gate / up steps (K slab, hidden tile)
  // fragment buffers of the gate / up and of the W2 contractions (reads
  // FR - 1, WR - 1 steps ahead; 4 and 5 measured no faster)
  constexpr int FR = 3, WR = 3;
  static_assert(NV1 * 8 * NTH == G1 && NV2 * 8 * NTH == S2 && NTH % (D / 8) == 0, "stage split");
  static_assert(NST == 16 && 2 * NV1 + 2 * NV2 <= IT, "step plan");
  using LY = ApplySoloLds<D>;
  static_assert(LY::S13 == 2 * S1 && LY::S2 == S2, "layout");

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = lane & 15, g = lane >> 4;
  const int tiles = (int)((a.n_tok + 127) / 128);
  const int head = lid / tiles, tile = lid % tiles;
  if (head >= a.bh) return;
  const int dh = a.dh;
  const int64_t tok0 = (int64_t)tile * 128 + 32 * wave;

  const bf16* q = reinterpret_cast<const bf16*>(a.q) + (int64_t)head * a.q_sbh;
  bf16* o = reinterpret_cast<bf16*>(a.o) + (int64_t)head * a.o_sbh;
  const bf16* sb = reinterpret_cast<const bf16*>(a.sh.base) + (int64_t)head * a.sh.per_head;
  const bf16* w1 = sb + a.sh.off_w1;
  const bf16* w3 = sb + a.sh.off_w3;
  const bf16* w2 = sb + a.sh.off_w2;

  // q^T fragments (B operand, K = features): token 16 tt + c, features 32 ks + 8 g ..
  bf16x8 qf[2][KS];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    const int64_t t = tok0 + 16 * tt + c;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (t < a.n_tok) {
        qf[tt][ks] = ld8(q + t * a.q_st + 32 * ks + 8 * g);
      } else {
#pragma unroll
        for (int m = 0; m < 8; ++m) qf[tt][ks][m] = (bf16)0.f;
      }
    }
  }
  f32x4 acc[IT][2];
#pragma unroll
  for (int it = 0; it < IT; ++it)
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) acc[it][tt] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int NB = dh / HB;
  bf16x8 r1[NV1], r3[NV1], r2[NV2];
  // block JB of W1 / W3 rows (contiguous: vector x of a thread is elements
  // 8 (tid + x NTH) ..) and of W2 columns (vector x: row tid / 4 + 64 x,
  // columns JB HB + 8 (tid % 4) ..), through one descriptor per matrix and
  // block: per-lane offsets go1 / go2, the x part uniform
  const uint32_t go1 = (uint32_t)tid * 16u;
  const uint32_t go2 = (uint32_t)(((tid >> 2) * dh + (tid & 3) * 8) * 2);
  const uint32_t n2 = (uint32_t)(((D - 1) * dh + HB) * 2);
#define LACT_AS_GLOAD13(JB)                                                            \
  {                                                                                    \
    const __amdgpu_buffer_rsrc_t b1_ = buf_rsrc(w1 + (int64_t)(JB) * G1, G1 * 2);      \
    const __amdgpu_buffer_rsrc_t b3_ = buf_rsrc(w3 + (int64_t)(JB) * G1, G1 * 2);      \
    _Pragma("unroll") for (int x = 0; x < NV1; ++x) {                                  \
      r1[x] = buf_ld8(b1_, go1, x * NTH * 16);                                         \
      r3[x] = buf_ld8(b3_, go1, x * NTH * 16);                                         \
    }                                                                                  \
  }
#define LACT_AS_GLOAD2(JB)                                                             \
  {                                                                                    \
    const __amdgpu_buffer_rsrc_t b2_ = buf_rsrc(w2 + (int64_t)(JB) * HB, n2);          \
    _Pragma("unroll") for (int x = 0; x < NV2; ++x) r2[x] = buf_ld8(b2_, go2, x * (NTH / 4) * dh * 2); \
  }
  // staging store number X of the block (X < 2 NV1 + 2 NV2), at a per-lane
  // base plus an immediate: W1 / W3 vector x is row tid / (D / 8) + x RX of
  // the padded block; W2 vector x is row tid / 4 + 64 x, whose swz32 key
  // repeats every 16 rows (slot pair ru = 2 (tid % 4) + half)
  constexpr int RX = NTH / (D / 8);
  const int so1 = opaque(tpad<D>(tid / (D / 8), (tid % (D / 8)) * 8));
  int so2[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int ru = 2 * (tid & 3) + h;
    so2[h] = opaque(swz32(tid >> 2, 2 * (ru & 3) + (ru >> 2)));
  }
#define LACT_AS_LSTORE1(S13_, S2_, X)                                                  \
  {                                                                                    \
    if ((X) < 2 * NV1) {                                                               \
      const int x_ = (X) >> 1;                                                         \
      bf16* d_ = (S13_) + so1 + (((X) & 1) ? S1 : 0) + x_ * RX * (D + 16);             \
      *reinterpret_cast<bf16x8*>(d_) = ((X) & 1) ? r3[x_] : r1[x_];                    \
    } else {                                                                           \
      const int y_ = (X) - 2 * NV1, x_ = y_ >> 1;                                      \
      bf16* s2_ = (S2_) + so2[y_ & 1] + x_ * (NTH / 4) * HB;                           \
      if ((y_ & 1) == 0)                                                               \
        *reinterpret_cast<bf16x4*>(s2_) = __builtin_shufflevector(r2[x_], r2[x_], 0, 1, 2, 3); \
      else                                                                             \
        *reinterpret_cast<bf16x4*>(s2_) = __builtin_shufflevector(r2[x_], r2[x_], 4, 5, 6, 7); \
    }                                                                                  \
  }

  // per-lane offsets (laundered: the stage is a runtime choice, every read
  // should be this base + an immediate): gate / up A fragments (row c,
  // features 8 g ..) and W2 A fragments (row c, slots 2 g, 2 g + 1)
  const int fo = opaque(tpad<D>(c, 8 * g));
  const int wo = opaque(swz32(c, 2 * g));
  f32x4 P[2][2], U[2][2];  // [hidden tile jt][token half tt]
  bf16x8 hf[2];
  // gate / up contractions of the block in stage BUF into Pn, Un; with BW,
  // h = silu(g) u of the previous block (Pc, Uc) between the steps
  auto forward = [&](int buf, f32x4 (&Pn)[2][2], f32x4 (&Un)[2][2], bool bw,
                     const f32x4 (&Pc)[2][2], const f32x4 (&Uc)[2][2]) {
#pragma unroll
    for (int jt = 0; jt < 2; ++jt)
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        Pn[jt][tt] = f32x4{0.f, 0.f, 0.f, 0.f};
        Un[jt][tt] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    const bf16* s1 = lds + opaque(LY::w13(buf) + fo);  // every read below: s1 + an immediate
    bf16x8 f1[FR], f3[FR];
    // step s = 2 ks + jt: rows 16 jt + c, features 32 ks + 8 g ..
#define LACT_AS_FRAG(S)                                                                \
  {                                                                                    \
    f1[(S) % FR] = ld8(s1 + 16 * ((S) & 1) * (D + 16) + 32 * ((S) >> 1));               \
    f3[(S) % FR] = ld8(s1 + S1 + 16 * ((S) & 1) * (D + 16) + 32 * ((S) >> 1));          \
  }
#pragma unroll
    for (int s_ = 0; s_ < FR - 1; ++s_) LACT_AS_FRAG(s_);
#pragma unroll
    for (int st = 0; st < NST; ++st) {
      if (st + FR - 1 < NST) LACT_AS_FRAG(st + FR - 1);
      const int jt = st & 1, ks = st >> 1;
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        mma(Pn[jt][tt], f1[st % FR], qf[tt][ks]);
        mma(Un[jt][tt], f3[st % FR], qf[tt][ks]);
      }
      if (bw) {
        // element (token half te, hidden tile je, row ie) of h: one per step
        const int te = st >> 3, je = (st >> 2) & 1, ie = st & 3;
        const float p = Pc[je][te][ie];
        hf[te][4 * je + ie] = (bf16)(p * sigmoid_fast(p) * Uc[je][te][ie]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#undef LACT_AS_FRAG
  };

  // Two stages each: the W1 / W3 rows of block b in their stage b % 2,
  // staged two iterations ahead (its gate / up run one iteration ahead of
  // its W2 contraction), the W2 block in its stage b % 2, staged one
  // iteration ahead: in iteration jb the gate / up read W1 / W3 stage
  // (jb + 1) % 2 and the W2 contraction W2 stage jb % 2, while the stores
  // fill W1 / W3 stage jb % 2 and W2 stage (jb + 1) % 2, whose last readers
  // were before the previous barrier.
  LACT_AS_GLOAD13(0);
  LACT_AS_GLOAD2(0);
#pragma unroll
  for (int x = 0; x < 2 * NV1 + 2 * NV2; ++x) LACT_AS_LSTORE1(lds + LY::w13(0), lds + LY::w2(0), x);
  LACT_AS_GLOAD13(min(1, NB - 1));
#pragma unroll
  for (int x = 0; x < 2 * NV1; ++x) LACT_AS_LSTORE1(lds + LY::w13(1), lds + LY::w2(1), x);
  __syncthreads();
  forward(0, P, U, false, P, U);
  for (int jb = 0; jb < NB; ++jb) {
    const int cb = jb % 2, nb = (jb + 1) % 2;
    // W1 / W3 of block jb + 2 and W2 of block jb + 1 (the last block again
    // at the end: its copy lands in a free stage)
    LACT_AS_GLOAD13(min(jb + 2, NB - 1));
    LACT_AS_GLOAD2(min(jb + 1, NB - 1));
    __builtin_amdgcn_sched_barrier(0);
    // ---- region 1: gate / up of block jb + 1 (past the last block: stale
    // stage, results unused) with h of block jb ----
    f32x4 Pn[2][2], Un[2][2];
    forward(nb, Pn, Un, true, P, U);
    // ---- region 2: o^T += W2[:, block jb] h^T, W2 reads two steps ahead,
    // the staging stores of W1 / W3 block jb + 2 and W2 block jb + 1
    // between them ----
    {
      const bf16* s2 = lds + opaque(LY::w2(cb) + wo);
      bf16* sl13 = lds + LY::w13(cb);
      bf16* sl2 = lds + LY::w2(nb);
      bf16x8 f2[WR];
#pragma unroll
      for (int i_ = 0; i_ < WR - 1; ++i_) f2[i_] = ld8(s2 + 16 * HB * i_);
#pragma unroll
      for (int it = 0; it < IT; ++it) {
        if (it + WR - 1 < IT) f2[(it + WR - 1) % WR] = ld8(s2 + 16 * HB * (it + WR - 1));
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) mma(acc[it][tt], f2[it % WR], hf[tt]);
        if (it < 2 * NV1 + 2 * NV2) LACT_AS_LSTORE1(sl13, sl2, it);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __syncthreads();
#pragma unroll
    for (int jt = 0; jt < 2; ++jt)
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        P[jt][tt] = Pn[jt][tt];
        U[jt][tt] = Un[jt][tt];
      }
  }
#undef LACT_AS_GLOAD13
#undef LACT_AS_GLOAD2
#undef LACT_AS_LSTORE1

#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    const int64_t t = tok0 + 16 * tt + c;
    if (t < a.n_tok) {
#pragma unroll
      for (int it = 0; it < IT; ++it)
        st4(o + t * a.o_st + 16 * it + 4 * g, acc[it][tt][0], acc[it][tt][1], acc[it][tt][2],
            acc[it][tt][3]);
    }
  }
}

}  // namespace lact
