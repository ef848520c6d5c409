// Fused SwiGLU fast-weight kernels: read (apply) and the chunk gradient.
//
// Read (LaCT rebuttal page, apply step of both pseudocode functions):
//   o_t = W2 (silu(W1 q_t) * (W3 q_t)).
// Write gradient (same page, "compute the gradient" block; summary page
// section 3.2, Eq. 4-5), descent direction of -sum_t eta_t <f_W(k_t), v_t>:
//   g = W1 k, u = W3 k, e = W2^T v, s = silu(g), h = s * u,
//   G2 += eta2 v h^T, G3 += eta3 (e * s) k^T, G1 += eta1 (e * u * silu'(g)) k^T.
// The hidden activations never leave the chip: they are produced in MFMA
// accumulators and consumed from registers by the next contraction.
#include "lact_internal.hpp"
#include "mfma.hpp"
#include "k_apply.hpp"

namespace lact {

// ----------------------------------------------------------------- apply --
// The workgroup body (apply_block) and the LDS layout helpers live in
// k_apply.hpp (shared with the fused Newton-Schulz + apply launch).
template <class T, int D, int NTW, int WAVES>
__global__ __launch_bounds__(WAVES * 64, 1) void k_apply(ApplyArgs a) {
  __shared__ __attribute__((aligned(16))) T lds[ApplyLds<T, D>::ELEMS];
  apply_block<T, D, NTW, WAVES>(a, xcd_logical_id(blockIdx.x, gridDim.x), lds);
}

// One 128-token tile per workgroup; or, launched with fewer workgroups than
// tiles (to leave compute units to Newton-Schulz on another stream), XCD x
// works through the tiles [x N / 8, (x + 1) N / 8) with its own
// workgroups, so that a head's weights stay in one L2.
template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void k_apply_solo(ApplyArgs a) {
  __shared__ __attribute__((aligned(16))) bf16 lds[ApplySoloLds<D>::ELEMS];
  const int total = (int)((a.n_tok + 127) / 128) * a.bh;
  const int nwg = (int)gridDim.x;
  if (nwg >= total) {
    apply_solo_block<D>(a, xcd_logical_id(blockIdx.x, nwg), lds);
  } else if (nwg < 8) {
    for (int t = blockIdx.x; t < total; t += nwg) apply_solo_block<D>(a, t, lds);
  } else {
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const int nw = (nwg - xcd + 7) >> 3;  // workgroups on this XCD
    const int t0 = (int)((int64_t)total * xcd / 8), t1 = (int)((int64_t)total * (xcd + 1) / 8);
    for (int t = t0 + slot; t < t1; t += nw) apply_solo_block<D>(a, t, lds);
  }
}

// ------------------------------------------------------------- gradient --
// One workgroup = WAVES waves x JW hidden units each, over one token split of
// one head.  Each wave keeps, for the whole token loop:
//   * its W1 / W3 / W2^T rows as B fragments (K = d),
//   * fp32 accumulators of G1^T, G3^T (d x JW) and G2 (d x JW).
// Per token tile (32 tokens): k, v are staged in LDS both row-major (A
// operand of the forward contractions, K = d) and transposed (A operand of
// the gradient contractions, K = tokens).  The forward results (tokens x
// hidden, in MFMA accumulators) go through the SwiGLU backward and the eta
// scaling in registers and feed the gradient contractions directly.
// PERCH: per-channel learning rates (eta1, eta3 [bh][*][D] scale k channel
// by channel, eta2 [bh][*][dh] the hidden activations): the gradient
// contractions of G1 and G3 then read (eta1 k)^T and (eta3 k)^T tiles staged
// beside k^T, and each token's eta2 values for the workgroup's hidden units
// are staged in LDS.
template <class T, int D, int JW, int WAVES, bool PERCH = false>
__global__ __launch_bounds__(WAVES * 64, 1) void k_grad(GradArgs a) {
  constexpr int NTH = WAVES * 64;
  constexpr int NT = 32;                 // tokens per tile (one K slab)
  constexpr int KS = D / 32;
  constexpr int JT = JW / 16;
  constexpr int IT = D / 16;
  constexpr int V = 16 / sizeof(T);
  constexpr int PR = D + V;              // pitch of row-major k / v tiles
  constexpr int PT = NT + 8;             // pitch of transposed tiles (elements)
  constexpr int NVT = NT * D / V;        // 16-byte vectors per tile
  static_assert(NVT % NTH == 0 || NTH % NVT == 0, "tile split");

  __shared__ __attribute__((aligned(16))) T sK[NT * PR];
  __shared__ __attribute__((aligned(16))) T sV[NT * PR];
  __shared__ __attribute__((aligned(16))) T sKt[D * PT];
  __shared__ __attribute__((aligned(16))) T sVt[D * PT];
  __shared__ float sEta[3][NT];
  constexpr int WB = WAVES * JW;         // hidden units per workgroup
  __shared__ __attribute__((aligned(16))) T sK1t[PERCH ? D * PT : 1];
  __shared__ __attribute__((aligned(16))) T sK3t[PERCH ? D * PT : 1];
  __shared__ float sE2[PERCH ? NT * WB : 1];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = lane & 15, g = lane >> 4;
  const int hblocks = (a.dh + WAVES * JW - 1) / (WAVES * JW);
  const int lid = xcd_logical_id(blockIdx.x, gridDim.x);
  // logical id -> (head, split, hidden block); hidden blocks of one head and
  // split are neighbours so they share k / v tiles in L2.
  const int hb = lid % hblocks;
  const int rest = lid / hblocks;
  const int split = rest % a.nsplit;
  const int head = rest / a.nsplit;
  if (head >= a.bh) return;
  const int64_t s0 = (int64_t)split * a.split_len;
  const int64_t s1 = (s0 + a.split_len < a.n_tok) ? s0 + a.split_len : a.n_tok;
  const int jw0 = hb * WAVES * JW + wave * JW;
  const bool active = jw0 < a.dh;  // dh need not fill the last block

  const T* kp = reinterpret_cast<const T*>(a.k) + (int64_t)head * a.k_sbh;
  const T* vp = reinterpret_cast<const T*>(a.v) + (int64_t)head * a.v_sbh;
  // per token (or, PERCH, per token and channel: eta_sbh counts tokens)
  const float* e1 = a.eta1 + (int64_t)head * a.eta_sbh * (PERCH ? D : 1);
  const float* e3 = a.eta3 + (int64_t)head * a.eta_sbh * (PERCH ? D : 1);
  const float* e2 = a.eta2 + (int64_t)head * a.eta_sbh * (PERCH ? a.dh : 1);
  const T* sb = reinterpret_cast<const T*>(a.sh.base) + (int64_t)head * a.sh.per_head;
  const T* w1 = sb + a.sh.off_w1;
  const T* w3 = sb + a.sh.off_w3;
  const T* w2t = sb + a.sh.off_w2t;

  // Weight B fragments: lane holds W[j = jw0 + 16jt + c][32ks + 8g ..].
  frag_t<T> b1[JT][KS], b3[JT][KS], b2[JT][KS];
#pragma unroll
  for (int jt = 0; jt < JT; ++jt)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int jrow = active ? jw0 + 16 * jt + c : c;  // idle waves read row c
      const int64_t off = (int64_t)jrow * D + 32 * ks + 8 * g;
      b1[jt][ks] = ld8(w1 + off);
      b3[jt][ks] = ld8(w3 + off);
      b2[jt][ks] = ld8(w2t + off);
    }
  wait_global_loads();

  f32x4 G1[IT][JT], G3[IT][JT], G2[IT][JT];
#pragma unroll
  for (int it = 0; it < IT; ++it)
#pragma unroll
    for (int jt = 0; jt < JT; ++jt) {
      G1[it][jt] = f32x4{0.f, 0.f, 0.f, 0.f};
      G3[it][jt] = f32x4{0.f, 0.f, 0.f, 0.f};
      G2[it][jt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

  for (int64_t t0 = s0; t0 < s1; t0 += NT) {
    // ---- stage the token tile (zero beyond the split end) ----
    for (int vi = tid; vi < NVT; vi += NTH) {
      const int r = vi / (D / V), col = (vi % (D / V)) * V;
      const int64_t t = t0 + r;
      uint4 kv = uint4{0u, 0u, 0u, 0u}, vv = uint4{0u, 0u, 0u, 0u};
      if (t < s1) {
        kv = *reinterpret_cast<const uint4*>(kp + t * a.k_st + col);
        vv = *reinterpret_cast<const uint4*>(vp + t * a.v_st + col);
      }
      *reinterpret_cast<uint4*>(sK + r * PR + col) = kv;
      *reinterpret_cast<uint4*>(sV + r * PR + col) = vv;
      const T* ke = reinterpret_cast<const T*>(&kv);
      const T* ve = reinterpret_cast<const T*>(&vv);
#pragma unroll
      for (int e = 0; e < V; ++e) {
        sKt[(col + e) * PT + r] = ke[e];
        sVt[(col + e) * PT + r] = ve[e];
      }
      if constexpr (PERCH) {
#pragma unroll
        for (int e = 0; e < V; ++e) {
          const float x1 = t < s1 ? e1[t * D + col + e] : 0.f;
          const float x3 = t < s1 ? e3[t * D + col + e] : 0.f;
          sK1t[(col + e) * PT + r] = to_t<T>(x1 * to_f(ke[e]));
          sK3t[(col + e) * PT + r] = to_t<T>(x3 * to_f(ke[e]));
        }
      }
    }
    if constexpr (PERCH) {
      for (int x = tid; x < NT * WB; x += NTH) {
        const int r = x / WB, jj = x % WB;
        const int64_t t = t0 + r;
        const int j = hb * WB + jj;
        sE2[x] = (t < s1 && j < a.dh) ? e2[t * a.dh + j] : 0.f;
      }
    }
    if (!PERCH && tid < NT) {
      const int64_t t = t0 + tid;
      const bool in = t < s1;
      sEta[0][tid] = in ? e1[t] : 0.f;
      sEta[1][tid] = in ? e3[t] : 0.f;
      sEta[2][tid] = in ? e2[t] : 0.f;
    }
    __syncthreads();
    if (active) {
    // ---- forward on keys / back-prop of v: tokens x hidden ----
    f32x4 P[2][JT], U[2][JT], E[2][JT];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int jt = 0; jt < JT; ++jt) {
        P[tt][jt] = f32x4{0.f, 0.f, 0.f, 0.f};
        U[tt][jt] = f32x4{0.f, 0.f, 0.f, 0.f};
        E[tt][jt] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const frag_t<T> ak = ld8(sK + (16 * tt + c) * PR + 32 * ks + 8 * g);
        const frag_t<T> av = ld8(sV + (16 * tt + c) * PR + 32 * ks + 8 * g);
#pragma unroll
        for (int jt = 0; jt < JT; ++jt) {
          mma(P[tt][jt], ak, b1[jt][ks]);
          mma(U[tt][jt], ak, b3[jt][ks]);
          mma(E[tt][jt], av, b2[jt][ks]);
        }
      }

    // ---- SwiGLU backward + eta, packed as B operands (K = 32 tokens) ----
    frag_t<T> fh[JT], fu[JT], fg[JT];
#pragma unroll
    for (int jt = 0; jt < JT; ++jt)
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * tt + 4 * g + i;   // token row inside the tile
          const float p = P[tt][jt][i], u = U[tt][jt][i], e = E[tt][jt][i];
          const float sg = sigmoidf_(p);
          const float sl = p * sg;
          const float dsl = sg * (1.f + p * (1.f - sg));
          if constexpr (PERCH) {
            fh[jt][4 * tt + i] = to_t<T>(sE2[r * WB + wave * JW + 16 * jt + c] * sl * u);
            fu[jt][4 * tt + i] = to_t<T>(e * sl);
            fg[jt][4 * tt + i] = to_t<T>(e * u * dsl);
          } else {
            fh[jt][4 * tt + i] = to_t<T>(sEta[2][r] * sl * u);
            fu[jt][4 * tt + i] = to_t<T>(sEta[1][r] * e * sl);
            fg[jt][4 * tt + i] = to_t<T>(sEta[0][r] * e * u * dsl);
          }
        }

    // ---- gradient contractions over the tile's tokens ----
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const T* kr = sKt + (16 * it + c) * PT;
      const T* vr = sVt + (16 * it + c) * PT;
      const frag_t<T> avt = ld4x2(vr + 4 * g, vr + 16 + 4 * g);
      if constexpr (PERCH) {
        const T* k1 = sK1t + (16 * it + c) * PT;
        const T* k3 = sK3t + (16 * it + c) * PT;
        const frag_t<T> ak1 = ld4x2(k1 + 4 * g, k1 + 16 + 4 * g);
        const frag_t<T> ak3 = ld4x2(k3 + 4 * g, k3 + 16 + 4 * g);
#pragma unroll
        for (int jt = 0; jt < JT; ++jt) {
          mma(G1[it][jt], ak1, fg[jt]);
          mma(G3[it][jt], ak3, fu[jt]);
          mma(G2[it][jt], avt, fh[jt]);
        }
      } else {
        const frag_t<T> akt = ld4x2(kr + 4 * g, kr + 16 + 4 * g);
#pragma unroll
        for (int jt = 0; jt < JT; ++jt) {
          mma(G1[it][jt], akt, fg[jt]);
          mma(G3[it][jt], akt, fu[jt]);
          mma(G2[it][jt], avt, fh[jt]);
        }
      }
    }
    }  // active
    __syncthreads();
  }
  // momentum: the head's mean coefficient, once per head
  if (a.mom != nullptr && hb == 0 && split == 0)
    block_mean<NTH>(a.mom + (int64_t)head * a.mom_sbh, a.n_tok, a.beta + head);
  if (!active) return;

  // ---- partials, [split][head][3][dh][d]: lane holds 4 consecutive d ----
  const int64_t mat = (int64_t)a.dh * D;
  float* out = a.partial + ((int64_t)split * a.bh + head) * 3 * mat;
#pragma unroll
  for (int it = 0; it < IT; ++it)
#pragma unroll
    for (int jt = 0; jt < JT; ++jt) {
      const int64_t off = (int64_t)(jw0 + 16 * jt + c) * D + 16 * it + 4 * g;
      st4(out + off, G1[it][jt][0], G1[it][jt][1], G1[it][jt][2], G1[it][jt][3]);
      st4(out + mat + off, G3[it][jt][0], G3[it][jt][1], G3[it][jt][2], G3[it][jt][3]);
      st4(out + 2 * mat + off, G2[it][jt][0], G2[it][jt][1], G2[it][jt][2], G2[it][jt][3]);
    }
}

// ----------------------------------------------------- gradient, bf16 --
// bf16 operands.  One workgroup = WAVES waves x 16 hidden units each (one MFMA
// column tile), over one token split of one head.  Per wave, for the whole
// token loop: its W1 / W3 / W2^T rows as B fragments (K = d) and the fp32
// accumulators of G1^T, G3^T, G2 (d x 16).  Token tiles of 32 are staged once
// in LDS, row-major, two per barrier in three stage buffers (the next stage's
// global loads are in flight while the current one is computed).  The
// forward contractions read
// k / v rows (K = d); the gradient contractions read k^T / v^T fragments
// (K = tokens) from the same tiles with LDS transpose reads.
// Tile layout: rows of D bf16 at the padded pitch of tpad.
template <int D, int WAVES, int HT>
__global__ __launch_bounds__(WAVES * 64) void k_grad_bf16(GradArgs a) {
  constexpr int NTH = WAVES * 64;
  constexpr int NT = 32;
  constexpr int KS = D / 32;
  constexpr int IT = D / 16;
  constexpr int TILE = NT * (D + 16);      // one k or v tile (rows padded: tpad)
  constexpr int NV = NT * D / 8;           // 16-byte vectors per tile
  constexpr int VPT = (NV + NTH - 1) / NTH;
  static_assert(NV % NTH == 0 || NTH % NV == 0, "tile split");

  // SUB tiles per barrier, three stage buffers (stage st read, st+1 written,
  // st-1 still read by the waves that defer their last gradient contraction)
  constexpr int NBUF = 3;
  constexpr int SUB = 2;
  __shared__ __attribute__((aligned(16))) bf16 sKV[NBUF * SUB][2 * TILE];
  __shared__ float sEta[NBUF * SUB][3][NT];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = lane & 15, g = lane >> 4;
  const int hblocks = (a.dh + WAVES * 16 * HT - 1) / (WAVES * 16 * HT);
  const int lid = xcd_logical_id(blockIdx.x, gridDim.x);
  const int hb = lid % hblocks;
  const int rest = lid / hblocks;
  const int split = rest % a.nsplit;
  const int head = rest / a.nsplit;
  if (head >= a.bh) return;
  const int64_t s0 = (int64_t)split * a.split_len;
  const int64_t s1 = (s0 + a.split_len < a.n_tok) ? s0 + a.split_len : a.n_tok;
  const int j0 = (hb * WAVES + wave) * 16 * HT;  // dh % 64 == 0: all HT tiles valid or none
  const bool active = j0 < a.dh;

  const bf16* kp = reinterpret_cast<const bf16*>(a.k) + (int64_t)head * a.k_sbh;
  const bf16* vp = reinterpret_cast<const bf16*>(a.v) + (int64_t)head * a.v_sbh;
  const float* e1 = a.eta1 + (int64_t)head * a.eta_sbh;
  const float* e3 = a.eta3 + (int64_t)head * a.eta_sbh;
  const float* e2 = a.eta2 + (int64_t)head * a.eta_sbh;
  // one learning rate for all three matrices (the pages' usual case): the
  // SwiGLU backward shares its eta products
  const bool same_eta = a.eta1 == a.eta3 && a.eta3 == a.eta2;
  const bf16* sb = reinterpret_cast<const bf16*>(a.sh.base) + (int64_t)head * a.sh.per_head;

  // W B fragments: lane holds W[j0 + 16 h + c][32 ks + 8 g ..]
  bf16x8 b1[HT][KS], b3[HT][KS], b2[HT][KS];
#pragma unroll
  for (int h = 0; h < HT; ++h) {
    const int64_t row = (int64_t)(active ? j0 + 16 * h + c : c) * D + 8 * g;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      b1[h][ks] = ld8(sb + a.sh.off_w1 + row + 32 * ks);
      b3[h][ks] = ld8(sb + a.sh.off_w3 + row + 32 * ks);
      b2[h][ks] = ld8(sb + a.sh.off_w2t + row + 32 * ks);
    }
  }
  wait_global_loads();
  f32x4 G1[HT][IT], G3[HT][IT], G2[HT][IT];
#pragma unroll
  for (int h = 0; h < HT; ++h)
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      G1[h][it] = f32x4{0.f, 0.f, 0.f, 0.f};
      G3[h][it] = f32x4{0.f, 0.f, 0.f, 0.f};
      G2[h][it] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  // momentum folded in: split 0 starts from beta M_old (M wide: element
  // (feature i, hidden j) at i dh + j), so that the split sum is G + beta M
  // (loads in flight while the first tiles are staged and contracted)
  if (a.mo1 != nullptr && split == 0) {
    const float beta = block_mean_all<NTH>(a.mom + (int64_t)head * a.mom_sbh, a.n_tok);
    if (active) {
      const int64_t hm = (int64_t)head * a.dh * D;
#pragma unroll
      for (int h = 0; h < HT; ++h)
#pragma unroll
        for (int it = 0; it < IT; ++it)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int64_t o = hm + (int64_t)(16 * it + 4 * g + e) * a.dh + j0 + 16 * h + c;
            G1[h][it][e] = beta * a.mo1[o];
            G3[h][it][e] = beta * a.mo3[o];
            G2[h][it][e] = beta * a.mo2[o];
          }
    }
  }

  // staging: thread tid moves 16-byte vectors vi = tid + x NTH of the k and v
  // tiles (row vi / (D/8), chunk vi % (D/8)) and, for tid < 3 NT, one eta
  const float* ep = tid < NT ? e1 : (tid < 2 * NT ? e3 : e2);
  const int er = tid % NT;
  uint4 rk[VPT], rv[VPT];
  float re = 0.f;
  // A whole tile inside the split, when every thread moves a vector of it
  // (d = 128): vector x of a thread is row tid / (D / 8) + x RX, piece
  // tid % (D / 8), loaded from a uniform row base plus the thread's 32-bit
  // byte offset (token strides below 2^24 elements keep it in range).  Else
  // every row is checked and rows past the split read as zeros.
  constexpr bool kWhole = NV % NTH == 0;
  constexpr int RX = NTH / (D / 8);
  const bool fast_ok = kWhole && a.k_st < (1 << 24) && a.v_st < (1 << 24);
  const uint32_t kob = (uint32_t)(((tid / (D / 8)) * (uint32_t)a.k_st + (tid % (D / 8)) * 8) * 2u);
  const uint32_t vob = (uint32_t)(((tid / (D / 8)) * (uint32_t)a.v_st + (tid % (D / 8)) * 8) * 2u);
#define LACT_GRAD_GLOAD(T0)                                                         \
  {                                                                                 \
    if (fast_ok && (T0) + NT <= s1) {                                               \
      _Pragma("unroll") for (int x = 0; x < VPT; ++x) {                             \
        const char* kb_ = reinterpret_cast<const char*>(kp + ((T0) + x * RX) * a.k_st); \
        const char* vb_ = reinterpret_cast<const char*>(vp + ((T0) + x * RX) * a.v_st); \
        rk[x] = *reinterpret_cast<const uint4*>(kb_ + kob);                         \
        rv[x] = *reinterpret_cast<const uint4*>(vb_ + vob);                         \
      }                                                                             \
    } else {                                                                        \
      _Pragma("unroll") for (int x = 0; x < VPT; ++x) {                             \
        const int vi = tid + x * NTH;                                               \
        const int64_t t = (T0) + vi / (D / 8);                                      \
        rk[x] = uint4{0u, 0u, 0u, 0u};                                              \
        rv[x] = uint4{0u, 0u, 0u, 0u};                                              \
        if (vi < NV && t < s1) {                                                    \
          rk[x] = *reinterpret_cast<const uint4*>(kp + t * a.k_st + (vi % (D / 8)) * 8); \
          rv[x] = *reinterpret_cast<const uint4*>(vp + t * a.v_st + (vi % (D / 8)) * 8); \
        }                                                                           \
      }                                                                             \
    }                                                                               \
    if (tid < 3 * NT) re = ((T0) + er < s1) ? ep[(T0) + er] : 0.f;                  \
  }
#define LACT_GRAD_LSTORE(BUF)                                                       \
  {                                                                                 \
    bf16* sK_ = sKV[BUF];                                                           \
    _Pragma("unroll") for (int x = 0; x < VPT; ++x) {                               \
      const int vi = tid + x * NTH;                                                 \
      if (vi < NV) {                                                                \
        const int o = tpad<D>(vi / (D / 8), (vi % (D / 8)) * 8);                     \
        *reinterpret_cast<uint4*>(sK_ + o) = rk[x];                                 \
        *reinterpret_cast<uint4*>(sK_ + TILE + o) = rv[x];                          \
      }                                                                             \
    }                                                                               \
    if (tid < 3 * NT) sEta[BUF][tid / NT][er] = re;                                 \
  }

  // per-lane element offsets in a tile, laundered so that each read below is
  // this base plus an immediate: forward fragments (row c, features 8 g ..)
  // and transpose reads (rows 4 g + c / 4, features 4 (c % 4) ..)
  const int fo = opaque(tpad<D>(c, 8 * g));
  const int to = opaque(tpad<D>(4 * g + (c >> 2), 4 * (c & 3)));
  // forward contractions of one tile: P = W1 k, U = W3 k, E = W2^T v
#define LACT_GRAD_FWD(BUF)                                                          \
  {                                                                                 \
    const bf16* pk_ = sKV[BUF] + fo;                                                \
    _Pragma("unroll") for (int h = 0; h < HT; ++h)                                  \
      _Pragma("unroll") for (int tt = 0; tt < 2; ++tt) {                            \
        P[h][tt] = f32x4{0.f, 0.f, 0.f, 0.f};                                       \
        U[h][tt] = f32x4{0.f, 0.f, 0.f, 0.f};                                       \
        E[h][tt] = f32x4{0.f, 0.f, 0.f, 0.f};                                       \
      }                                                                             \
    _Pragma("unroll") for (int ks = 0; ks < KS; ++ks)                               \
      _Pragma("unroll") for (int tt = 0; tt < 2; ++tt) {                            \
        const bf16x8 ak = ld8(pk_ + 16 * tt * (D + 16) + 32 * ks);                  \
        const bf16x8 av = ld8(pk_ + TILE + 16 * tt * (D + 16) + 32 * ks);           \
        _Pragma("unroll") for (int h = 0; h < HT; ++h) {                            \
          mma(P[h][tt], ak, b1[h][ks]);                                             \
          mma(U[h][tt], ak, b3[h][ks]);                                             \
          mma(E[h][tt], av, b2[h][ks]);                                             \
        }                                                                           \
      }                                                                             \
  }
  // SwiGLU backward + eta, packed as B operands (K = 32 tokens, kappa order)
#define LACT_GRAD_EW(BUF)                                                           \
  {                                                                                 \
    _Pragma("unroll") for (int tt = 0; tt < 2; ++tt) {                              \
      const f32x4 n1 = *reinterpret_cast<const f32x4*>(&sEta[BUF][0][16 * tt + 4 * g]); \
      const f32x4 n3 = *reinterpret_cast<const f32x4*>(&sEta[BUF][1][16 * tt + 4 * g]); \
      const f32x4 n2 = *reinterpret_cast<const f32x4*>(&sEta[BUF][2][16 * tt + 4 * g]); \
      if (same_eta) {                                                               \
        _Pragma("unroll") for (int h = 0; h < HT; ++h)                              \
        _Pragma("unroll") for (int i = 0; i < 4; ++i) {                             \
          const float p = P[h][tt][i], u = U[h][tt][i], e = E[h][tt][i];            \
          const float sg = sigmoid_fast(p);                                         \
          const float sl = p * sg;                                                  \
          const float dsl = __builtin_fmaf(sl, 1.f - sg, sg);                       \
          const float sn = n1[i] * sl;                                              \
          fh[h][4 * tt + i] = (bf16)(sn * u);                                       \
          fu[h][4 * tt + i] = (bf16)(sn * e);                                       \
          fg[h][4 * tt + i] = (bf16)((n1[i] * dsl) * (e * u));                      \
        }                                                                           \
      } else {                                                                      \
        _Pragma("unroll") for (int h = 0; h < HT; ++h)                              \
        _Pragma("unroll") for (int i = 0; i < 4; ++i) {                             \
          const float p = P[h][tt][i], u = U[h][tt][i], e = E[h][tt][i];            \
          const float sg = sigmoid_fast(p);                                         \
          const float sl = p * sg;                                                  \
          const float dsl = __builtin_fmaf(sl, 1.f - sg, sg);                       \
          fh[h][4 * tt + i] = (bf16)((n2[i] * sl) * u);                             \
          fu[h][4 * tt + i] = (bf16)((n3[i] * sl) * e);                             \
          fg[h][4 * tt + i] = (bf16)((n1[i] * dsl) * (e * u));                      \
        }                                                                           \
      }                                                                             \
    }                                                                               \
  }
  // gradient contractions: lane j of each 16-lane group reads token row
  // 4g + j/4 (+16), features 16 it + 4 (j%4); transposed, that is the A
  // fragment with tokens in kappa order.
#define LACT_GRAD_GG(BUF)                                                           \
  {                                                                                 \
    const bf16* qk_ = sKV[BUF] + to;                                                \
    _Pragma("unroll") for (int it = 0; it < IT; ++it) {                             \
      const bf16x8 akt = cat8(ld_tr4(qk_ + 16 * it), ld_tr4(qk_ + 16 * (D + 16) + 16 * it)); \
      const bf16x8 avt = cat8(ld_tr4(qk_ + TILE + 16 * it),                         \
                              ld_tr4(qk_ + TILE + 16 * (D + 16) + 16 * it));        \
      _Pragma("unroll") for (int h = 0; h < HT; ++h) {                              \
        mma(G1[h][it], akt, fg[h]);                                                 \
        mma(G3[h][it], akt, fu[h]);                                                 \
        mma(G2[h][it], avt, fh[h]);                                                 \
      }                                                                             \
    }                                                                               \
  }

  const int ntile = s0 < s1 ? (int)((s1 - s0 + NT - 1) / NT) : 0;
  f32x4 P[HT][2], U[HT][2], E[HT][2];
  bf16x8 fh[HT], fu[HT], fg[HT];
  // Two token tiles per barrier: stage st reads slots (st % 3) SUB + 0, 1
  // and stages the next stage's tiles into ((st + 1) % 3) SUB + 0, 1.
  // Waves WAVES/2.. (which share their SIMDs with waves 0..WAVES/2-1) run
  // the gradient contractions of their second tile at the start of the
  // next stage, so the two waves of a SIMD are out of phase: one wave's
  // SwiGLU backward (VALU) overlaps the other's MFMA phases.
  static_assert(SUB == 2, "stage = two tiles");
  const bool late = wave >= WAVES / 2;
  const int nst = (ntile + SUB - 1) / SUB;
#pragma unroll
  for (int sb = 0; sb < SUB; ++sb)
    if (sb < ntile) {
      LACT_GRAD_GLOAD(s0 + (int64_t)sb * NT);
      LACT_GRAD_LSTORE(sb);
    }
  __syncthreads();
  for (int st = 0; st < nst; ++st) {
    const int cur = (st % 3) * SUB, nxt = ((st + 1) % 3) * SUB, prv = ((st + 2) % 3) * SUB;
    const int ta = st * SUB, tb = ta + 1;
    if (late && active && st > 0) LACT_GRAD_GG(prv + 1);  // deferred tile
    if (ta + SUB < ntile) LACT_GRAD_GLOAD(s0 + (int64_t)(ta + SUB) * NT);
    if (active) {
      LACT_GRAD_FWD(cur);
      LACT_GRAD_EW(cur);
      LACT_GRAD_GG(cur);
    }
    if (ta + SUB < ntile) LACT_GRAD_LSTORE(nxt);
    if (tb + SUB < ntile) LACT_GRAD_GLOAD(s0 + (int64_t)(tb + SUB) * NT);
    if (active && tb < ntile) {
      LACT_GRAD_FWD(cur + 1);
      LACT_GRAD_EW(cur + 1);
      if (!late) LACT_GRAD_GG(cur + 1);
    }
    if (tb + SUB < ntile) LACT_GRAD_LSTORE(nxt + 1);
    __syncthreads();
  }
  // the last stage's second tile (late waves), if it exists
  if (late && active && nst > 0 && (nst - 1) * SUB + 1 < ntile)
    LACT_GRAD_GG(((nst - 1) % 3) * SUB + 1);
#undef LACT_GRAD_FWD
#undef LACT_GRAD_EW
#undef LACT_GRAD_GG
#undef LACT_GRAD_GLOAD
#undef LACT_GRAD_LSTORE
  // momentum: the head's mean coefficient, once per head
  if (a.mom != nullptr && hb == 0 && split == 0)
    block_mean<NTH>(a.mom + (int64_t)head * a.mom_sbh, a.n_tok, a.beta + head);
  if (!active) return;

  // ---- partials, [split][head][3][dh][d]: lane holds 4 consecutive d ----
  const int64_t mat = (int64_t)a.dh * D;
  float* out = a.partial + ((int64_t)split * a.bh + head) * 3 * mat + (int64_t)(j0 + c) * D + 4 * g;
#pragma unroll
  for (int h = 0; h < HT; ++h)
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      float* o = out + 16 * h * D + 16 * it;
      st4(o, G1[h][it][0], G1[h][it][1], G1[h][it][2], G1[h][it][3]);
      st4(o + mat, G3[h][it][0], G3[h][it][1], G3[h][it][2], G3[h][it][3]);
      st4(o + 2 * mat, G2[h][it][0], G2[h][it][1], G2[h][it][2], G2[h][it][3]);
    }
}

// ------------------------------------------------- gradient, bf16, solo --
// One wave per SIMD holding 16 HW hidden units over all D features: its W
// fragments (3 HW D / 8 registers) and G1^T, G3^T, G2 accumulators
// (6 HW D / 4, in AGPRs) take a whole SIMD's register file.  Launched for
// D = 256 with HW = 1 only: at D = 128, HW = 2 (every k / v fragment feeding
// two hidden tiles) measured slower than k_grad_bf16 (77.5 vs 73.3 us on
// 32 heads x 2048 tokens, dh = 512).  (For d = 256, two waves per SIMD
// would have to split the features, exchange the forward partials through
// LDS and both run the SwiGLU backward: measured 20-30 % slower.)
// 4 waves = 64 HW hidden units share the staged k / v tiles.  Software
// pipeline over 32-token tiles, three stage buffers, one barrier per tile:
// iteration n runs the forward contractions of tile n + 1 with the SwiGLU
// backward of tile n spread between them, then the gradient contractions
// of tile n with the staging stores of tile n + 2 between its last steps
// (as late as possible: the tile's loads, issued at the top of the
// iteration, then have both regions to arrive); fragment reads ahead of
// their MFMAs (below), the order held by scheduling fences.
// SAME: one learning-rate array for the three matrices (the η products of
// the SwiGLU backward are shared; one η row per token in registers).
// RING, TRING: fragment buffers of the forward and of the gradient
// contractions (reads RING - 1, TRING - 1 steps ahead of their MFMAs).
// Measured on long-context (4 heads x 16384 tokens): with one rate,
// TRING = 6 (226 us per launch) beats 4 (231), 5 (228) and 8 (226-227),
// RING = 2 is 5 % slower; three rates keep 3 / 3 (TRING = 4 was 2.5 %
// slower there: the register allocation, not the instruction count, moves
// the time).
template <int D, int HW, bool SAME = false, int RING = 3, int TRING = 3>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void k_grad_solo(GradArgs a) {
  constexpr int NTH = 256, NT = 32;
  constexpr int KS = D / 32;           // K slabs of the forward contractions
  constexpr int IT = D / 16;           // feature tiles of the gradient
  constexpr int TILE = NT * (D + 16);  // rows at a padded pitch (tpad)
  constexpr int NV = NT * D / 8;       // 16-byte vectors per tile
  constexpr int VPT = NV / NTH;
  constexpr int NBUF = 3;
  constexpr int NST = 2 * KS;          // forward steps (K slab, token half)
  constexpr int EPS_ = 8 * HW / NST;   // backward elements per forward step
  constexpr int EVERY = NST / (8 * HW) > 0 ? NST / (8 * HW) : 1;  // steps per element
  static_assert(NV % NTH == 0 && VPT <= IT, "tile split");
  static_assert(EPS_ * NST == 8 * HW || EVERY * 8 * HW == NST, "backward spread");
  __shared__ __attribute__((aligned(16))) bf16 sKV[NBUF][2 * TILE];
  __shared__ float sEta[NBUF][3][NT];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = lane & 15, g = lane >> 4;
  const int hblocks = a.dh / (64 * HW);
  const int lid = xcd_logical_id(blockIdx.x, gridDim.x);
  const int hb = lid % hblocks;
  const int rest = lid / hblocks;
  const int split = rest % a.nsplit;
  const int head = rest / a.nsplit;
  if (head >= a.bh) return;
  const int64_t s0 = (int64_t)split * a.split_len;
  const int64_t s1 = (s0 + a.split_len < a.n_tok) ? s0 + a.split_len : a.n_tok;
  const int j0 = (hb * 4 + wave) * 16 * HW;

  const bf16* kp = reinterpret_cast<const bf16*>(a.k) + (int64_t)head * a.k_sbh;
  const bf16* vp = reinterpret_cast<const bf16*>(a.v) + (int64_t)head * a.v_sbh;
  const float* e1 = a.eta1 + (int64_t)head * a.eta_sbh;
  const float* e3 = a.eta3 + (int64_t)head * a.eta_sbh;
  const float* e2 = a.eta2 + (int64_t)head * a.eta_sbh;
  const bf16* sb = reinterpret_cast<const bf16*>(a.sh.base) + (int64_t)head * a.sh.per_head;

  // W B fragments: lane holds W[j0 + 16 h + c][32 ks + 8 g ..]
  bf16x8 b1[HW][KS], b3[HW][KS], b2[HW][KS];
#pragma unroll
  for (int h = 0; h < HW; ++h) {
    const int64_t row = (int64_t)(j0 + 16 * h + c) * D + 8 * g;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      b1[h][ks] = ld8(sb + a.sh.off_w1 + row + 32 * ks);
      b3[h][ks] = ld8(sb + a.sh.off_w3 + row + 32 * ks);
      b2[h][ks] = ld8(sb + a.sh.off_w2t + row + 32 * ks);
    }
  }
  f32x4 G1[HW][IT], G3[HW][IT], G2[HW][IT];
#pragma unroll
  for (int h = 0; h < HW; ++h)
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      G1[h][it] = f32x4{0.f, 0.f, 0.f, 0.f};
      G3[h][it] = f32x4{0.f, 0.f, 0.f, 0.f};
      G2[h][it] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

  // staging: 16-byte vectors vi = tid + x NTH of the k and v tiles, and for
  // tid < 3 NT one eta (zero past the split: no contribution)
  const float* ep = tid < NT ? e1 : (tid < 2 * NT ? e3 : e2);
  const int er = tid % NT;
  uint4 rk[VPT], rv[VPT];
  float re = 0.f;
  // Staging loads through one buffer descriptor per tensor and tile: base =
  // the tile's first row, range = the tile's rows that lie inside the split
  // (rows past the split, and whole tiles past the last, read as zeros: the
  // range check); vector x of a thread is row tid / (D / 8) + x RX, piece
  // tid % (D / 8), at a 32-bit byte offset from the base (token strides
  // below 2^24 elements).  Larger strides take a checked per-lane path.
  constexpr int RX = NTH / (D / 8);
  static_assert(NTH % (D / 8) == 0, "rows per vector step");
  const bool fast_ok = a.k_st < (1 << 24) && a.v_st < (1 << 24) && s1 - s0 < (1 << 30);
  const int nrow = (int)(s1 - s0);
  uint32_t kox[VPT], vox[VPT];
#pragma unroll
  for (int x = 0; x < VPT; ++x) {
    const uint32_t row = (uint32_t)(tid / (D / 8) + x * RX), piece = (uint32_t)(tid % (D / 8)) * 16u;
    kox[x] = row * (uint32_t)a.k_st * 2u + piece;
    vox[x] = row * (uint32_t)a.v_st * 2u + piece;
  }
  // bytes from row t0 to the end of the tile's last row inside the split (0
  // from s1 on)
  auto span = [&](int64_t t0, int st) -> uint32_t {
    const int rows = min(nrow - (int)(t0 - s0), NT);
    return rows <= 0 ? 0u : (uint32_t)(((rows - 1) * st + D) * 2);
  };
#define LACT_GS_GLOAD(T0)                                                           \
  {                                                                                 \
    if (fast_ok) {                                                                  \
      const __amdgpu_buffer_rsrc_t kr_ = buf_rsrc(kp + (T0) * a.k_st, span((T0), (int)a.k_st)); \
      const __amdgpu_buffer_rsrc_t vr_ = buf_rsrc(vp + (T0) * a.v_st, span((T0), (int)a.v_st)); \
      _Pragma("unroll") for (int x = 0; x < VPT; ++x) {                             \
        rk[x] = buf_ld16(kr_, kox[x]);                                              \
        rv[x] = buf_ld16(vr_, vox[x]);                                              \
      }                                                                             \
    } else {                                                                        \
      /* (an opaque row base: no per-lane pointers carried across tiles) */         \
      const int64_t t0_ = opaque_s(T0);                                             \
      _Pragma("unroll") for (int x = 0; x < VPT; ++x) {                             \
        const int vi = tid + x * NTH;                                               \
        const int64_t t = t0_ + vi / (D / 8);                                       \
        rk[x] = uint4{0u, 0u, 0u, 0u};                                              \
        rv[x] = uint4{0u, 0u, 0u, 0u};                                              \
        if (t < s1) {                                                               \
          rk[x] = *reinterpret_cast<const uint4*>(kp + t * a.k_st + (vi % (D / 8)) * 8); \
          rv[x] = *reinterpret_cast<const uint4*>(vp + t * a.v_st + (vi % (D / 8)) * 8); \
        }                                                                           \
      }                                                                             \
    }                                                                               \
    if (tid < 3 * NT) re = ((T0) + er < s1) ? ep[(T0) + er] : 0.f;                  \
  }
#define LACT_GS_LSTORE(BUF)                                                         \
  {                                                                                 \
    bf16* sK_ = sKV[BUF];                                                           \
    _Pragma("unroll") for (int x = 0; x < VPT; ++x) {                               \
      const int vi = tid + x * NTH;                                                 \
      const int o = tpad<D>(vi / (D / 8), (vi % (D / 8)) * 8);                       \
      *reinterpret_cast<uint4*>(sK_ + o) = rk[x];                                   \
      *reinterpret_cast<uint4*>(sK_ + TILE + o) = rv[x];                            \
    }                                                                               \
    if (tid < 3 * NT) sEta[BUF][tid / NT][er] = re;                                 \
  }

  // per-lane element offsets in a tile (laundered: the stage buffer is a
  // runtime choice, and every read should be this base + an immediate):
  // forward fragments (row c, features 8 g ..) and transpose reads (rows
  // 4 g + c / 4, features 4 (c % 4) ..)
  const int fo = opaque(tpad<D>(c, 8 * g));
  const int to = opaque(tpad<D>(4 * g + (c >> 2), 4 * (c & 3)));
  // forward contractions of the tile in buffer BUF (gate, up from k rows,
  // W2^T v from v rows): tokens 16 tt + 4 g + i, hidden 16 h + c.  With
  // BW, the SwiGLU backward of the previous tile runs between the steps.
  f32x4 P[HW][2], U[HW][2], E[HW][2];
  bf16x8 fh[HW], fu[HW], fg[HW];
  auto forward = [&](int buf, f32x4 (&Pn)[HW][2], f32x4 (&Un)[HW][2], f32x4 (&En)[HW][2],
                     bool bw, int eb, const f32x4 (&Pc)[HW][2], const f32x4 (&Uc)[HW][2],
                     const f32x4 (&Ec)[HW][2]) {
    f32x4 n1[2], n2[2], n3[2];
    if (bw) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        n1[tt] = *reinterpret_cast<const f32x4*>(&sEta[eb][0][16 * tt + 4 * g]);
        if constexpr (!SAME) {
          n3[tt] = *reinterpret_cast<const f32x4*>(&sEta[eb][1][16 * tt + 4 * g]);
          n2[tt] = *reinterpret_cast<const f32x4*>(&sEta[eb][2][16 * tt + 4 * g]);
        }
      }
    }
#pragma unroll
    for (int h = 0; h < HW; ++h)
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        Pn[h][tt] = f32x4{0.f, 0.f, 0.f, 0.f};
        Un[h][tt] = f32x4{0.f, 0.f, 0.f, 0.f};
        En[h][tt] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    const bf16* pk = sKV[buf] + fo;
    bf16x8 rk_[RING], rv_[RING];
    // step s = KS tt + ks reads row block tt, K slab ks: token half 0 first,
    // as the backward below, so that the two tiles' halves overlap in
    // registers instead of the whole of both
#define LACT_GS_FRAG(S)                                                             \
  {                                                                                 \
    rk_[(S) % RING] = ld8(pk + 16 * ((S) / KS) * (D + 16) + 32 * ((S) % KS));       \
    rv_[(S) % RING] = ld8(pk + TILE + 16 * ((S) / KS) * (D + 16) + 32 * ((S) % KS)); \
  }
#pragma unroll
    for (int st = 0; st < RING - 1; ++st) LACT_GS_FRAG(st);
#pragma unroll
    for (int st = 0; st < NST; ++st) {
      if (st + RING - 1 < NST) LACT_GS_FRAG(st + RING - 1);
      const int tt = st / KS, ks = st % KS;
#pragma unroll
      for (int h = 0; h < HW; ++h) {
        mma(Pn[h][tt], rk_[st % RING], b1[h][ks]);
        mma(Un[h][tt], rk_[st % RING], b3[h][ks]);
        mma(En[h][tt], rv_[st % RING], b2[h][ks]);
      }
      if (bw) {
#pragma unroll
        for (int q = 0; q < EPS_ + (EPS_ == 0 ? 1 : 0); ++q) {
          if (EPS_ == 0 && (st % EVERY) != EVERY - 1) continue;
          // backward element e8 = (token half te, h, row ie)
          const int e8 = EPS_ > 0 ? st * EPS_ + q : st / EVERY;
          const int te = e8 / (4 * HW), h = (e8 >> 2) % HW, ie = e8 & 3;
          const float p = Pc[h][te][ie], u = Uc[h][te][ie], e = Ec[h][te][ie];
          const float sg = sigmoid_fast(p);
          const float sl = p * sg;
          const float dsl = __builtin_fmaf(sl, 1.f - sg, sg);
          if constexpr (SAME) {
            const float sn = n1[te][ie] * sl;
            fh[h][4 * te + ie] = (bf16)(sn * u);
            fu[h][4 * te + ie] = (bf16)(sn * e);
          } else {
            fh[h][4 * te + ie] = (bf16)((n2[te][ie] * sl) * u);
            fu[h][4 * te + ie] = (bf16)((n3[te][ie] * sl) * e);
          }
          fg[h][4 * te + ie] = (bf16)((n1[te][ie] * dsl) * (e * u));
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#undef LACT_GS_FRAG
  };

  const int ntile = s0 < s1 ? (int)((s1 - s0 + NT - 1) / NT) : 0;
  if (ntile > 0) {
    LACT_GS_GLOAD(s0);
    LACT_GS_LSTORE(0);
  }
  if (ntile > 1) {
    LACT_GS_GLOAD(s0 + NT);
    LACT_GS_LSTORE(1);
  }
  __syncthreads();
  forward(0, P, U, E, false, 0, P, U, E);  // (unused when there is no tile)
  for (int n = 0; n < ntile; ++n) {
    const int cb = n % NBUF, nb = (n + 1) % NBUF, lb = (n + 2) % NBUF;
    // tile n + 2 (rows past the split read as zeros; past the last tile the
    // store below goes to a free buffer)
    LACT_GS_GLOAD(s0 + (int64_t)(n + 2) * NT);
    __builtin_amdgcn_sched_barrier(0);
    // ---- region 1: forward contractions of tile n + 1 (past the last
    // tile: stale buffer, results unused) with the backward of tile n ----
    f32x4 Pn[HW][2], Un[HW][2], En[HW][2];
    forward(nb, Pn, Un, En, true, cb, P, U, E);
    // ---- region 2: gradient contractions of tile n, transpose reads two
    // steps ahead, the staging stores of tile n + 2 between them ----
    {
      const bf16* qk = sKV[cb] + to;
      constexpr int TR = TRING;
      bf16x8 tk_[TR], tv_[TR];
#define LACT_GS_TFRAG(IT_)                                                          \
  {                                                                                 \
    tk_[(IT_) % TR] = cat8(ld_tr4(qk + 16 * (IT_)), ld_tr4(qk + 16 * (D + 16) + 16 * (IT_))); \
    tv_[(IT_) % TR] = cat8(ld_tr4(qk + TILE + 16 * (IT_)),                          \
                           ld_tr4(qk + TILE + 16 * (D + 16) + 16 * (IT_)));         \
  }
#pragma unroll
      for (int it = 0; it < TR - 1; ++it) LACT_GS_TFRAG(it);
      bf16* sK_ = sKV[lb];
#pragma unroll
      for (int it = 0; it < IT; ++it) {
        if (it + TR - 1 < IT) LACT_GS_TFRAG(it + TR - 1);
#pragma unroll
        for (int h = 0; h < HW; ++h) {
          mma(G1[h][it], tk_[it % TR], fg[h]);
          mma(G3[h][it], tk_[it % TR], fu[h]);
          mma(G2[h][it], tv_[it % TR], fh[h]);
        }
        if (it >= IT - VPT) {
          const int x = it - (IT - VPT), vi = tid + x * NTH;
          const int o = tpad<D>(vi / (D / 8), (vi % (D / 8)) * 8);
          *reinterpret_cast<uint4*>(sK_ + o) = rk[x];
          *reinterpret_cast<uint4*>(sK_ + TILE + o) = rv[x];
        }
        __builtin_amdgcn_sched_barrier(0);
      }
#undef LACT_GS_TFRAG
      if (tid < 3 * NT) sEta[lb][tid / NT][er] = re;
    }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < HW; ++h)
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        P[h][tt] = Pn[h][tt];
        U[h][tt] = Un[h][tt];
        E[h][tt] = En[h][tt];
      }
  }
#undef LACT_GS_GLOAD
#undef LACT_GS_LSTORE
  // momentum: the head's mean coefficient, once per head
  if (a.mom != nullptr && hb == 0 && split == 0)
    block_mean<NTH>(a.mom + (int64_t)head * a.mom_sbh, a.n_tok, a.beta + head);

  // ---- partials, [split][head][3][dh][d]: lane holds 4 consecutive d ----
  const int64_t mat = (int64_t)a.dh * D;
  float* out = a.partial + ((int64_t)split * a.bh + head) * 3 * mat + (int64_t)(j0 + c) * D + 4 * g;
#pragma unroll
  for (int h = 0; h < HW; ++h)
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      float* o = out + 16 * h * D + 16 * it;
      st4(o, G1[h][it][0], G1[h][it][1], G1[h][it][2], G1[h][it][3]);
      st4(o + mat, G3[h][it][0], G3[h][it][1], G3[h][it][2], G3[h][it][3]);
      st4(o + 2 * mat, G2[h][it][0], G2[h][it][1], G2[h][it][2], G2[h][it][3]);
    }
}

// --------------------------------------------------------------- launch --
static hipError_t run_apply_solo(const ApplyArgs& a, hipStream_t s, int max_blocks) {
  int64_t blocks = (a.n_tok + 127) / 128 * a.bh;
  if (blocks <= 0) return hipSuccess;
  if (max_blocks > 0 && blocks > max_blocks) blocks = max_blocks;
  hipLaunchKernelGGL((k_apply_solo<256>), dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <class T, int D, int NTW, int WAVES>
static hipError_t run_apply(const ApplyArgs& a, hipStream_t s) {
  const int64_t tiles = (a.n_tok + (int64_t)WAVES * NTW - 1) / ((int64_t)WAVES * NTW);
  const int64_t blocks = tiles * a.bh;
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL((k_apply<T, D, NTW, WAVES>), dim3((unsigned)blocks), dim3(WAVES * 64), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_apply(int dtype, const ApplyArgs& a, hipStream_t s, int max_blocks) {
  if (dtype == 1) {
    switch (a.d) {
      case 64: return run_apply<bf16, 64, 64, 4>(a, s);
      case 128: return run_apply<bf16, 128, 32, 8>(a, s);
      case 256: return run_apply_solo(a, s, max_blocks);
    }
  } else {
    switch (a.d) {
      case 64: return run_apply<float, 64, 32, 4>(a, s);
      case 128: return run_apply<float, 128, 32, 4>(a, s);
    }
  }
  return hipErrorInvalidValue;
}

int grad_hidden_per_block(int dtype, int d, bool generic) {
  if (dtype == 1 && !generic) return d == 256 ? 4 * 16 : 128;   // k_grad_bf16: WAVES x 16 x HT (d = 64, 128: 8 x 16)
  return 4 * (d == 64 ? 32 : 16);                               // k_grad: WAVES x JW
}

template <int D, int WAVES, int HT>
static hipError_t run_grad_bf16(const GradArgs& a, hipStream_t s) {
  const int hblocks = (a.dh + WAVES * 16 * HT - 1) / (WAVES * 16 * HT);
  const int64_t blocks = (int64_t)hblocks * a.nsplit * a.bh;
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL((k_grad_bf16<D, WAVES, HT>), dim3((unsigned)blocks), dim3(WAVES * 64), 0, s, a);
  return hipGetLastError();
}

template <int D, int HW>
static hipError_t run_grad_solo(const GradArgs& a, hipStream_t s) {
  const int64_t blocks = (int64_t)(a.dh / (64 * HW)) * a.nsplit * a.bh;
  if (blocks <= 0) return hipSuccess;
  if (a.eta1 == a.eta3 && a.eta3 == a.eta2)
    hipLaunchKernelGGL((k_grad_solo<D, HW, true, 3, 6>), dim3((unsigned)blocks), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((k_grad_solo<D, HW, false, 3, 3>), dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <class T, int D, int JW, int WAVES, bool PERCH = false>
static hipError_t run_grad(const GradArgs& a, hipStream_t s) {
  const int hblocks = (a.dh + WAVES * JW - 1) / (WAVES * JW);
  const int64_t blocks = (int64_t)hblocks * a.nsplit * a.bh;
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL((k_grad<T, D, JW, WAVES, PERCH>), dim3((unsigned)blocks), dim3(WAVES * 64), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_grad(int dtype, const GradArgs& a, hipStream_t s) {
  // folding the old momentum in is a k_grad_bf16 feature
  if (a.mo1 != nullptr && !(dtype == 1 && a.d <= 128 && a.mom != nullptr && !a.eta_per_channel))
    return hipErrorInvalidValue;
  if (a.eta_per_channel) {
    // per-channel learning rates: the generic kernel, d <= 128
    if (dtype == 1) {
      switch (a.d) {
        case 64: return run_grad<bf16, 64, 32, 4, true>(a, s);
        case 128: return run_grad<bf16, 128, 16, 4, true>(a, s);
      }
    } else {
      switch (a.d) {
        case 64: return run_grad<float, 64, 32, 4, true>(a, s);
        case 128: return run_grad<float, 128, 16, 4, true>(a, s);
      }
    }
    return hipErrorInvalidValue;
  }
  if (dtype == 1) {
    switch (a.d) {
      case 64: return run_grad_bf16<64, 8, 1>(a, s);
      case 128: return run_grad_bf16<128, 8, 1>(a, s);
      case 256: return run_grad_solo<256, 1>(a, s);
    }
  } else {
    switch (a.d) {
      case 64: return run_grad<float, 64, 32, 4>(a, s);
      case 128: return run_grad<float, 128, 16, 4>(a, s);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace lact
