// Streaming read of a few tokens per head (decode): o_t = W2 (silu(W1 q_t) *
// (W3 q_t)) for n <= 8 tokens (LaCT rebuttal page, apply step of both
// pseudocode functions; uTTT page section 2: one read per token, a write
// only when a chunk has filled).
//
// With so few tokens the read is a matrix-vector product bound by reading
// the weights: hidden unit j needs the rows W1[j], W3[j] and W2^T[j] of the
// operand copies (3 d values) once, for every token.  Workgroup (head, blk)
// streams the hidden units [blk HB, (blk + 1) HB) of one head:
//   * a row of d values is LPR = d * sizeof(T) / 16 lanes of 16 bytes, so a
//     wave covers RPW = 64 / LPR rows per load;
//   * per token, g = W1[j] q and u = W3[j] q are sums over the LPR lanes of
//     the row (butterflies within the lane group), h = silu(g) u in fp32,
//     and each lane adds h W2^T[j] to its 16-byte slot of the token's output;
//   * the rows' contributions are summed over the lane groups of a wave and
//     over the four waves in a fixed order, and the workgroup writes its
//     partial output [n][d] (fp32) to the workspace.
// k_decode_sum adds a head's partials in block order and writes o.  (The
// partials cross XCDs, whose L2s are not coherent with each other, so a
// last-workgroup-sums scheme in one launch would need device-scope fences,
// each an L2 write-back; measured 3x slower than the second launch.)
#include "lact_internal.hpp"
#include "mfma.hpp"

namespace lact {

template <class T> struct Vec16;
template <> struct Vec16<bf16> { typedef bf16x8 type; static constexpr int N = 8; };
template <> struct Vec16<float> { typedef f32x4 type; static constexpr int N = 4; };

template <class T, int D, int NMAX>
__global__ __launch_bounds__(256) void k_decode(DecodeArgs a) {
  typedef typename Vec16<T>::type vec;
  constexpr int V = Vec16<T>::N;          // values per 16-byte slot
  constexpr int LPR = D / V;              // lanes per row
  constexpr int RPW = 64 / LPR;           // rows per wave load
  static_assert(LPR >= 1 && LPR <= 64 && 64 % LPR == 0, "row split");
  __shared__ float red[4][NMAX][D];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int head = blockIdx.x / a.nblk, blk = blockIdx.x % a.nblk;
  const int slot = lane % LPR, rg = lane / LPR;
  const int n = a.n;
  const int hb = a.dh / a.nblk;           // hidden units of this workgroup
  const int j0 = blk * hb;

  // this lane's slot of every token
  float qv[NMAX][V];
  const T* qp = reinterpret_cast<const T*>(a.q) + (int64_t)head * a.q_sbh;
#pragma unroll
  for (int t = 0; t < NMAX; ++t) {
    if (t < n) {
      const vec x = *reinterpret_cast<const vec*>(qp + (int64_t)t * a.q_st + V * slot);
#pragma unroll
      for (int v = 0; v < V; ++v) qv[t][v] = to_f(x[v]);
    } else {
#pragma unroll
      for (int v = 0; v < V; ++v) qv[t][v] = 0.f;
    }
  }
  float acc[NMAX][V];
#pragma unroll
  for (int t = 0; t < NMAX; ++t)
#pragma unroll
    for (int v = 0; v < V; ++v) acc[t][v] = 0.f;

  const T* sb = reinterpret_cast<const T*>(a.sh.base) + (int64_t)head * a.sh.per_head;
  const T* w1 = sb + a.sh.off_w1;
  const T* w3 = sb + a.sh.off_w3;
  const T* w2t = sb + a.sh.off_w2t;
  // rows j0 + 4 RPW p + RPW wave + rg, p = 0 .. hb / (4 RPW) - 1
#pragma unroll 2
  for (int r = RPW * wave + rg; r < hb; r += 4 * RPW) {
    const int64_t off = (int64_t)(j0 + r) * D + V * slot;
    const vec x1 = *reinterpret_cast<const vec*>(w1 + off);
    const vec x3 = *reinterpret_cast<const vec*>(w3 + off);
    const vec x2 = *reinterpret_cast<const vec*>(w2t + off);
#pragma unroll
    for (int t = 0; t < NMAX; ++t) {
      if (t < n) {
        float g = 0.f, u = 0.f;
#pragma unroll
        for (int v = 0; v < V; ++v) {
          g += to_f(x1[v]) * qv[t][v];
          u += to_f(x3[v]) * qv[t][v];
        }
#pragma unroll
        for (int o = 1; o < LPR; o <<= 1) {
          g += __shfl_xor(g, o);
          u += __shfl_xor(u, o);
        }
        const float h = g * sigmoidf_(g) * u;
#pragma unroll
        for (int v = 0; v < V; ++v) acc[t][v] += h * to_f(x2[v]);
      }
    }
  }
  // sum over the lane groups of the wave (same slot), then over the waves
#pragma unroll
  for (int t = 0; t < NMAX; ++t) {
    if (t < n) {
#pragma unroll
      for (int v = 0; v < V; ++v) {
        float x = acc[t][v];
#pragma unroll
        for (int o = LPR; o < 64; o <<= 1) x += __shfl_xor(x, o);
        acc[t][v] = x;
      }
    }
  }
  if (rg == 0) {
#pragma unroll
    for (int t = 0; t < NMAX; ++t)
      if (t < n) {
#pragma unroll
        for (int v = 0; v < V; ++v) red[wave][t][V * slot + v] = acc[t][v];
      }
  }
  __syncthreads();
  float* part = a.part + ((int64_t)head * a.nblk + blk) * n * D;
  for (int e = tid; e < n * D; e += 256) {
    const int t = e / D, i = e % D;
    part[e] = (red[0][t][i] + red[1][t][i]) + (red[2][t][i] + red[3][t][i]);
  }
}

// o[head][t][i] = the sum over hidden blocks, in block order, of the
// partials: 64 output values per workgroup.
template <class T>
__global__ __launch_bounds__(64) void k_decode_sum(DecodeArgs a) {
  const int nd = a.n * a.d;
  const int per = (nd + 63) / 64;
  const int head = blockIdx.x / per;
  const int e = (blockIdx.x % per) * 64 + threadIdx.x;
  if (e >= nd) return;
  const float* p = a.part + (int64_t)head * a.nblk * nd + e;
  float x = 0.f;
#pragma unroll 8
  for (int b = 0; b < a.nblk; ++b) x += p[(int64_t)b * nd];
  const int t = e / a.d, i = e % a.d;
  reinterpret_cast<T*>(a.o)[(int64_t)head * a.o_sbh + (int64_t)t * a.o_st + i] = to_t<T>(x);
}

// Hidden blocks per head: about one workgroup per compute unit, each a
// whole number of wave loads.
int decode_blocks(int dtype, int bh, int d, int dh) {
  const int lpr = d * (dtype == 1 ? 2 : 4) / 16;
  const int rows = 4 * (64 / lpr);  // rows per workgroup pass
  int nb = (256 + bh - 1) / bh;
  const int cap = dh / rows;
  if (nb > cap) nb = cap;
  while (nb > 1 && (dh % nb != 0 || (dh / nb) % rows != 0)) --nb;
  return nb < 1 ? 1 : nb;
}

template <class T, int D>
static hipError_t run_decode(const DecodeArgs& a, hipStream_t s) {
  // registers for as many tokens as there are (1, 2, 4 or 8)
  const dim3 grid((unsigned)(a.bh * a.nblk));
  if (a.n == 1) hipLaunchKernelGGL((k_decode<T, D, 1>), grid, dim3(256), 0, s, a);
  else if (a.n == 2) hipLaunchKernelGGL((k_decode<T, D, 2>), grid, dim3(256), 0, s, a);
  else if (a.n <= 4) hipLaunchKernelGGL((k_decode<T, D, 4>), grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((k_decode<T, D, 8>), grid, dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int per = (a.n * a.d + 63) / 64;
  hipLaunchKernelGGL((k_decode_sum<T>), dim3((unsigned)(a.bh * per)), dim3(64), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_decode(int dtype, const DecodeArgs& a, hipStream_t s) {
  if (a.n < 1 || a.n > 8) return hipErrorInvalidValue;
  if (dtype == 1) {
    switch (a.d) {
      case 64: return run_decode<bf16, 64>(a, s);
      case 128: return run_decode<bf16, 128>(a, s);
      case 256: return run_decode<bf16, 256>(a, s);
    }
  } else {
    switch (a.d) {
      case 64: return run_decode<float, 64>(a, s);
      case 128: return run_decode<float, 128>(a, s);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace lact
