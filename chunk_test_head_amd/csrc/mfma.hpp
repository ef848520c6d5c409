// MFMA fragment helpers for gfx950 (CDNA4), wave64.
//
// Every contraction in this library is written on one tile shape: the
// 16x16x32 bf16 MFMA,  C[16x16] += A[16x32] * B[32x16].  With lane l,
// c = l & 15 and g = l >> 4 (0..3):
//   A fragment: lane holds A[c][8g + m], m = 0..7       (8 elements)
//   B fragment: lane holds B[8g + m][c], m = 0..7
//   C tile    : lane holds C[4g + i][c], i = 0..3        (4 floats)
// The fp32 operand path keeps the same fragment (8 fp32 per lane) and issues
// eight 16x16x4 f32 MFMAs; MFMA number m contracts slot m of the four lane
// groups, so both paths contract exactly the same pairs of elements.
//
// Because the order of the K index inside one contraction is free, a C tile
// pair can feed the next contraction directly from registers: for the K slab
// made of C tiles t0 (rows 0..15) and t1 (rows 16..31), slot m of lane
// (c, g) is row kappa(g, m) = m < 4 ? 4g + m : 16 + 4g + (m - 4), and the
// other operand is read with the same kappa (two runs of four elements).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lact {

typedef __bf16 bf16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(8 * sizeof(float)))) float f32x8;

template <class T> struct FragOf;
template <> struct FragOf<bf16> { typedef bf16x8 type; };
template <> struct FragOf<float> { typedef f32x8 type; };
template <class T> using frag_t = typename FragOf<T>::type;

__device__ __forceinline__ void mma(f32x4& c, const bf16x8& a, const bf16x8& b) {
  c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x4& c, const f32x8& a, const f32x8& b) {
#pragma unroll
  for (int m = 0; m < 8; ++m) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[m], b[m], c, 0, 0, 0);
}

// 8 contiguous elements (16 B for bf16, 32 B for fp32; 16-byte aligned).
__device__ __forceinline__ bf16x8 ld8(const bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }
__device__ __forceinline__ f32x8 ld8(const float* p) {
  f32x4 a = *reinterpret_cast<const f32x4*>(p);
  f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
  f32x8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = a[2]; r[3] = a[3];
  r[4] = b[0]; r[5] = b[1]; r[6] = b[2]; r[7] = b[3];
  return r;
}
// slots 0..3 from p0[0..3], slots 4..7 from p1[0..3] (kappa order).
__device__ __forceinline__ bf16x8 ld4x2(const bf16* p0, const bf16* p1) {
  bf16x4 a = *reinterpret_cast<const bf16x4*>(p0);
  bf16x4 b = *reinterpret_cast<const bf16x4*>(p1);
  bf16x8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = a[2]; r[3] = a[3];
  r[4] = b[0]; r[5] = b[1]; r[6] = b[2]; r[7] = b[3];
  return r;
}
__device__ __forceinline__ f32x8 ld4x2(const float* p0, const float* p1) {
  f32x4 a = *reinterpret_cast<const f32x4*>(p0);
  f32x4 b = *reinterpret_cast<const f32x4*>(p1);
  f32x8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = a[2]; r[3] = a[3];
  r[4] = b[0]; r[5] = b[1]; r[6] = b[2]; r[7] = b[3];
  return r;
}

// Raw buffer loads: a wave-uniform descriptor over [base, base + bytes)
// (gfx9 descriptor word 3: 32-bit data format) and a per-lane 32-bit byte
// offset; a load past the range returns zeros (the hardware's range check),
// and no 64-bit address arithmetic runs per lane.
typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint4 buf_ld16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
// 8 bf16 at the per-lane offset plus a wave-uniform one (bytes)
__device__ __forceinline__ bf16x8 buf_ld8(__amdgpu_buffer_rsrc_t r, uint32_t off, int soff) {
  return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, off, soff, 0));
}

// LDS transpose read (ds_read_b64_tr_b16), per 16-lane group: lane j gives
// the address of 4 consecutive 16-bit elements of row j/4 (columns
// 4 (j%4) .. +3) of a 4 x 16 block; lane i receives column i of the 4 rows.
// Stored N-contiguous, this is the K-per-lane MFMA fragment layout.
typedef short i16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ bf16x4 ld_tr4(const bf16* p) {
  i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(const_cast<bf16*>(p)));
  return __builtin_bit_cast(bf16x4, r);
}
__device__ __forceinline__ bf16x8 cat8(bf16x4 a, bf16x4 b) {
  bf16x8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = a[2]; r[3] = a[3];
  r[4] = b[0]; r[5] = b[1]; r[6] = b[2]; r[7] = b[3];
  return r;
}

template <class T> __device__ __forceinline__ T to_t(float x);
template <> __device__ __forceinline__ bf16 to_t<bf16>(float x) { return (bf16)x; }
template <> __device__ __forceinline__ float to_t<float>(float x) { return x; }

__device__ __forceinline__ float to_f(bf16 x) { return (float)x; }
__device__ __forceinline__ float to_f(float x) { return x; }

// 4 contiguous elements from 4 floats (8 B bf16 / 16 B fp32 store).
__device__ __forceinline__ void st4(bf16* p, float a, float b, float c, float d) {
  bf16x4 v;
  v[0] = (bf16)a; v[1] = (bf16)b; v[2] = (bf16)c; v[3] = (bf16)d;
  *reinterpret_cast<bf16x4*>(p) = v;
}
__device__ __forceinline__ void st4(float* p, float a, float b, float c, float d) {
  f32x4 v;
  v[0] = a; v[1] = b; v[2] = c; v[3] = d;
  *reinterpret_cast<f32x4*>(p) = v;
}

__device__ __forceinline__ float sigmoidf_(float x) { return 1.0f / (1.0f + __expf(-x)); }
// sigmoid with the hardware reciprocal (about 1 ulp) instead of an IEEE divide
__device__ __forceinline__ float sigmoid_fast(float x) {
  return __builtin_amdgcn_rcpf(1.0f + __expf(-x));
}

// An opaque copy of a value: address arithmetic derived from it is redone
// where it is used instead of being hoisted out of a loop and kept live in
// registers (one per distinct swizzled address).
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}
// The same for a wave-uniform 64-bit value (kept in a scalar register pair).
__device__ __forceinline__ int64_t opaque_s(int64_t x) {
  asm volatile("" : "+s"(x));
  return x;
}

// Waits until every global load the wave has issued has returned (vmcnt(0);
// expcnt and lgkmcnt left open).  Called after the loads of register-resident
// operands that a loop then reuses (weight fragments): the compiler's wait
// analysis then counts them as complete inside the loop.  Without it, a loop
// whose own loads are conditional (the tile loads of a ragged tail) cannot
// bound how many loads follow them, and waits for every outstanding load,
// the next tile's prefetch included, at their first use in every iteration.
__device__ __forceinline__ void wait_global_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Mean of x[0 .. n) by the whole workgroup in a fixed order (thread-strided
// partial sums, wave butterflies, waves in index order), returned to every
// thread; every thread must call it.
template <int NTH>
__device__ __forceinline__ float block_mean_all(const float* x, int64_t n) {
  __shared__ float red_bm[NTH / 64 + 1];
  const int tid = threadIdx.x;
  float q0 = 0.f, q1 = 0.f, q2 = 0.f, q3 = 0.f;
  int64_t t = tid;
  for (; t + 3 * NTH < n; t += 4 * NTH) {
    q0 += x[t];
    q1 += x[t + NTH];
    q2 += x[t + 2 * NTH];
    q3 += x[t + 3 * NTH];
  }
  for (; t < n; t += NTH) q0 += x[t];
  float q = (q0 + q1) + (q2 + q3);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) q += __shfl_xor(q, o);
  __syncthreads();
  if ((tid & 63) == 0) red_bm[tid >> 6] = q;
  __syncthreads();
  if (tid == 0) {
    float tot = 0.f;
#pragma unroll
    for (int w = 0; w < NTH / 64; ++w) tot += red_bm[w];
    red_bm[NTH / 64] = n > 0 ? tot / (float)n : 0.f;
  }
  __syncthreads();
  return red_bm[NTH / 64];
}

// The same mean, written by thread 0 to *out.
template <int NTH>
__device__ __forceinline__ void block_mean(const float* x, int64_t n, float* out) {
  const float m = block_mean_all<NTH>(x, n);
  if (threadIdx.x == 0) *out = m;
}

// Workgroups are dealt to the 8 XCDs round-robin (id % 8).  Renumber them so
// that each XCD runs one contiguous range of logical ids: neighbouring tiles
// (same head, same weights) then share that XCD's L2.
__device__ __forceinline__ int xcd_logical_id(int id, int n) {
  const int q = n >> 3, r = n & 7;
  const int x = id & 7, s = id >> 3;
  return (x < r) ? x * (q + 1) + s : r * (q + 1) + (x - r) * q + s;
}

}  // namespace lact
