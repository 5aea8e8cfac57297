// Device-side building blocks shared by the gfx950 kernels: element types,
// 16-byte vector loads, MFMA wrappers with one operand layout for fp32 and
// bf16, and wave64 reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float floatx4;

// 16 bytes seen as 8 bf16, 4 floats or 4 dwords.
union V16 {
  uint4 u;
  bf16x8 b;
  floatx4 f;
};

__device__ __forceinline__ V16 ld16(const void* p) {
  V16 v;
  v.u = *reinterpret_cast<const uint4*>(p);
  return v;
}
__device__ __forceinline__ void st16(void* p, const V16& v) { *reinterpret_cast<uint4*>(p) = v.u; }
__device__ __forceinline__ V16 zero16() {
  V16 v;
  v.u = make_uint4(0, 0, 0, 0);
  return v;
}

__device__ __forceinline__ float to_f(float x) { return x; }
__device__ __forceinline__ float to_f(bf16 x) { return static_cast<float>(x); }
template <typename T> __device__ __forceinline__ T from_f(float x);
template <> __device__ __forceinline__ float from_f<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f<bf16>(float x) { return static_cast<bf16>(x); }

// Element i of a 16-byte vector of T.
template <typename T> __device__ __forceinline__ float v16_get(const V16& v, int i);
template <> __device__ __forceinline__ float v16_get<float>(const V16& v, int i) { return v.f[i]; }
template <> __device__ __forceinline__ float v16_get<bf16>(const V16& v, int i) {
  return static_cast<float>(v.b[i]);
}

// ---------------------------------------------------------------------------
// MFMA 16x16 tiles with fp32 accumulation.
//
// Operand layout used everywhere: with lane = 16*g + c (g = lane/16, c = lane%16)
// each lane supplies one 16-byte vector of A row c and one of B column c, at
// K offset g*VEC inside a "vector step" of KSTEP = 4*VEC elements.  For bf16
// (VEC 8) that is exactly one v_mfma_f32_16x16x32_bf16.  For fp32 (VEC 4) it
// is four v_mfma_f32_16x16x4_f32, the i-th consuming element i of both
// vectors: the K index is permuted identically on both operands, which leaves
// the dot product unchanged.  The 16x16 result lives as acc[i] =
// C[row 4*g + i][col c].
// ---------------------------------------------------------------------------
template <typename T> struct Mfma;

template <> struct Mfma<bf16> {
  static constexpr int VEC = 8;
  static constexpr int KSTEP = 32;
  __device__ __forceinline__ static void mac(floatx4& acc, const V16& a, const V16& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.b, b.b, acc, 0, 0, 0);
  }
};

template <> struct Mfma<float> {
  static constexpr int VEC = 4;
  static constexpr int KSTEP = 16;
  __device__ __forceinline__ static void mac(floatx4& acc, const V16& a, const V16& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.f[0], b.f[0], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.f[1], b.f[1], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.f[2], b.f[2], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.f[3], b.f[3], acc, 0, 0, 0);
  }
};

// Split an fp32 vector operand of the 16-byte MFMA layout into bf16 hi/lo
// halves (bf16 MFMA) or pass it through (fp32 MFMA).  src holds VEC floats.
template <typename T> struct SplitOperand;
template <> struct SplitOperand<bf16> {
  static constexpr int PARTS = 2;
  __device__ __forceinline__ static void make(const float* src, V16* out) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const bf16 h = static_cast<bf16>(src[i]);
      out[0].b[i] = h;
      out[1].b[i] = static_cast<bf16>(src[i] - static_cast<float>(h));
    }
  }
};
// Four fp32 values stored as bf16 hi halves (hi = bf16(v)) and lo halves
// (lo = bf16(v - hi)), 8 bytes to each plane: the activation planes that the
// bf16 GEMMs multiply (in LDS, or in memory when a producer writes them).
__device__ __forceinline__ void store_hi_lo4(bf16* hi, bf16* lo, const float4& x) {
  const float v[4] = {x.x, x.y, x.z, x.w};
  bf16x4 h, l;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    h[i] = static_cast<bf16>(v[i]);
    l[i] = static_cast<bf16>(v[i] - static_cast<float>(h[i]));
  }
  *reinterpret_cast<bf16x4*>(hi) = h;
  *reinterpret_cast<bf16x4*>(lo) = l;
}
template <> struct SplitOperand<float> {
  static constexpr int PARTS = 1;
  __device__ __forceinline__ static void make(const float* src, V16* out) {
#pragma unroll
    for (int i = 0; i < 4; ++i) out[0].f[i] = src[i];
  }
};

// ---------------------------------------------------------------------------
// wave64 / block reductions
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Sum over a block of NW waves; `red` is __shared__ float[NW].  Every thread
// gets the total.
template <int NW>
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float t = 0.f;
#pragma unroll
  for (int i = 0; i < NW; ++i) t += red[i];
  __syncthreads();
  return t;
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// Pins prefetched registers at their point of use: an empty volatile asm that
// takes the values and gives them back, ordered with the barriers around it.
// Without it the scheduler hoists the pure-ALU conversion of a prefetched
// operand (fp32 -> bf16 hi/lo) above the previous step's barrier, up to just
// after its load, and the wait for that load then stalls the step that issued
// it -- two slabs of prefetch collapse to none.
template <int N>
__device__ __forceinline__ void hold_regs(float4 (&r)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) asm volatile("" : "+v"(r[i].x), "+v"(r[i].y), "+v"(r[i].z), "+v"(r[i].w));
}

// ---------------------------------------------------------------------------
// Split-K partial sums: acc[i] += sum over s < S of p[i][s * stride] (float4),
// in split order, for NV vectors at once.  The split count is dispatched once
// and every load of a group of up to eight splits is issued before any add:
// a load under a runtime condition (or in a loop with a runtime trip count)
// makes the compiler wait for all earlier loads where the paths join, which
// turns S independent reads into S round trips.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void add4(float4& a, const float4& v) {
  a.x += v.x;
  a.y += v.y;
  a.z += v.z;
  a.w += v.w;
}

template <int NS, int NV>
__device__ __forceinline__ void sum_splits_fixed(float4 (&acc)[NV], const float* const (&p)[NV],
                                                 size_t off, size_t stride) {
  float4 v[NV][NS];
#pragma unroll
  for (int k = 0; k < NS; ++k)
#pragma unroll
    for (int i = 0; i < NV; ++i)
      v[i][k] = *reinterpret_cast<const float4*>(p[i] + off + (size_t)k * stride);
#pragma unroll
  for (int i = 0; i < NV; ++i)
#pragma unroll
    for (int k = 0; k < NS; ++k) add4(acc[i], v[i][k]);
}

// G: most splits loaded at once (8, or less to bound the registers a
// kernel with many vectors holds for the largest case).
template <int NV, int G = 8>
__device__ __forceinline__ void add_splits(float4 (&acc)[NV], const float* const (&p)[NV],
                                           size_t stride, int S) {
  static_assert(G >= 1 && G <= 8, "group of 1..8 splits");
  int s = 0;
  for (; S - s > G; s += G) sum_splits_fixed<G, NV>(acc, p, (size_t)s * stride, stride);
  const size_t off = (size_t)s * stride;
  switch (S - s) {
    case 1: sum_splits_fixed<1, NV>(acc, p, off, stride); break;
    case 2: if constexpr (G >= 2) sum_splits_fixed<2, NV>(acc, p, off, stride); break;
    case 3: if constexpr (G >= 3) sum_splits_fixed<3, NV>(acc, p, off, stride); break;
    case 4: if constexpr (G >= 4) sum_splits_fixed<4, NV>(acc, p, off, stride); break;
    case 5: if constexpr (G >= 5) sum_splits_fixed<5, NV>(acc, p, off, stride); break;
    case 6: if constexpr (G >= 6) sum_splits_fixed<6, NV>(acc, p, off, stride); break;
    case 7: if constexpr (G >= 7) sum_splits_fixed<7, NV>(acc, p, off, stride); break;
    case 8: if constexpr (G >= 8) sum_splits_fixed<8, NV>(acc, p, off, stride); break;
    default: break;
  }
}
