// Row-wise kernels of the denoising step: window embedding (hard or
// iteration-smoothed), residual add + RMSNorm, QKV split-K reduction + RoPE +
// vicinity scatter into the KV cache, SwiGLU, and the final norm of the block
// rows.  All are HBM/latency-bound and touch each element once.
#include "common.h"
#include "kernels.h"

namespace dinfer {

namespace {

constexpr int kThreads = 256;

// Input embedding of every row of a pass.  Still-masked block positions that
// carry smoothing state take (1-alpha) E[MASK] + alpha * sum_j p~_j E[id_j]
// (dInfer news article, section "解码的艺术", iteration smoothing bullet);
// every other row takes its token's embedding.
// Token ids outside [0, V) are read as MASK (never an out-of-range row).
template <typename T>
__global__ __launch_bounds__(kThreads) void embed_kernel(PassTable tb, const int* __restrict__ tokens,
                                                         int max_len, const T* __restrict__ emb, int d,
                                                         int V, int mask_id, float alpha,
                                                         const int* __restrict__ smooth_id,
                                                         const float* __restrict__ smooth_p,
                                                         const uint8_t* __restrict__ smooth_valid,
                                                         int B, float* __restrict__ x) {
  const int m = blockIdx.x;
  if (m >= *tb.nrows) return;
  const int r = tb.row_req[m];
  const int p = tb.row_pos[m];
  int tok = tokens[(size_t)r * max_len + p];
  if (tok < 0 || tok >= V) tok = mask_id;
  const int j = p - tb.req_bs[r];
  const bool soft = alpha != 0.f && tok == mask_id && j >= 0 && j < B &&
                    smooth_valid[r * B + j] != 0;
  float* xr = x + (size_t)m * d;
  if (!soft) {
    const T* e = emb + (size_t)tok * d;
    for (int i = threadIdx.x; i < d; i += kThreads) xr[i] = to_f(e[i]);
    return;
  }
  const int* ids = smooth_id + (size_t)(r * B + j) * 8;
  const float* ps = smooth_p + (size_t)(r * B + j) * 8;
  const T* em = emb + (size_t)mask_id * d;
  for (int i = threadIdx.x; i < d; i += kThreads) {
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int id = ids[k];
      if (id >= 0 && id < V) s += ps[k] * to_f(emb[(size_t)id * d + i]);
    }
    xr[i] = (1.f - alpha) * to_f(em[i]) + alpha * s;
  }
}

// x[m] += sum_s P[s][m] (split order); a[m] = x[m] / sqrt(mean(x^2) + eps) * g.
template <typename T>
__global__ __launch_bounds__(kThreads) void add_rmsnorm_kernel(const int* __restrict__ nrows, int m_cap,
                                                               float* __restrict__ x,
                                                               const float* __restrict__ P, int S,
                                                               size_t p_stride,
                                                               const T* __restrict__ g, float eps,
                                                               float* __restrict__ a, int d) {
  constexpr int MAXE = 32;   // d <= 8192
  __shared__ float red[kThreads / 64];
  const int m = blockIdx.x;
  if (m >= min(*nrows, m_cap)) return;
  float v[MAXE];
  float ss = 0.f;
  float* xr = x + (size_t)m * d;
#pragma unroll
  for (int e = 0; e < MAXE; ++e) {
    const int i = threadIdx.x + e * kThreads;
    if (i < d) {
      float xv = xr[i];
      for (int s = 0; s < S; ++s) xv += P[s * p_stride + (size_t)m * d + i];
      if (S > 0) xr[i] = xv;
      v[e] = xv;
      ss += xv * xv;
    }
  }
  const float tot = block_sum<kThreads / 64>(ss, red);
  const float inv = 1.f / sqrtf(tot / d + eps);
  float* ar = a + (size_t)m * d;
#pragma unroll
  for (int e = 0; e < MAXE; ++e) {
    const int i = threadIdx.x + e * kThreads;
    if (i < d) ar[i] = v[e] * inv * to_f(g[i]);
  }
}

// QKV: sum the split-K partials, rotate q and k (pair (j, j+hd/2) by the
// angle pos*theta^(-2j/hd), from a table built in fp64), write q for the
// attention and scatter k, v into the cache at the row's position -- before
// any query of this layer reads the cache (dInfer news article, section
// "削减计算成本：邻近KV缓存刷新": only the window's KV is recomputed).
template <typename T>
__global__ __launch_bounds__(kThreads) void qkv_rope_scatter_kernel(
    PassTable tb, int m_cap, const float* __restrict__ P, int S, size_t p_stride, int d, int H,
    int hd, const float* __restrict__ rope_cs, float* __restrict__ q_out, T* __restrict__ kc,
    T* __restrict__ vc, int max_len) {
  const int m = blockIdx.x;
  if (m >= min(*tb.nrows, m_cap)) return;
  const int r = tb.row_req[m];
  const int pos = tb.row_pos[m];
  const int half = hd / 2;
  const int N3 = 3 * d;
  const float* pr = P + (size_t)m * N3;
  const float* cs = rope_cs + (size_t)pos * hd;   // [pos][cos half | sin half]
  for (int i = threadIdx.x; i < H * half; i += kThreads) {
    const int h = i / half;
    const int j = i % half;
    const int c0 = h * hd + j;
    const int c1 = c0 + half;
    float q0 = 0.f, q1 = 0.f, k0 = 0.f, k1 = 0.f, v0 = 0.f, v1 = 0.f;
    for (int s = 0; s < S; ++s) {
      const float* ps = pr + s * p_stride;
      q0 += ps[c0];
      q1 += ps[c1];
      k0 += ps[d + c0];
      k1 += ps[d + c1];
      v0 += ps[2 * d + c0];
      v1 += ps[2 * d + c1];
    }
    const float c = cs[j];
    const float sn = cs[half + j];
    float* qr = q_out + (size_t)m * d;
    qr[c0] = q0 * c - q1 * sn;
    qr[c1] = q1 * c + q0 * sn;
    const size_t cb = (((size_t)r * H + h) * max_len + pos) * hd;
    kc[cb + j] = from_f<T>(k0 * c - k1 * sn);
    kc[cb + j + half] = from_f<T>(k1 * c + k0 * sn);
    vc[cb + j] = from_f<T>(v0);
    vc[cb + j + half] = from_f<T>(v1);
  }
}

// act[m][f] = silu(gate) * up with gate, up summed over the split-K partials
// of the fused [gate | up] projection.
__global__ __launch_bounds__(kThreads) void swiglu_kernel(const int* __restrict__ nrows, int m_cap,
                                                          const float* __restrict__ P, int S,
                                                          size_t p_stride, int F,
                                                          float* __restrict__ act) {
  const int M = min(*nrows, m_cap);
  const size_t total = (size_t)M * F;
  for (size_t idx = (size_t)blockIdx.x * kThreads + threadIdx.x; idx < total;
       idx += (size_t)gridDim.x * kThreads) {
    const size_t m = idx / F;
    const size_t f = idx % F;
    const float* pr = P + m * 2 * F;
    float g = 0.f, u = 0.f;
    for (int s = 0; s < S; ++s) {
      g += pr[s * p_stride + f];
      u += pr[s * p_stride + F + f];
    }
    act[idx] = g / (1.f + expf(-g)) * u;
  }
}

// Block rows only: residual add of the last layer, final RMSNorm, and the
// row's planting for the vocab statistics.
template <typename T>
__global__ __launch_bounds__(kThreads) void final_norm_kernel(
    PassTable tb, int B, const float* __restrict__ x, const float* __restrict__ P, int S,
    size_t p_stride, const T* __restrict__ g, float eps, float* __restrict__ out, int d,
    const int* __restrict__ plant_id, const float* __restrict__ plant_bias, int max_len,
    int* __restrict__ row_plant_id, float* __restrict__ row_plant_bias) {
  constexpr int MAXE = 32;
  __shared__ float red[kThreads / 64];
  const int rr = blockIdx.x;
  const int r = rr / B;
  const int j = rr % B;
  float* orow = out + (size_t)rr * d;
  if (!tb.req_active[r] || tb.req_nrows[r] == 0) {
    for (int i = threadIdx.x; i < d; i += kThreads) orow[i] = 0.f;
    if (threadIdx.x == 0) {
      row_plant_id[rr] = -1;
      row_plant_bias[rr] = 0.f;
    }
    return;
  }
  const int off = tb.req_row_off[r];
  const int lo = tb.row_pos[off];
  const int bs = tb.req_bs[r];
  const int m = off + (bs - lo) + j;
  float v[MAXE];
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < MAXE; ++e) {
    const int i = threadIdx.x + e * kThreads;
    if (i < d) {
      float xv = x[(size_t)m * d + i];
      for (int s = 0; s < S; ++s) xv += P[s * p_stride + (size_t)m * d + i];
      v[e] = xv;
      ss += xv * xv;
    }
  }
  const float tot = block_sum<kThreads / 64>(ss, red);
  const float inv = 1.f / sqrtf(tot / d + eps);
#pragma unroll
  for (int e = 0; e < MAXE; ++e) {
    const int i = threadIdx.x + e * kThreads;
    if (i < d) orow[i] = v[e] * inv * to_f(g[i]);
  }
  if (threadIdx.x == 0) {
    row_plant_id[rr] = plant_id ? plant_id[(size_t)r * max_len + bs + j] : -1;
    row_plant_bias[rr] = plant_bias ? plant_bias[r] : 0.f;
  }
}

}  // namespace

#define DISPATCH_T(t, ...)                   \
  if ((t) == DType::F32) {                   \
    using T = float;                         \
    __VA_ARGS__;                             \
  } else {                                   \
    using T = bf16;                          \
    __VA_ARGS__;                             \
  }

hipError_t launch_embed(DType t, PassTable tb, int m_cap, const int* tokens, int max_len,
                        const void* emb, int d, int V, int mask_id, float alpha, const int* smooth_id,
                        const float* smooth_p, const uint8_t* smooth_valid, int B, float* x,
                        hipStream_t st) {
  DISPATCH_T(t, hipLaunchKernelGGL((embed_kernel<T>), dim3(m_cap), dim3(kThreads), 0, st, tb,
                                   tokens, max_len, static_cast<const T*>(emb), d, V, mask_id, alpha,
                                   smooth_id, smooth_p, smooth_valid, B, x));
  return hipGetLastError();
}

hipError_t launch_add_rmsnorm(DType t, const int* nrows, int m_cap, float* x, const float* P,
                              int S, size_t p_stride, const void* g, float eps, float* a, int d,
                              hipStream_t st) {
  if (d > 32 * kThreads) return hipErrorInvalidValue;
  DISPATCH_T(t, hipLaunchKernelGGL((add_rmsnorm_kernel<T>), dim3(m_cap), dim3(kThreads), 0, st,
                                   nrows, m_cap, x, P, S, p_stride, static_cast<const T*>(g), eps,
                                   a, d));
  return hipGetLastError();
}

hipError_t launch_qkv_rope_scatter(DType t, PassTable tb, int m_cap, const float* P, int S,
                                   size_t p_stride, int d, int H, int hd, const float* rope_cs,
                                   float* q_out, void* kc, void* vc, int max_len, hipStream_t st) {
  DISPATCH_T(t, hipLaunchKernelGGL((qkv_rope_scatter_kernel<T>), dim3(m_cap), dim3(kThreads), 0,
                                   st, tb, m_cap, P, S, p_stride, d, H, hd, rope_cs, q_out,
                                   static_cast<T*>(kc),
                                   static_cast<T*>(vc), max_len));
  return hipGetLastError();
}

hipError_t launch_swiglu(const int* nrows, int m_cap, const float* P, int S, size_t p_stride,
                         int F, float* act, hipStream_t st) {
  size_t total = (size_t)m_cap * F;
  int blocks = (int)((total + kThreads - 1) / kThreads);
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(swiglu_kernel, dim3(blocks), dim3(kThreads), 0, st, nrows, m_cap, P, S,
                     p_stride, F, act);
  return hipGetLastError();
}

hipError_t launch_final_norm(DType t, PassTable tb, int batch, int B, const float* x,
                             const float* P, int S, size_t p_stride, const void* g, float eps,
                             float* out, int d, const int* plant_id, const float* plant_bias,
                             int max_len, int* row_plant_id, float* row_plant_bias,
                             hipStream_t st) {
  if (d > 32 * kThreads) return hipErrorInvalidValue;
  DISPATCH_T(t, hipLaunchKernelGGL((final_norm_kernel<T>), dim3(batch * B), dim3(kThreads), 0, st,
                                   tb, B, x, P, S, p_stride, static_cast<const T*>(g), eps,
                                   out, d, plant_id, plant_bias, max_len,
                                   row_plant_id, row_plant_bias));
  return hipGetLastError();
}

}  // namespace dinfer
