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
  constexpr int EV = 16 / sizeof(T);   // elements per 16-byte vector (d % EV == 0)
  if (!soft) {
    const T* e = emb + (size_t)tok * d;
    for (int c = threadIdx.x; c < d / EV; c += kThreads) {
      const V16 v = ld16(e + c * EV);
#pragma unroll
      for (int q = 0; q < EV; q += 4)
        *reinterpret_cast<float4*>(xr + c * EV + q) =
            make_float4(v16_get<T>(v, q), v16_get<T>(v, q + 1), v16_get<T>(v, q + 2),
                        v16_get<T>(v, q + 3));
    }
    return;
  }
  // an id outside [0, V) contributes nothing: it reads the MASK row with
  // weight 0, so that the eight rows' loads of a vector are issued together
  const int* ids = smooth_id + (size_t)(r * B + j) * 8;
  const float* ps = smooth_p + (size_t)(r * B + j) * 8;
  const T* em = emb + (size_t)mask_id * d;
  const T* er[8];
  float pk[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int id = ids[k];
    const bool ok = id >= 0 && id < V;
    er[k] = emb + (size_t)(ok ? id : mask_id) * d;
    pk[k] = ok ? ps[k] : 0.f;
  }
  for (int c = threadIdx.x; c < d / EV; c += kThreads) {
    const V16 mv = ld16(em + c * EV);
    V16 ev[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) ev[k] = ld16(er[k] + c * EV);
    float o[EV];
#pragma unroll
    for (int q = 0; q < EV; ++q) {
      float sm = 0.f;
#pragma unroll
      for (int k = 0; k < 8; ++k) sm += pk[k] * v16_get<T>(ev[k], q);
      o[q] = (1.f - alpha) * v16_get<T>(mv, q) + alpha * sm;
    }
#pragma unroll
    for (int q = 0; q < EV; q += 4)
      *reinterpret_cast<float4*>(xr + c * EV + q) = make_float4(o[q], o[q + 1], o[q + 2], o[q + 3]);
  }
}

constexpr int kNormThreads = 1024;

// x[m] += sum_s P[s][m] (split order); a[m] = x[m] / sqrt(mean(x^2) + eps) * g.
// One workgroup of 1024 threads per row, one float4 (d <= 4096) or two per
// thread.
// Sum of squares of one row after its split-K partials are added, NV float4
// per thread (threads past the row end read its last vector and add nothing).
template <int NV>
__device__ __forceinline__ float load_row(float4 (&v)[NV], const float* xrow, const float* prow,
                                          int S, size_t p_stride, int d4) {
  const float* pp[NV];
#pragma unroll
  for (int e = 0; e < NV; ++e) {
    const int i = min((int)threadIdx.x + e * kNormThreads, d4 - 1);
    v[e] = reinterpret_cast<const float4*>(xrow)[i];
    pp[e] = prow + 4 * i;
  }
  add_splits<NV>(v, pp, p_stride, S);
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < NV; ++e)
    if ((int)threadIdx.x + e * kNormThreads < d4)
      ss += v[e].x * v[e].x + v[e].y * v[e].y + v[e].z * v[e].z + v[e].w * v[e].w;
  return ss;
}

// out[i] = v * inv * g for this thread's in-range vectors
template <typename T, int NV>
__device__ __forceinline__ void store_norm(float4* orow, const float4 (&v)[NV], float inv,
                                           const T* __restrict__ g, int d4) {
#pragma unroll
  for (int e = 0; e < NV; ++e) {
    const int i = threadIdx.x + e * kNormThreads;
    if (i < d4) {
      const T* gi = g + 4 * i;
      orow[i] = make_float4(v[e].x * inv * to_f(gi[0]), v[e].y * inv * to_f(gi[1]),
                            v[e].z * inv * to_f(gi[2]), v[e].w * inv * to_f(gi[3]));
    }
  }
}

// The same as bf16 hi and lo planes: hi [m][d] at a_hi, lo at a_hi + aps.
template <typename T, int NV>
__device__ __forceinline__ void store_norm_planes(bf16* a_hi, size_t aps, const float4 (&v)[NV],
                                                  float inv, const T* __restrict__ g, int d4) {
#pragma unroll
  for (int e = 0; e < NV; ++e) {
    const int i = threadIdx.x + e * kNormThreads;
    if (i < d4) {
      const T* gi = g + 4 * i;
      store_hi_lo4(a_hi + 4 * i, a_hi + aps + 4 * i,
                   make_float4(v[e].x * inv * to_f(gi[0]), v[e].y * inv * to_f(gi[1]),
                               v[e].z * inv * to_f(gi[2]), v[e].w * inv * to_f(gi[3])));
    }
  }
}

// x[m] += sum_s P[s][m] (split order); a[m] = rmsnorm(x[m]) * g, fp32, or
// (aps > 0) as bf16 hi and lo planes aps elements apart.  One row per
// workgroup, NV = ceil(d / 4096) float4 per thread.
template <typename T, int NV>
__global__ __launch_bounds__(kNormThreads) void add_rmsnorm_kernel(
    const int* __restrict__ nrows, int m_cap, float* __restrict__ x, const float* __restrict__ P,
    int S, size_t p_stride, const T* __restrict__ g, float eps, float* __restrict__ a, int d,
    size_t aps) {
  __shared__ float red[kNormThreads / 64];
  const int m = blockIdx.x;
  // the row count is read together with the row (every row below m_cap is
  // readable): one memory round trip before the reduction instead of two
  const int nr = *nrows;
  const int d4 = d / 4;
  float4 v[NV];
  const float ss = load_row<NV>(v, x + (size_t)m * d, P + (size_t)m * d, S, p_stride, d4);
  if (m >= min(nr, m_cap)) return;
  if (S > 0) {
    float4* xr = reinterpret_cast<float4*>(x + (size_t)m * d);
#pragma unroll
    for (int e = 0; e < NV; ++e)
      if ((int)threadIdx.x + e * kNormThreads < d4) xr[threadIdx.x + e * kNormThreads] = v[e];
  }
  const float tot = block_sum<kNormThreads / 64>(ss, red);
  const float inv = 1.f / sqrtf(tot / d + eps);
  if (aps)
    store_norm_planes<T, NV>(reinterpret_cast<bf16*>(a) + (size_t)m * d, aps, v, inv, g, d4);
  else
    store_norm<T, NV>(reinterpret_cast<float4*>(a + (size_t)m * d), v, inv, g, d4);
}

// QKV: sum the split-K partials, rotate q and k (pair (j, j+hd/2) by the
// angle pos*theta^(-2j/hd), from a table built in fp64), write q for the
// attention and scatter k, v into the cache at the row's position -- before
// any query of this layer reads the cache (dInfer news article, section
// "削减计算成本：邻近KV缓存刷新": only the window's KV is recomputed).
// K goes to [request][head][Lp][hd]; V to transposed tiles of 32 positions,
// [request][head][Lp/32][hd][32], through an LDS tile, so that consecutive
// threads store consecutive positions.  A workgroup takes 8 rows of one head
// (16 threads per row), so a 64-row window still spreads over 256 workgroups.
constexpr int kQkvRows = 8;
constexpr int kQkvThreads = 128;

template <typename T, int G>
__global__ __launch_bounds__(kQkvThreads) void qkv_rope_scatter_kernel(
    PassTable tb, int m_cap, const float* __restrict__ P, int S, size_t p_stride, int d, int H,
    int hd, const float* __restrict__ rope_cs, float* __restrict__ q_out, T* __restrict__ kc,
    T* __restrict__ vt, int Lp) {
  __shared__ float vs[128 * (kQkvRows + 1)];
  __shared__ int s_req[kQkvRows], s_pos[kQkvRows];
  const int m0 = blockIdx.x * kQkvRows;
  const int h = blockIdx.y;
  const int half = hd / 2;
  const int rr = threadIdx.x / 16;                // row of the tile
  const int m = m0 + rr;
  // The row count, the row's table entries and its partials are loaded
  // together (rows past the pass read row min(m, m_cap - 1), which is
  // readable; nothing of theirs is stored).  One vector of each half of the
  // head per thread (hd <= 128); threads past half load a clamped column.
  const int nr = *tb.nrows;
  const int mm = min(m, m_cap - 1);
  const int r = tb.row_req[mm];
  const int pos = tb.row_pos[mm];
  const int j = (threadIdx.x % 16) * 4;
  const int jj = min(j, half - 4);
  const float* pr = P + (size_t)mm * 3 * d;
  const int c0 = h * hd + jj;
  const int c1 = c0 + half;
  const float4 z4 = make_float4(0.f, 0.f, 0.f, 0.f);
  float4 t[6] = {z4, z4, z4, z4, z4, z4};
  const float* const pp[6] = {pr + c0, pr + c1, pr + d + c0, pr + d + c1, pr + 2 * d + c0,
                              pr + 2 * d + c1};
  add_splits<6, G>(t, pp, p_stride, S);
  const int M = min(nr, m_cap);
  if (m0 >= M) return;
  if (threadIdx.x % 16 == 0) {
    s_req[rr] = r;
    s_pos[rr] = pos;
  }
  if (m < M && j < half) {
    const float* cs = rope_cs + (size_t)pos * hd;   // [pos][cos half | sin half]
    T* kp = kc + (((size_t)r * H + h) * Lp + pos) * hd;
    float* qr = q_out + (size_t)m * d + h * hd;
    const float4 q0 = t[0], q1 = t[1], k0 = t[2], k1 = t[3], v0 = t[4], v1 = t[5];
    const float4 c = *reinterpret_cast<const float4*>(cs + j);
    const float4 sn = *reinterpret_cast<const float4*>(cs + half + j);
    *reinterpret_cast<float4*>(qr + j) =
        make_float4(q0.x * c.x - q1.x * sn.x, q0.y * c.y - q1.y * sn.y,
                    q0.z * c.z - q1.z * sn.z, q0.w * c.w - q1.w * sn.w);
    *reinterpret_cast<float4*>(qr + j + half) =
        make_float4(q1.x * c.x + q0.x * sn.x, q1.y * c.y + q0.y * sn.y,
                    q1.z * c.z + q0.z * sn.z, q1.w * c.w + q0.w * sn.w);
    const float ka[4] = {k0.x * c.x - k1.x * sn.x, k0.y * c.y - k1.y * sn.y,
                         k0.z * c.z - k1.z * sn.z, k0.w * c.w - k1.w * sn.w};
    const float kb[4] = {k1.x * c.x + k0.x * sn.x, k1.y * c.y + k0.y * sn.y,
                         k1.z * c.z + k0.z * sn.z, k1.w * c.w + k0.w * sn.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      kp[j + e] = from_f<T>(ka[e]);
      kp[j + half + e] = from_f<T>(kb[e]);
    }
    const float va[4] = {v0.x, v0.y, v0.z, v0.w};
    const float vb[4] = {v1.x, v1.y, v1.z, v1.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      vs[(j + e) * (kQkvRows + 1) + rr] = va[e];
      vs[(j + half + e) * (kQkvRows + 1) + rr] = vb[e];
    }
  }
  __syncthreads();
  // V^T: element (dim hi, tile row rr2), rows fastest
  for (int e = threadIdx.x; e < hd * kQkvRows; e += kQkvThreads) {
    const int rr2 = e % kQkvRows;
    const int hi = e / kQkvRows;
    if (m0 + rr2 >= M) continue;
    const int r2 = s_req[rr2];
    const int pos2 = s_pos[rr2];
    vt[(((size_t)r2 * H + h) * Lp + (pos2 & ~31)) * hd + hi * 32 + (pos2 & 31)] =
        from_f<T>(vs[hi * (kQkvRows + 1) + rr2]);
  }
}

// act[m][f] = silu(gate) * up with gate, up summed over the split-K partials
// of the fused [gate | up] projection (float4 per thread).
template <int G>
__global__ __launch_bounds__(kThreads) void swiglu_kernel(const int* __restrict__ nrows, int m_cap,
                                                          const float* __restrict__ P, int S,
                                                          size_t p_stride, int F,
                                                          float* __restrict__ act, size_t aps) {
  // rows up to m_cap are read (all readable) while the row count loads;
  // only the pass's rows are stored
  const int nr = *nrows;
  const int F4 = F / 4;
  const size_t total = (size_t)m_cap * F4;
  const float4 z4 = make_float4(0.f, 0.f, 0.f, 0.f);
  for (size_t idx = (size_t)blockIdx.x * kThreads + threadIdx.x; idx < total;
       idx += (size_t)gridDim.x * kThreads) {
    const size_t m = idx / F4;
    const size_t f = (idx % F4) * 4;
    const float* pr = P + m * 2 * F;
    float4 t[2] = {z4, z4};
    const float* const pp[2] = {pr + f, pr + F + f};
    add_splits<2, G>(t, pp, p_stride, S);
    const float4 g = t[0], u = t[1];
    if ((int)m < min(nr, m_cap)) {
      const float4 y = make_float4(g.x / (1.f + expf(-g.x)) * u.x, g.y / (1.f + expf(-g.y)) * u.y,
                                   g.z / (1.f + expf(-g.z)) * u.z, g.w / (1.f + expf(-g.w)) * u.w);
      if (aps) {
        bf16* hi = reinterpret_cast<bf16*>(act) + m * F + f;
        store_hi_lo4(hi, hi + aps, y);
      } else {
        *reinterpret_cast<float4*>(act + m * F + f) = y;
      }
    }
  }
}

// Block rows only: residual add of the last layer, final RMSNorm, and the
// row's planting for the vocab statistics.
template <typename T, int NV>
__global__ __launch_bounds__(kNormThreads) void final_norm_kernel(
    PassTable tb, int B, const float* __restrict__ x, const float* __restrict__ P, int S,
    size_t p_stride, const T* __restrict__ g, float eps, float* __restrict__ out, int d,
    const int* __restrict__ plant_id, const float* __restrict__ plant_bias, int max_len,
    int* __restrict__ row_plant_id, float* __restrict__ row_plant_bias) {
  __shared__ float red[kNormThreads / 64];
  const int rr = blockIdx.x;
  const int r = rr / B;
  const int j = rr % B;
  const int d4 = d / 4;
  float4* orow = reinterpret_cast<float4*>(out + (size_t)rr * d);
  if (!tb.req_active[r] || tb.req_nrows[r] == 0) {
    for (int i = threadIdx.x; i < d4; i += kNormThreads) orow[i] = make_float4(0.f, 0.f, 0.f, 0.f);
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
  float4 v[NV];
  const float ss = load_row<NV>(v, x + (size_t)m * d, P + (size_t)m * d, S, p_stride, d4);
  const float tot = block_sum<kNormThreads / 64>(ss, red);
  const float inv = 1.f / sqrtf(tot / d + eps);
  store_norm<T, NV>(orow, v, inv, g, d4);
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
  if (d % 8 != 0) return hipErrorInvalidValue;   // whole 16-byte vectors per row
  DISPATCH_T(t, hipLaunchKernelGGL((embed_kernel<T>), dim3(m_cap), dim3(kThreads), 0, st, tb,
                                   tokens, max_len, static_cast<const T*>(emb), d, V, mask_id, alpha,
                                   smooth_id, smooth_p, smooth_valid, B, x));
  return hipGetLastError();
}

hipError_t launch_add_rmsnorm(DType t, const int* nrows, int m_cap, float* x, const float* P,
                              int S, size_t p_stride, const void* g, float eps, float* a, int d,
                              hipStream_t st, size_t aps) {
  if (d > 8 * kNormThreads || d % 4 != 0) return hipErrorInvalidValue;
  if (d <= 4 * kNormThreads) {
    DISPATCH_T(t, hipLaunchKernelGGL((add_rmsnorm_kernel<T, 1>), dim3(m_cap), dim3(kNormThreads),
                                     0, st, nrows, m_cap, x, P, S, p_stride,
                                     static_cast<const T*>(g), eps, a, d, aps));
  } else {
    DISPATCH_T(t, hipLaunchKernelGGL((add_rmsnorm_kernel<T, 2>), dim3(m_cap), dim3(kNormThreads),
                                     0, st, nrows, m_cap, x, P, S, p_stride,
                                     static_cast<const T*>(g), eps, a, d, aps));
  }
  return hipGetLastError();
}

hipError_t launch_qkv_rope_scatter(DType t, PassTable tb, int m_cap, const float* P, int S,
                                   size_t p_stride, int d, int H, int hd, const float* rope_cs,
                                   float* q_out, void* kc, void* vt, int Lp, hipStream_t st) {
  if (hd > 128 || hd % 8 != 0 || m_cap < 1) return hipErrorInvalidValue;
  const dim3 grid((m_cap + kQkvRows - 1) / kQkvRows, H);
  // unsplit input (many-row passes): a small register set keeps occupancy up
  if (S <= 1) {
    DISPATCH_T(t, hipLaunchKernelGGL((qkv_rope_scatter_kernel<T, 1>), grid, dim3(kQkvThreads), 0,
                                     st, tb, m_cap, P, S, p_stride, d, H, hd, rope_cs, q_out,
                                     static_cast<T*>(kc), static_cast<T*>(vt), Lp));
  } else {
    DISPATCH_T(t, hipLaunchKernelGGL((qkv_rope_scatter_kernel<T, 8>), grid, dim3(kQkvThreads), 0,
                                     st, tb, m_cap, P, S, p_stride, d, H, hd, rope_cs, q_out,
                                     static_cast<T*>(kc), static_cast<T*>(vt), Lp));
  }
  return hipGetLastError();
}

hipError_t launch_swiglu(const int* nrows, int m_cap, const float* P, int S, size_t p_stride,
                         int F, float* act, hipStream_t st, size_t aps) {
  if (F % 4 != 0) return hipErrorInvalidValue;
  size_t total = (size_t)m_cap * F / 4;
  int blocks = (int)((total + kThreads - 1) / kThreads);
  if (blocks > 8192) blocks = 8192;
  if (S <= 1)   // unsplit input (many-row passes): fewer registers, more waves
    hipLaunchKernelGGL(swiglu_kernel<1>, dim3(blocks), dim3(kThreads), 0, st, nrows, m_cap, P, S,
                       p_stride, F, act, aps);
  else
    hipLaunchKernelGGL(swiglu_kernel<8>, dim3(blocks), dim3(kThreads), 0, st, nrows, m_cap, P, S,
                       p_stride, F, act, aps);
  return hipGetLastError();
}

hipError_t launch_final_norm(DType t, PassTable tb, int batch, int B, const float* x,
                             const float* P, int S, size_t p_stride, const void* g, float eps,
                             float* out, int d, const int* plant_id, const float* plant_bias,
                             int max_len, int* row_plant_id, float* row_plant_bias,
                             hipStream_t st) {
  if (d > 8 * kNormThreads || d % 4 != 0) return hipErrorInvalidValue;
  if (d <= 4 * kNormThreads) {
    DISPATCH_T(t, hipLaunchKernelGGL((final_norm_kernel<T, 1>), dim3(batch * B), dim3(kNormThreads),
                                     0, st, tb, B, x, P, S, p_stride, static_cast<const T*>(g), eps,
                                     out, d, plant_id, plant_bias, max_len, row_plant_id,
                                     row_plant_bias));
  } else {
    DISPATCH_T(t, hipLaunchKernelGGL((final_norm_kernel<T, 2>), dim3(batch * B), dim3(kNormThreads),
                                     0, st, tb, B, x, P, S, p_stride, static_cast<const T*>(g), eps,
                                     out, d, plant_id, plant_bias, max_len, row_plant_id,
                                     row_plant_bias));
  }
  return hipGetLastError();
}

}  // namespace dinfer
