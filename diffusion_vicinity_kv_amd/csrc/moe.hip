// Mixture-of-experts FFN of the MoE dLLM (dInfer abstract: MoE model; TIDE
// abstract: expert activations are stable within a block, which the router's
// per-block preference bias of the workload reproduces).
//
//   route  : router logits r = f W_r^T + bias[request][layer][block] (fp32,
//            kept per row), softmax over the experts, the top_k by (logit
//            desc, id asc), gates renormalised over the selected experts
//   plan   : per-expert counts, offsets and row lists of the (row, slot)
//            assignments, in row order (deterministic), plus each
//            assignment's position in the packed list
//   experts: grouped projections (gemm.hip) over the packed list, SwiGLU
//   combine: x[m] += shared-expert partials (split order) + sum over slots of
//            gate * expert output (slot order)
#include "common.h"
#include "kernels.h"

#include <climits>

namespace dinfer {

namespace {

constexpr int kMaxE = 64;
constexpr int kMaxTopK = 8;

// One workgroup (256 threads) per row.
template <typename T>
__global__ __launch_bounds__(256) void moe_route_kernel(PassTable tb, int m_cap,
                                                        const float* __restrict__ f, int d,
                                                        const T* __restrict__ Wr, int E, int top_k,
                                                        const float* __restrict__ router_bias,
                                                        int n_layers, int n_blocks, int layer,
                                                        int* __restrict__ sel,
                                                        float* __restrict__ gate,
                                                        float* __restrict__ rlog) {
  __shared__ float logit[kMaxE];
  const int m = blockIdx.x;
  if (m >= min(*tb.nrows, m_cap)) return;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const float* fr = f + (size_t)m * d;
  for (int e = wave; e < E; e += 4) {
    const T* w = Wr + (size_t)e * d;
    float s = 0.f;
    for (int k = lane * 4; k < d; k += 256) {
      const float4 x = *reinterpret_cast<const float4*>(fr + k);
      s += x.x * to_f(w[k]) + x.y * to_f(w[k + 1]) + x.z * to_f(w[k + 2]) + x.w * to_f(w[k + 3]);
    }
    s = wave_sum(s);
    if (lane == 0) logit[e] = s;
  }
  __syncthreads();
  if (wave != 0) return;
  const int r = tb.row_req[m];
  float v = -INFINITY;
  if (lane < E) {
    v = logit[lane];
    if (router_bias)
      v += router_bias[(((size_t)r * n_layers + layer) * n_blocks + tb.req_blk[r]) * E + lane];
    rlog[(size_t)m * E + lane] = v;
  }
  const float mx = wave_max(v);
  // top_k by (value desc, id asc); the selected lanes drop out one by one
  float cand = v;
  int chosen_id[kMaxTopK];
  float chosen_v[kMaxTopK];
#pragma unroll
  for (int k = 0; k < kMaxTopK; ++k) {
    if (k >= top_k) break;
    float bv = cand;
    int bi = lane < E ? lane : INT_MAX;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(bv, o, 64);
      const int oi = __shfl_xor(bi, o, 64);
      if (ov > bv || (ov == bv && oi < bi)) {
        bv = ov;
        bi = oi;
      }
    }
    chosen_id[k] = bi;
    chosen_v[k] = bv;
    if (lane == bi) cand = -INFINITY;
  }
  float z = 0.f;
#pragma unroll
  for (int k = 0; k < kMaxTopK; ++k)
    if (k < top_k) z += expf(chosen_v[k] - mx);
#pragma unroll
  for (int k = 0; k < kMaxTopK; ++k)
    if (k < top_k && lane == k) {
      sel[(size_t)m * top_k + k] = chosen_id[k];
      gate[(size_t)m * top_k + k] = expf(chosen_v[k] - mx) / z;
    }
}

// One workgroup of E*G threads: thread (e, g) owns expert e over the g-th
// range of assignments.  Counts per (e, g), an exclusive scan in (e, g)
// order, then positions: assignments of an expert appear in row order.
constexpr int kPlanGroups = 16;

__global__ __launch_bounds__(kMaxE * kPlanGroups) void moe_plan_kernel(
    const int* __restrict__ nrows, int m_cap, const int* __restrict__ sel, int E, int top_k,
    int* __restrict__ e_count, int* __restrict__ e_off, int* __restrict__ row_of,
    int* __restrict__ pos, int* __restrict__ n_assign) {
  __shared__ int cnt[kMaxE * kPlanGroups];
  const int t = threadIdx.x;
  const int e = t / kPlanGroups;
  const int g = t % kPlanGroups;
  const int M = min(*nrows, m_cap);
  const int total = M * top_k;
  const int a0 = (int)((long long)total * g / kPlanGroups);
  const int a1 = (int)((long long)total * (g + 1) / kPlanGroups);
  int c = 0;
  if (e < E)
    for (int a = a0; a < a1; ++a) c += (sel[a] == e);
  // exclusive scan of the counts in thread order (= (expert, group) order)
  __shared__ int wsum[kMaxE * kPlanGroups / 64];
  const int lane = t & 63;
  const int wave = t >> 6;
  int incl = c;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o, 64);
    if (lane >= o) incl += y;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  if (t == 0) {
    int run = 0;
    for (int w = 0; w < kMaxE * kPlanGroups / 64; ++w) {
      const int x = wsum[w];
      wsum[w] = run;
      run += x;
    }
    *n_assign = run;
  }
  __syncthreads();
  cnt[t] = wsum[wave] + incl - c;
  __syncthreads();
  if (e < E) {
    int p = cnt[t];
    if (g == 0) {
      e_off[e] = p;
      const int next = (e + 1 < E) ? cnt[(e + 1) * kPlanGroups] : *n_assign;
      e_count[e] = next - p;
    }
    for (int a = a0; a < a1; ++a)
      if (sel[a] == e) {
        row_of[p] = a / top_k;
        pos[a] = p;
        ++p;
      }
  }
}

// x[m] += sum_s P[s][m] + sum_k gate[m][k] * Y[pos[m][k]]  (float4 per thread)
__global__ __launch_bounds__(256) void moe_combine_kernel(
    const int* __restrict__ nrows, int m_cap, float* __restrict__ x, const float* __restrict__ P,
    int S, size_t p_stride, const float* __restrict__ Y, const int* __restrict__ pos,
    const float* __restrict__ gate, int top_k, int d) {
  const int m = blockIdx.x;
  if (m >= min(*nrows, m_cap)) return;
  const int d4 = d / 4;
  for (int i = threadIdx.x; i < d4; i += 256) {
    float4 acc = reinterpret_cast<float4*>(x + (size_t)m * d)[i];
    for (int s = 0; s < S; ++s) {
      const float4 v = *reinterpret_cast<const float4*>(P + s * p_stride + (size_t)m * d + 4 * i);
      acc.x += v.x;
      acc.y += v.y;
      acc.z += v.z;
      acc.w += v.w;
    }
    for (int k = 0; k < top_k; ++k) {
      const float gk = gate[(size_t)m * top_k + k];
      const float4 v =
          *reinterpret_cast<const float4*>(Y + (size_t)pos[(size_t)m * top_k + k] * d + 4 * i);
      acc.x += gk * v.x;
      acc.y += gk * v.y;
      acc.z += gk * v.z;
      acc.w += gk * v.w;
    }
    reinterpret_cast<float4*>(x + (size_t)m * d)[i] = acc;
  }
}

}  // namespace

hipError_t launch_moe_route(DType t, PassTable tb, int m_cap, const float* f, int d,
                            const void* Wr, int E, int top_k, const float* router_bias,
                            int n_layers, int n_blocks, int layer, int* sel, float* gate,
                            float* rlog, hipStream_t st) {
  if (E > kMaxE || top_k > kMaxTopK || top_k > E || d % 4 != 0) return hipErrorInvalidValue;
  if (t == DType::F32)
    hipLaunchKernelGGL(moe_route_kernel<float>, dim3(m_cap), dim3(256), 0, st, tb, m_cap, f, d,
                       static_cast<const float*>(Wr), E, top_k, router_bias, n_layers, n_blocks,
                       layer, sel, gate, rlog);
  else
    hipLaunchKernelGGL(moe_route_kernel<bf16>, dim3(m_cap), dim3(256), 0, st, tb, m_cap, f, d,
                       static_cast<const bf16*>(Wr), E, top_k, router_bias, n_layers, n_blocks,
                       layer, sel, gate, rlog);
  return hipGetLastError();
}

hipError_t launch_moe_plan(const int* nrows, int m_cap, const int* sel, int E, int top_k,
                           int* e_count, int* e_off, int* row_of, int* pos, int* n_assign,
                           hipStream_t st) {
  if (E > kMaxE) return hipErrorInvalidValue;
  hipLaunchKernelGGL(moe_plan_kernel, dim3(1), dim3(kMaxE * kPlanGroups), 0, st, nrows, m_cap, sel,
                     E, top_k, e_count, e_off, row_of, pos, n_assign);
  return hipGetLastError();
}

hipError_t launch_moe_combine(const int* nrows, int m_cap, float* x, const float* P, int S,
                              size_t p_stride, const float* Y, const int* pos, const float* gate,
                              int top_k, int d, hipStream_t st) {
  if (d % 4 != 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(moe_combine_kernel, dim3(m_cap), dim3(256), 0, st, nrows, m_cap, x, P, S,
                     p_stride, Y, pos, gate, top_k, d);
  return hipGetLastError();
}

}  // namespace dinfer
