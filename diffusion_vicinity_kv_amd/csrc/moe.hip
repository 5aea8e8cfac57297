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
#include "vocab_common.h"

#include <climits>

namespace dinfer {

namespace {

constexpr int kMaxE = 64;
constexpr int kMaxTopK = 8;

// One workgroup of sixteen waves per row (measured 0.7% faster on the MoE
// window step than eight waves of eight experts).  Wave w takes experts
// [w*epw, (w+1)*epw) (epw = ceil(E/16) <= 4): its lanes walk the row d in
// 16-byte steps, every lane loading the same stretch of each of the wave's
// router rows (one contiguous kilobyte per load instruction) and of the
// activation row, and keeping one partial dot product per expert; the
// partials are summed across the wave, the logits meet in LDS, and wave 0
// picks the top_k by repeated wave argmax.  The row count and the row's
// request are read together with the row.
constexpr int kRouteWaves = 16;

template <typename T>
__global__ __launch_bounds__(64 * kRouteWaves) void moe_route_kernel(PassTable tb, int m_cap,
                                                        const float* __restrict__ f, int d,
                                                        const T* __restrict__ Wr, int E, int top_k,
                                                        const float* __restrict__ router_bias,
                                                        int n_layers, int n_blocks, int layer,
                                                        int* __restrict__ sel,
                                                        float* __restrict__ gate,
                                                        float* __restrict__ rlog) {
  constexpr int VEC = 16 / sizeof(T);          // weights per 16-byte load
  constexpr int EPW = kMaxE / kRouteWaves;     // most experts a wave takes
  __shared__ float logit[kMaxE];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int m = blockIdx.x;                    // < m_cap: the row is readable
  const int nr = *tb.nrows;
  const int r = tb.row_req[m];
  const int epw = (E + kRouteWaves - 1) / kRouteWaves;
  const int e0 = wave * epw;
  const float* fr = f + (size_t)m * d;
  // rows past the wave's experts repeat the last expert (not stored)
  const T* wr[EPW];
#pragma unroll
  for (int i = 0; i < EPW; ++i) wr[i] = Wr + (size_t)min(e0 + min(i, epw - 1), E - 1) * d;
  float s[EPW];
#pragma unroll
  for (int i = 0; i < EPW; ++i) s[i] = 0.f;
#pragma unroll 2
  for (int k0 = lane * VEC; k0 < d; k0 += 64 * VEC) {
    float xv[VEC];
#pragma unroll
    for (int q = 0; q < VEC; q += 4) {
      const float4 x = *reinterpret_cast<const float4*>(fr + k0 + q);
      xv[q] = x.x;
      xv[q + 1] = x.y;
      xv[q + 2] = x.z;
      xv[q + 3] = x.w;
    }
    V16 wv[EPW];
#pragma unroll
    for (int i = 0; i < EPW; ++i) wv[i] = ld16(wr[i] + k0);
#pragma unroll
    for (int i = 0; i < EPW; ++i)
#pragma unroll
      for (int q = 0; q < VEC; ++q) s[i] += xv[q] * v16_get<T>(wv[i], q);
  }
#pragma unroll
  for (int i = 0; i < EPW; ++i) s[i] = wave_sum(s[i]);
  if (m >= min(nr, m_cap)) return;             // the whole workgroup
  if (lane == 0)
#pragma unroll
    for (int i = 0; i < EPW; ++i)
      if (i < epw && e0 + i < E) logit[e0 + i] = s[i];
  __syncthreads();
  if (wave != 0) return;
  float v = -INFINITY;
  if (lane < E) {
    v = logit[lane];
    if (router_bias)
      v += router_bias[(((size_t)r * n_layers + layer) * n_blocks + tb.req_blk[r]) * E + lane];
    rlog[(size_t)m * E + lane] = v;
  }
  const float mx = vocab::wave_max_rot(v);
  // top_k by (value desc, id asc); the selected lanes drop out one by one
  float cand = v;
  int chosen_id[kMaxTopK];
  float chosen_v[kMaxTopK];
#pragma unroll
  for (int k = 0; k < kMaxTopK; ++k) {
    if (k >= top_k) break;
    float bv = cand;
    int bi = lane < E ? lane : INT_MAX;
    vocab::wave_best(bv, bi);                  // the whole wave takes part
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

// Plan of the (row, slot) assignments: per-expert counts, offsets (experts
// in id order) and row lists, rows ascending within an expert -- a stable
// counting sort, deterministic.  One workgroup of 16 waves; the list
// (row-major [row][slot]) is staged in LDS in chunks of 64 assignments.
//  1. each wave takes whole chunks: a lane finds the lanes of its chunk with
//     the same expert by six ballots over the bits of the expert id (its
//     rank among them and their count) and the chunk's first such lane
//     records the count per (chunk, expert);
//  2. one thread per expert sums its chunk counts in chunk order (its
//     per-chunk bases); an exclusive scan over experts gives the offsets;
//  3. each assignment's packed position = offset of its expert + base of its
//     chunk for that expert + its rank in the chunk.
// Lists longer than kPlanLds assignments use moe_plan_wide_kernel.
constexpr int kPlanWaves = 16;
constexpr int kPlanLds = 16384;                 // assignments staged in LDS
constexpr int kPlanChunks = kPlanLds / 64;

__global__ __launch_bounds__(64 * kPlanWaves) void moe_plan_kernel(
    const int* __restrict__ nrows, int m_cap, const int* __restrict__ sel_g, int E, int top_k,
    int* __restrict__ e_count, int* __restrict__ e_off, int* __restrict__ row_of,
    int* __restrict__ pos, int* __restrict__ n_assign) {
  __shared__ int sel_s[kPlanLds];
  __shared__ unsigned short ccnt[kPlanChunks][kMaxE];   // per (chunk, expert): count, then base
  __shared__ int off[kMaxE + 1];
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int M = min(*nrows, m_cap);
  const int total = M * top_k;                  // <= kPlanLds (checked at launch)
  const int nch = (total + 63) / 64;
  for (int a = t; a < total; a += 64 * kPlanWaves) sel_s[a] = sel_g[a];
  for (int i = t; i < nch * kMaxE; i += 64 * kPlanWaves) ccnt[i / kMaxE][i % kMaxE] = 0;
  __syncthreads();
  const unsigned long long below = (1ull << lane) - 1ull;
  // 1. per-chunk counts and ranks (ranks kept in registers, up to 16 chunks
  //    per wave)
  constexpr int kMaxOwn = kPlanChunks / kPlanWaves;
  int rank[kMaxOwn];
#pragma unroll
  for (int i = 0; i < kMaxOwn; ++i) {
    const int ch = wave + i * kPlanWaves;
    rank[i] = 0;
    if (ch >= nch) continue;                     // wave-uniform
    const int a = ch * 64 + lane;
    const bool live = a < total;
    const int e = live ? sel_s[a] : kMaxE;      // kMaxE: no expert (7 bits)
    unsigned long long peers = ~0ull;
#pragma unroll
    for (int b = 0; b < 7; ++b) {
      const unsigned long long bb = __ballot((e >> b) & 1);
      peers &= ((e >> b) & 1) ? bb : ~bb;
    }
    rank[i] = __popcll(peers & below);
    if (live && rank[i] == 0) ccnt[ch][e] = (unsigned short)__popcll(peers);
  }
  __syncthreads();
  // 2. per-expert chunk bases (chunk order), then offsets over experts
  if (t < E) {
    int run = 0;
    for (int ch = 0; ch < nch; ++ch) {
      const int c = ccnt[ch][t];
      ccnt[ch][t] = (unsigned short)run;
      run += c;
    }
    off[t] = run;                                // count, scanned below
  }
  __syncthreads();
  if (t == 0) {
    int run = 0;
    for (int e = 0; e < E; ++e) {
      const int c = off[e];
      off[e] = run;
      run += c;
    }
    off[E] = run;
    *n_assign = run;
  }
  __syncthreads();
  if (t < E) {
    e_off[t] = off[t];
    e_count[t] = off[t + 1] - off[t];
  }
  // 3. packed positions
#pragma unroll
  for (int i = 0; i < kMaxOwn; ++i) {
    const int ch = wave + i * kPlanWaves;
    if (ch >= nch) continue;
    const int a = ch * 64 + lane;
    if (a >= total) continue;
    const int e = sel_s[a];
    const int q = off[e] + ccnt[ch][e] + rank[i];
    row_of[q] = a / top_k;
    pos[a] = q;
  }
}

// Lists longer than kPlanLds (many-row refreshes of several requests): one
// workgroup of 16 waves, wave w owns experts w, w+16, ...; an expert's
// assignments are found 64 at a time by ballot, a first pass counts them,
// an exclusive scan over experts gives the offsets, a second pass writes
// each assignment's position (its rank among the expert's matches in list
// order) -- the same result as moe_plan_kernel.
__global__ __launch_bounds__(64 * kPlanWaves) void moe_plan_wide_kernel(
    const int* __restrict__ nrows, int m_cap, const int* __restrict__ sel, int E, int top_k,
    int* __restrict__ e_count, int* __restrict__ e_off, int* __restrict__ row_of,
    int* __restrict__ pos, int* __restrict__ n_assign) {
  __shared__ int cnt[kMaxE];
  __shared__ int off[kMaxE + 1];
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int M = min(*nrows, m_cap);
  const int total = M * top_k;
  const unsigned long long below = (1ull << lane) - 1ull;
  for (int e = wave; e < E; e += kPlanWaves) {
    int c = 0;
    for (int a0 = 0; a0 < total; a0 += 64) {
      const int a = a0 + lane;
      c += __popcll(__ballot(a < total && sel[a] == e));
    }
    if (lane == 0) cnt[e] = c;
  }
  __syncthreads();
  if (t == 0) {
    int run = 0;
    for (int e = 0; e < E; ++e) {
      off[e] = run;
      run += cnt[e];
    }
    off[E] = run;
    *n_assign = run;
  }
  __syncthreads();
  for (int e = wave; e < E; e += kPlanWaves) {
    if (lane == 0) {
      e_off[e] = off[e];
      e_count[e] = cnt[e];
    }
    int p = off[e];
    for (int a0 = 0; a0 < total; a0 += 64) {
      const int a = a0 + lane;
      const bool hit = a < total && sel[a] == e;
      const unsigned long long mask = __ballot(hit);
      if (hit) {
        const int q = p + __popcll(mask & below);
        row_of[q] = a / top_k;
        pos[a] = q;
      }
      p += __popcll(mask);
    }
  }
}

// x[m] += sum_s P[s][m] + sum_k gate[m][k] * Y[pos[m][k]]: one float4 of one
// row per thread, partials in split order, experts in slot order.
__global__ __launch_bounds__(256) void moe_combine_kernel(
    const int* __restrict__ nrows, int m_cap, float* __restrict__ x, const float* __restrict__ P,
    int S, size_t p_stride, const float* __restrict__ Y, const int* __restrict__ pos,
    const float* __restrict__ gate, int top_k, int d) {
  const int d4 = d / 4;
  const int idx = blockIdx.x * 256 + threadIdx.x;
  const int m = idx / d4;
  const int i = idx % d4;
  if (m >= min(*nrows, m_cap)) return;
  float4 acc[1] = {reinterpret_cast<float4*>(x + (size_t)m * d)[i]};
  const float* const pp[1] = {P + (size_t)m * d + 4 * i};
  add_splits<1>(acc, pp, p_stride, S);
  // expert slots: indices and gates first, then every slot's row load, then
  // the sum in slot order (top_k <= 8; slots past top_k repeat the last one
  // and are not added)
  int pk[kMaxTopK];
  float gk[kMaxTopK];
#pragma unroll
  for (int k = 0; k < kMaxTopK; ++k) {
    const size_t slot = (size_t)m * top_k + min(k, top_k - 1);
    pk[k] = pos[slot];
    gk[k] = gate[slot];
  }
  float4 v[kMaxTopK];
#pragma unroll
  for (int k = 0; k < kMaxTopK; ++k)
    v[k] = *reinterpret_cast<const float4*>(Y + (size_t)pk[k] * d + 4 * i);
  float4 a = acc[0];
#pragma unroll
  for (int k = 0; k < kMaxTopK; ++k)
    if (k < top_k) {
      a.x += gk[k] * v[k].x;
      a.y += gk[k] * v[k].y;
      a.z += gk[k] * v[k].z;
      a.w += gk[k] * v[k].w;
    }
  reinterpret_cast<float4*>(x + (size_t)m * d)[i] = a;
}

// One wave: lane e takes expert e (E <= 64).
__global__ __launch_bounds__(64) void expert_usage_kernel(const int* __restrict__ e_count, int E,
                                                          const int* __restrict__ resident,
                                                          int* __restrict__ counts,
                                                          long long* __restrict__ acct) {
  const int e = threadIdx.x;
  const int c = e < E ? e_count[e] : 0;
  const bool res = e < E && resident[e] != 0;
  if (e < E) counts[e] += c;
  const unsigned long long used = __ballot(c > 0);
  const unsigned long long hit = __ballot(c > 0 && res);
  int rh = (c > 0 && res) ? c : 0;
  int rm = (c > 0 && !res) ? c : 0;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    rh += __shfl_xor(rh, o, 64);
    rm += __shfl_xor(rm, o, 64);
  }
  if (e == 0) {
    acct[0] += __popcll(hit);
    acct[1] += __popcll(used & ~hit);
    acct[2] += rh;
    acct[3] += rm;
  }
}

}  // namespace

hipError_t launch_expert_usage(const int* e_count, int E, const int* resident, int* counts,
                               long long* acct, hipStream_t st) {
  if (E < 1 || E > kMaxE) return hipErrorInvalidValue;
  hipLaunchKernelGGL(expert_usage_kernel, dim3(1), dim3(64), 0, st, e_count, E, resident, counts,
                     acct);
  return hipGetLastError();
}

hipError_t launch_moe_route(DType t, PassTable tb, int m_cap, const float* f, int d,
                            const void* Wr, int E, int top_k, const float* router_bias,
                            int n_layers, int n_blocks, int layer, int* sel, float* gate,
                            float* rlog, hipStream_t st) {
  const int vec = t == DType::F32 ? 4 : 8;
  if (E > kMaxE || top_k > kMaxTopK || top_k > E || d % (64 * vec) != 0 || m_cap < 1)
    return hipErrorInvalidValue;
  const dim3 grid(m_cap);
  if (t == DType::F32)
    hipLaunchKernelGGL(moe_route_kernel<float>, grid, dim3(64 * kRouteWaves), 0, st, tb, m_cap, f,
                       d, static_cast<const float*>(Wr), E, top_k, router_bias, n_layers, n_blocks,
                       layer, sel, gate, rlog);
  else
    hipLaunchKernelGGL(moe_route_kernel<bf16>, grid, dim3(64 * kRouteWaves), 0, st, tb, m_cap, f,
                       d, static_cast<const bf16*>(Wr), E, top_k, router_bias, n_layers, n_blocks,
                       layer, sel, gate, rlog);
  return hipGetLastError();
}

hipError_t launch_moe_plan(const int* nrows, int m_cap, const int* sel, int E, int top_k,
                           int* e_count, int* e_off, int* row_of, int* pos, int* n_assign,
                           hipStream_t st) {
  if (E > kMaxE) return hipErrorInvalidValue;
  if ((size_t)m_cap * top_k <= (size_t)kPlanLds)
    hipLaunchKernelGGL(moe_plan_kernel, dim3(1), dim3(64 * kPlanWaves), 0, st, nrows, m_cap, sel,
                       E, top_k, e_count, e_off, row_of, pos, n_assign);
  else
    hipLaunchKernelGGL(moe_plan_wide_kernel, dim3(1), dim3(64 * kPlanWaves), 0, st, nrows, m_cap,
                       sel, E, top_k, e_count, e_off, row_of, pos, n_assign);
  return hipGetLastError();
}

hipError_t launch_moe_combine(const int* nrows, int m_cap, float* x, const float* P, int S,
                              size_t p_stride, const float* Y, const int* pos, const float* gate,
                              int top_k, int d, hipStream_t st) {
  if (d % 4 != 0) return hipErrorInvalidValue;
  const int blocks = (int)(((size_t)m_cap * (d / 4) + 255) / 256);
  hipLaunchKernelGGL(moe_combine_kernel, dim3(blocks), dim3(256), 0, st, nrows, m_cap, x, P, S,
                     p_stride, Y, pos, gate, top_k, d);
  return hipGetLastError();
}

}  // namespace dinfer
