// Vocab statistics of the block rows: planting bias, MASK exclusion, argmax
// (lowest id on ties), max softmax probability, log-sum-exp and top-8 --
// everything the decoding strategy consumes (dInfer news article, section
// "扩散模型的“理论翅膀”与“现实枷锁”": confidence of the most likely token;
// section "解码的艺术": the probability distribution kept for iteration
// smoothing).
//
// One pass over the fp32 logits.  The vocabulary of a row is split across
// workgroups so that a few rows still fill the chip; each thread keeps an
// online (max, sum of exp) and a sorted top-8 in registers, fed through a
// wave-wide threshold so that few entries need an insertion, a workgroup
// merges them with wave64 exchanges, and a second kernel merges the splits of
// a row (one wave per row) in split order.
#include "common.h"
#include "kernels.h"
#include "vocab_common.h"

#include <climits>
#include <type_traits>

namespace dinfer {

namespace {

using namespace vocab;

constexpr int kThreads = 256;

// part_f [rows][n_split][2 + 8] = (max, sum exp(z - max), top-8 values);
// part_i [rows][n_split][8] = top-8 ids.
__global__ __launch_bounds__(kThreads) void vocab_partial_kernel(
    const float* __restrict__ logits, int V, int n_split, int chunk, const int* __restrict__ plant_id,
    const float* __restrict__ plant_bias, int mask_id, float* __restrict__ part_f,
    int* __restrict__ part_i) {
  __shared__ float s_m[kThreads / 64], s_s[kThreads / 64];
  __shared__ float s_tv[kThreads / 64][kTop];
  __shared__ int s_ti[kThreads / 64][kTop];
  const int split = blockIdx.x;
  const int row = blockIdx.y;
  const int c0 = split * chunk;
  const int c1 = min(V, c0 + chunk);
  const int pid = plant_id ? plant_id[row] : -1;
  const float pb = plant_bias ? plant_bias[row] : 0.f;
  const float* z = logits + (size_t)row * V;

  float m = -INFINITY, s = 0.f;
  float tv[kTop];
  int ti[kTop];
#pragma unroll
  for (int k = 0; k < kTop; ++k) {
    tv[k] = -INFINITY;
    ti[k] = INT_MAX;
  }
  // c0, c1 and V are multiples of 4, so every float4 lies wholly inside or
  // outside the split (c1 > c0 for every launched split).  A thread takes
  // kE = 4 kU entries per round, kU float4 loaded together; entry i of the
  // round has id b0 + (i/4) 4 kThreads + i%4 -- increasing in i and over
  // rounds.
  //  * softmax: the round's maximum first, then one rescale of the running
  //    sum and one exp per entry;
  //  * top-8: an entry can reach the row's top 8 only if it is >= T, the
  //    largest 8th-best value over the wave's lanes (that lane holds eight
  //    entries >= T, so anything smaller has eight strictly larger
  //    entries), and it enters this lane's list only if it beats the list's
  //    8th entry; after the first rounds few entries pass both tests.
  constexpr int kU = 4;
  constexpr int kE = 4 * kU;
  // Every lane runs the same number of rounds (the wave-wide threshold is a
  // cross-lane reduction), rounded up to even; entries past the split are
  // -inf.  The loads of round r+1 are issued before round r is processed
  // (two register sets alternate; loads past the split are clamped).
  float T = -INFINITY;
  constexpr int kRound = 4 * kThreads * kU;    // entries of the split per round
  const int rounds = ((c1 - c0 + kRound - 1) / kRound + 1) / 2 * 2;
  auto issue = [&](float4 (&xv)[kU], int r) {
    const int b0 = c0 + 4 * threadIdx.x + r * kRound;
#pragma unroll
    for (int u = 0; u < kU; ++u)
      xv[u] = *reinterpret_cast<const float4*>(z + min(b0 + u * 4 * kThreads, c1 - 4));
  };
  auto process = [&](const float4 (&xv)[kU], int r, auto sparse) {
    const int b0 = c0 + 4 * threadIdx.x + r * kRound;
    float v[kE];
    float gm = -INFINITY;
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int base = b0 + u * 4 * kThreads;
      const float xs[4] = {xv[u].x, xv[u].y, xv[u].z, xv[u].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int id = base + e;
        float x = xs[e];
        if (id == pid) x += pb;
        if (id == mask_id || base >= c1) x = -INFINITY;
        v[4 * u + e] = x;
        gm = fmaxf(gm, x);
      }
    }
    const float mn = fmaxf(m, gm);
    if (mn != -INFINITY) {
      float add = 0.f;
#pragma unroll
      for (int i = 0; i < kE; ++i) add += exp2f((v[i] - mn) * kLog2e);
      s = s * exp2f((m - mn) * kLog2e) + add;
      m = mn;
    }
    if constexpr (decltype(sparse)::value) {
      // few entries pass: collect them, then insert one at a time in id order
      unsigned pend = 0;
#pragma unroll
      for (int i = 0; i < kE; ++i) pend |= (v[i] > tv[kTop - 1] && v[i] >= T) ? 1u << i : 0u;
      while (pend != 0) {
        const int i = __builtin_ctz(pend);
        pend &= pend - 1;
        float cv = v[0];
#pragma unroll
        for (int j = 1; j < kE; ++j) cv = i == j ? v[j] : cv;
        insert_top8(tv, ti, cv, b0 + (i >> 2) * 4 * kThreads + (i & 3));
      }
    } else {
#pragma unroll
      for (int i = 0; i < kE; ++i)
        if (v[i] >= T) insert_top8(tv, ti, v[i], b0 + (i >> 2) * 4 * kThreads + (i & 3));
    }
    T = wave_max(tv[kTop - 1]);
  };
  // The first two rounds fill the lists (most entries enter): each entry is
  // tried in turn.  Later rounds collect the few passing entries first.
  using Dense = std::integral_constant<bool, false>;
  using Sparse = std::integral_constant<bool, true>;
  float4 xa[kU], xb[kU];
  issue(xa, 0);
  issue(xb, 1);
  process(xa, 0, Dense{});
  issue(xa, 2);
  process(xb, 1, Dense{});
  for (int r = 2; r < rounds; r += 2) {
    issue(xb, r + 1);
    process(xa, r, Sparse{});
    issue(xa, r + 2);
    process(xb, r + 1, Sparse{});
  }
  // workgroup merge: (max, sum) then top-8
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  float wm = wave_max(m);
  float ws = (m == -INFINITY) ? 0.f : s * exp2f((m - wm) * kLog2e);
  ws = wave_sum(ws);
  float ov[kTop];
  int oi[kTop];
  wave_top8(tv, ti, ov, oi);
  if (lane == 0) {
    s_m[wave] = wm;
    s_s[wave] = ws;
#pragma unroll
    for (int k = 0; k < kTop; ++k) {
      s_tv[wave][k] = ov[k];
      s_ti[wave][k] = oi[k];
    }
  }
  __syncthreads();
  if (wave != 0) return;
  float bm = -INFINITY;
#pragma unroll
  for (int w = 0; w < kThreads / 64; ++w) bm = fmaxf(bm, s_m[w]);
  float bs = 0.f;
#pragma unroll
  for (int w = 0; w < kThreads / 64; ++w)
    if (s_m[w] != -INFINITY) bs += s_s[w] * exp2f((s_m[w] - bm) * kLog2e);
  // 32 candidates, one per lane (lanes 32..63 empty): extract 8 in order
  float cv = -INFINITY;
  int ci = INT_MAX;
  if (lane < (kThreads / 64) * kTop) {
    cv = s_tv[lane / kTop][lane % kTop];
    ci = s_ti[lane / kTop][lane % kTop];
  }
  float* pf = part_f + ((size_t)row * n_split + split) * (2 + kTop);
  int* pi = part_i + ((size_t)row * n_split + split) * kTop;
#pragma unroll
  for (int k = 0; k < kTop; ++k) {
    float v = cv;
    int id = ci;
    wave_best(v, id);
    if (cv == v && ci == id) {
      cv = -INFINITY;
      ci = INT_MAX;
    }
    if (lane == 0) {
      pf[2 + k] = v;
      pi[k] = id;
    }
  }
  if (lane == 0) {
    pf[0] = bm;
    pf[1] = bs;
  }
}

// One wave per row: merge the splits (lane = split) and emit the statistics.
__global__ __launch_bounds__(64) void vocab_merge_kernel(int rows, int n_split,
                                                         const float* __restrict__ part_f,
                                                         const int* __restrict__ part_i,
                                                         int* __restrict__ argmax,
                                                         float* __restrict__ conf,
                                                         float* __restrict__ lse,
                                                         int* __restrict__ topk_id,
                                                         float* __restrict__ topk_p) {
  const int row = blockIdx.x;
  const int lane = threadIdx.x;
  float m = -INFINITY, s = 0.f;
  float tv[kTop];
  int ti[kTop];
#pragma unroll
  for (int k = 0; k < kTop; ++k) {
    tv[k] = -INFINITY;
    ti[k] = INT_MAX;
  }
  if (lane < n_split) {
    const float* pf = part_f + ((size_t)row * n_split + lane) * (2 + kTop);
    const int* pi = part_i + ((size_t)row * n_split + lane) * kTop;
    m = pf[0];
    s = pf[1];
#pragma unroll
    for (int k = 0; k < kTop; ++k) {
      tv[k] = pf[2 + k];
      ti[k] = pi[k];
    }
  }
  const float M = wave_max(m);
  const float Z = wave_sum(m == -INFINITY ? 0.f : s * exp2f((m - M) * kLog2e));
  float ov[kTop];
  int oi[kTop];
  wave_top8(tv, ti, ov, oi);
  if (lane < kTop) {
    float v = ov[0];
    int id = oi[0];
#pragma unroll
    for (int k = 1; k < kTop; ++k)
      if (lane == k) {
        v = ov[k];
        id = oi[k];
      }
    topk_id[(size_t)row * kTop + lane] = id;
    topk_p[(size_t)row * kTop + lane] = exp2f((v - M) * kLog2e) / Z;
  }
  if (lane == 0) {
    argmax[row] = oi[0];
    conf[row] = 1.f / Z;
    lse[row] = M + logf(Z);
  }
}

// Merge of the LM head's per-(row, column tile) records: one workgroup per
// row.  Thread t folds tiles t, t + 256, ... (ascending, so ids arrive in
// increasing order for equal values) into an online (max, sum of exp) and a
// sorted top-8, the waves merge theirs with wave64 exchanges, and wave 0
// merges the four waves' and emits the statistics.
__global__ __launch_bounds__(kThreads) void vocab_merge_tiles_kernel(
    int n_tiles, const float* __restrict__ rec_f, const int* __restrict__ rec_i,
    int* __restrict__ argmax, float* __restrict__ conf, float* __restrict__ lse,
    int* __restrict__ topk_id, float* __restrict__ topk_p) {
  __shared__ float s_m[kThreads / 64], s_s[kThreads / 64];
  __shared__ float s_tv[kThreads / 64][kTop];
  __shared__ int s_ti[kThreads / 64][kTop];
  const int row = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  float m = -INFINITY, s = 0.f;
  float tv[kTop];
  int ti[kTop];
#pragma unroll
  for (int k = 0; k < kTop; ++k) {
    tv[k] = -INFINITY;
    ti[k] = INT_MAX;
  }
  for (int t = threadIdx.x; t < n_tiles; t += kThreads) {
    const float* pf = rec_f + ((size_t)row * n_tiles + t) * kRecF;
    const int* pi = rec_i + ((size_t)row * n_tiles + t) * kTop;
    float f[kRecF];
    int id[kTop];
#pragma unroll
    for (int k = 0; k < kRecF; ++k) f[k] = pf[k];
#pragma unroll
    for (int k = 0; k < kTop; ++k) id[k] = pi[k];
    const float mn = fmaxf(m, f[0]);
    if (mn != -INFINITY) {
      s = (m == -INFINITY ? 0.f : s * exp2f((m - mn) * kLog2e)) +
          (f[0] == -INFINITY ? 0.f : f[1] * exp2f((f[0] - mn) * kLog2e));
      m = mn;
    }
#pragma unroll
    for (int k = 0; k < kTop; ++k) insert_top8(tv, ti, f[2 + k], id[k]);
  }
  const float wm = wave_max(m);
  float ws = (m == -INFINITY) ? 0.f : s * exp2f((m - wm) * kLog2e);
  ws = wave_sum(ws);
  float ov[kTop];
  int oi[kTop];
  wave_top8(tv, ti, ov, oi);
  if (lane == 0) {
    s_m[wave] = wm;
    s_s[wave] = ws;
#pragma unroll
    for (int k = 0; k < kTop; ++k) {
      s_tv[wave][k] = ov[k];
      s_ti[wave][k] = oi[k];
    }
  }
  __syncthreads();
  if (wave != 0) return;
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < kThreads / 64; ++w) M = fmaxf(M, s_m[w]);
  float Z = 0.f;
#pragma unroll
  for (int w = 0; w < kThreads / 64; ++w)
    if (s_m[w] != -INFINITY) Z += s_s[w] * exp2f((s_m[w] - M) * kLog2e);
  float cv = -INFINITY;
  int ci = INT_MAX;
  if (lane < (kThreads / 64) * kTop) {
    cv = s_tv[lane / kTop][lane % kTop];
    ci = s_ti[lane / kTop][lane % kTop];
  }
#pragma unroll
  for (int k = 0; k < kTop; ++k) {
    float v = cv;
    int id = ci;
    wave_best(v, id);
    if (cv == v && ci == id) {
      cv = -INFINITY;
      ci = INT_MAX;
    }
    if (lane == 0) {
      topk_id[(size_t)row * kTop + k] = id;
      topk_p[(size_t)row * kTop + k] = exp2f((v - M) * kLog2e) / Z;
      if (k == 0) {
        argmax[row] = id;
        conf[row] = 1.f / Z;
        lse[row] = M + logf(Z);
      }
    }
  }
}

}  // namespace

hipError_t launch_vocab_merge_tiles(int rows, int n_tiles, const float* rec_f, const int* rec_i,
                                    int* argmax, float* conf, float* lse, int* topk_id,
                                    float* topk_p, hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  if (n_tiles < 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL(vocab_merge_tiles_kernel, dim3(rows), dim3(kThreads), 0, st, n_tiles, rec_f,
                     rec_i, argmax, conf, lse, topk_id, topk_p);
  return hipGetLastError();
}

size_t vocab_record_bytes(int rows, int n_tiles) {
  return (size_t)rows * n_tiles * (vocab::kRecF * sizeof(float) + vocab::kTop * sizeof(int));
}

VocabPlan plan_vocab(int rows, int V, int target_wgs) {
  VocabPlan p{};
  int ns = (target_wgs + rows - 1) / rows;
  const int max_ns = (V + 2047) / 2048;        // at least ~2K entries per split
  if (ns > max_ns) ns = max_ns;
  if (ns > 64) ns = 64;
  if (ns < 1) ns = 1;
  int chunk = (V + ns - 1) / ns;
  chunk = (chunk + 3) / 4 * 4;                 // float4-aligned splits
  p.chunk = chunk;
  p.n_split = (V + chunk - 1) / chunk;
  return p;
}

size_t vocab_scratch_bytes(const VocabPlan& p, int rows) {
  return (size_t)rows * p.n_split * ((2 + kTop) * sizeof(float) + kTop * sizeof(int));
}

hipError_t launch_vocab_stats(const VocabPlan& p, const float* logits, int rows, int V,
                              const int* plant_id, const float* plant_bias, int mask_id,
                              void* scratch, int* argmax, float* conf, float* lse, int* topk_id,
                              float* topk_p, hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  float* part_f = static_cast<float*>(scratch);
  int* part_i = reinterpret_cast<int*>(part_f + (size_t)rows * p.n_split * (2 + kTop));
  hipLaunchKernelGGL(vocab_partial_kernel, dim3(p.n_split, rows), dim3(kThreads), 0, st, logits, V,
                     p.n_split, p.chunk, plant_id, plant_bias, mask_id, part_f, part_i);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(vocab_merge_kernel, dim3(rows), dim3(64), 0, st, rows, p.n_split, part_f,
                     part_i, argmax, conf, lse, topk_id, topk_p);
  return hipGetLastError();
}

}  // namespace dinfer
