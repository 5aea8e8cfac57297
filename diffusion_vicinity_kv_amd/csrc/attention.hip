// Bidirectional attention of the window queries over the full cached KV of
// their request (no causal mask: every position attends to every position;
// dInfer news article, section "扩散模型的“理论翅膀”与“现实枷锁”").
//
// Split-KV flash attention on gfx950 MFMA.  A workgroup takes one (request,
// head, 64-query tile, key range); each of its four waves owns 16 queries.
// Per 64-key chunk, K is staged in LDS as [key][hd] and V transposed as
// [hd][key].  Scores are computed transposed, S^T = K Q^T, so that a lane
// holds the scores of query (lane % 16) for keys 4*(lane/16)+i: exactly the
// B-operand layout of the next product O^T = V^T P^T, which therefore needs no
// data movement; the online-softmax statistics of a query also live in the
// lanes that hold its output column.  Softmax runs in fp32 in the log2
// domain.  Each split writes (m, l, unnormalised O) in fp32; a merge kernel
// combines the splits of a query in split order.
//
// Queries stay fp32 and the probabilities are fp32: with a bf16 cache both
// enter the bf16 MFMAs as hi + lo halves, so the only rounding left in the
// attention is the cache's own storage of K and V.
#include "common.h"
#include "kernels.h"

namespace dinfer {

namespace {

constexpr int QT = 64;   // queries per workgroup
constexpr int KT = 64;   // keys per LDS chunk

template <typename T, int HD>
__global__ __launch_bounds__(256) void attn_split_kernel(
    PassTable tb, int q_tiles, int keys_per_split, int m_cap, const float* __restrict__ q,
    const T* __restrict__ kc, const T* __restrict__ vc, int H, int max_len, float scale_log2,
    float* __restrict__ o_part, float* __restrict__ ml_part) {
  using MF = Mfma<T>;
  constexpr int VEC = MF::VEC;
  constexpr int KSTEP = MF::KSTEP;
  constexpr int QV = HD / KSTEP;               // vector steps over the head dim
  constexpr int KSTR = HD + 16 / sizeof(T);    // K rows in LDS
  constexpr int VSTR = KT + 8;                 // V^T rows in LDS (elements)
  constexpr int HT = HD / 16;                  // 16-wide output tiles over hd
  constexpr int VPK = HD / VEC;                // 16-byte vectors per key row
  __shared__ __attribute__((aligned(16))) T Ks[KT * KSTR];
  __shared__ __attribute__((aligned(16))) T Vt[HD * VSTR];

  const int split = blockIdx.x;
  const int h = blockIdx.y;
  const int r = blockIdx.z / q_tiles;
  const int qt = blockIdx.z % q_tiles;
  const int nq = tb.req_nrows[r];
  if (qt * QT >= nq) return;
  const int L = tb.req_len[r];
  const int k0 = split * keys_per_split;
  if (k0 >= L) return;
  const int k1 = min(L, k0 + keys_per_split);

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int lc = lane & 15;
  const int lg = lane >> 4;
  const int qloc = qt * QT + wave * 16 + lc;    // query index inside the request's rows
  const bool qvalid = qloc < nq;
  const int qrow = tb.req_row_off[r] + qloc;
  const int d = H * HD;

  using SO = SplitOperand<T>;
  constexpr int QP = SO::PARTS;
  V16 qf[QV][QP];
#pragma unroll
  for (int kk = 0; kk < QV; ++kk) {
    float qv[VEC];
#pragma unroll
    for (int e = 0; e < VEC; e += 4) {
      const float4 x = qvalid ? *reinterpret_cast<const float4*>(
                                    q + (size_t)qrow * d + h * HD + kk * KSTEP + lg * VEC + e)
                              : make_float4(0.f, 0.f, 0.f, 0.f);
      qv[e] = x.x;
      qv[e + 1] = x.y;
      qv[e + 2] = x.z;
      qv[e + 3] = x.w;
    }
    SO::make(qv, qf[kk]);
  }

  floatx4 o[HT];
#pragma unroll
  for (int t = 0; t < HT; ++t) o[t] = floatx4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;
  float l_run = 0.f;

  const size_t head_base = ((size_t)r * H + h) * max_len;
  for (int kb = k0; kb < k1; kb += KT) {
    __syncthreads();
    for (int v = threadIdx.x; v < KT * VPK; v += 256) {
      const int key = v / VPK;
      const int cv = v % VPK;
      V16 kv = zero16(), vv = zero16();
      if (kb + key < k1) {
        kv = ld16(kc + (head_base + kb + key) * HD + cv * VEC);
        vv = ld16(vc + (head_base + kb + key) * HD + cv * VEC);
      }
      st16(&Ks[key * KSTR + cv * VEC], kv);
      const T* ve = reinterpret_cast<const T*>(&vv);
#pragma unroll
      for (int e = 0; e < VEC; ++e) Vt[(cv * VEC + e) * VSTR + key] = ve[e];
    }
    __syncthreads();

    // S^T tiles: s[t][i] = score(query lc, key kb + 16 t + 4 lg + i)
    floatx4 s[KT / 16];
#pragma unroll
    for (int t = 0; t < KT / 16; ++t) {
      s[t] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < QV; ++kk) {
        const V16 a = *reinterpret_cast<const V16*>(&Ks[(t * 16 + lc) * KSTR + kk * KSTEP + lg * VEC]);
#pragma unroll
        for (int p = 0; p < QP; ++p) MF::mac(s[t], a, qf[kk][p]);
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < KT / 16; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = kb + t * 16 + lg * 4 + i;
        const float v = key < k1 ? s[t][i] * scale_log2 : -INFINITY;
        s[t][i] = v;
        mx = fmaxf(mx, v);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx);      // finite: the chunk holds at least one key
    const float alpha = exp2f(m_run - m_new);
    float ps = 0.f;
#pragma unroll
    for (int t = 0; t < KT / 16; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = exp2f(s[t][i] - m_new);
        s[t][i] = p;
        ps += p;
      }
    ps += __shfl_xor(ps, 16, 64);
    ps += __shfl_xor(ps, 32, 64);
    l_run = l_run * alpha + ps;
    m_run = m_new;
#pragma unroll
    for (int t = 0; t < HT; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) o[t][i] *= alpha;

    // O^T[hd][q] += V^T[hd][key] * P^T[key][q]
#pragma unroll
    for (int t = 0; t < KT / 16; ++t) {
      float pv[4] = {s[t][0], s[t][1], s[t][2], s[t][3]};
#pragma unroll
      for (int ht = 0; ht < HT; ++ht) {
        const T* vr = &Vt[(ht * 16 + lc) * VSTR + t * 16 + lg * 4];
        float av[4] = {to_f(vr[0]), to_f(vr[1]), to_f(vr[2]), to_f(vr[3])};
        Mfma4<T>::mac_split_b(o[ht], av, pv);
      }
    }
  }

  if (!qvalid) return;
  const size_t base = ((size_t)split * m_cap + qrow) * H + h;
  float* op = o_part + base * HD;
#pragma unroll
  for (int ht = 0; ht < HT; ++ht)
#pragma unroll
    for (int i = 0; i < 4; ++i) op[ht * 16 + lg * 4 + i] = o[ht][i];
  if (lg == 0) {
    ml_part[base * 2] = m_run;
    ml_part[base * 2 + 1] = l_run;
  }
}

// Combine the key splits of each (row, head): out = sum_s 2^(m_s - M) O_s /
// sum_s 2^(m_s - M) l_s, splits taken in order.
template <int HD>
__global__ __launch_bounds__(64) void attn_merge_kernel(PassTable tb, int keys_per_split,
                                                        int n_split, int m_cap,
                                                        const float* __restrict__ o_part,
                                                        const float* __restrict__ ml_part, int H,
                                                        float* __restrict__ out) {
  const int m = blockIdx.x;
  const int h = blockIdx.y;
  if (m >= min(*tb.nrows, m_cap)) return;
  const int r = tb.row_req[m];
  const int L = tb.req_len[r];
  int ns = (L + keys_per_split - 1) / keys_per_split;
  if (ns > n_split) ns = n_split;
  float M = -INFINITY;
  for (int s = 0; s < ns; ++s) M = fmaxf(M, ml_part[(((size_t)s * m_cap + m) * H + h) * 2]);
  float lsum = 0.f;
  float acc[HD / 64];
#pragma unroll
  for (int e = 0; e < HD / 64; ++e) acc[e] = 0.f;
  for (int s = 0; s < ns; ++s) {
    const size_t base = ((size_t)s * m_cap + m) * H + h;
    const float w = exp2f(ml_part[base * 2] - M);
    lsum += w * ml_part[base * 2 + 1];
#pragma unroll
    for (int e = 0; e < HD / 64; ++e) acc[e] += w * o_part[base * HD + threadIdx.x + 64 * e];
  }
  const float inv = 1.f / lsum;
  float* orow = out + (size_t)m * H * HD + h * HD;
#pragma unroll
  for (int e = 0; e < HD / 64; ++e) orow[threadIdx.x + 64 * e] = acc[e] * inv;
}

template <typename T, int HD>
hipError_t run(const AttnPlan& p, PassTable tb, int batch, int m_cap, const float* q,
               const void* kc, const void* vc, int H, int max_len, float* o_part, float* ml_part,
               float* o, hipStream_t st) {
  const float scale_log2 = 1.4426950408889634f / sqrtf((float)HD);
  dim3 grid(p.n_split, H, batch * p.q_tiles);
  hipLaunchKernelGGL((attn_split_kernel<T, HD>), grid, dim3(256), 0, st, tb, p.q_tiles,
                     p.keys_per_split, m_cap, q, static_cast<const T*>(kc),
                     static_cast<const T*>(vc), H, max_len, scale_log2, o_part, ml_part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((attn_merge_kernel<HD>), dim3(m_cap, H), dim3(64), 0, st, tb,
                     p.keys_per_split, p.n_split, m_cap, o_part, ml_part, H, o);
  return hipGetLastError();
}

}  // namespace

AttnPlan plan_attention(int batch, int max_rows_per_req, int max_keys, int H, int target_wgs) {
  AttnPlan p{};
  p.q_tiles = (max_rows_per_req + QT - 1) / QT;
  if (p.q_tiles < 1) p.q_tiles = 1;
  const int chunks = (max_keys + KT - 1) / KT;
  const int base = batch * p.q_tiles * H;
  int ns = (target_wgs + base - 1) / base;
  if (ns < 1) ns = 1;
  if (ns > chunks) ns = chunks;
  int kps = (chunks + ns - 1) / ns * KT;
  p.keys_per_split = kps;
  p.n_split = (max_keys + kps - 1) / kps;
  return p;
}

hipError_t launch_attention(DType t, const AttnPlan& p, PassTable tb, int batch, int m_cap,
                            const float* q, const void* kc, const void* vc, int H, int hd,
                            int max_len, float* o_part, float* ml_part, float* o,
                            hipStream_t st) {
  if (t == DType::F32) {
    if (hd == 64) return run<float, 64>(p, tb, batch, m_cap, q, kc, vc, H, max_len, o_part, ml_part, o, st);
    if (hd == 128) return run<float, 128>(p, tb, batch, m_cap, q, kc, vc, H, max_len, o_part, ml_part, o, st);
  } else {
    if (hd == 64) return run<bf16, 64>(p, tb, batch, m_cap, q, kc, vc, H, max_len, o_part, ml_part, o, st);
    if (hd == 128) return run<bf16, 128>(p, tb, batch, m_cap, q, kc, vc, H, max_len, o_part, ml_part, o, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace dinfer
