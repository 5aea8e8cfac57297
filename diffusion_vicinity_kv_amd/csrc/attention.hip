// Bidirectional attention of the window queries over the full cached KV of
// their request (no causal mask: every position attends to every position;
// dInfer news article, section "扩散模型的“理论翅膀”与“现实枷锁”").
//
// Cache layouts (per layer): K [request][head][Lp][hd] -- one key's head
// vector contiguous -- and V in transposed tiles of 32 keys,
// [request][head][Lp/32][hd][32] -- within a tile one head dimension's values
// over consecutive keys are contiguous, and a whole tile (8 KB in bf16) is
// contiguous; Lp = max_len rounded up to 64.  Every MFMA operand of both
// products is then a 16-byte piece of memory in its fragment layout.
//
// A workgroup takes (request, head, block of 64 * QTW queries, key range) on
// two groups of four waves; each wave owns QTW tiles of 16 queries, and the
// groups take alternate steps of KS keys (32 for bf16, 16 for fp32) and merge
// at the end.  A step's K and V fragments (NF kilobytes) are loaded once for
// the group -- a quarter by each wave, two steps ahead, through registers --
// and stored to LDS in fragment order, so that every wave reads each fragment
// as one contiguous, conflict-free 16-byte-per-lane load.  Then:
//   S^T = K Q^T with the keys as MFMA rows.  For bf16 the two 16-key tiles
//   take their rows in the order key(t, j) = 8*(j/4) + 4t + j%4, so lane
//   (query c, group g) ends up holding the scores of keys 8g..8g+7;
//   O^T += V^T P^T then takes those eight probabilities as its B operand
//   directly, against eight consecutive keys of a V^T tile row.
// Softmax is fp32 in the log2 domain.  Each lane keeps its own partial sum
// of probabilities (reduced across lanes once, at the end), and the scale m
// shared by a query's lanes is raised only when some score passes it by more
// than kSlack (so most steps need no cross-lane reduction; probabilities stay
// below 2^kSlack).  Queries (fp32) and probabilities enter the bf16 MFMAs as
// hi + lo halves, so the only rounding left is the cache's own storage.  With
// one key split the kernel writes the output; otherwise each split writes
// (m, l, unnormalised O) and a merge kernel combines the splits of a row in
// split order.
#include "common.h"
#include "kernels.h"

namespace dinfer {

namespace {

constexpr float kSlack = 8.f;

// 2^x by the hardware instruction alone; results below 2^-126 come out as
// zero (exp2f adds a rescaling step per call for them).  A probability that
// small, next to a row maximum of at least 1, changes no sum in fp32.
__device__ __forceinline__ float exp2_ftz(float x) { return __builtin_amdgcn_exp2f(x); }

// The probabilities' operand of O^T += V^T P^T: hi + lo halves like the
// queries (PLO), or bf16(p) alone (a precision option: one MFMA per V
// fragment instead of two).
template <typename T, bool PLO> struct ProbOperand : SplitOperand<T> {};
template <> struct ProbOperand<bf16, true> {
  static constexpr int PARTS = 2;
  // per pair of probabilities: one packed conversion gives both hi halves;
  // each hi half, widened back, leaves the remainder that the second packed
  // conversion rounds to the lo halves
  __device__ __forceinline__ static void make(const float* src, V16* out) {
    typedef float f2 __attribute__((ext_vector_type(2)));
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    unsigned hw[4], lw[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f2 x = {src[2 * i], src[2 * i + 1]};
      hw[i] = __builtin_bit_cast(unsigned, __builtin_convertvector(x, b2));
      const f2 hx = {__builtin_bit_cast(float, hw[i] << 16),
                     __builtin_bit_cast(float, hw[i] & 0xffff0000u)};
      lw[i] = __builtin_bit_cast(unsigned, __builtin_convertvector(x - hx, b2));
    }
    out[0].u = make_uint4(hw[0], hw[1], hw[2], hw[3]);
    out[1].u = make_uint4(lw[0], lw[1], lw[2], lw[3]);
  }
};
template <> struct ProbOperand<bf16, false> {
  static constexpr int PARTS = 1;
  __device__ __forceinline__ static void make(const float* src, V16* out) {
#pragma unroll
    for (int i = 0; i < 8; ++i) out[0].b[i] = static_cast<bf16>(src[i]);
  }
};
constexpr int kKeyGroups = 2;   // groups of four waves taking alternate steps

template <typename T, int HD, int QTW, bool PLO>
__global__ __launch_bounds__(256 * kKeyGroups) void attn_kernel(
    PassTable tb, int q_blocks, int keys_per_split, int n_split, int m_cap,
    const float* __restrict__ q, const T* __restrict__ kc, const T* __restrict__ vt, int H,
    int Lp, float scale_log2, float* __restrict__ o_part, float* __restrict__ ml_part,
    float* __restrict__ out, size_t o_aps) {
  using MF = Mfma<T>;
  using SO = SplitOperand<T>;
  using SP = ProbOperand<T, PLO>;
  constexpr int VEC = MF::VEC;
  constexpr int KS = MF::KSTEP;        // keys per step
  constexpr int NTS = KS / 16;         // 16-key score tiles per step
  constexpr int QV = HD / KS;          // vector steps over the head dim
  constexpr int HT = HD / 16;          // 16-row output tiles over the head dim
  constexpr int PL = SO::PARTS;
  constexpr int PP = SP::PARTS;       // parts of the probabilities (B of O^T)
  constexpr int QB = 64 * QTW;         // queries per workgroup
  constexpr int NK = NTS * QV;         // K fragments per step
  constexpr int NF = NK + HT;          // K and V fragments per step
  constexpr int FW = NF / 4;           // fragments each wave loads
  constexpr int KG = kKeyGroups;
  static_assert(NF % 4 == 0, "fragments must split over four waves");
  __shared__ V16 frag[KG][2][NF][64];

  const int split = blockIdx.x;
  const int h = blockIdx.y;
  const int r = blockIdx.z / q_blocks;
  const int qb = blockIdx.z % q_blocks;
  // the request's three table entries are loaded together
  const int nq = tb.req_nrows[r];
  const int L = tb.req_len[r];
  const int row_off = tb.req_row_off[r];
  if (qb * QB >= nq) return;
  const int k0 = split * keys_per_split;
  if (k0 >= L) return;
  const int k1 = min(L, k0 + keys_per_split);
  const int n_steps = (k1 - k0 + KS - 1) / KS;

  const int lane = threadIdx.x & 63;
  // wave-uniform indices read as scalars: the step's key base, its range
  // test and the fragment addresses then take scalar instructions, not the
  // vector ALUs the softmax needs
  const int kg = __builtin_amdgcn_readfirstlane(threadIdx.x >> 8);   // key group: steps kg, kg + KG, ...
  const int wave = __builtin_amdgcn_readfirstlane((threadIdx.x >> 6) & 3);   // query tile(s)
  const int lc = lane & 15;
  const int lg = lane >> 4;
  const int d = H * HD;
  const int n_local = (n_steps + KG - 1) / KG; // steps per group (the last may be empty)

  // query fragments (B operand of S^T): query lc of each tile, hd g*VEC..
  // The raw rows are loaded here, unconditionally (a query past the block
  // reads the request's first row, zeroed below), and split only after the
  // first K/V loads are issued: the three reads share one memory round trip
  // (a conditional load here put each in a branch of its own, with a full
  // wait at a join, before any K/V load left).
  V16 qf[QTW][QV][PL];
  int qrow[QTW];
  bool qvalid[QTW];
  float4 qraw[QTW][QV][VEC / 4];
#pragma unroll
  for (int u = 0; u < QTW; ++u) {
    const int qloc = qb * QB + (wave * QTW + u) * 16 + lc;
    qvalid[u] = qloc < nq;
    qrow[u] = row_off + (qvalid[u] ? qloc : 0);
#pragma unroll
    for (int kk = 0; kk < QV; ++kk)
#pragma unroll
      for (int e = 0; e < VEC; e += 4)
        qraw[u][kk][e / 4] = *reinterpret_cast<const float4*>(
            q + (size_t)qrow[u] * d + h * HD + kk * KS + lg * VEC + e);
  }
  auto split_queries = [&]() {
#pragma unroll
    for (int u = 0; u < QTW; ++u)
#pragma unroll
      for (int kk = 0; kk < QV; ++kk) {
        // scaled into the log2 domain here, once, instead of every score
        const float sc = qvalid[u] ? scale_log2 : 0.f;
        float qv[VEC];
#pragma unroll
        for (int e = 0; e < VEC; e += 4) {
          const float4 x = qraw[u][kk][e / 4];
          qv[e] = x.x * sc;
          qv[e + 1] = x.y * sc;
          qv[e + 2] = x.z * sc;
          qv[e + 3] = x.w * sc;
        }
        SO::make(qv, qf[u][kk]);
      }
  };

  floatx4 o[QTW][HT];
  float m_run[QTW], l_run[QTW];
#pragma unroll
  for (int u = 0; u < QTW; ++u) {
#pragma unroll
    for (int t = 0; t < HT; ++t) o[u][t] = floatx4{0.f, 0.f, 0.f, 0.f};
    m_run[u] = -INFINITY;
    l_run[u] = 0.f;
  }

  const size_t head = (size_t)r * H + h;
  // score-tile row j of tile t holds key key_of(t, j) of the step
  const int krow0 = NTS == 2 ? 8 * (lc >> 2) + (lc & 3) : lc;

  // fragment f of a step, as lane `lane` holds it: f < NK is K tile t = f /
  // QV, head-dim step kk = f % QV; the rest are V^T row tiles ht = f - NK.
  // A wave loads fragments of one kind only, so its lane's offset within a
  // fragment is fixed (one register) and each load adds it to a scalar
  // address.  Keys of the step past the range are read (every row below Lp
  // is inside the cache, and finite: zeroed at set-up, written with keys
  // since) and masked out of the scores.
  static_assert(NK % FW == 0, "a wave's fragments are all K or all V");
  const bool loads_k = wave * FW < NK;
  const unsigned lane_off =
      (unsigned)(loads_k ? krow0 * HD + lg * VEC : lc * 32 + lg * VEC) * sizeof(T);
  const T* kv_head = (loads_k ? kc : vt) + head * Lp * HD;
  int frag_off[FW];                            // a fragment's offset within its step
#pragma unroll
  for (int j = 0; j < FW; ++j) {
    const int f = wave * FW + j;
    frag_off[j] = loads_k ? 4 * (f / QV) * HD + (f % QV) * KS : (f - NK) * 16 * 32;
  }
  auto load = [&](V16 (&reg)[FW], int i) {     // this group's local step i
    const int kb = k0 + min(kg + i * KG, n_steps - 1) * KS;   // past the end: repeat the last
    // K rows kb.. start at kb * HD; so does the V^T tile of kb when a step
    // is a whole tile (KS 32), else (KS 16) it starts inside one
    const size_t step_off =
        KS == 32 || loads_k ? (size_t)kb * HD : (size_t)(kb >> 5) * HD * 32 + (kb & 31);
    const T* sbase = kv_head + step_off;
#pragma unroll
    for (int j = 0; j < FW; ++j)
      reg[j] = ld16(reinterpret_cast<const char*>(sbase + frag_off[j]) + lane_off);
  };
  auto store = [&](const V16 (&reg)[FW], int buf) {
#pragma unroll
    for (int i = 0; i < FW; ++i) frag[kg][buf][wave * FW + i][lane] = reg[i];
  };

  // Scores of every query tile first (each K fragment read from LDS once and
  // used by all of the wave's tiles), then the softmax update of each tile,
  // then P V with each V fragment likewise read once.
  auto compute = [&](int buf, int i) {
    const int s = kg + i * KG;
    if (s >= n_steps) return;                  // this group's slot past the range
    const int kb = k0 + s * KS;
    floatx4 sc[QTW][NTS];
#pragma unroll
    for (int u = 0; u < QTW; ++u)
#pragma unroll
      for (int t = 0; t < NTS; ++t) sc[u][t] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < NTS; ++t)
#pragma unroll
      for (int kk = 0; kk < QV; ++kk) {
        const V16 kf = frag[kg][buf][t * QV + kk][lane];
#pragma unroll
        for (int u = 0; u < QTW; ++u)
#pragma unroll
          for (int p = 0; p < PL; ++p) MF::mac(sc[u][t], kf, qf[u][kk][p]);
      }
    // lane (query lc, group lg) holds keys kb + lg*VEC + e, e = 4t + i; keys
    // past the range occur only in a split's last step
    if (kb + KS > k1) {
#pragma unroll
      for (int u = 0; u < QTW; ++u)
#pragma unroll
        for (int t = 0; t < NTS; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (kb + lg * VEC + 4 * t + i >= k1) sc[u][t][i] = -INFINITY;
    }
    V16 pf[QTW][PP];
#pragma unroll
    for (int u = 0; u < QTW; ++u) {
      float pv[VEC];
      float mloc = -INFINITY;
#pragma unroll
      for (int t = 0; t < NTS; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pv[4 * t + i] = sc[u][t][i];
          mloc = fmaxf(mloc, sc[u][t][i]);
        }
      if (__any(mloc > m_run[u] + kSlack)) {      // wave-uniform: raise the scale
        float mx = fmaxf(mloc, __shfl_xor(mloc, 16, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const float m_new = fmaxf(m_run[u], mx);  // finite after the first step
        const float alpha = exp2_ftz(m_run[u] - m_new);
        l_run[u] *= alpha;
#pragma unroll
        for (int ht = 0; ht < HT; ++ht)
#pragma unroll
          for (int i = 0; i < 4; ++i) o[u][ht][i] *= alpha;
        m_run[u] = m_new;
      }
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        pv[e] = exp2_ftz(pv[e] - m_run[u]);
        l_run[u] += pv[e];
      }
      SP::make(pv, pf[u]);
    }
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      const V16 vf = frag[kg][buf][NK + ht][lane];
#pragma unroll
      for (int u = 0; u < QTW; ++u)
#pragma unroll
        for (int p = 0; p < PP; ++p) MF::mac(o[u][ht], vf, pf[u][p]);
    }
  };

  // Per group, registers hold the loads of its next two steps; at local step
  // i the loads of i+2 are issued, step i is computed from LDS, the
  // registers of i+1 are stored to the group's other LDS buffer, and a
  // barrier (shared by the groups, which advance together) ends the step.
  // Three register sets rotate through a three-times unrolled loop (a copy
  // would wait for the loads just issued); every step loads (clamped), so
  // the waits stay two steps deep on every path.
  V16 r0[FW], r1[FW], r2[FW];
  auto step = [&](int i, V16 (&next)[FW], V16 (&ahead)[FW]) {
    load(ahead, i + 2);
    compute(i & 1, i);
    store(next, (i + 1) & 1);
    __syncthreads();
  };
  load(r0, 0);
  load(r1, 1);
  split_queries();
  store(r0, 0);
  __syncthreads();
  // whole groups of three steps unconditionally, the rest after the loop
  // (conditional steps inside the loop let the compiler sink the prefetch
  // loads into their use and drain the pipeline at every iteration)
  int i = 0;
  for (; i + 3 <= n_local; i += 3) {
    step(i, r1, r2);
    step(i + 1, r2, r0);
    step(i + 2, r0, r1);
  }
  if (i < n_local) {
    step(i, r1, r2);
    if (i + 1 < n_local) step(i + 1, r2, r0);
  }

  // each lane summed its own keys: total over the query's four lanes
#pragma unroll
  for (int u = 0; u < QTW; ++u) {
    l_run[u] += __shfl_xor(l_run[u], 16, 64);
    l_run[u] += __shfl_xor(l_run[u], 32, 64);
  }

  // key groups 1.. hand (m, l, O) to group 0 through the (now idle) fragment
  // buffers, one query tile of each wave per round; group 0 merges them in
  // order
  static_assert((KG - 1) * 4 * (HT + 1) <= KG * 2 * NF, "merge area fits the fragment buffers");
  V16* xch = &frag[0][0][0][0];
#pragma unroll
  for (int u = 0; u < QTW; ++u) {
    if (u > 0) __syncthreads();   // the previous round's records have been read
    if (kg > 0) {
      const int slot = (kg - 1) * 4 + wave;
#pragma unroll
      for (int ht = 0; ht < HT; ++ht) xch[(slot * (HT + 1) + ht) * 64 + lane].f = o[u][ht];
      xch[(slot * (HT + 1) + HT) * 64 + lane].f = floatx4{m_run[u], l_run[u], 0.f, 0.f};
    }
    __syncthreads();
    if (kg == 0) {
      float M = m_run[u];
#pragma unroll
      for (int k = 1; k < KG; ++k)
        M = fmaxf(M, xch[(((k - 1) * 4 + wave) * (HT + 1) + HT) * 64 + lane].f[0]);
      const float w0 = M == -INFINITY ? 0.f : exp2f(m_run[u] - M);
      float l = l_run[u] * w0;
#pragma unroll
      for (int ht = 0; ht < HT; ++ht)
#pragma unroll
        for (int i = 0; i < 4; ++i) o[u][ht][i] *= w0;
#pragma unroll
      for (int k = 1; k < KG; ++k) {
        const int slot = (k - 1) * 4 + wave;
        const floatx4 ml = xch[(slot * (HT + 1) + HT) * 64 + lane].f;
        const float w = ml[0] == -INFINITY ? 0.f : exp2f(ml[0] - M);
        l += w * ml[1];
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) {
          const floatx4 v = xch[(slot * (HT + 1) + ht) * 64 + lane].f;
#pragma unroll
          for (int i = 0; i < 4; ++i) o[u][ht][i] += w * v[i];
        }
      }
      m_run[u] = M;
      l_run[u] = l;
    }
  }
  if (kg > 0) return;

#pragma unroll
  for (int u = 0; u < QTW; ++u) {
    if (!qvalid[u]) continue;
    if (n_split == 1) {
      const float inv = 1.f / l_run[u];
      const size_t ro = (size_t)qrow[u] * d + h * HD;
#pragma unroll
      for (int ht = 0; ht < HT; ++ht) {
        const float4 y = make_float4(o[u][ht][0] * inv, o[u][ht][1] * inv, o[u][ht][2] * inv,
                                     o[u][ht][3] * inv);
        if (o_aps) {
          bf16* hi = reinterpret_cast<bf16*>(out) + ro + ht * 16 + lg * 4;
          store_hi_lo4(hi, hi + o_aps, y);
        } else {
          *reinterpret_cast<float4*>(out + ro + ht * 16 + lg * 4) = y;
        }
      }
    } else {
      const size_t base = ((size_t)split * m_cap + qrow[u]) * H + h;
      float* op = o_part + base * HD;
#pragma unroll
      for (int ht = 0; ht < HT; ++ht)
        *reinterpret_cast<float4*>(op + ht * 16 + lg * 4) =
            make_float4(o[u][ht][0], o[u][ht][1], o[u][ht][2], o[u][ht][3]);
      if (lg == 0) {
        ml_part[base * 2] = m_run[u];
        ml_part[base * 2 + 1] = l_run[u];
      }
    }
  }
}

// Combine the key splits of each row: out = sum_s 2^(m_s - M) O_s /
// sum_s 2^(m_s - M) l_s per head, splits taken in order; float4 of the row
// per thread.  With at most sixteen splits every record a row may have is
// loaded first -- before the row's request and key count are known, which
// only decide how many of them count (ns) -- so the row's loads take one
// memory round trip; records past ns are ignored (never read as numbers).
template <int HD, int NS>
__device__ __forceinline__ float4 merge_fixed(const float* __restrict__ o_part,
                                              const float* __restrict__ ml_part, size_t base0,
                                              size_t sstride, int i4,
                                              const int* __restrict__ req_len, int r, int kps,
                                              bool valid) {
  float2 ml[NS];
  float4 v[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const size_t base = base0 + s * sstride;
    ml[s] = *reinterpret_cast<const float2*>(ml_part + base * 2);
    v[s] = *reinterpret_cast<const float4*>(o_part + base * HD + (i4 * 4) % HD);
  }
  // a row past the pass has no request to look up (its table entry may be
  // anything); its result is not stored
  const int L = valid ? req_len[r] : 0;
  const int ns = min(NS, (L + kps - 1) / kps);
  if (ns <= 0) return make_float4(0.f, 0.f, 0.f, 0.f);   // no split covers the row
  float M = -INFINITY;
#pragma unroll
  for (int s = 0; s < NS; ++s)
    if (s < ns) M = fmaxf(M, ml[s].x);
  float lsum = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    if (s < ns) {
      const float w = exp2f(ml[s].x - M);
      lsum += w * ml[s].y;
      acc.x += w * v[s].x;
      acc.y += w * v[s].y;
      acc.z += w * v[s].z;
      acc.w += w * v[s].w;
    }
  }
  const float inv = 1.f / lsum;
  return make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
}

// Any split count (more than sixteen splits).
template <int HD>
__device__ __forceinline__ float4 merge_loop(int ns, const float* __restrict__ o_part,
                                             const float* __restrict__ ml_part, size_t base0,
                                             size_t sstride, int i4) {
  if (ns <= 0) return make_float4(0.f, 0.f, 0.f, 0.f);
  float M = -INFINITY;
  for (int s = 0; s < ns; ++s) M = fmaxf(M, ml_part[(base0 + s * sstride) * 2]);
  float lsum = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s = 0; s < ns; ++s) {
    const size_t base = base0 + s * sstride;
    const float w = exp2f(ml_part[base * 2] - M);
    lsum += w * ml_part[base * 2 + 1];
    const float4 v = *reinterpret_cast<const float4*>(o_part + base * HD + (i4 * 4) % HD);
    acc.x += w * v.x;
    acc.y += w * v.y;
    acc.z += w * v.z;
    acc.w += w * v.w;
  }
  const float inv = 1.f / lsum;
  return make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
}

template <int HD>
__global__ __launch_bounds__(256) void attn_merge_kernel(PassTable tb, int keys_per_split,
                                                         int n_split, int m_cap,
                                                         const float* __restrict__ o_part,
                                                         const float* __restrict__ ml_part,
                                                         int H, float* __restrict__ out,
                                                         size_t o_aps) {
  const int m = blockIdx.x;                    // < m_cap: every row's records are readable
  const int i4 = blockIdx.y * 256 + threadIdx.x;
  if (i4 * 4 >= H * HD) return;
  const int nr = *tb.nrows;
  const int r = tb.row_req[m];
  const bool valid = m < min(nr, m_cap);
  const int h = i4 * 4 / HD;
  const size_t base0 = (size_t)m * H + h;
  const size_t sstride = (size_t)m_cap * H;   // between splits, in (m, h) records
  float4 res;
  switch (n_split) {
    case 1: res = merge_fixed<HD, 1>(o_part, ml_part, base0, sstride, i4, tb.req_len, r, keys_per_split, valid); break;
    case 2: res = merge_fixed<HD, 2>(o_part, ml_part, base0, sstride, i4, tb.req_len, r, keys_per_split, valid); break;
    case 3: res = merge_fixed<HD, 3>(o_part, ml_part, base0, sstride, i4, tb.req_len, r, keys_per_split, valid); break;
    case 4: res = merge_fixed<HD, 4>(o_part, ml_part, base0, sstride, i4, tb.req_len, r, keys_per_split, valid); break;
    case 5: res = merge_fixed<HD, 5>(o_part, ml_part, base0, sstride, i4, tb.req_len, r, keys_per_split, valid); break;
    case 6: res = merge_fixed<HD, 6>(o_part, ml_part, base0, sstride, i4, tb.req_len, r, keys_per_split, valid); break;
    case 7: res = merge_fixed<HD, 7>(o_part, ml_part, base0, sstride, i4, tb.req_len, r, keys_per_split, valid); break;
    case 8: res = merge_fixed<HD, 8>(o_part, ml_part, base0, sstride, i4, tb.req_len, r, keys_per_split, valid); break;
    case 9: res = merge_fixed<HD, 9>(o_part, ml_part, base0, sstride, i4, tb.req_len, r, keys_per_split, valid); break;
    case 10: res = merge_fixed<HD, 10>(o_part, ml_part, base0, sstride, i4, tb.req_len, r, keys_per_split, valid); break;
    case 11: res = merge_fixed<HD, 11>(o_part, ml_part, base0, sstride, i4, tb.req_len, r, keys_per_split, valid); break;
    case 12: res = merge_fixed<HD, 12>(o_part, ml_part, base0, sstride, i4, tb.req_len, r, keys_per_split, valid); break;
    case 13: res = merge_fixed<HD, 13>(o_part, ml_part, base0, sstride, i4, tb.req_len, r, keys_per_split, valid); break;
    case 14: res = merge_fixed<HD, 14>(o_part, ml_part, base0, sstride, i4, tb.req_len, r, keys_per_split, valid); break;
    case 15: res = merge_fixed<HD, 15>(o_part, ml_part, base0, sstride, i4, tb.req_len, r, keys_per_split, valid); break;
    case 16: res = merge_fixed<HD, 16>(o_part, ml_part, base0, sstride, i4, tb.req_len, r, keys_per_split, valid); break;
    default: {
      const int L = valid ? tb.req_len[r] : 0;
      const int ns = min(n_split, (L + keys_per_split - 1) / keys_per_split);
      res = merge_loop<HD>(ns, o_part, ml_part, base0, sstride, i4);
    }
  }
  if (!valid) return;
  if (o_aps) {
    bf16* hi = reinterpret_cast<bf16*>(out) + (size_t)m * H * HD + i4 * 4;
    store_hi_lo4(hi, hi + o_aps, res);
  } else {
    *reinterpret_cast<float4*>(out + (size_t)m * H * HD + i4 * 4) = res;
  }
}

template <typename T, int HD, int QTW, bool PLO>
hipError_t run(const AttnPlan& p, PassTable tb, int batch, int m_cap, const float* q,
               const void* kc, const void* vt, int H, int Lp, float* o_part, float* ml_part,
               float* o, hipStream_t st, size_t o_aps) {
  const float scale_log2 = 1.4426950408889634f / sqrtf((float)HD);
  dim3 grid(p.n_split, H, batch * p.q_blocks);
  hipLaunchKernelGGL((attn_kernel<T, HD, QTW, PLO>), grid, dim3(256 * kKeyGroups), 0, st, tb,
                     p.q_blocks,
                     p.keys_per_split, p.n_split, m_cap, q, static_cast<const T*>(kc),
                     static_cast<const T*>(vt), H, Lp, scale_log2, o_part, ml_part, o, o_aps);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.n_split == 1) return e;
  const int blocks_y = (H * HD / 4 + 255) / 256;
  hipLaunchKernelGGL((attn_merge_kernel<HD>), dim3(m_cap, blocks_y), dim3(256), 0, st, tb,
                     p.keys_per_split, p.n_split, m_cap, o_part, ml_part, H, o, o_aps);
  return hipGetLastError();
}

template <typename T, int HD, bool PLO>
hipError_t run_q(const AttnPlan& p, PassTable tb, int batch, int m_cap, const float* q,
                 const void* kc, const void* vt, int H, int Lp, float* o_part, float* ml_part,
                 float* o, hipStream_t st, size_t o_aps) {
  if (p.qtw == 1) return run<T, HD, 1, PLO>(p, tb, batch, m_cap, q, kc, vt, H, Lp, o_part, ml_part, o, st, o_aps);
  if (p.qtw == 2) return run<T, HD, 2, PLO>(p, tb, batch, m_cap, q, kc, vt, H, Lp, o_part, ml_part, o, st, o_aps);
  return hipErrorInvalidValue;
}

}  // namespace

int attn_cache_len(int max_len) { return (max_len + 63) / 64 * 64; }

// Blocks of 64 queries, one 16-query tile per wave, while a request has at
// most 64 query rows (batch-1 and batch-16 windows of 32 + 2 * 16 positions;
// measured faster than fewer, wider workgroups there).  With more rows
// (refresh, wider windows) blocks of 128 queries, two tiles per wave: each
// K/V fragment is read from the cache and from LDS once for twice the
// queries (refresh of the 8K-prompt workload 6% faster, its window steps 3%).
// Then key splits while the grid stays within target_wgs (256: about one
// workgroup of eight waves per CU) and every split keeps at least 192 keys
// (shorter splits cost more in fixed work and partials than they gain in
// parallelism).
AttnPlan plan_attention(int batch, int max_rows_per_req, int max_keys, int H, int target_wgs) {
  AttnPlan p{};
  p.qtw = max_rows_per_req > 64 ? 2 : 1;
  p.q_blocks = (max_rows_per_req + 64 * p.qtw - 1) / (64 * p.qtw);
  if (p.q_blocks < 1) p.q_blocks = 1;
  const int steps = (max_keys + 31) / 32;
  const int base = batch * p.q_blocks * H;
  int ns = target_wgs / base;
  if (ns > max_keys / 192) ns = max_keys / 192;
  if (ns < 1) ns = 1;
  p.keys_per_split = (steps + ns - 1) / ns * 32;
  p.n_split = (max_keys + p.keys_per_split - 1) / p.keys_per_split;
  return p;
}

hipError_t launch_attention(DType t, const AttnPlan& p, PassTable tb, int batch, int m_cap,
                            const float* q, const void* kc, const void* vt, int H, int hd,
                            int Lp, float* o_part, float* ml_part, float* o, hipStream_t st,
                            bool p_lo, size_t o_aps) {
  if (Lp % 64 != 0 || p.keys_per_split % 32 != 0) return hipErrorInvalidValue;
  if (t == DType::F32) {
    if (hd == 64) return run_q<float, 64, true>(p, tb, batch, m_cap, q, kc, vt, H, Lp, o_part, ml_part, o, st, o_aps);
    if (hd == 128) return run_q<float, 128, true>(p, tb, batch, m_cap, q, kc, vt, H, Lp, o_part, ml_part, o, st, o_aps);
  } else if (p_lo) {
    if (hd == 64) return run_q<bf16, 64, true>(p, tb, batch, m_cap, q, kc, vt, H, Lp, o_part, ml_part, o, st, o_aps);
    if (hd == 128) return run_q<bf16, 128, true>(p, tb, batch, m_cap, q, kc, vt, H, Lp, o_part, ml_part, o, st, o_aps);
  } else {
    if (hd == 64) return run_q<bf16, 64, false>(p, tb, batch, m_cap, q, kc, vt, H, Lp, o_part, ml_part, o, st, o_aps);
    if (hd == 128) return run_q<bf16, 128, false>(p, tb, batch, m_cap, q, kc, vt, H, Lp, o_part, ml_part, o, st, o_aps);
  }
  return hipErrorInvalidValue;
}

}  // namespace dinfer
