// Linear layers of the denoising step on gfx950 MFMA: out = A * W^T with A
// [M][K] fp32 activations and W [N][K] weights (Linear storage, fp32 or bf16),
// fp32 accumulation.
//
// Activations stay fp32 between kernels.  With bf16 weights each activation
// is split into hi = bf16(a) and lo = bf16(a - hi) and both halves go through
// the bf16 MFMA against the same weight fragment: the product then carries
// the weights' own precision only (no activation rounding), for one extra
// MFMA per weight fragment -- free wherever the layer is a weight stream.
//
// Weights are read in a packed layout (pack_kernel below; gemm_split.h): the
// 1 KB MFMA B operand of every 16 rows x KSTEP columns is stored
// contiguously, in lane order, so that each weight load of a wave is one
// contiguous kilobyte -- whole 128-byte lines -- and the blocks of one k-step
// of all rows are adjacent, so that the workgroups of a K split, advancing
// together, stream one narrow window of addresses through the matrix.  Read
// row-major, each load would touch 64
// bytes of 16 different rows and the vector L1 would issue twice as many
// half-line requests, stalling the address unit.
//
// Kernels:
//  * skinny (M <= 128): the vicinity window holds tens of rows, so a layer is
//    a weight stream.  A workgroup of NW waves owns 16*NT*NW output columns
//    (64 to 256) over all rows (or one of two 64-row tiles, for 65..128 rows)
//    and one K slice.  Each wave streams its own
//    packed weight blocks straight into registers (one 16-byte load per lane
//    per MFMA B operand), two K chunks ahead; the activation chunk is
//    split into hi/lo planes in LDS, double-buffered, and shared by the
//    waves -- wide column groups keep that fp32 re-read small next to the
//    weights.  K splits bring the workgroup count to about one per CU; each
//    split writes an fp32 partial that the consumer kernel sums in split
//    order (deterministic; the kernel boundary orders the writes).
//  * fat (M > 128: block-start refresh, batched steps): gemm_fat.hip.
// Also the grouped projection of the MoE experts, and the plans.
#include <algorithm>

#include "common.h"
#include "gemm_split.h"
#include "kernels.h"
#include "vocab_common.h"

namespace dinfer {

namespace {

// ---------------------------------------------------------------------------
// GUARD = false: A has at least 16*MT readable rows (rows >= M hold anything
// finite or not -- they only feed output rows that are never stored), so the
// activation loads and MFMAs carry no per-row conditions.  GUARD = true: rows
// >= M are read as zeros (exact-size operands of the standalone entry point).
//
// One workgroup's tile: rows [0, M) of A (row r at A + (arow ? arow[r] : r) * K)
// times weight rows [n_tile, n_tile + 16*NT*NW) of W (N rows) over K chunks
// [c_begin, c_end), written to out[row * ldo + column].
//
// VS = true (LM head): instead of storing the tile (or besides it, when out
// is not null) the workgroup stages it in LDS and reduces every row of it to
// its vocab record (vocab_common.h), rows numbered from vrow0.
template <typename TW, int MT, int NT, int NW, bool GUARD, bool VS = false, bool LO = true,
          int U = 4>
__device__ __forceinline__ void skinny_tile(const float* __restrict__ A,
                                            const int* __restrict__ arow, int M,
                                            const TW* __restrict__ W, int N, int K,
                                            float* __restrict__ out, int ldo, int n_tile,
                                            int c_begin, int c_end,
                                            const VocabEpi* ve = nullptr, int vrow0 = 0) {
  using MF = Mfma<TW>;
  using AS = ASplit<TW, LO>;
  constexpr int PL = AS::PLANES;
  constexpr int VEC = MF::VEC;
  constexpr int KSTEP = MF::KSTEP;
  // U vector steps per K chunk: KC = 128 (bf16, U 4) or 64 (U 2) K per
  // chunk; the LDS rows keep the 128-element stride (+16 B) either way
  constexpr int KC = U * KSTEP;
  constexpr int ROWS = 16 * MT;
  constexpr int STR = 4 * KSTEP + 16 / sizeof(TW);
  constexpr int NTH = NW * 64;                  // threads per workgroup
  constexpr int F4R = KC / 4;                   // float4 of A per chunk row
  constexpr int AF4 = ROWS * F4R;               // float4 of A per chunk
  constexpr int AV = (AF4 + NTH - 1) / NTH;     // float4 of A per thread per chunk
  // (when the threads do not divide the chunk, the surplus ones repeat its
  // last float4: the same value to the same LDS address)
  static_assert(U == 2 || U == 4, "two or four vector steps per chunk");
  __shared__ __attribute__((aligned(16))) TW As[2][PL][ROWS * STR];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int lc = lane & 15;
  const int lg = lane >> 4;
  const int n0 = n_tile + wave * (16 * NT);

  floatx4 acc[MT][NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = floatx4{0.f, 0.f, 0.f, 0.f};

  // packed weights: block (16-row group, vector step) of 64 * VEC elements;
  // a wave's groups sit in one tile, so they share the k-step stride
  constexpr int BE = 64 * VEC;
  const int KS = K / KSTEP;
  const int NG = N / 16;
  const size_t wstep = (size_t)packed_kstride(n0 / 16, NG) * BE;
  const TW* wrow[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
    wrow[nt] = W + packed_block(n0 / 16 + nt, 0, KS, NG) * BE + lane * VEC;

  // Weight fragments and raw activations of three consecutive chunks live in
  // registers.  At chunk c the loads of chunk c+2 are issued (activations
  // first), chunk c is multiplied from LDS, and the activations of chunk c+1
  // -- loaded one chunk earlier -- are split into LDS for the next chunk.
  // Memory operations complete in issue order, so that wait leaves the
  // weights of c+1 and everything of c+2 in flight.  The loop is unrolled
  // three times so buffers change roles without register copies (a copy
  // would wait for loads just issued).
  V16 b0[U][NT], b1[U][NT], b2[U][NT];
  float4 a0[AV], a1[AV], a2[AV];
  auto load_w = [&](V16 (&b)[U][NT], int c) {
#pragma unroll
    for (int j = 0; j < U; ++j)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) b[j][nt] = ld16(wrow[nt] + (c * U + j) * wstep);
  };
  auto load_a = [&](float4 (&areg)[AV], int c) {
#pragma unroll
    for (int i = 0; i < AV; ++i) {
      const int v = AF4 % NTH ? min((int)threadIdx.x + NTH * i, AF4 - 1) : threadIdx.x + NTH * i;
      const int r = v / F4R;
      const int cv = v % F4R;
      const size_t ar = arow ? (size_t)arow[GUARD ? min(r, M - 1) : r] : (size_t)r;
      if (GUARD)
        areg[i] = r < M ? *reinterpret_cast<const float4*>(A + ar * K + c * KC + cv * 4)
                        : make_float4(0.f, 0.f, 0.f, 0.f);
      else
        areg[i] = *reinterpret_cast<const float4*>(A + ar * K + c * KC + cv * 4);
    }
  };
  auto store_a = [&](const float4 (&areg)[AV], int buf) {
#pragma unroll
    for (int i = 0; i < AV; ++i) {
      const int v = AF4 % NTH ? min((int)threadIdx.x + NTH * i, AF4 - 1) : threadIdx.x + NTH * i;
      const int r = v / F4R;
      const int cv = v % F4R;
      AS::store4(&As[buf][0][r * STR + cv * 4], &As[buf][PL - 1][r * STR + cv * 4], areg[i]);
    }
  };
  // Activation fragments of one vector step for every row tile and plane,
  // read from LDS one vector step ahead of the MFMAs that use them.
  auto read_frags = [&](V16 (&f)[MT][PL], int buf, int j) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int p = 0; p < PL; ++p)
        f[mt][p] = *reinterpret_cast<const V16*>(
            &As[buf][p][(mt * 16 + lc) * STR + j * KSTEP + lg * VEC]);
  };
  // bc/ac: chunk c (weights; activations already staged), an: activations of
  // c+1 (to stage), bl/al: targets of the chunk c+2 loads.  Every step issues
  // its loads, clamped to the last chunk near the end (a repeated read of
  // data just fetched): loads under a condition make the compiler's wait
  // counts at the join points assume the short path and drain the prefetch.
  auto step = [&](int c, V16 (&bc)[U][NT], float4 (&an)[AV], V16 (&bl)[U][NT],
                  float4 (&al)[AV]) {
    const int buf = (c - c_begin) & 1;
    const int cl = min(c + 2, c_end - 1);
    load_a(al, cl);
    load_w(bl, cl);
    if constexpr (MT * PL <= 12) {
      V16 af[2][MT][PL];
      read_frags(af[0], buf, 0);
#pragma unroll
      for (int j = 0; j < U; ++j) {
        if (j + 1 < U) read_frags(af[(j + 1) & 1], buf, j + 1);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int p = 0; p < PL; ++p)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) MF::mac(acc[mt][nt], af[j & 1][mt][p], bc[j][nt]);
      }
    } else {   // many row tiles: no registers to spare for a fragment buffer
#pragma unroll
      for (int j = 0; j < U; ++j)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int p = 0; p < PL; ++p) {
            const V16 a = *reinterpret_cast<const V16*>(
                &As[buf][p][(mt * 16 + lc) * STR + j * KSTEP + lg * VEC]);
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) MF::mac(acc[mt][nt], a, bc[j][nt]);
          }
    }
    store_a(an, buf ^ 1);   // past the end: staged into a buffer nobody reads
    __syncthreads();
  };

  if (c_begin < c_end) {
    load_a(a0, c_begin);
    load_w(b0, c_begin);
    const int c1 = min(c_begin + 1, c_end - 1);
    load_a(a1, c1);
    load_w(b1, c1);
    store_a(a0, 0);
  }
  __syncthreads();
  // (Whole groups of three unconditional steps with the remainder after the
  // loop, which keeps the compiler from draining the prefetch at the loop's
  // join points, measured 3-10% slower here; the fat kernel takes it.)
  for (int c = c_begin; c < c_end; c += 3) {
    step(c, b0, a1, b2, a2);
    if (c + 1 < c_end) step(c + 1, b1, a2, b0, a0);
    if (c + 2 < c_end) step(c + 2, b2, a0, b1, a1);
  }

  if constexpr (VS) {
    // the logit tile [ROWS][NCOL] in the (now idle) activation staging
    // buffer; rows padded so the four row groups of a store fall on
    // different banks
    constexpr int NCOL = 16 * NT * NW;
    constexpr int LDZ = NCOL + (sizeof(TW) == 2 ? 16 : 8);
    static_assert(ROWS * LDZ * sizeof(float) <= sizeof(As), "logit tile fits the staging buffer");
    float* zt = reinterpret_cast<float*>(&As[0][0][0]);
    __syncthreads();
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = mt * 16 + lg * 4 + i;
          const int col = wave * (16 * NT) + nt * 16 + lc;
          zt[row * LDZ + col] = acc[mt][nt][i];
          if (out != nullptr && row < M) out[(size_t)row * ldo + n0 + nt * 16 + lc] = acc[mt][nt][i];
        }
    __syncthreads();
    vocab::tile_records<NCOL, NW>(zt, LDZ, M, vrow0, n_tile, N, n_tile / NCOL, ve->n_tiles,
                                  ve->row_plant_id, ve->row_plant_bias, ve->mask_id, ve->rec_f,
                                  ve->rec_i);
  } else {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = mt * 16 + lg * 4 + i;
          if (row < M) out[(size_t)row * ldo + n0 + nt * 16 + lc] = acc[mt][nt][i];
        }
  }
}

template <typename TW, int MT, int NT, int NW, bool GUARD, bool LO, int U>
__global__ __launch_bounds__(NW * 64) void gemm_skinny_kernel(const float* __restrict__ A,
                                                              const TW* __restrict__ W,
                                                              float* __restrict__ P,
                                                              const int* __restrict__ m_dev,
                                                              int m_cap, int N, int K,
                                                              int n_tiles, int S, int m_tiles) {
  constexpr int KC = U * Mfma<TW>::KSTEP;
  constexpr int ROWS = 16 * MT;
  // work item (split, column group) = split * n_tiles + tile; its m_tiles row
  // tiles get workgroup ids 8 apart, so they run side by side on one XCD and
  // share the weights through its L2 (ids past the items exit)
  const int bid = blockIdx.x;
  const int grp = bid / (8 * m_tiles);
  const int rem = bid % (8 * m_tiles);
  const int mt = rem / 8;
  const int item = grp * 8 + rem % 8;
  if (item >= n_tiles * S) return;
  const int tile = item % n_tiles;
  const int split = item / n_tiles;
  const int C = K / KC;
  const int M = (m_dev ? min(*m_dev, m_cap) : m_cap) - mt * ROWS;
  if (M <= 0) return;
  skinny_tile<TW, MT, NT, NW, GUARD, false, LO, U>(A + (size_t)mt * ROWS * K, nullptr, min(M, ROWS), W, N, K,
                                     P + ((size_t)split * m_cap + (size_t)mt * ROWS) * N, N,
                                     tile * (16 * NT * NW), (split * C) / S, ((split + 1) * C) / S);
}

// Vector steps per K chunk of a skinny projection: 64-element chunks (two
// 32-element MFMA steps) for the eight-wave bf16 groups -- 32 KB of weights
// per workgroup and chunk, 64 KB in flight two chunks ahead -- and 128 for
// the rest.  Measured on the dense 8B window (64 rows): QKV 26.9 -> 24.5 us,
// gate|up 49.3 -> 47.3 us; the four-wave O and down projections (128-column
// groups, K 4096 and 12288) were 2% faster and 3% slower.  The LM head and
// the MoE grouped experts (eight-wave groups) take the same: dense step
// 4.78 -> 4.76 ms, MoE step 5.09 -> 5.00 ms.
template <typename TW, int NW> constexpr int skinny_u() {
  return sizeof(TW) == 2 && NW == 8 ? 2 : 4;
}

// LM head: the skinny projection of the block rows over the whole
// vocabulary (one K slice), each workgroup reducing its tile to vocab
// records instead of storing logits (also stored when ve.logits is set).
template <typename TW, int MT, int NT, int NW, bool GUARD>
__global__ __launch_bounds__(NW * 64) void gemm_skinny_lmhead_kernel(
    const float* __restrict__ A, const TW* __restrict__ W, const int* __restrict__ m_dev,
    int m_cap, int N, int K, int n_tiles, int m_tiles, VocabEpi ve) {
  constexpr int SU = skinny_u<TW, NW>();
  constexpr int KC = SU * Mfma<TW>::KSTEP;
  constexpr int ROWS = 16 * MT;
  const int bid = blockIdx.x;
  const int grp = bid / (8 * m_tiles);
  const int rem = bid % (8 * m_tiles);
  const int mt = rem / 8;
  const int tile = grp * 8 + rem % 8;
  if (tile >= n_tiles) return;
  const int M = (m_dev ? min(*m_dev, m_cap) : m_cap) - mt * ROWS;
  if (M <= 0) return;
  skinny_tile<TW, MT, NT, NW, GUARD, true, true, SU>(
      A + (size_t)mt * ROWS * K, nullptr, min(M, ROWS), W, N, K,
      ve.logits ? ve.logits + (size_t)mt * ROWS * N : nullptr, N, tile * (16 * NT * NW), 0,
      K / KC, &ve, mt * ROWS);
}

// Grouped projection of the MoE experts: workgroup (expert e, column group,
// 64-row tile) multiplies rows [off_e + 64 t, min(off_e + count_e, +64)) of
// the packed assignment list -- gathered from A through row_of[] when given,
// else read in place -- with expert e's weights Wtab[e] (one packed [N][K]
// matrix: in HBM, or in pinned host memory the kernel reads directly when an
// expert cache holds only some experts in HBM).  The row tiles of
// one (expert, column group) get workgroup ids 8 apart: workgroups are dealt
// to the eight XCDs in id order, so they run side by side on one XCD and
// the second reads the weights the first brings into that XCD's L2 (an
// expert that many rows prefer needs two row tiles).
template <typename TW, int NT, int NW>
__global__ __launch_bounds__(NW * 64) void gemm_grouped_kernel(
    const float* __restrict__ A, const int* __restrict__ row_of, const int* __restrict__ e_count,
    const int* __restrict__ e_off, const TW* const* __restrict__ Wtab, float* __restrict__ out,
    int N, int K, int n_tiles, int m_tiles, int n_pairs) {
  constexpr int SU = skinny_u<TW, NW>();
  constexpr int KC = SU * Mfma<TW>::KSTEP;
  const int bid = blockIdx.x;
  const int grp = bid / (8 * m_tiles);
  const int rem = bid % (8 * m_tiles);
  const int mt = rem / 8;
  const int pair = grp * 8 + rem % 8;          // e * n_tiles + tile
  if (pair >= n_pairs) return;
  const int tile = pair % n_tiles;
  const int e = pair / n_tiles;
  const int cnt = e_count[e];
  const int M = min(64, cnt - mt * 64);
  if (M <= 0) return;
  const int base = e_off[e] + mt * 64;
  const float* a = row_of ? A : A + (size_t)base * K;
  const int* ar = row_of ? row_of + base : nullptr;
  skinny_tile<TW, 4, NT, NW, true, false, true, SU>(a, ar, M, Wtab[e], N, K, out + (size_t)base * N, N,
                                   tile * (16 * NT * NW), 0, K / KC);
}


// Packs W [N][K] (row-major; blockIdx.y selects one of a stack of such
// matrices) into the block layout the GEMMs read (packed_block): block
// (group g = n / 16, k-step s = k / KSTEP) holds 64 * VEC elements and its
// slot 16 q + c holds W[16 g + c][s * KSTEP + q * VEC, + VEC) -- the MFMA
// operand of lane 16 q + c.
template <typename TW>
__global__ __launch_bounds__(256) void pack_kernel(const TW* __restrict__ W, TW* __restrict__ P,
                                                   int N, int K) {
  constexpr int VEC = Mfma<TW>::VEC;
  constexpr int KSTEP = Mfma<TW>::KSTEP;
  const int KS = K / KSTEP;
  const int NG = N / 16;
  const size_t blk = (size_t)blockIdx.x * 4 + (threadIdx.x >> 6);   // source order: g, then s
  if (blk >= (size_t)NG * KS) return;
  const size_t mat = (size_t)blockIdx.y * N * K;
  const int lane = threadIdx.x & 63;
  const int g = (int)(blk / KS);
  const int s = (int)(blk % KS);
  st16(P + mat + packed_block(g, s, KS, NG) * 64 * VEC + lane * VEC,
       ld16(W + mat + ((size_t)g * 16 + (lane & 15)) * K + s * KSTEP + (lane >> 4) * VEC));
}

// ---------------------------------------------------------------------------
template <typename TW, int MT, int NT, int NW, bool LO>
hipError_t run_skinny(const GemmPlan& p, const float* A, const void* W, float* out,
                      const int* m_dev, int m_cap, int N, int K, hipStream_t st) {
  constexpr int SU = skinny_u<TW, NW>();
  const int n_tiles = N / (16 * NT * NW);
  const int mtiles = p.mtiles > 1 ? p.mtiles : 1;
  if (m_cap > 16 * MT * mtiles) return hipErrorInvalidValue;
  const dim3 grid((n_tiles * p.splits + 7) / 8 * 8 * mtiles);
  if (p.guard)
    hipLaunchKernelGGL((gemm_skinny_kernel<TW, MT, NT, NW, true, LO, SU>), grid, dim3(NW * 64), 0, st, A,
                       static_cast<const TW*>(W), out, m_dev, m_cap, N, K, n_tiles, p.splits,
                       mtiles);
  else
    hipLaunchKernelGGL((gemm_skinny_kernel<TW, MT, NT, NW, false, LO, SU>), grid, dim3(NW * 64), 0, st, A,
                       static_cast<const TW*>(W), out, m_dev, m_cap, N, K, n_tiles, p.splits,
                       mtiles);
  return hipGetLastError();
}

template <typename TW, int MT, int NT, int NW>
hipError_t run_skinny_lmhead(const GemmPlan& p, const float* A, const void* W, const int* m_dev,
                             int m_cap, int N, int K, const VocabEpi& e, hipStream_t st) {
  const int n_tiles = N / (16 * NT * NW);
  const int mtiles = p.mtiles > 1 ? p.mtiles : 1;
  if (m_cap > 16 * MT * mtiles || p.splits != 1 || e.n_tiles != n_tiles) return hipErrorInvalidValue;
  const dim3 grid((n_tiles + 7) / 8 * 8 * mtiles);
  if (p.guard)
    hipLaunchKernelGGL((gemm_skinny_lmhead_kernel<TW, MT, NT, NW, true>), grid, dim3(NW * 64), 0,
                       st, A, static_cast<const TW*>(W), m_dev, m_cap, N, K, n_tiles, mtiles, e);
  else
    hipLaunchKernelGGL((gemm_skinny_lmhead_kernel<TW, MT, NT, NW, false>), grid, dim3(NW * 64), 0,
                       st, A, static_cast<const TW*>(W), m_dev, m_cap, N, K, n_tiles, mtiles, e);
  return hipGetLastError();
}

template <typename TW, int NT, int NW>
hipError_t lmhead_mt(const GemmPlan& p, const float* A, const void* W, const int* m_dev,
                     int m_cap, int N, int K, const VocabEpi& e, hipStream_t st) {
  switch (p.mt) {
    case 1: return run_skinny_lmhead<TW, 1, NT, NW>(p, A, W, m_dev, m_cap, N, K, e, st);
    case 2: return run_skinny_lmhead<TW, 2, NT, NW>(p, A, W, m_dev, m_cap, N, K, e, st);
    case 3: return run_skinny_lmhead<TW, 3, NT, NW>(p, A, W, m_dev, m_cap, N, K, e, st);
    case 4: return run_skinny_lmhead<TW, 4, NT, NW>(p, A, W, m_dev, m_cap, N, K, e, st);
    default: break;
  }
  if constexpr (NW == 8) {
    return hipErrorInvalidValue;
  } else {
    switch (p.mt) {
      case 5: return run_skinny_lmhead<TW, 5, NT, NW>(p, A, W, m_dev, m_cap, N, K, e, st);
      case 6: return run_skinny_lmhead<TW, 6, NT, NW>(p, A, W, m_dev, m_cap, N, K, e, st);
      case 7: return run_skinny_lmhead<TW, 7, NT, NW>(p, A, W, m_dev, m_cap, N, K, e, st);
      case 8: return run_skinny_lmhead<TW, 8, NT, NW>(p, A, W, m_dev, m_cap, N, K, e, st);
      default: return hipErrorInvalidValue;
    }
  }
}

template <typename TW>
hipError_t lmhead_dispatch(const GemmPlan& p, const float* A, const void* W, const int* m_dev,
                           int m_cap, int N, int K, const VocabEpi& e, hipStream_t st) {
  if (p.kind == 1)
    return launch_gemm_fat_lmhead(sizeof(TW) == 2 ? DType::BF16 : DType::F32, p.nw, A, W, m_dev,
                                  m_cap, N, K, e, st);
  if constexpr (sizeof(TW) == 2) {
    if (p.nw == 8) return lmhead_mt<TW, 2, 8>(p, A, W, m_dev, m_cap, N, K, e, st);
  }
  return p.nt == 2 ? lmhead_mt<TW, 2, 4>(p, A, W, m_dev, m_cap, N, K, e, st)
                   : lmhead_mt<TW, 1, 4>(p, A, W, m_dev, m_cap, N, K, e, st);
}

template <typename TW, int NT, int NW, bool LO>
hipError_t dispatch_mt(const GemmPlan& p, const float* A, const void* W, float* out,
                       const int* m_dev, int m_cap, int N, int K, hipStream_t st) {
  switch (p.mt) {
    case 1: return run_skinny<TW, 1, NT, NW, LO>(p, A, W, out, m_dev, m_cap, N, K, st);
    case 2: return run_skinny<TW, 2, NT, NW, LO>(p, A, W, out, m_dev, m_cap, N, K, st);
    case 3: return run_skinny<TW, 3, NT, NW, LO>(p, A, W, out, m_dev, m_cap, N, K, st);
    case 4: return run_skinny<TW, 4, NT, NW, LO>(p, A, W, out, m_dev, m_cap, N, K, st);
    default: break;
  }
  if constexpr (NW == 8) {
    return hipErrorInvalidValue;   // 8-wave groups: at most 64 rows
  } else {
    switch (p.mt) {
      case 5: return run_skinny<TW, 5, NT, NW, LO>(p, A, W, out, m_dev, m_cap, N, K, st);
      case 6: return run_skinny<TW, 6, NT, NW, LO>(p, A, W, out, m_dev, m_cap, N, K, st);
      case 7: return run_skinny<TW, 7, NT, NW, LO>(p, A, W, out, m_dev, m_cap, N, K, st);
      case 8: return run_skinny<TW, 8, NT, NW, LO>(p, A, W, out, m_dev, m_cap, N, K, st);
      default: return hipErrorInvalidValue;
    }
  }
}

template <typename TW, bool LO>
hipError_t dispatch_lo(const GemmPlan& p, const float* A, const void* W, float* out,
                       const int* m_dev, int m_cap, int N, int K, hipStream_t st) {
  if constexpr (sizeof(TW) == 2) {   // 8-wave groups: bf16 weights only
    if (p.nw == 8) return dispatch_mt<TW, 2, 8, LO>(p, A, W, out, m_dev, m_cap, N, K, st);
  }
  return p.nt == 2 ? dispatch_mt<TW, 2, 4, LO>(p, A, W, out, m_dev, m_cap, N, K, st)
                   : dispatch_mt<TW, 1, 4, LO>(p, A, W, out, m_dev, m_cap, N, K, st);
}

template <typename TW>
hipError_t dispatch(const GemmPlan& p, const float* A, const void* W, float* out,
                    const int* m_dev, int m_cap, int N, int K, hipStream_t st) {
  if (p.kind == 1)
    return launch_gemm_fat(sizeof(TW) == 2 ? DType::BF16 : DType::F32, p.nw, p.splits, A, W,
                           out, m_dev, m_cap, N, K, st, p.lo != 0, p.ap != 0);
  if (p.ap) return hipErrorInvalidValue;   // planar activations: fat plans only
  if constexpr (sizeof(TW) == 2) {   // activations in bf16 only: a bf16-weight option
    if (!p.lo) return dispatch_lo<TW, false>(p, A, W, out, m_dev, m_cap, N, K, st);
  }
  return dispatch_lo<TW, true>(p, A, W, out, m_dev, m_cap, N, K, st);
}

}  // namespace

int gemm_k_chunk(DType t) { return t == DType::F32 ? 64 : 128; }

hipError_t launch_gemm_grouped(DType t, const float* A, const int* row_of, const int* e_count,
                               const int* e_off, int E, int max_rows, const void* const* Wtab,
                               float* out, int N, int K, hipStream_t st) {
  if (N % 128 != 0 || K % gemm_k_chunk(t) != 0) return hipErrorInvalidValue;
  const int m_tiles = (max_rows + 63) / 64;
  // bf16 with 256-column groups: eight waves x 32 columns (two waves per
  // SIMD hide each other's latency; four waves of this tile need one SIMD
  // each); else four waves x 32 columns
  const bool wide = t == DType::BF16 && N % 256 == 0;
  const int n_tiles = N / (wide ? 256 : 128);
  const int n_pairs = E * n_tiles;
  const dim3 grid((n_pairs + 7) / 8 * 8 * m_tiles);
  if (t == DType::F32)
    hipLaunchKernelGGL((gemm_grouped_kernel<float, 2, 4>), grid, dim3(256), 0, st, A, row_of,
                       e_count, e_off, reinterpret_cast<const float* const*>(Wtab), out, N, K, n_tiles, m_tiles,
                       n_pairs);
  else if (wide)
    hipLaunchKernelGGL((gemm_grouped_kernel<bf16, 2, 8>), grid, dim3(512), 0, st, A, row_of,
                       e_count, e_off, reinterpret_cast<const bf16* const*>(Wtab), out, N, K, n_tiles, m_tiles,
                       n_pairs);
  else
    hipLaunchKernelGGL((gemm_grouped_kernel<bf16, 2, 4>), grid, dim3(256), 0, st, A, row_of,
                       e_count, e_off, reinterpret_cast<const bf16* const*>(Wtab), out, N, K, n_tiles, m_tiles,
                       n_pairs);
  return hipGetLastError();
}

hipError_t launch_pack_linear(DType t, const void* W, void* P, int n_mats, int N, int K,
                              hipStream_t st) {
  const int kstep = t == DType::F32 ? Mfma<float>::KSTEP : Mfma<bf16>::KSTEP;
  if (n_mats < 1 || n_mats > 65535 || N < 16 || N % 16 != 0 || K < kstep || K % kstep != 0)
    return hipErrorInvalidValue;
  const size_t wgs = ((size_t)(N / 16) * (K / kstep) + 3) / 4;   // four 1 KB blocks per workgroup
  if (wgs > (size_t)INT32_MAX) return hipErrorInvalidValue;
  const dim3 grid((unsigned)wgs, (unsigned)n_mats);
  if (t == DType::F32)
    hipLaunchKernelGGL(pack_kernel<float>, grid, dim3(256), 0, st, static_cast<const float*>(W),
                       static_cast<float*>(P), N, K);
  else
    hipLaunchKernelGGL(pack_kernel<bf16>, grid, dim3(256), 0, st, static_cast<const bf16*>(W),
                       static_cast<bf16*>(P), N, K);
  return hipGetLastError();
}

bool gemm_shape_ok(DType t, int N, int K) {
  return N > 0 && K > 0 && N % 128 == 0 && K % gemm_k_chunk(t) == 0;
}

// Fat plan: 128 x 256 tiles (128 x 128 when N has a single tile), and the K
// split count s <= 4 that minimises the estimated time
//   ceil(tiles * s / target_wgs) / s * K * c_round  +  (s - 1) * M * N * c_part
// -- rounds of one workgroup per CU, each a 1/s share of the full-K tile work,
// plus the extra fp32 partial written and read back for each added split
// (c_round and c_part measured on the dense 8B shapes: a full-K round takes
// about 112 us at K = 4096; a partial element costs 8 bytes at about 4 TB/s).
// Splitting pays where the tile count leaves a last round mostly empty.
//
// Skinny plan: up to 64 rows, 256-column groups (8 waves x 32) where that
// gives at least 32 groups, else 128 (4 x 32) where it gives 16, else 64
// (4 x 16); 65..128 rows with N % 256 == 0: two 64-row tiles on 256-column
// eight-wave groups; then K splits so that the grid is about target_wgs
// workgroups.
GemmPlan plan_gemm(DType t, int m_cap, int N, int K, int target_wgs) {
  GemmPlan p{};
  p.lo = 1;
  if (m_cap > 128) {
    p.kind = 1;
    p.mtiles = 1;
    p.mt = p.nt = 0;
    p.nw = N > 128 ? 4 : 2;
    const int mtiles = (m_cap + 127) / 128;
    const int tiles = ((N + 64 * p.nw - 1) / (64 * p.nw)) * mtiles;
    const int max_s = std::min(4, K / (t == DType::F32 ? 32 : 64));
    const double c_round = 112.0 / 4096, c_part = 8.0 / 4e6;   // us per K element; us per partial
    double best = 0.0;
    p.splits = 1;
    for (int s = 1; s <= max_s; ++s) {
      const double rounds = (double)((tiles * s + target_wgs - 1) / target_wgs);
      const double cost = rounds / s * K * c_round + (s - 1) * (double)m_cap * N * c_part;
      if (s == 1 || cost < best) {
        best = cost;
        p.splits = s;
      }
    }
    p.grid = tiles * p.splits;
    return p;
  }
  p.kind = 0;
  p.mt = (m_cap + 15) / 16;
  if (p.mt < 1) p.mt = 1;
  p.mtiles = 1;
  p.guard = (m_cap % 16) != 0;   // exact-size operands with ragged rows only
  const int chunks = K / gemm_k_chunk(t);
  if (t == DType::BF16 && N % 256 == 0 && N / 256 >= 32 && p.mt <= 4) {
    p.nt = 2;
    p.nw = 8;
  } else if (t == DType::BF16 && N % 256 == 0 && p.mt > 4) {
    // 65..128 rows: two 64-row tiles on eight-wave groups (two waves per
    // SIMD; one 128-row tile needs four waves of 400+ registers, one per
    // SIMD), the tiles of a column group sharing its weights through L2
    p.mt = 4;
    p.mtiles = 2;
    p.nt = 2;
    p.nw = 8;
    p.guard = (m_cap % 64) != 0;   // the second tile reads rows 64..127
  } else if (N % 128 == 0 && N / 128 >= 16) {
    p.nt = 2;
    p.nw = 4;
  } else {
    p.nt = 1;
    p.nw = 4;
  }
  const int n_tiles = N / (16 * p.nt * p.nw);
  // as many K splits as still fit one round of target_wgs workgroups: a
  // partial round costs a whole round, and each split adds an fp32 partial
  int s = target_wgs / (n_tiles * p.mtiles);
  if (s < 1) s = 1;
  if (s > chunks) s = chunks;
  p.splits = s;
  p.grid = n_tiles * s * p.mtiles;
  return p;
}

int gemm_lmhead_tiles(const GemmPlan& p, int N) {
  const int cols = p.kind == 1 ? 64 * p.nw : 16 * p.nt * p.nw;
  return (N + cols - 1) / cols;
}

hipError_t launch_gemm_lmhead(const GemmPlan& p, DType t, const float* A, const void* W,
                              const int* m_dev, int m_cap, int N, int K, const VocabEpi& e,
                              hipStream_t st) {
  if (!e.row_plant_id || !e.row_plant_bias || !e.rec_f || !e.rec_i ||
      e.n_tiles != gemm_lmhead_tiles(p, N))
    return hipErrorInvalidValue;
  if (t == DType::F32) return lmhead_dispatch<float>(p, A, W, m_dev, m_cap, N, K, e, st);
  return lmhead_dispatch<bf16>(p, A, W, m_dev, m_cap, N, K, e, st);
}

hipError_t launch_gemm(const GemmPlan& p, DType t, const float* A, const void* W, float* out,
                       const int* m_dev, int m_cap, int N, int K, hipStream_t st) {
  if (t == DType::F32) return dispatch<float>(p, A, W, out, m_dev, m_cap, N, K, st);
  return dispatch<bf16>(p, A, W, out, m_dev, m_cap, N, K, st);
}

}  // namespace dinfer
