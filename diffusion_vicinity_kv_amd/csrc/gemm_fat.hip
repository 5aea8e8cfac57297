// Dense projections with many rows (block-start refresh, batched steps) on
// gfx950 MFMA: out[s] = A * W^T over the s-th K slice, A [M][K] fp32
// activations, W [N][K] weights (fp32 or bf16) in the packed block layout of
// launch_pack_linear, fp32 accumulation.  K splits (grid z) only even out the
// last round of workgroups; their partials are summed by the consumer.
#include <type_traits>

#include "common.h"
#include "gemm_split.h"
#include "kernels.h"
#include "vocab_common.h"

namespace dinfer {

namespace {

// Fat kernel: 128 x 64*WN output tile per workgroup of 2 x WN waves (each
// 64 x 64 as 4 x 4 MFMA tiles; WN = 4: two waves per SIMD, used when the grid
// still has a workgroup per CU, else WN = 2), K slabs of BK = 64 (bf16)
// / 32 (fp32) elements double-buffered in LDS with the activations split into
// hi/lo planes on the way in (or taking planes a producer already split).
// Activation rows in LDS are unpadded 128-byte lines with an XOR swizzle of
// their 16-byte chunks; the weights keep their packed 1 KB operand blocks,
// so both are read and written without bank conflicts (measured: matrix
// cores about 38% busy; a slab takes about twice its MFMA time, spent on the
// LDS fragment reads, the staging, the barrier and waits on global loads,
// which hit L2 three times in four).  Global loads run
// two slabs ahead through three register sets (a three-times unrolled loop,
// as in the skinny kernel), all unconditional: rows past M read row M-1 and
// columns past N read the last 16-column group (their outputs are not
// stored).
constexpr int kFatM = 128;
// Vector steps per K slab: two (128-byte LDS rows: 64 bf16 / 32 fp32).
// Measured against one step of 32 bf16 (64-byte rows, 64 KB of slab
// buffers): 5% slower at the same occupancy, and 35% slower when held to
// four waves per SIMD so that two workgroups share a CU (the register limit
// of 128 spills).
template <typename TW> constexpr int kFatKK = 2;

//
// VS = true (LM head, one K split): the 128 x 64*WN tile is reduced to vocab
// records (vocab_common.h) through LDS, 64 rows at a time, instead of being
// stored (stored as well when ve.logits is set).
// The 128 KB of LDS admit one workgroup per CU (2 x WN / 4 waves per SIMD),
// which leaves each wave up to 256 registers; saying so keeps the compiler
// from squeezing into 128 by reloading the prefetched slabs just before use.
//
// AP = true (bf16 weights): A holds the activations already split, as bf16 hi
// and lo planes of [m_cap][K], the lo plane aps elements after the hi plane
// (written by the producing kernel with store_hi_lo4: the bits the in-kernel
// split would make).  Each 16-byte load is then one LDS chunk of a plane and
// is stored unchanged -- no conversion in the slab loop, which every column
// tile of a row tile would otherwise repeat.
//
// SG = true (gate|up projection of a SwiGLU FFN, one K split, WN = 4): the
// workgroup's 256 columns are the gate columns f0..f0+127 (waves wn 0, 1)
// and the up columns F+f0..F+f0+127 (waves 2, 3) of W [2F][K], f0 = 128 bx,
// and its epilogue writes act = silu(gate) * up (the SwiGLU kernel's
// arithmetic on the same fp32 sums) as bf16 hi/lo planes of [m_cap][F]
// (lo plane aps_out elements after hi) instead of the [m_cap][2F] product:
// the up waves hand their tiles to the gate waves through LDS.
template <typename TW, int WN, bool VS, bool LO, bool AP = false, bool SG = false>
__global__ __launch_bounds__(128 * WN)
__attribute__((amdgpu_waves_per_eu(1, WN / 2))) void gemm_fat_kernel(const float* __restrict__ A,
                                                            const TW* __restrict__ W,
                                                            float* __restrict__ Cout,
                                                            const int* __restrict__ m_dev,
                                                            int m_cap, int N, int K, VocabEpi ve,
                                                            size_t aps, size_t aps_out) {
  constexpr int kFatN = 64 * WN, kFatThreads = 128 * WN;
  using MF = Mfma<TW>;
  using AS = ASplit<TW, LO>;
  constexpr int PL = AS::PLANES;
  constexpr int VEC = MF::VEC;
  constexpr int KSTEP = MF::KSTEP;
  constexpr int KK = kFatKK<TW>;               // vector steps per slab
  constexpr int BK = KK * KSTEP;               // K elements per slab
  constexpr int STR = BK;                      // LDS row: NC 16-byte chunks, unpadded
  constexpr int CH = 16 / sizeof(TW);          // elements per chunk
  constexpr int NC = BK / CH;                  // chunks per row: 4 or 8
  static_assert(NC == 4 || NC == 8, "the swizzle takes rows of 64 or 128 bytes");
  // LDS reads serve 16 lanes (256 bytes, every bank once) at a time.  Chunk j
  // of row r lives at chunk j ^ ((r / RS) % NC), RS = 256 / row bytes rows
  // sharing a bank window: the 16 rows of a fragment read then fall on 16
  // distinct 16-byte bank groups.
  constexpr int RS = 256 / (NC * 16);
  auto sw = [](int r, int e) {
    return r * STR + ((((e / CH) ^ (r / RS)) & (NC - 1)) * CH) + e % CH;
  };
  static_assert(!AP || (sizeof(TW) == 2 && !VS), "activation planes: bf16 projections only");
  static_assert(!SG || (sizeof(TW) == 2 && !VS && WN == 4), "SwiGLU epilogue: bf16, 256 columns");
  constexpr int F4R = BK / 4;                  // float4 of A per slab row
  constexpr int AV = kFatM * F4R / kFatThreads;     // float4 of A per thread per slab
  // AP: 16-byte chunks (CH elements) of one plane; PL planes of kFatM rows
  constexpr int APC = kFatM * NC;              // chunks of one plane per slab
  constexpr int AU = AP ? PL * APC / kFatThreads : 1;   // chunks per thread per slab
  static_assert(!AP || PL * APC % kFatThreads == 0, "plane chunks must split evenly");
  using AReg = std::conditional_t<AP, V16, float4>;
  constexpr int NA = AP ? AU : AV;             // activation registers per thread per slab
  constexpr int BE = 64 * VEC;                 // elements of one packed weight block
  constexpr int BV = (kFatN / 16) * KK * 64 / kFatThreads;   // W vectors per thread per slab
  static_assert((kFatN / 16) * KK * 64 % kFatThreads == 0, "weight slab must split evenly");
  // one LDS block: activation planes, then weight slabs (the LM head's
  // epilogue reuses all of it)
  constexpr size_t kAsBytes = (size_t)2 * PL * kFatM * STR * sizeof(TW);
  constexpr size_t kBsBytes = (size_t)2 * kFatN * STR * sizeof(TW);
  __shared__ __attribute__((aligned(16))) unsigned char smem[kAsBytes + kBsBytes];
  auto& As = *reinterpret_cast<TW(*)[2][PL][kFatM * STR]>(smem);
  auto& Bs = *reinterpret_cast<TW(*)[2][kFatN * STR]>(smem + kAsBytes);

  const int M = m_dev ? min(*m_dev, m_cap) : m_cap;
  // The LM head's grid is one-dimensional: the row tiles of a column tile
  // get workgroup ids 8 apart, so they run side by side on one XCD and read
  // the tile's weights from HBM once (its column tiles are not a multiple of
  // 8: in a 2-D grid the row tiles of a column would fall on different XCDs,
  // rounds apart, and the 1 GB head would stream once per row tile).
  int bx = blockIdx.x, by = blockIdx.y;
  if constexpr (VS) {
    const int mtiles = (m_cap + kFatM - 1) / kFatM;
    const int grp = blockIdx.x / (8 * mtiles);
    const int rem = blockIdx.x % (8 * mtiles);
    by = rem / 8;
    bx = grp * 8 + rem % 8;
    if (bx * kFatN >= N) return;
  }
  const int m0 = by * kFatM;
  const int n0 = bx * kFatN;
  if (m0 >= M) return;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int lc = lane & 15;
  const int lg = lane >> 4;
  const int wm = wave / WN;                    // 2 row halves
  const int wn = wave % WN;                    // WN column groups
  // this workgroup's K slabs: split blockIdx.z of gridDim.z
  const int nk_all = K / BK;
  const int kb = (int)(blockIdx.z * nk_all / gridDim.z);
  const int nk = (int)((blockIdx.z + 1) * nk_all / gridDim.z) - kb;
  Cout += (size_t)blockIdx.z * m_cap * N;

  floatx4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

  // row offsets of this thread's slab elements (fixed over K); with AP the
  // thread's chunk i is plane v / APC, row (v % APC) / NC, chunk v % NC
  const float* arow[AV];
  const TW* aprow[AU];
  if constexpr (AP) {
    const TW* Ab = reinterpret_cast<const TW*>(A);
#pragma unroll
    for (int i = 0; i < AU; ++i) {
      const int v = threadIdx.x + kFatThreads * i;
      aprow[i] = Ab + (v / APC) * aps + (size_t)min(m0 + (v % APC) / NC, M - 1) * K +
                 (v % NC) * CH;
    }
  } else {
#pragma unroll
    for (int i = 0; i < AV; ++i) {
      const int v = threadIdx.x + kFatThreads * i;
      arow[i] = A + (size_t)min(m0 + v / F4R, M - 1) * K + (v % F4R) * 4;
    }
  }
  // weight vector v of a slab: block v / 64 = (16-column group, vector step),
  // lane slot v % 64; the slab's blocks sit in LDS in that order
  const int KS = K / KSTEP;
  const int NG = N / 16;
  const TW* wrow[BV];
  size_t wstep[BV];   // elements between slabs
#pragma unroll
  for (int i = 0; i < BV; ++i) {
    const int v = threadIdx.x + kFatThreads * i;
    // SG: groups 0..7 of the tile are gate groups 8 bx.., 8..15 up groups
    const int j = (v / 64) / KK;
    const int grp = SG ? (j < 8 ? 8 * bx + j : NG / 2 + 8 * bx + j - 8)
                       : min(n0 / 16 + j, NG - 1);
    wrow[i] = W + packed_block(grp, (v / 64) % KK, KS, NG) * BE + (v % 64) * VEC;
    wstep[i] = (size_t)KK * packed_kstride(grp, NG) * BE;
  }
  auto gload = [&](AReg (&ra)[NA], V16 (&rb)[BV], int kt) {
    kt = kb + min(kt, nk - 1);   // past the end: repeat the last slab
    if constexpr (AP) {
#pragma unroll
      for (int i = 0; i < AU; ++i) ra[i] = ld16(aprow[i] + kt * BK);
    } else {
#pragma unroll
      for (int i = 0; i < AV; ++i) ra[i] = *reinterpret_cast<const float4*>(arow[i] + kt * BK);
    }
#pragma unroll
    for (int i = 0; i < BV; ++i) rb[i] = ld16(wrow[i] + kt * wstep[i]);
  };
  auto sstore = [&](AReg (&ra)[NA], const V16 (&rb)[BV], int buf) {
    if constexpr (AP) {
#pragma unroll
      for (int i = 0; i < AU; ++i) {
        const int v = threadIdx.x + kFatThreads * i;
        st16(&As[buf][v / APC][sw((v % APC) / NC, (v % NC) * CH)], ra[i]);
      }
    } else {
      hold_regs(ra);
#pragma unroll
      for (int i = 0; i < AV; ++i) {
        const int v = threadIdx.x + kFatThreads * i;
        const int r = v / F4R;
        const int cv = v % F4R;
        AS::store4(&As[buf][0][sw(r, cv * 4)], &As[buf][PL - 1][sw(r, cv * 4)], ra[i]);
      }
    }
#pragma unroll
    for (int i = 0; i < BV; ++i) st16(&Bs[buf][(threadIdx.x + kFatThreads * i) * VEC], rb[i]);
  };
  auto mma = [&](int buf) {
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      V16 b[4];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
        b[nt] = *reinterpret_cast<const V16*>(&Bs[buf][((wn * 4 + nt) * KK + kk) * BE + lane * VEC]);
#pragma unroll
      for (int p = 0; p < PL; ++p) {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          const V16 a = *reinterpret_cast<const V16*>(
              &As[buf][p][sw(wm * 64 + mt * 16 + lc, kk * KSTEP + lg * VEC)]);
#pragma unroll
          for (int nt = 0; nt < 4; ++nt) MF::mac(acc[mt][nt], a, b[nt]);
        }
      }
    }
  };
  // slab kt: issue the loads of kt+2, multiply slab kt from LDS, stage the
  // registers of kt+1 into the other buffer, barrier
  AReg a0[NA], a1[NA], a2[NA];
  V16 b0[BV], b1[BV], b2[BV];
  auto step = [&](int kt, AReg (&an)[NA], V16 (&bn)[BV], AReg (&al)[NA], V16 (&bl)[BV]) {
    gload(al, bl, kt + 2);
    mma(kt & 1);
    sstore(an, bn, (kt + 1) & 1);
    __syncthreads();
  };
  gload(a0, b0, 0);
  gload(a1, b1, 1);
  sstore(a0, b0, 0);
  __syncthreads();
  // whole groups of three steps unconditionally, the rest after the loop
  // (conditional steps inside the loop let the compiler sink the prefetch
  // loads into their use and drain the pipeline at every iteration)
  int kt = 0;
  for (; kt + 3 <= nk; kt += 3) {
    step(kt, a1, b1, a2, b2);
    step(kt + 1, a2, b2, a0, b0);
    step(kt + 2, a0, b0, a1, b1);
  }
  if (kt < nk) {
    step(kt, a1, b1, a2, b2);
    if (kt + 1 < nk) step(kt + 1, a2, b2, a0, b0);
  }

  if constexpr (VS) {
    constexpr int LDZ = kFatN + 16;              // padded rows: stores spread over banks
    // rows staged per pass: 64 when they fit the LDS block, else 32
    constexpr int RP = (size_t)64 * LDZ * sizeof(float) <= kAsBytes + kBsBytes ? 64 : 32;
    static_assert((size_t)RP * LDZ * sizeof(float) <= kAsBytes + kBsBytes, "pass fits LDS");
    float* zt = reinterpret_cast<float*>(smem);
    for (int h = 0; h < kFatM / RP; ++h) {      // each pass: the waves holding its rows stage them
      __syncthreads();
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const int rb = wm * 64 + mt * 16;       // wave-uniform
        if (rb / RP != h) continue;
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            zt[(rb % RP + lg * 4 + i) * LDZ + wn * 64 + nt * 16 + lc] = acc[mt][nt][i];
      }
      __syncthreads();
      const int r0 = m0 + h * RP;
      if (r0 < M)
        vocab::tile_records<kFatN, 2 * WN>(zt, LDZ, min(RP, M - r0), r0, n0, N, bx,
                                           ve.n_tiles, ve.row_plant_id, ve.row_plant_bias,
                                           ve.mask_id, ve.rec_f, ve.rec_i);
    }
    Cout = ve.logits;
    if (Cout == nullptr) return;
  }
  if constexpr (SG) {
    // the up waves (wn 2, 3) park their 128 x 128 tile in LDS (free since
    // the loop's last barrier); the gate waves pair each element with it
    constexpr int LDU = 128 + 4;
    static_assert((size_t)128 * LDU * sizeof(float) <= kAsBytes + kBsBytes, "up tile fits LDS");
    float* ut = reinterpret_cast<float*>(smem);
    if (wn >= 2) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            ut[(wm * 64 + mt * 16 + lg * 4 + i) * LDU + (wn - 2) * 64 + nt * 16 + lc] = acc[mt][nt][i];
    }
    __syncthreads();
    if (wn >= 2) return;
    const int F = N / 2;
    bf16* hi = reinterpret_cast<bf16*>(Cout);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = wm * 64 + mt * 16 + lg * 4 + i;
          const int c = wn * 64 + nt * 16 + lc;
          if (m0 + r >= M) continue;
          const float g = acc[mt][nt][i], u = ut[r * LDU + c];
          const float y = g / (1.f + expf(-g)) * u;
          const bf16 h = static_cast<bf16>(y);
          const size_t at = (size_t)(m0 + r) * F + 128 * bx + c;
          hi[at] = h;
          hi[at + aps_out] = static_cast<bf16>(y - static_cast<float>(h));
        }
    return;
  }
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = m0 + wm * 64 + mt * 16 + lg * 4 + i;
        const int col = n0 + wn * 64 + nt * 16 + lc;
        if (row < M && col < N) Cout[(size_t)row * N + col] = acc[mt][nt][i];
      }
}

template <bool VS, bool LO, bool AP = false, bool SG = false>
hipError_t fat_launch(DType t, int wn, int splits, const float* A, const void* W, float* out,
                      const int* m_dev, int m_cap, int N, int K, const VocabEpi& ve,
                      hipStream_t st) {
  const size_t aps = AP ? (size_t)m_cap * K : 0;   // plane stride of planar activations
  const size_t aps_out = SG ? (size_t)m_cap * (N / 2) : 0;   // ... of the SwiGLU output
  if (SG && (wn != 4 || splits != 1 || N % 256 != 0 || t != DType::BF16)) return hipErrorInvalidValue;
  const int bk = t == DType::F32 ? 16 * kFatKK<float> : 32 * kFatKK<bf16>;   // K per slab
  if ((wn != 2 && wn != 4) || splits < 1 || splits > K / bk) return hipErrorInvalidValue;
  const int n_tiles = (N + 64 * wn - 1) / (64 * wn), m_tiles = (m_cap + kFatM - 1) / kFatM;
  const dim3 grid = VS ? dim3((n_tiles + 7) / 8 * 8 * m_tiles, 1, 1)   // see the kernel
                       : dim3(n_tiles, m_tiles, splits);
  if (t == DType::F32) {
    if constexpr (AP) return hipErrorInvalidValue;
    if (wn == 4)
      hipLaunchKernelGGL((gemm_fat_kernel<float, 4, VS, true>), grid, dim3(512), 0, st, A,
                         static_cast<const float*>(W), out, m_dev, m_cap, N, K, ve, aps, aps_out);
    else
      hipLaunchKernelGGL((gemm_fat_kernel<float, 2, VS, true>), grid, dim3(256), 0, st, A,
                         static_cast<const float*>(W), out, m_dev, m_cap, N, K, ve, aps, aps_out);
  } else {
    if (wn == 4)
      hipLaunchKernelGGL((gemm_fat_kernel<bf16, 4, VS, LO, AP, SG>), grid, dim3(512), 0, st, A,
                         static_cast<const bf16*>(W), out, m_dev, m_cap, N, K, ve, aps, aps_out);
    else if constexpr (!SG)
      hipLaunchKernelGGL((gemm_fat_kernel<bf16, 2, VS, LO, AP>), grid, dim3(256), 0, st, A,
                         static_cast<const bf16*>(W), out, m_dev, m_cap, N, K, ve, aps, aps_out);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_fat(DType t, int wn, int splits, const float* A, const void* W,
                           float* out, const int* m_dev, int m_cap, int N, int K, hipStream_t st,
                           bool lo, bool ap) {
  if (ap && t != DType::BF16) return hipErrorInvalidValue;
  if (!lo && t == DType::BF16)
    return ap ? fat_launch<false, false, true>(t, wn, splits, A, W, out, m_dev, m_cap, N, K,
                                               VocabEpi{}, st)
              : fat_launch<false, false>(t, wn, splits, A, W, out, m_dev, m_cap, N, K, VocabEpi{}, st);
  return ap ? fat_launch<false, true, true>(t, wn, splits, A, W, out, m_dev, m_cap, N, K,
                                            VocabEpi{}, st)
            : fat_launch<false, true>(t, wn, splits, A, W, out, m_dev, m_cap, N, K, VocabEpi{}, st);
}

hipError_t launch_gemm_fat_swiglu(DType t, const float* A, const void* W, float* act,
                                  const int* m_dev, int m_cap, int N, int K, hipStream_t st,
                                  bool lo) {
  if (t != DType::BF16) return hipErrorInvalidValue;
  return lo ? fat_launch<false, true, true, true>(t, 4, 1, A, W, act, m_dev, m_cap, N, K,
                                                  VocabEpi{}, st)
            : fat_launch<false, false, true, true>(t, 4, 1, A, W, act, m_dev, m_cap, N, K,
                                                   VocabEpi{}, st);
}

hipError_t launch_gemm_fat_lmhead(DType t, int wn, const float* A, const void* W,
                                  const int* m_dev, int m_cap, int N, int K, const VocabEpi& e,
                                  hipStream_t st) {
  if (e.n_tiles != (N + 64 * wn - 1) / (64 * wn)) return hipErrorInvalidValue;
  return fat_launch<true, true>(t, wn, 1, A, W, e.logits, m_dev, m_cap, N, K, e, st);
}

}  // namespace dinfer
