// Device helpers of the vocab statistics shared by the standalone vocab pass
// (vocab.hip) and the LM-head epilogue of the projection kernels: the order
// every top-k here uses (larger value first, then smaller id), wave64 best
// and top-8 extraction, and sorted insertion into a per-thread top-8.  The
// MoE router's top-k takes the same wave64 best (the same order).
#pragma once

#include <climits>

#include "common.h"

namespace dinfer {
namespace vocab {

constexpr int kTop = 8;
constexpr float kLog2e = 1.4426950408889634f;

// Order used everywhere: larger value first, then smaller id.
__device__ __forceinline__ bool better(float va, int ia, float vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

// One exchange of a wave-wide reduction: each lane takes the better of its
// own pair and the partner's.  Within a row of 16 lanes the partner comes
// from a DPP rotation of the row (row_ror:n, control 0x120 + n); across rows
// from the gfx950 row swaps (v_permlane16_swap: odd rows of the first
// operand with even rows of the second; v_permlane32_swap: the upper half of
// the first with the lower half of the second), which with both operands the
// same value give each lane its partner row's value in one of the two
// results.  All of these are vector-ALU moves (no LDS round trip as
// ds_bpermute takes).  The order is a total order, so any reduction tree
// gives the same pair.
template <int CTRL>
__device__ __forceinline__ void best_rot(float& v, int& id) {
  const float ov =
      __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                             0xf, 0xf, false));
  const int oi = __builtin_amdgcn_update_dpp(0, id, CTRL, 0xf, 0xf, false);
  if (better(ov, oi, v, id)) {
    v = ov;
    id = oi;
  }
}
template <bool HALF>   // false: partner row (lane ^ 16); true: partner half (lane ^ 32)
__device__ __forceinline__ void best_swap(float& v, int& id) {
  const unsigned vb = __builtin_bit_cast(unsigned, v), ib = (unsigned)id;
  const int lane = threadIdx.x & 63;
  if constexpr (HALF) {
    const auto sv = __builtin_amdgcn_permlane32_swap(vb, vb, false, false);
    const auto si = __builtin_amdgcn_permlane32_swap(ib, ib, false, false);
    const bool lo = lane < 32;
    const float ov = __builtin_bit_cast(float, lo ? sv[1] : sv[0]);
    const int oi = (int)(lo ? si[1] : si[0]);
    if (better(ov, oi, v, id)) {
      v = ov;
      id = oi;
    }
  } else {
    const auto sv = __builtin_amdgcn_permlane16_swap(vb, vb, false, false);
    const auto si = __builtin_amdgcn_permlane16_swap(ib, ib, false, false);
    const bool even = ((lane >> 4) & 1) == 0;
    const float ov = __builtin_bit_cast(float, even ? sv[1] : sv[0]);
    const int oi = (int)(even ? si[1] : si[0]);
    if (better(ov, oi, v, id)) {
      v = ov;
      id = oi;
    }
  }
}

// Wave-wide best (value, id) pair: rotations by 8, 4, 2, 1 within each row
// give every lane its row's best, the two swaps combine the rows.
__device__ __forceinline__ void wave_best(float& v, int& id) {
  best_rot<0x128>(v, id);
  best_rot<0x124>(v, id);
  best_rot<0x122>(v, id);
  best_rot<0x121>(v, id);
  best_swap<false>(v, id);
  best_swap<true>(v, id);
}

// Wave-wide maximum the same way (exact: max is order-free).
__device__ __forceinline__ float wave_max_rot(float v) {
  int id = 0;
  wave_best(v, id);
  return v;
}

// Extract the wave's top-8 from per-lane sorted lists (pop-front on the
// winning lane).  Results are uniform across the wave.
__device__ __forceinline__ void wave_top8(float (&tv)[kTop], int (&ti)[kTop], float (&ov)[kTop],
                                          int (&oi)[kTop]) {
#pragma unroll
  for (int k = 0; k < kTop; ++k) {
    float v = tv[0];
    int id = ti[0];
    wave_best(v, id);
    ov[k] = v;
    oi[k] = id;
    if (tv[0] == v && ti[0] == id) {
#pragma unroll
      for (int j = 0; j < kTop - 1; ++j) {
        tv[j] = tv[j + 1];
        ti[j] = ti[j + 1];
      }
      tv[kTop - 1] = -INFINITY;
      ti[kTop - 1] = INT_MAX;
    }
  }
}

__device__ __forceinline__ void insert_top8(float (&tv)[kTop], int (&ti)[kTop], float v, int id) {
  // ids reach a thread in increasing order, so an equal value never displaces
  // an entry already kept (that entry has the smaller id).  The insertion is
  // a chain of selects (no per-slot branches): once a slot takes the new
  // entry, every later slot takes its predecessor.
  if (!(v > tv[kTop - 1])) return;
  bool carry = false;
  float cv = v;
  int ci = id;
#pragma unroll
  for (int k = 0; k < kTop; ++k) {
    const bool take = carry || cv > tv[k];
    const float tvk = tv[k];
    const int tik = ti[k];
    tv[k] = take ? cv : tvk;
    ti[k] = take ? ci : tik;
    cv = take ? tvk : cv;
    ci = take ? tik : ci;
    carry = take;
  }
}


// Record of one (row, column tile) of logits, merged over the tiles of a row
// by the merge kernel: rec_f[row][tile] = (max, sum of exp(z - max), top-8
// values), rec_i[row][tile] = top-8 ids; entries past the row's candidates
// are (-inf, INT_MAX).
constexpr int kRecF = 2 + kTop;

// Vocab records of a tile of logits staged in LDS: z[r * ldz + c] holds the
// logit of tile row r (global row row0 + r, r < nrows) and column col0 + c
// (c < NCOL).  Per row, the planting bias is added to its planted column,
// the MASK column and columns past V are excluded (-inf), and the record of
// (row, tile) is written.  The NW waves of the workgroup take rows w,
// w + NW, ...; lane l takes columns l + 64 j, so the lane's entries come in
// increasing id order.
template <int NCOL, int NW>
__device__ __forceinline__ void tile_records(const float* z, int ldz, int nrows, int row0,
                                             int col0, int V, int tile, int n_tiles,
                                             const int* __restrict__ row_pid,
                                             const float* __restrict__ row_pb, int mask_id,
                                             float* __restrict__ rec_f, int* __restrict__ rec_i) {
  static_assert(NCOL % 64 == 0 && NCOL <= 512, "64..512 columns per tile");
  constexpr int PJ = NCOL / 64;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  for (int r = wave; r < nrows; r += NW) {
    const int row = row0 + r;
    const int pid = row_pid[row];
    const float pb = row_pb[row];
    float tv[kTop];
    int ti[kTop];
#pragma unroll
    for (int k = 0; k < kTop; ++k) {
      tv[k] = -INFINITY;
      ti[k] = INT_MAX;
    }
    float m = -INFINITY;
#pragma unroll
    for (int j = 0; j < PJ; ++j) {
      const int c = lane + 64 * j;
      const int id = col0 + c;
      float x = z[r * ldz + c];
      if (id == pid) x += pb;
      if (id == mask_id || id >= V) x = -INFINITY;
      m = fmaxf(m, x);
      insert_top8(tv, ti, x, id);      // ids increase with j: ties keep the lower id
    }
    const float wm = wave_max_rot(m);
    float s = 0.f;
    if (wm != -INFINITY) {
#pragma unroll
      for (int j = 0; j < PJ; ++j)
        if (j < kTop && tv[j] != -INFINITY) s += exp2f((tv[j] - wm) * kLog2e);
    }
    const float ws = wave_sum(s);
    float ov[kTop];
    int oi[kTop];
    wave_top8(tv, ti, ov, oi);
    if (lane == 0) {
      float* pf = rec_f + ((size_t)row * n_tiles + tile) * kRecF;
      int* pi = rec_i + ((size_t)row * n_tiles + tile) * kTop;
      pf[0] = wm;
      pf[1] = ws;
#pragma unroll
      for (int k = 0; k < kTop; ++k) {
        pf[2 + k] = ov[k];
        pi[k] = oi[k];
      }
    }
  }
}

}  // namespace vocab
}  // namespace dinfer
