// Device helpers of the vocab statistics shared by the standalone vocab pass
// (vocab.hip) and the LM-head epilogue of the projection kernels: the order
// every top-k here uses (larger value first, then smaller id), wave64 best
// and top-8 extraction, and sorted insertion into a per-thread top-8.
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

// Wave-wide best (value, id) pair.
__device__ __forceinline__ void wave_best(float& v, int& id) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float ov = __shfl_xor(v, o, 64);
    const int oi = __shfl_xor(id, o, 64);
    if (better(ov, oi, v, id)) {
      v = ov;
      id = oi;
    }
  }
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
    const float wm = wave_max(m);
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
