// Operand formats shared by the GEMM kernels: the activation staging of the
// bf16 GEMMs (fp32 activations become two bf16 planes, hi = bf16(a) and lo =
// bf16(a - hi), so that the two bf16 MFMAs against the same weight fragment
// carry the weights' precision only; fp32 weights take fp32 activations
// unchanged, one plane) and the packed weight layout.
#pragma once

#include "common.h"

namespace dinfer {
namespace {

template <typename TW> struct ASplit;
// bf16 weights: two LDS planes (hi, lo) of bf16 activations.
template <> struct ASplit<bf16> {
  static constexpr int PLANES = 2;
  __device__ __forceinline__ static void store4(bf16* hi, bf16* lo, const float4& x) {
    const float v[4] = {x.x, x.y, x.z, x.w};
    bf16x4 h, l;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      h[i] = static_cast<bf16>(v[i]);
      l[i] = static_cast<bf16>(v[i] - static_cast<float>(h[i]));
    }
    *reinterpret_cast<bf16x4*>(hi) = h;
    *reinterpret_cast<bf16x4*>(lo) = l;
  }
};
// fp32 weights: one plane of fp32 activations.
template <> struct ASplit<float> {
  static constexpr int PLANES = 1;
  __device__ __forceinline__ static void store4(float* p, float*, const float4& x) {
    *reinterpret_cast<float4*>(p) = x;
  }
};

// Packed weight layout (written by pack_kernel in gemm.hip).  One block is
// the 1 KB MFMA operand of 16 rows (a "group") x one vector step of KSTEP
// columns, slot 16q + c holding row c, columns [q VEC, (q+1) VEC).  Groups
// come in tiles of kPackTile = 16 (256 rows); a tile's blocks are stored
// k-step by k-step, the tile's groups consecutive within a k-step, so that a
// workgroup streaming a 256-row (or 128-row) column tile reads one
// contiguous run per k-step.  The last tile of a matrix may hold fewer
// groups.  Block index of (group g, k-step s), with KS k-steps and NG groups:
constexpr int kPackTile = 16;
__host__ __device__ __forceinline__ size_t packed_block(int g, int s, int KS, int NG) {
  const int t = g / kPackTile;
  const int tb = min(kPackTile, NG - t * kPackTile);   // groups in this tile
  return (size_t)t * kPackTile * KS + (size_t)s * tb + (g - t * kPackTile);
}
// Distance in blocks between consecutive k-steps of group g.
__host__ __device__ __forceinline__ int packed_kstride(int g, int NG) {
  return min(kPackTile, NG - (g / kPackTile) * kPackTile);
}

}  // namespace
}  // namespace dinfer
