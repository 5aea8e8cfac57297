// Operand formats shared by the GEMM kernels: the activation staging of the
// bf16 GEMMs (fp32 activations become two bf16 planes, hi = bf16(a) and lo =
// bf16(a - hi), so that the two bf16 MFMAs against the same weight fragment
// carry the weights' precision only; fp32 weights take fp32 activations
// unchanged, one plane) and the packed weight layout.
#pragma once

#include "common.h"

namespace dinfer {
namespace {

// LO = false (bf16 only): the activations enter the MFMA as bf16(a) alone --
// one plane, one MFMA per weight fragment, the activation's own rounding
// kept (a per-projection precision option of the library).
template <typename TW, bool LO = true> struct ASplit;
// bf16 weights: two LDS planes (hi, lo) of bf16 activations.
template <> struct ASplit<bf16, true> {
  static constexpr int PLANES = 2;
  __device__ __forceinline__ static void store4(bf16* hi, bf16* lo, const float4& x) {
    store_hi_lo4(hi, lo, x);
  }
};
template <> struct ASplit<bf16, false> {
  static constexpr int PLANES = 1;
  __device__ __forceinline__ static void store4(bf16* hi, bf16*, const float4& x) {
    bf16x4 h;
    h[0] = static_cast<bf16>(x.x);
    h[1] = static_cast<bf16>(x.y);
    h[2] = static_cast<bf16>(x.z);
    h[3] = static_cast<bf16>(x.w);
    *reinterpret_cast<bf16x4*>(hi) = h;
  }
};
// fp32 weights: one plane of fp32 activations.
template <bool LO> struct ASplit<float, LO> {
  static constexpr int PLANES = 1;
  __device__ __forceinline__ static void store4(float* p, float*, const float4& x) {
    *reinterpret_cast<float4*>(p) = x;
  }
};

// Packed weight layout (written by pack_kernel in gemm.hip).  One block is
// the 1 KB MFMA operand of 16 rows (a "group") x one vector step of KSTEP
// columns, slot 16q + c holding row c, columns [q VEC, (q+1) VEC).  Blocks
// are stored k-step-major: all NG groups of k-step 0, then of k-step 1, ...
// A wave's weight load is one contiguous kilobyte, a workgroup's column tile
// is one contiguous run per k-step, and the workgroups of one K split, which
// advance through their k-steps at about the same pace, read neighbouring
// runs at any moment -- a narrow window of addresses sweeping through the
// matrix, which streams from HBM measurably faster (+4-5% on the dense 8B
// projections) than one separate sequential run per workgroup.  Block index
// of (group g, k-step s), with NG groups:
__host__ __device__ __forceinline__ size_t packed_block(int g, int s, int /*KS*/, int NG) {
  return (size_t)s * NG + g;
}
// Distance in blocks between consecutive k-steps of one group.
__host__ __device__ __forceinline__ int packed_kstride(int /*g*/, int NG) { return NG; }

}  // namespace
}  // namespace dinfer
