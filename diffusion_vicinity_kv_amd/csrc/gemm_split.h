// Activation staging of the bf16 GEMMs: fp32 activations become two bf16
// planes, hi = bf16(a) and lo = bf16(a - hi), so that the two bf16 MFMAs
// against the same weight fragment carry the weights' precision only.  fp32
// weights take fp32 activations unchanged (one plane).
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

}  // namespace
}  // namespace dinfer
