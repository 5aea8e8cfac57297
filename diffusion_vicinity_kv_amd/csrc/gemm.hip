// Linear layers of the denoising step on gfx950 MFMA: out = A * W^T with A
// [M][K] activations and W [N][K] weights (Linear storage), fp32 accumulation.
//
// Two kernels:
//  * skinny (M <= 128): the vicinity window holds tens of rows, so each layer
//    is a weight stream.  A workgroup owns 64*NT output columns over all rows
//    and one K slice; its activations are staged in LDS chunk by chunk and
//    shared by four waves, while every wave streams its own weight rows
//    straight into registers (one 16-byte load per lane per MFMA B operand),
//    issued ahead of the LDS staging so their latency overlaps it.  K splits
//    raise the workgroup count; each split writes an fp32 partial that the
//    consumer kernel sums in split order (deterministic).
//  * fat (M > 128: block-start refresh, batched steps): 128x128 output tiles,
//    128-byte K slabs of both operands double-buffered in LDS, four waves each
//    computing 64x64 with 16x16 MFMA tiles.
#include "common.h"
#include "kernels.h"

namespace dinfer {

namespace {

// ---------------------------------------------------------------------------
template <typename T, int MT, int NT>
__global__ __launch_bounds__(256) void gemm_skinny_kernel(const T* __restrict__ A,
                                                          const T* __restrict__ W,
                                                          float* __restrict__ P,
                                                          const int* __restrict__ m_dev,
                                                          int m_cap, int N, int K, int n_tiles,
                                                          int S) {
  using MF = Mfma<T>;
  constexpr int VEC = MF::VEC;
  constexpr int KSTEP = MF::KSTEP;
  constexpr int KC = 512 / sizeof(T);             // K elements per LDS chunk (512 B / row)
  constexpr int U = KC / KSTEP;                   // vector steps per chunk
  constexpr int ROWS = 16 * MT;
  constexpr int STR = KC + 16 / sizeof(T);        // LDS row stride, +16 B against bank conflicts
  constexpr int VPR = KC / VEC;                   // 16-byte vectors per staged row (32)
  __shared__ __attribute__((aligned(16))) T As[ROWS * STR];

  const int bid = blockIdx.x;
  const int tile = bid % n_tiles;
  const int split = bid / n_tiles;
  const int C = K / KC;
  const int c_begin = (split * C) / S;
  const int c_end = ((split + 1) * C) / S;
  const int M = m_dev ? min(*m_dev, m_cap) : m_cap;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int lc = lane & 15;
  const int lg = lane >> 4;
  const int n0 = tile * (64 * NT) + wave * (16 * NT);

  floatx4 acc[MT][NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = floatx4{0.f, 0.f, 0.f, 0.f};

  const T* wrow[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) wrow[nt] = W + (size_t)(n0 + nt * 16 + lc) * K + lg * VEC;

  for (int c = c_begin; c < c_end; ++c) {
    const int kb = c * KC;
    V16 b[U][NT];
#pragma unroll
    for (int j = 0; j < U; ++j)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) b[j][nt] = ld16(wrow[nt] + kb + j * KSTEP);
    __syncthreads();  // every wave is done reading the previous chunk
    for (int v = threadIdx.x; v < ROWS * VPR; v += 256) {
      const int r = v / VPR;
      const int cv = v % VPR;
      const V16 x = (r < M) ? ld16(A + (size_t)r * K + kb + cv * VEC) : zero16();
      st16(&As[r * STR + cv * VEC], x);
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < U; ++j) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        if (mt * 16 < M) {
          const V16 a = *reinterpret_cast<const V16*>(&As[(mt * 16 + lc) * STR + j * KSTEP + lg * VEC]);
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) MF::mac(acc[mt][nt], a, b[j][nt]);
        }
      }
    }
  }

  float* out = P + (size_t)split * m_cap * N;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = mt * 16 + lg * 4 + i;
        if (row < M) out[(size_t)row * N + n0 + nt * 16 + lc] = acc[mt][nt][i];
      }
}

// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void gemm_fat_kernel(const T* __restrict__ A,
                                                       const T* __restrict__ W,
                                                       float* __restrict__ Cout,
                                                       const int* __restrict__ m_dev, int m_cap,
                                                       int N, int K) {
  using MF = Mfma<T>;
  constexpr int VEC = MF::VEC;
  constexpr int KSTEP = MF::KSTEP;
  constexpr int BK = 128 / sizeof(T);      // K elements per slab (128 B per row)
  constexpr int STEPS = BK / KSTEP;
  constexpr int STR = BK + 16 / sizeof(T);
  constexpr int VPR = BK / VEC;            // 8 vectors per slab row
  __shared__ __attribute__((aligned(16))) T As[2][128 * STR];
  __shared__ __attribute__((aligned(16))) T Bs[2][128 * STR];

  const int M = m_dev ? min(*m_dev, m_cap) : m_cap;
  const int m0 = blockIdx.y * 128;
  const int n0 = blockIdx.x * 128;
  if (m0 >= M) return;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int lc = lane & 15;
  const int lg = lane >> 4;
  const int wm = wave >> 1;
  const int wn = wave & 1;

  floatx4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

  V16 ra[4], rb[4];
  auto gload = [&](int kt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int v = threadIdx.x + 256 * i;
      const int r = v / VPR;
      const int cv = v % VPR;
      ra[i] = (m0 + r < M) ? ld16(A + (size_t)(m0 + r) * K + kt * BK + cv * VEC) : zero16();
      rb[i] = (n0 + r < N) ? ld16(W + (size_t)(n0 + r) * K + kt * BK + cv * VEC) : zero16();
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int v = threadIdx.x + 256 * i;
      const int r = v / VPR;
      const int cv = v % VPR;
      st16(&As[buf][r * STR + cv * VEC], ra[i]);
      st16(&Bs[buf][r * STR + cv * VEC], rb[i]);
    }
  };

  const int nk = K / BK;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
#pragma unroll
    for (int s = 0; s < STEPS; ++s) {
      V16 a[4], b[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
        a[mt] = *reinterpret_cast<const V16*>(
            &As[cur][(wm * 64 + mt * 16 + lc) * STR + s * KSTEP + lg * VEC]);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
        b[nt] = *reinterpret_cast<const V16*>(
            &Bs[cur][(wn * 64 + nt * 16 + lc) * STR + s * KSTEP + lg * VEC]);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) MF::mac(acc[mt][nt], a[mt], b[nt]);
    }
    if (kt + 1 < nk) sstore(cur ^ 1);
    __syncthreads();
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

template <typename T, int MT, int NT>
hipError_t run_skinny(const GemmPlan& p, const void* A, const void* W, float* out,
                      const int* m_dev, int m_cap, int N, int K, hipStream_t st) {
  const int n_tiles = N / (64 * NT);
  hipLaunchKernelGGL((gemm_skinny_kernel<T, MT, NT>), dim3(n_tiles * p.splits), dim3(256), 0, st,
                     static_cast<const T*>(A), static_cast<const T*>(W), out, m_dev, m_cap, N, K,
                     n_tiles, p.splits);
  return hipGetLastError();
}

template <typename T, int NT>
hipError_t dispatch_mt(const GemmPlan& p, const void* A, const void* W, float* out,
                       const int* m_dev, int m_cap, int N, int K, hipStream_t st) {
  switch (p.mt) {
    case 1: return run_skinny<T, 1, NT>(p, A, W, out, m_dev, m_cap, N, K, st);
    case 2: return run_skinny<T, 2, NT>(p, A, W, out, m_dev, m_cap, N, K, st);
    case 3: return run_skinny<T, 3, NT>(p, A, W, out, m_dev, m_cap, N, K, st);
    case 4: return run_skinny<T, 4, NT>(p, A, W, out, m_dev, m_cap, N, K, st);
    case 5: return run_skinny<T, 5, NT>(p, A, W, out, m_dev, m_cap, N, K, st);
    case 6: return run_skinny<T, 6, NT>(p, A, W, out, m_dev, m_cap, N, K, st);
    case 7: return run_skinny<T, 7, NT>(p, A, W, out, m_dev, m_cap, N, K, st);
    case 8: return run_skinny<T, 8, NT>(p, A, W, out, m_dev, m_cap, N, K, st);
    default: return hipErrorInvalidValue;
  }
}

template <typename T>
hipError_t dispatch(const GemmPlan& p, const void* A, const void* W, float* out, const int* m_dev,
                    int m_cap, int N, int K, hipStream_t st) {
  if (p.kind == 1) {
    dim3 grid((N + 127) / 128, (m_cap + 127) / 128);
    hipLaunchKernelGGL((gemm_fat_kernel<T>), grid, dim3(256), 0, st, static_cast<const T*>(A),
                       static_cast<const T*>(W), out, m_dev, m_cap, N, K);
    return hipGetLastError();
  }
  return p.nt == 2 ? dispatch_mt<T, 2>(p, A, W, out, m_dev, m_cap, N, K, st)
                   : dispatch_mt<T, 1>(p, A, W, out, m_dev, m_cap, N, K, st);
}

}  // namespace

bool gemm_shape_ok(DType t, int N, int K) {
  const int kc = t == DType::F32 ? 128 : 256;   // skinny chunk; the fat slab divides it
  return N > 0 && K > 0 && N % 128 == 0 && K % kc == 0;
}

GemmPlan plan_gemm(DType t, int m_cap, int N, int K, int target_wgs) {
  GemmPlan p{};
  if (m_cap > 128) {
    p.kind = 1;
    p.mt = p.nt = 0;
    p.splits = 1;
    p.grid = ((N + 127) / 128) * ((m_cap + 127) / 128);
    return p;
  }
  p.kind = 0;
  p.mt = (m_cap + 15) / 16;
  if (p.mt < 1) p.mt = 1;
  const int kc = t == DType::F32 ? 128 : 256;
  const int chunks = K / kc;
  p.nt = (N / 128 >= target_wgs / 2) ? 2 : 1;
  const int n_tiles = N / (64 * p.nt);
  int s = (target_wgs + n_tiles - 1) / n_tiles;
  if (s < 1) s = 1;
  if (s > chunks) s = chunks;
  p.splits = s;
  p.grid = n_tiles * s;
  return p;
}

hipError_t launch_gemm(const GemmPlan& p, DType t, const void* A, const void* W, float* out,
                       const int* m_dev, int m_cap, int N, int K, hipStream_t st) {
  if (t == DType::F32) return dispatch<float>(p, A, W, out, m_dev, m_cap, N, K, st);
  return dispatch<bf16>(p, A, W, out, m_dev, m_cap, N, K, st);
}

}  // namespace dinfer
