// Standalone feature map phi: X [rows][D] (I/O type) -> Phi [rows][R] fp32.
//
// ELU(x)+1 (alpha = 1) and the identity are pointwise ("Choice of phi" on the
// linear-attention-kernel page; "Efficient attention variants" sec. 4), so the
// kernel is a pure stream: contiguous vector loads and 16-byte stores, grid
// stride, HBM-bound.
//
// FAVOR+ ("Efficient attention variants" sec. 6): x = u / D^(1/4),
// phi(u)_f = exp(w_f . x - |x|^2 / 2) / sqrt(R).  A workgroup keeps one omega
// row per thread in registers and walks a block of input rows staged in LDS.
#include "la_common.h"
#include "la_prefill.h"

namespace la {

// One group of 4 elements per lane and step: the loads (8 bytes per lane for
// bf16, 16 for fp32) and the 16-byte fp32 stores are both contiguous across
// the lanes of every instruction, so each instruction covers whole cache
// lines in both directions.
template <typename T, int PHI>
__global__ __launch_bounds__(kThreads) void la_phi_pointwise_kernel(const T* __restrict__ X,
                                                                    float* __restrict__ Y, long long n_quad) {
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  const long long stride = (long long)gridDim.x * kThreads;
  for (long long i = (long long)blockIdx.x * kThreads + threadIdx.x; i < n_quad; i += stride) {
    float f[4];
    if constexpr (sizeof(T) == 2) {
      const u32x2 u = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(X) + i);
      f[0] = bf16_lo(u.x); f[1] = bf16_hi(u.x);
      f[2] = bf16_lo(u.y); f[3] = bf16_hi(u.y);
    } else {
      const u32x4 u = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(X) + i);
      unpack16<float>(u, f);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) f[e] = phi_pointwise<PHI>(f[e]);
    __builtin_nontemporal_store(f32x4{f[0], f[1], f[2], f[3]}, reinterpret_cast<f32x4*>(Y) + i);
  }
}

template <typename T, int D, int R>
__global__ __launch_bounds__(kThreads) void la_phi_favor_kernel(const T* __restrict__ X, float* __restrict__ Y,
                                                                 long long rows,
                                                                 const float* __restrict__ omega) {
  static_assert(R % kThreads == 0, "one or more features per thread");
  constexpr int FPT = R / kThreads;  // features per thread
  constexpr int RB = 16;             // rows staged per step
  __shared__ float xs[RB][D];
  __shared__ float hs[RB];           // |x|^2 / 2 per staged row
  const int tid = threadIdx.x;
  float wreg[FPT][D];
#pragma unroll
  for (int j = 0; j < FPT; ++j)
#pragma unroll
    for (int i = 0; i < D; ++i) wreg[j][i] = omega[(size_t)(tid + j * kThreads) * D + i];
  const float scale = 1.0f / sqrtf(sqrtf(static_cast<float>(D)));
  const float inv_sqrt_r = 1.0f / sqrtf(static_cast<float>(R));
  for (long long r0 = (long long)blockIdx.x * RB; r0 < rows; r0 += (long long)gridDim.x * RB) {
    __syncthreads();
    for (int e = tid; e < RB * D; e += kThreads) {
      const long long row = r0 + e / D;
      float x = 0.f;
      if (row < rows) {
        if constexpr (sizeof(T) == 2) x = static_cast<float>(X[row * D + e % D]);
        else x = X[row * D + e % D];
      }
      xs[e / D][e % D] = x * scale;
    }
    __syncthreads();
    if (tid < RB) {
      float s = 0.f;
      for (int i = 0; i < D; ++i) s += xs[tid][i] * xs[tid][i];
      hs[tid] = 0.5f * s;
    }
    __syncthreads();
    for (int rr = 0; rr < RB; ++rr) {
      const long long row = r0 + rr;
      if (row >= rows) break;
#pragma unroll
      for (int j = 0; j < FPT; ++j) {
        float p = 0.f;
#pragma unroll
        for (int i = 0; i < D; ++i) p += wreg[j][i] * xs[rr][i];
        Y[row * R + tid + j * kThreads] = __expf(p - hs[rr]) * inv_sqrt_r;
      }
    }
  }
}

bool feature_supported(int io, int phi, int d, int r) {
  if (io != 0 && io != 1) return false;
  if (phi == PHI_FAVOR) return (d == 64 || d == 128) && r == 256;
  if (phi == PHI_ELU1 || phi == PHI_IDENTITY) return r == d && d % 8 == 0 && d > 0;
  return false;
}

template <typename T>
static hipError_t feature_io(const FeatureArgs& a) {
  hipStream_t st = static_cast<hipStream_t>(a.stream);
  if (a.rows == 0) return hipSuccess;
  (void)hipGetLastError();  // drop a stale error left by an unrelated earlier runtime call
  if (a.phi == PHI_FAVOR) {
    const long long blocks = (a.rows + 15) / 16;
    const int grid = static_cast<int>(blocks < 4096 ? blocks : 4096);
    if (a.d == 64)
      hipLaunchKernelGGL((la_phi_favor_kernel<T, 64, 256>), dim3(grid), dim3(kThreads), 0, st,
                         static_cast<const T*>(a.X), a.Y, a.rows, a.omega);
    else
      hipLaunchKernelGGL((la_phi_favor_kernel<T, 128, 256>), dim3(grid), dim3(kThreads), 0, st,
                         static_cast<const T*>(a.X), a.Y, a.rows, a.omega);
    return hipGetLastError();
  }
  const long long n_quad = a.rows * a.d / 4;
  const long long blocks = (n_quad + kThreads - 1) / kThreads;
  const int grid = static_cast<int>(blocks < 8192 ? blocks : 8192);
  if (a.phi == PHI_ELU1)
    hipLaunchKernelGGL((la_phi_pointwise_kernel<T, PHI_ELU1>), dim3(grid), dim3(kThreads), 0, st,
                       static_cast<const T*>(a.X), a.Y, n_quad);
  else
    hipLaunchKernelGGL((la_phi_pointwise_kernel<T, PHI_IDENTITY>), dim3(grid), dim3(kThreads), 0, st,
                       static_cast<const T*>(a.X), a.Y, n_quad);
  return hipGetLastError();
}

hipError_t feature_launch(const FeatureArgs& a) {
  return a.io == 1 ? feature_io<bf16>(a) : feature_io<float>(a);
}

}  // namespace la
