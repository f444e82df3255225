// One autoregressive decode step of causal kernelized linear attention.
//
// For every (batch, head) with state S [R][DV] (fp32) and z [R] (fp32) and a
// new token (q, k, v):
//   S' = S + phi(k) v^T,  z' = z + phi(k),  o = phi(q)^T S' / phi(q)^T z'
// ("Efficient attention variants" sec. 5: write the token first, then read;
// the state is O(R*DV) and a step costs O(R*DV) work).
// With a fixed per-head decay gamma ("Efficient attention variants" sec. 7.1)
// the old state is multiplied by gamma first: S' = gamma S + phi(k) v^T,
// z' = gamma z + phi(k); without one gamma = 1, which changes no bit.  With
// a per-token gate a ("Linear attention and SSM", Mamba-2 SSD section:
// A_t = a_t I) the same with a in place of gamma, given as log a per
// (batch, head); a gate under 2^-126 (zero included) acts as 2^-126, as in
// the gated prefill.  With normalize = 0 the read-out is phi(q)^T S' (no
// division).
//
// The step streams S once (read 4*R*DV bytes, write 4*R*DV bytes); its
// arithmetic intensity is ~0.5 flop/byte, so it is HBM-bound and runs on the
// vector ALUs.  One workgroup per (batch, head); a thread owns 4 consecutive
// value columns of every (256 / (DV/4))-th state row and keeps its partial
// read-out in registers; S' may alias S (every element is read and then
// written by the same thread), and z' may alias z.
#include "la_common.h"
#include "la_prefill.h"

namespace la {

template <typename T>
__device__ __forceinline__ float load_io(const T* p);
template <>
__device__ __forceinline__ float load_io<bf16>(const bf16* p) { return static_cast<float>(*p); }
template <>
__device__ __forceinline__ float load_io<float>(const float* p) { return *p; }

__device__ __forceinline__ float block_sum(float v, float* scratch) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) scratch[w] = v;
  __syncthreads();
  float t = 0.f;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) t += scratch[i];
  return t;
}

// Features of one input vector u (length D) into out[R] (LDS), fp32.
// FAVOR+ ("Efficient attention variants" sec. 6): x = u / D^(1/4),
// phi(u)_f = exp(w_f . x - |x|^2 / 2) / sqrt(R) with w_f the f-th row of omega.
// For the query (query_row) the row's constant exp(4 |x| - |x|^2 / 2) is
// taken out, exp(w_f . x - 4 |x|) / sqrt(R): it cancels in the normalised
// read-out (FAVOR+ decode is always normalised) and keeps phi(q) . S within
// fp32's range for queries of large norm, as in the prefill.
template <typename T, int D, int R, int PHI>
__device__ __forceinline__ void features_to_lds(const T* u, const float* __restrict__ omega, float* out,
                                                float* xbuf, float* scratch, bool query_row) {
  const int tid = threadIdx.x;
  if constexpr (PHI == PHI_FAVOR) {
    const float scale = 1.0f / sqrtf(sqrtf(static_cast<float>(D)));
    float sq = 0.f;
    for (int i = tid; i < D; i += kThreads) {
      const float x = load_io<T>(u + i) * scale;
      xbuf[i] = x;
      sq += x * x;
    }
    sq = block_sum(sq, scratch);  // contains a barrier: xbuf is visible after it
    const float inv_sqrt_r = 1.0f / sqrtf(static_cast<float>(R));
    const float shift = query_row ? 4.0f * sqrtf(sq) : 0.5f * sq;
    for (int f = tid; f < R; f += kThreads) {
      const float* wrow = omega + (size_t)f * D;
      float p = 0.f;
#pragma unroll 8
      for (int i = 0; i < D; ++i) p += wrow[i] * xbuf[i];
      out[f] = __expf(p - shift) * inv_sqrt_r;
    }
    __syncthreads();
  } else {
    for (int f = tid; f < R; f += kThreads) out[f] = phi_pointwise<PHI>(load_io<T>(u + f));
  }
}

template <typename T>
__device__ __forceinline__ void store_io(T* p, float x);
template <>
__device__ __forceinline__ void store_io<bf16>(bf16* p, float x) { *p = static_cast<bf16>(x); }
template <>
__device__ __forceinline__ void store_io<float>(float* p, float x) { *p = x; }

template <typename T, int D, int R, int DV, int PHI>
__global__ __launch_bounds__(kThreads) void la_decode_kernel(const float* S, const float* z,
                                                             const T* __restrict__ q, const T* __restrict__ k,
                                                             const T* __restrict__ v, T* __restrict__ o,
                                                             float* S_new, float* z_new,
                                                             const float* __restrict__ omega,
                                                             const float* __restrict__ gamma, int H,
                                                             int normalize, const float* __restrict__ log_a,
                                                             const float* __restrict__ log_a_ch) {
  constexpr int TPR = DV / 4;          // threads per state row
  constexpr int RPP = kThreads / TPR;  // rows per pass
  static_assert(R % RPP == 0, "state rows must split evenly");
  __shared__ float fq[R], fk[R], vv[DV], xbuf[D], gch[R];
  __shared__ float red[RPP * DV];
  __shared__ float scratch[2][kWaves];
  const int bh = blockIdx.x;
  const int tid = threadIdx.x;
  const float gm = log_a ? __builtin_amdgcn_exp2f(fmaxf(log_a[bh] * 1.4426950408889634f, -126.f))
                        : gamma ? gamma[bh % H] : 1.f;

  const int c4 = tid % TPR;
  const int r0 = tid / TPR;
  const float* Sh = S + (size_t)bh * R * DV + 4 * c4;
  float* Sn = S_new + (size_t)bh * R * DV + 4 * c4;
  // S_new may alias S, so every S load comes before the first store (a store
  // could not be moved above a later load, and the loads would serialise).
  // With a pointwise map S is requested first and the token's few loads and
  // its features overlap the S stream: one round trip to memory, not two.
  // FAVOR+ forms its features from omega first and requests S after them.
  constexpr bool EARLY = PHI != PHI_FAVOR && R <= kThreads && DV <= kThreads;
  f32x4 s[R / RPP];
  auto load_state = [&]() {
#pragma unroll
    for (int it = 0; it < R / RPP; ++it)
      s[it] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(Sh + (size_t)(r0 + it * RPP) * DV));
  };
  float zx = 0.f;  // pointwise maps: z[tid] (state row f = tid, tid < R)
  if constexpr (EARLY) {
    load_state();
    // every thread loads (rows and columns wrapped), with no branch around
    // the loads
    const int f = tid % R, c = tid % DV;
    const T qr = q[(size_t)bh * D + f], kr = k[(size_t)bh * D + f], vr = v[(size_t)bh * DV + c];
    const float ar = (log_a_ch ? log_a_ch : z)[(size_t)bh * R + f];
    zx = z[(size_t)bh * R + f];
    if (tid < R) {
      fq[tid] = phi_pointwise<PHI>(static_cast<float>(qr));
      fk[tid] = phi_pointwise<PHI>(static_cast<float>(kr));
      // per-channel gates (state row f keeps a_f of itself; the floor of the
      // per-channel gated prefill, log2 a >= -14)
      gch[tid] = log_a_ch ? __builtin_amdgcn_exp2f(fmaxf(ar * 1.4426950408889634f, -14.f)) : gm;
    }
    if (tid < DV) vv[tid] = static_cast<float>(vr);
  } else {
    features_to_lds<T, D, R, PHI>(q + (size_t)bh * D, omega, fq, xbuf, scratch[0], true);
    features_to_lds<T, D, R, PHI>(k + (size_t)bh * D, omega, fk, xbuf, scratch[1], false);
    for (int c = tid; c < DV; c += kThreads) vv[c] = load_io<T>(v + (size_t)bh * DV + c);
    for (int f = tid; f < R; f += kThreads)
      gch[f] = log_a_ch ? __builtin_amdgcn_exp2f(fmaxf(log_a_ch[(size_t)bh * R + f] * 1.4426950408889634f, -14.f))
                        : gm;
  }
  __syncthreads();
  if constexpr (!EARLY) load_state();
  const f32x4 v4 = f32x4{vv[4 * c4], vv[4 * c4 + 1], vv[4 * c4 + 2], vv[4 * c4 + 3]};
  f32x4 num = zero4();
#pragma unroll
  for (int it = 0; it < R / RPP; ++it) {
    const int f = r0 + it * RPP;
    s[it] = s[it] * gch[f] + fk[f] * v4;
    __builtin_nontemporal_store(s[it], reinterpret_cast<f32x4*>(Sn + (size_t)f * DV));
    num += fq[f] * s[it];
  }
  red[r0 * DV + 4 * c4 + 0] = num[0];
  red[r0 * DV + 4 * c4 + 1] = num[1];
  red[r0 * DV + 4 * c4 + 2] = num[2];
  red[r0 * DV + 4 * c4 + 3] = num[3];

  float dpart = 0.f;
  for (int f = tid; f < R; f += kThreads) {
    const float zn = (EARLY ? zx : z[(size_t)bh * R + f]) * gch[f] + fk[f];
    z_new[(size_t)bh * R + f] = zn;
    dpart += fq[f] * zn;
  }
  const float den = block_sum(dpart, scratch[0] /* reused after the barrier above */);

  for (int c = tid; c < DV; c += kThreads) {
    float n = 0.f;
#pragma unroll
    for (int rr = 0; rr < RPP; ++rr) n += red[rr * DV + c];
    store_io<T>(o + (size_t)bh * DV + c, normalize ? n / den : n);
  }
}

template <typename T, int D, int R, int DV, int PHI>
static hipError_t launch_decode(const DecodeArgs& a) {
  const int BH = a.B * a.H;
  if (BH == 0) return hipSuccess;
  (void)hipGetLastError();  // drop a stale error left by an unrelated earlier runtime call
  hipLaunchKernelGGL((la_decode_kernel<T, D, R, DV, PHI>), dim3(BH), dim3(kThreads), 0,
                     static_cast<hipStream_t>(a.stream), a.S, a.z, static_cast<const T*>(a.q),
                     static_cast<const T*>(a.k), static_cast<const T*>(a.v), static_cast<T*>(a.o), a.S_new,
                     a.z_new, a.omega, a.gamma, a.H > 0 ? a.H : 1, a.normalize, a.log_a, a.log_a_ch);
  return hipGetLastError();
}

template <typename T, int PHI>
static hipError_t decode_dims(const DecodeArgs& a) {
  if constexpr (PHI == PHI_FAVOR) {
    if (a.d == 64 && a.r == 256 && a.dv == 64) return launch_decode<T, 64, 256, 64, PHI>(a);
    if (a.d == 128 && a.r == 256 && a.dv == 128) return launch_decode<T, 128, 256, 128, PHI>(a);
  } else {
    if (a.d == 64 && a.dv == 64) return launch_decode<T, 64, 64, 64, PHI>(a);
    if (a.d == 128 && a.dv == 128) return launch_decode<T, 128, 128, 128, PHI>(a);
  }
  return hipErrorInvalidValue;
}

bool decode_supported(int io, int phi, int d, int dv, int r) {
  if (io != 0 && io != 1) return false;
  if (phi == PHI_FAVOR) return r == 256 && ((d == 64 && dv == 64) || (d == 128 && dv == 128));
  if (phi == PHI_ELU1 || phi == PHI_IDENTITY) return r == d && d == dv && (d == 64 || d == 128);
  return false;
}

hipError_t decode_launch(const DecodeArgs& a) {
  if (a.io == 1) {
    if (a.phi == PHI_ELU1) return decode_dims<bf16, PHI_ELU1>(a);
    if (a.phi == PHI_IDENTITY) return decode_dims<bf16, PHI_IDENTITY>(a);
    return decode_dims<bf16, PHI_FAVOR>(a);
  }
  if (a.phi == PHI_ELU1) return decode_dims<float, PHI_ELU1>(a);
  if (a.phi == PHI_IDENTITY) return decode_dims<float, PHI_IDENTITY>(a);
  return decode_dims<float, PHI_FAVOR>(a);
}

}  // namespace la
