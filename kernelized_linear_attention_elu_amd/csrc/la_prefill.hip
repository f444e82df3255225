// Chunkwise prefill of causal (and non-causal) kernelized linear attention
// for gfx950.
//
// What is computed (per batch*head, tokens t = 0..N-1):
//   S_t = S_{t-1} + phi(k_t) v_t^T,  z_t = z_{t-1} + phi(k_t),
//   o_t = phi(q_t)^T S_t / phi(q_t)^T z_t,
// i.e. the recurrence of "Efficient attention variants" sec. 5 (and the
// "Recurrent form" section of the linear-attention-kernel page), evaluated
// chunkwise as sec. 8 of the same page describes: inside a chunk of C tokens
// the masked weights phi(Q_c) phi(K_c)^T (diagonal kept) are applied
// directly; across chunks the history enters through the running state.
// Non-causal mode uses the full-sequence sums S, z of sec. 4.
//
// Three kernels, one workgroup per (head, span of L tokens):
//   la_state_kernel  - dS_span = phi(K_span)^T V_span, dz_span = sum phi(K_span)
//                      (bf16 MFMA, fp32 accumulation) -> workspace;
//   la_scan_kernel   - fp32 exclusive prefix of (dS, dz) over spans, plus the
//                      total (final state / non-causal sums);
//   la_output_kernel - walks its span chunk by chunk carrying (S, z) in
//                      registers: per chunk the masked intra-chunk product,
//                      the read-out of the carried state, the denominator and
//                      the divide, then the state update.
//
// Data layout: Q, K [B*H][N][D], V, O [B*H][N][DV] (I/O type T), workspace
// fp32 [B*H][n_span+1][R*DV + R] holding S (row-major [R][DV]) then z.
#include "la_common.h"
#include "la_prefill.h"

namespace la {

template <typename T, int D_, int R_, int DV_, int C_, int PHI_>
struct Cfg {
  using IO = T;
  using OP = T;                               // MFMA operand type
  static constexpr int D = D_, R = R_, DV = DV_, C = C_, PHI = PHI_;
  static constexpr int EPL = Vec16<T>::N;     // elements per 16-byte vector
  static constexpr int PAD = EPL;             // LDS row padding (elements)
  static constexpr int QS = R + PAD;          // row stride of phi(Q), phi(K)  [C][QS]
  static constexpr int TS = C + PAD;          // row stride of phi(K)^T, V^T   [R][TS], [DV][TS]
  static constexpr int SS = R + PAD;          // row stride of the state copy  [DV][SS]
  static constexpr int KS = Op<OP>::K;
  static constexpr int PL = Op<OP>::PL;
  static constexpr int RB = C / 16;           // 16-token row blocks per chunk
  static constexpr int CT = DV / 16;          // 16-wide value-column tiles
  static constexpr int FT = R / 16;           // 16-wide feature tiles
  static constexpr int NTILE = CT * FT;       // 16x16 tiles of the state
  static constexpr int TPW = NTILE / kWaves;  // state tiles owned per wave
  static constexpr int VQ = C * D / EPL;      // 16-byte vectors of one Q/K chunk
  static constexpr int VV = C * DV / EPL;     // ... of one V chunk
  static constexpr int LQ = (VQ + kThreads - 1) / kThreads;
  static constexpr int LV = (VV + kThreads - 1) / kThreads;
  static constexpr int ZPT = (R * 4 + kThreads - 1) / kThreads;  // z partial sums per thread
  // causal output work split: waves per row block, row blocks per wave,
  // value-column tiles per wave
  static constexpr int WPR = RB >= kWaves ? 1 : kWaves / RB;
  static constexpr int RBW = RB >= kWaves ? RB / kWaves : 1;
  static constexpr int CTW = CT / WPR;
  static_assert(R == D, "pointwise feature maps keep the dimension");
  static_assert(NTILE % kWaves == 0, "state tiles must split evenly over waves");
  static_assert(C % 16 == 0 && C <= 128, "chunk must be 16, 32, 64 or 128");
  static_assert(CT % WPR == 0, "value tiles must split over the waves of a row block");
  static_assert((R * 4) % kThreads == 0 || R * 4 < kThreads, "z partial layout");
};

// ------------------------------------------------------------------ staging

template <class CF, bool WITH_Q>
struct ChunkRegs {
  u32x4 q[WITH_Q ? CF::LQ : 1];
  u32x4 k[CF::LQ];
  u32x4 v[CF::LV];
};

// Global -> registers for the chunk starting at token t0 (zero beyond N).
template <class CF, bool WITH_Q>
__device__ __forceinline__ void load_chunk(ChunkRegs<CF, WITH_Q>& cr, const typename CF::IO* Qh,
                                           const typename CF::IO* Kh, const typename CF::IO* Vh,
                                           int t0, int N) {
  using T = typename CF::IO;
  const int tid = threadIdx.x;
  constexpr int QV = CF::D / CF::EPL;   // vectors per Q/K row
  constexpr int VVR = CF::DV / CF::EPL; // vectors per V row
#pragma unroll
  for (int i = 0; i < CF::LQ; ++i) {
    const int vi = tid + i * kThreads;
    u32x4 kq = u32x4{0, 0, 0, 0}, qq = u32x4{0, 0, 0, 0};
    if (vi < CF::VQ) {
      const int t = t0 + vi / QV;
      const int col = (vi % QV) * CF::EPL;
      if (t < N) {
        kq = *reinterpret_cast<const u32x4*>(Kh + (size_t)t * CF::D + col);
        if constexpr (WITH_Q) qq = *reinterpret_cast<const u32x4*>(Qh + (size_t)t * CF::D + col);
      }
    }
    cr.k[i] = kq;
    if constexpr (WITH_Q) cr.q[i] = qq;
  }
#pragma unroll
  for (int i = 0; i < CF::LV; ++i) {
    const int vi = tid + i * kThreads;
    u32x4 vv = u32x4{0, 0, 0, 0};
    if (vi < CF::VV) {
      const int t = t0 + vi / VVR;
      const int col = (vi % VVR) * CF::EPL;
      if (t < N) vv = *reinterpret_cast<const u32x4*>(Vh + (size_t)t * CF::DV + col);
    }
    cr.v[i] = vv;
  }
  (void)sizeof(T);
}

// Registers -> LDS: applies phi to Q and K (fp32), rounds to the operand
// type, writes phi(Q), phi(K) row-major (if WITH_Q) and phi(K)^T, V^T
// (token-contiguous rows).  Keys beyond N get zero features so that they add
// nothing to the state.
template <class CF, bool WITH_Q>
__device__ __forceinline__ void stage_chunk(const ChunkRegs<CF, WITH_Q>& cr, typename CF::OP* sq,
                                            typename CF::OP* sk, typename CF::OP* skt,
                                            typename CF::OP* svt, int t0, int N) {
  using T = typename CF::IO;
  using OP = typename CF::OP;
  const int tid = threadIdx.x;
  constexpr int QV = CF::D / CF::EPL;
  constexpr int VVR = CF::DV / CF::EPL;
#pragma unroll
  for (int i = 0; i < CF::LQ; ++i) {
    const int vi = tid + i * kThreads;
    if (vi < CF::VQ) {
      const int tok = vi / QV;
      const int col = (vi % QV) * CF::EPL;
      const bool valid = t0 + tok < N;
      float f[CF::EPL];
      if constexpr (WITH_Q) {
        unpack16<T>(cr.q[i], f);
#pragma unroll
        for (int e = 0; e < CF::EPL; ++e) f[e] = phi_pointwise<CF::PHI>(f[e]);
        *reinterpret_cast<u32x4*>(sq + tok * CF::QS + col) = pack16<OP>(f);
      }
      unpack16<T>(cr.k[i], f);
#pragma unroll
      for (int e = 0; e < CF::EPL; ++e) f[e] = valid ? phi_pointwise<CF::PHI>(f[e]) : 0.f;
      if constexpr (WITH_Q) *reinterpret_cast<u32x4*>(sk + tok * CF::QS + col) = pack16<OP>(f);
#pragma unroll
      for (int e = 0; e < CF::EPL; ++e) skt[(col + e) * CF::TS + tok] = to_op<OP>(f[e]);
    }
  }
#pragma unroll
  for (int i = 0; i < CF::LV; ++i) {
    const int vi = tid + i * kThreads;
    if (vi < CF::VV) {
      const int tok = vi / VVR;
      const int col = (vi % VVR) * CF::EPL;
      float f[CF::EPL];
      unpack16<T>(cr.v[i], f);
#pragma unroll
      for (int e = 0; e < CF::EPL; ++e) svt[(col + e) * CF::TS + tok] = to_op<OP>(f[e]);
    }
  }
}

// ------------------------------------------------------------------ state update

// acc[i] += V_c^T phi(K_c) for the state tiles this wave owns.  Tile i of wave
// w is t = w + 4 i with value tile ct = t % CT and feature tile ft = t / CT;
// lane (g, li) ends up holding S[f = 16 ft + li][c = 16 ct + 4 g + r].
template <class CF>
__device__ __forceinline__ void state_mfma(f32x4 (&acc)[CF::TPW], const typename CF::OP* skt,
                                           const typename CF::OP* svt, int w, int g, int li) {
  using OP = typename CF::OP;
#pragma unroll
  for (int i = 0; i < CF::TPW; ++i) {
    const int t = w + kWaves * i;
    const int ct = t % CF::CT;
    const int ft = t / CF::CT;
    const OP* arow = svt + (16 * ct + li) * CF::TS;
    const OP* brow = skt + (16 * ft + li) * CF::TS;
    if constexpr (sizeof(OP) == 2) {
      if constexpr (CF::C % 32 == 0) {
#pragma unroll
        for (int ks = 0; ks < CF::C / 32; ++ks)
          acc[i] = mfma16(load_frag(arow + ks * 32 + 8 * g), load_frag(brow + ks * 32 + 8 * g), acc[i]);
      } else {  // C == 16: tokens 4g..4g+3 in the low half, zeros above
        const bf16x4 a4 = *reinterpret_cast<const bf16x4*>(arow + 4 * g);
        const bf16x4 b4 = *reinterpret_cast<const bf16x4*>(brow + 4 * g);
        const bf16x4 z4 = bf16x4{0, 0, 0, 0};
        acc[i] = mfma16(__builtin_shufflevector(a4, z4, 0, 1, 2, 3, 4, 5, 6, 7),
                        __builtin_shufflevector(b4, z4, 0, 1, 2, 3, 4, 5, 6, 7), acc[i]);
      }
    } else {
#pragma unroll
      for (int ks = 0; ks < CF::C / 4; ++ks) acc[i] = mfma16(arow[ks * 4 + g], brow[ks * 4 + g], acc[i]);
    }
  }
}

// zacc[j] += sum over the chunk's tokens of phi(k)[f] for the features this
// thread tracks: entry idx = tid + 256 j covers feature f = idx / 4, token
// quarter idx % 4; the four quarter sums are combined inside the quad, so
// every lane of the quad holds the full chunk sum for f.
template <class CF>
__device__ __forceinline__ void z_partial(float (&zacc)[CF::ZPT], const typename CF::OP* skt) {
  constexpr int QT = CF::C / 4;
#pragma unroll
  for (int j = 0; j < CF::ZPT; ++j) {
    const int idx = threadIdx.x + j * kThreads;
    const int f = idx >> 2;
    const int p = idx & 3;
    float s = 0.f;
    if (f < CF::R) {
#pragma unroll
      for (int t = 0; t < QT; ++t) s += from_op(skt[f * CF::TS + p * QT + t]);
    }
    s += __shfl_xor(s, 1);
    s += __shfl_xor(s, 2);
    zacc[j] += s;
  }
}

// ------------------------------------------------------------------ outputs

// Output rows of one chunk.  For row block ib (query tokens 16 ib .. +15):
//  * weights: tiles a[jb] = phi(K_jb) phi(Q_ib)^T for key blocks jb <= ib;
//    lane (g, li) holds A[i = li][j = 16 jb + 4 g + r]; the diagonal block is
//    masked to j <= i by selection (never by multiplication, so non-finite
//    future values cannot leak);
//  * numerator O^T = V^T A^T + S^T phi(Q)^T (MFMA), where the accumulator row
//    m of value tile ct maps to value column (DV/4)(m/4) + 4 ct + m%4, so that
//    every lane ends with 4*CTW consecutive columns of one row;
//  * denominator = rowsum(A) + phi(q_i).z  (fp32), then one divide per value.
// The weights and phi(Q) enter both sums exactly as rounded for the MFMA.
template <class CF, bool CAUSAL>
__device__ __forceinline__ void chunk_outputs(const typename CF::OP* sq, const typename CF::OP* sk,
                                              const typename CF::OP* svt, const typename CF::OP* sst,
                                              const float* sz, typename CF::IO* Oh, int t0, int N, int w,
                                              int g, int li) {
  using OP = typename CF::OP;
  using T = typename CF::IO;
  using frag = typename Op<OP>::frag;
  constexpr int KS = CF::KS, PL = CF::PL, RB = CF::RB, CTW = CF::CTW;
#pragma unroll
  for (int rbi = 0; rbi < CF::RBW; ++rbi) {
    const int ib = (RB >= kWaves) ? (w + kWaves * rbi) : (w % RB);
    const int ct0 = (RB >= kWaves) ? 0 : (w / RB) * CTW;
    frag qf[CF::R / KS];
#pragma unroll
    for (int ks = 0; ks < CF::R / KS; ++ks) qf[ks] = load_frag(sq + (16 * ib + li) * CF::QS + ks * KS + g * PL);

    float den = 0.f;
#pragma unroll
    for (int ks = 0; ks < CF::R / KS; ++ks) {
      if constexpr (PL == 1) {
        den += qf[ks] * sz[ks * KS + g];
      } else {
#pragma unroll
        for (int e = 0; e < PL; ++e) den += static_cast<float>(qf[ks][e]) * sz[ks * KS + g * PL + e];
      }
    }

    f32x4 o[CTW];
#pragma unroll
    for (int c = 0; c < CTW; ++c) o[c] = zero4();

    if constexpr (CAUSAL) {
      f32x4 a[RB];
#pragma unroll
      for (int jb = 0; jb < RB; ++jb) {
        a[jb] = zero4();
        if (jb <= ib) {
#pragma unroll
          for (int ks = 0; ks < CF::R / KS; ++ks)
            a[jb] = mfma16(load_frag(sk + (16 * jb + li) * CF::QS + ks * KS + g * PL), qf[ks], a[jb]);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float x = a[jb][r];
            x = (jb == ib && 4 * g + r > li) ? 0.f : x;
            x = round_op<OP>(x);
            a[jb][r] = x;
            den += x;
          }
        }
      }
#pragma unroll
      for (int cti = 0; cti < CTW; ++cti) {
        const int ct = ct0 + cti;
        const int c = (CF::DV / 4) * (li >> 2) + 4 * ct + (li & 3);
        const OP* vrow = svt + c * CF::TS;
        if constexpr (PL == 8) {
#pragma unroll
          for (int jp = 0; jp < (RB + 1) / 2; ++jp) {
            const int jb0 = 2 * jp, jb1 = 2 * jp + 1;
            if (jb0 <= ib) {
              const bf16x4 alo = *reinterpret_cast<const bf16x4*>(vrow + 16 * jb0 + 4 * g);
              const bf16x4 blo = bf16x4{to_op<bf16>(a[jb0][0]), to_op<bf16>(a[jb0][1]),
                                        to_op<bf16>(a[jb0][2]), to_op<bf16>(a[jb0][3])};
              bf16x4 ahi = bf16x4{0, 0, 0, 0}, bhi = bf16x4{0, 0, 0, 0};
              if (jb1 < RB && jb1 <= ib) {
                ahi = *reinterpret_cast<const bf16x4*>(vrow + 16 * jb1 + 4 * g);
                bhi = bf16x4{to_op<bf16>(a[jb1][0]), to_op<bf16>(a[jb1][1]), to_op<bf16>(a[jb1][2]),
                             to_op<bf16>(a[jb1][3])};
              }
              o[cti] = mfma16(__builtin_shufflevector(alo, ahi, 0, 1, 2, 3, 4, 5, 6, 7),
                              __builtin_shufflevector(blo, bhi, 0, 1, 2, 3, 4, 5, 6, 7), o[cti]);
            }
          }
        } else {
#pragma unroll
          for (int jb = 0; jb < RB; ++jb) {
            if (jb <= ib) {
#pragma unroll
              for (int r = 0; r < 4; ++r) o[cti] = mfma16(vrow[16 * jb + 4 * g + r], a[jb][r], o[cti]);
            }
          }
        }
      }
    }

    den = xor_sum16_32(den);

#pragma unroll
    for (int cti = 0; cti < CTW; ++cti) {
      const int ct = ct0 + cti;
      const int c = (CF::DV / 4) * (li >> 2) + 4 * ct + (li & 3);
      const OP* srow = sst + c * CF::SS;
#pragma unroll
      for (int ks = 0; ks < CF::R / KS; ++ks) o[cti] = mfma16(load_frag(srow + ks * KS + g * PL), qf[ks], o[cti]);
    }

    const int tok = t0 + 16 * ib + li;
    if (tok < N) {
      float vals[4 * CTW];
#pragma unroll
      for (int cti = 0; cti < CTW; ++cti)
#pragma unroll
        for (int r = 0; r < 4; ++r) vals[4 * cti + r] = o[cti][r] / den;
      T* dst = Oh + (size_t)tok * CF::DV + (CF::DV / 4) * g + 4 * ct0;
      constexpr int NV = 4 * CTW;                 // values per lane
      if constexpr (NV % CF::EPL == 0) {
#pragma unroll
        for (int vv = 0; vv < NV / CF::EPL; ++vv)
          *reinterpret_cast<u32x4*>(dst + vv * CF::EPL) = pack16<T>(vals + vv * CF::EPL);
      } else {  // bf16 with 4 values per lane
        const bf16x4 h = bf16x4{to_op<bf16>(vals[0]), to_op<bf16>(vals[1]), to_op<bf16>(vals[2]),
                                to_op<bf16>(vals[3])};
        *reinterpret_cast<bf16x4*>(dst) = h;
      }
    }
  }
}

// ------------------------------------------------------------------ kernels

template <class CF>
struct SmemState {
  typename CF::OP kt[CF::R * CF::TS];
  typename CF::OP vt[CF::DV * CF::TS];
};

template <class CF>
struct SmemOut {
  typename CF::OP q[CF::C * CF::QS];
  typename CF::OP k[CF::C * CF::QS];
  typename CF::OP kt[CF::R * CF::TS];
  typename CF::OP vt[CF::DV * CF::TS];
  typename CF::OP st[CF::DV * CF::SS];
  float z[CF::R];
};

// Per-span state: dS = phi(K_span)^T V_span, dz = sum phi(K_span) -> ws slot s.
template <class CF>
__global__ __launch_bounds__(kThreads) void la_state_kernel(const typename CF::IO* __restrict__ K,
                                                            const typename CF::IO* __restrict__ V,
                                                            float* __restrict__ ws, int N, int span,
                                                            int n_span) {
  __shared__ SmemState<CF> sm;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, g = l >> 4, li = l & 15;
  const int bh = blockIdx.x / n_span;
  const int s = blockIdx.x % n_span;
  const int t_begin = s * span;
  const int t_end = min(t_begin + span, N);
  const typename CF::IO* Kh = K + (size_t)bh * N * CF::D;
  const typename CF::IO* Vh = V + (size_t)bh * N * CF::DV;

  f32x4 acc[CF::TPW];
#pragma unroll
  for (int i = 0; i < CF::TPW; ++i) acc[i] = zero4();
  float zacc[CF::ZPT];
#pragma unroll
  for (int j = 0; j < CF::ZPT; ++j) zacc[j] = 0.f;

  ChunkRegs<CF, false> cr;
  load_chunk<CF, false>(cr, nullptr, Kh, Vh, t_begin, N);
  for (int t0 = t_begin; t0 < t_end; t0 += CF::C) {
    __syncthreads();
    stage_chunk<CF, false>(cr, nullptr, nullptr, sm.kt, sm.vt, t0, N);
    __syncthreads();
    if (t0 + CF::C < t_end) load_chunk<CF, false>(cr, nullptr, Kh, Vh, t0 + CF::C, N);
    state_mfma<CF>(acc, sm.kt, sm.vt, w, g, li);
    z_partial<CF>(zacc, sm.kt);
  }

  constexpr int E = CF::R * CF::DV + CF::R;
  float* slot = ws + ((size_t)bh * (n_span + 1) + s) * E;
#pragma unroll
  for (int i = 0; i < CF::TPW; ++i) {
    const int t = w + kWaves * i;
    const int ct = t % CF::CT, ft = t / CF::CT;
    *reinterpret_cast<f32x4*>(slot + (16 * ft + li) * CF::DV + 16 * ct + 4 * g) = acc[i];
  }
#pragma unroll
  for (int j = 0; j < CF::ZPT; ++j) {
    const int idx = tid + j * kThreads;
    if ((idx & 3) == 0 && (idx >> 2) < CF::R) slot[CF::R * CF::DV + (idx >> 2)] = zacc[j];
  }
}

// Exclusive fp32 prefix over spans, element-parallel: slot s becomes the
// state before span s (starting from S0/z0 or zero); slot n_span receives
// the total, which is also copied to S_out/z_out when given.  The summation
// order is fixed, so results are reproducible.
__global__ __launch_bounds__(kThreads) void la_scan_kernel(float* __restrict__ ws, int R, int DV, int n_span,
                                                           const float* __restrict__ S0,
                                                           const float* __restrict__ z0,
                                                           float* __restrict__ S_out,
                                                           float* __restrict__ z_out) {
  const int E = R * DV + R;
  const int e = blockIdx.x * kThreads + threadIdx.x;
  const int bh = blockIdx.y;
  if (e >= E) return;
  const bool is_s = e < R * DV;
  float acc = 0.f;
  if (is_s) {
    if (S0) acc = S0[(size_t)bh * R * DV + e];
  } else {
    if (z0) acc = z0[(size_t)bh * R + (e - R * DV)];
  }
  float* p = ws + (size_t)bh * (n_span + 1) * E + e;
  int s = 0;
  for (; s + 4 <= n_span; s += 4) {
    const float x0 = p[(size_t)(s + 0) * E], x1 = p[(size_t)(s + 1) * E];
    const float x2 = p[(size_t)(s + 2) * E], x3 = p[(size_t)(s + 3) * E];
    p[(size_t)(s + 0) * E] = acc; acc += x0;
    p[(size_t)(s + 1) * E] = acc; acc += x1;
    p[(size_t)(s + 2) * E] = acc; acc += x2;
    p[(size_t)(s + 3) * E] = acc; acc += x3;
  }
  for (; s < n_span; ++s) {
    const float x = p[(size_t)s * E];
    p[(size_t)s * E] = acc;
    acc += x;
  }
  p[(size_t)n_span * E] = acc;
  if (is_s) {
    if (S_out) S_out[(size_t)bh * R * DV + e] = acc;
  } else {
    if (z_out) z_out[(size_t)bh * R + (e - R * DV)] = acc;
  }
}

// Outputs of one span, carrying (S, z) from the span's prefix (causal) or
// reading the full-sequence sums (non-causal).
template <class CF, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void la_output_kernel(const typename CF::IO* __restrict__ Q,
                                                             const typename CF::IO* __restrict__ K,
                                                             const typename CF::IO* __restrict__ V,
                                                             typename CF::IO* __restrict__ O,
                                                             const float* __restrict__ ws, int N, int span,
                                                             int n_span) {
  using OP = typename CF::OP;
  __shared__ SmemOut<CF> sm;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, g = l >> 4, li = l & 15;
  const int bh = blockIdx.x / n_span;
  const int s = blockIdx.x % n_span;
  const int t_begin = s * span;
  const int t_end = min(t_begin + span, N);
  const typename CF::IO* Qh = Q + (size_t)bh * N * CF::D;
  const typename CF::IO* Kh = K + (size_t)bh * N * CF::D;
  const typename CF::IO* Vh = V + (size_t)bh * N * CF::DV;
  typename CF::IO* Oh = O + (size_t)bh * N * CF::DV;

  // carried state: this wave's tiles of S (fp32) and this thread's z entries
  constexpr int E = CF::R * CF::DV + CF::R;
  const float* pre = ws + ((size_t)bh * (n_span + 1) + (CAUSAL ? s : n_span)) * E;
  f32x4 sacc[CF::TPW];
#pragma unroll
  for (int i = 0; i < CF::TPW; ++i) {
    const int t = w + kWaves * i;
    const int ct = t % CF::CT, ft = t / CF::CT;
    sacc[i] = *reinterpret_cast<const f32x4*>(pre + (16 * ft + li) * CF::DV + 16 * ct + 4 * g);
  }
  float zacc[CF::ZPT];
#pragma unroll
  for (int j = 0; j < CF::ZPT; ++j) {
    const int f = (tid + j * kThreads) >> 2;
    zacc[j] = f < CF::R ? pre[CF::R * CF::DV + f] : 0.f;
  }

  ChunkRegs<CF, true> cr;
  load_chunk<CF, true>(cr, Qh, Kh, Vh, t_begin, N);
  bool first = true;
  for (int t0 = t_begin; t0 < t_end; t0 += CF::C) {
    // publish the carried state as an MFMA operand (and z for the divide)
    if (CAUSAL || first) {
#pragma unroll
      for (int i = 0; i < CF::TPW; ++i) {
        const int t = w + kWaves * i;
        const int ct = t % CF::CT, ft = t / CF::CT;
#pragma unroll
        for (int r = 0; r < 4; ++r) sm.st[(16 * ct + 4 * g + r) * CF::SS + 16 * ft + li] = to_op<OP>(sacc[i][r]);
      }
#pragma unroll
      for (int j = 0; j < CF::ZPT; ++j) {
        const int idx = tid + j * kThreads;
        if ((idx & 3) == 0 && (idx >> 2) < CF::R) sm.z[idx >> 2] = zacc[j];
      }
    }
    first = false;
    stage_chunk<CF, true>(cr, sm.q, sm.k, sm.kt, sm.vt, t0, N);
    __syncthreads();
    if (t0 + CF::C < t_end) load_chunk<CF, true>(cr, Qh, Kh, Vh, t0 + CF::C, N);
    chunk_outputs<CF, CAUSAL>(sm.q, sm.k, sm.vt, sm.st, sm.z, Oh, t0, N, w, g, li);
    if constexpr (CAUSAL) {
      state_mfma<CF>(sacc, sm.kt, sm.vt, w, g, li);
      z_partial<CF>(zacc, sm.kt);
    }
    __syncthreads();
  }
}

// ------------------------------------------------------------------ launcher

template <class CF>
static hipError_t launch_prefill(const PrefillArgs& a) {
  using T = typename CF::IO;
  const T* Q = static_cast<const T*>(a.Q);
  const T* K = static_cast<const T*>(a.K);
  const T* V = static_cast<const T*>(a.V);
  T* O = static_cast<T*>(a.O);
  float* ws = static_cast<float*>(a.workspace);
  const int BH = a.B * a.H;
  hipStream_t st = static_cast<hipStream_t>(a.stream);
  const int n_span = a.n_span;
  const int E = CF::R * CF::DV + CF::R;

  auto rec = [&](int i) {
    if (a.events && a.events[i]) (void)hipEventRecord(static_cast<hipEvent_t>(a.events[i]), st);
  };
  rec(0);
  if (n_span > 0 && BH > 0) {
    hipLaunchKernelGGL((la_state_kernel<CF>), dim3(BH * n_span), dim3(kThreads), 0, st, K, V, ws, a.N, a.span,
                       n_span);
  }
  rec(1);
  rec(2);
  if (BH > 0) {
    hipLaunchKernelGGL(la_scan_kernel, dim3((E + kThreads - 1) / kThreads, BH), dim3(kThreads), 0, st, ws, CF::R,
                       CF::DV, n_span, a.S0, a.z0, a.S_out, a.z_out);
  }
  rec(3);
  rec(4);
  if (n_span > 0 && BH > 0) {
    if (a.causal)
      hipLaunchKernelGGL((la_output_kernel<CF, true>), dim3(BH * n_span), dim3(kThreads), 0, st, Q, K, V, O, ws,
                         a.N, a.span, n_span);
    else
      hipLaunchKernelGGL((la_output_kernel<CF, false>), dim3(BH * n_span), dim3(kThreads), 0, st, Q, K, V, O, ws,
                         a.N, a.span, n_span);
  }
  rec(5);
  return hipGetLastError();
}

template <typename T, int D, int PHI>
static hipError_t dispatch_chunk(const PrefillArgs& a) {
  switch (a.chunk) {
    case 16: return launch_prefill<Cfg<T, D, D, D, 16, PHI>>(a);
    case 32: return launch_prefill<Cfg<T, D, D, D, 32, PHI>>(a);
    case 64: return launch_prefill<Cfg<T, D, D, D, 64, PHI>>(a);
    case 128:
      if constexpr (sizeof(T) == 2 && D == 64) return launch_prefill<Cfg<T, D, D, D, 128, PHI>>(a);
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
}

bool prefill_supported(int io, int phi, int d, int dv, int r, int chunk) {
  if (phi != PHI_ELU1 && phi != PHI_IDENTITY) return false;
  if (r != d || dv != d) return false;
  if (chunk != 16 && chunk != 32 && chunk != 64 && chunk != 128) return false;
  if (io == 1) {  // bf16
    if (d == 64) return true;
    if (d == 128) return chunk <= 64;
    return false;
  }
  if (io == 0) return d == 64 && chunk <= 64;  // fp32
  return false;
}

hipError_t prefill_launch(const PrefillArgs& a) {
  if (a.io == 1) {
    if (a.d == 64) return a.phi == PHI_ELU1 ? dispatch_chunk<bf16, 64, PHI_ELU1>(a) : dispatch_chunk<bf16, 64, PHI_IDENTITY>(a);
    if (a.d == 128)
      return a.phi == PHI_ELU1 ? dispatch_chunk<bf16, 128, PHI_ELU1>(a) : dispatch_chunk<bf16, 128, PHI_IDENTITY>(a);
  } else {
    if (a.d == 64) return a.phi == PHI_ELU1 ? dispatch_chunk<float, 64, PHI_ELU1>(a) : dispatch_chunk<float, 64, PHI_IDENTITY>(a);
  }
  return hipErrorInvalidValue;
}

}  // namespace la
