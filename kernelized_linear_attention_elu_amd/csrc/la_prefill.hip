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
//                      (bf16 MFMA, fp32 accumulation; phi(K) enters as a
//                      bf16 hi + lo pair so the fp32 state is accurate to
//                      ~2^-16 relative) -> workspace;
//   la_scan_kernel   - fp32 exclusive prefix of (dS, dz) over spans, plus the
//                      total (final state / non-causal sums);
//   la_output_kernel - walks its span chunk by chunk carrying (S, z) in
//                      registers: per chunk the masked intra-chunk product,
//                      the read-out of the carried state, the denominator and
//                      the divide, then the state update.
//
// LDS tiles are all row-major ([token][feature], [feature][value]) and are
// written with 16-byte stores.  MFMA operands whose k-slots run down a column
// (phi(K)^T and V^T over tokens, S^T over features) are fetched with the
// gfx950 transposing LDS read ds_read_b64_tr_b16: inside each 16-lane group,
// lane i reads 4 consecutive elements of row r0 + i/4 starting at column
// col_start(i%4), and output lane o receives rows r0..r0+3 of column
// col_start(o/4) + o%4.
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
  static constexpr int VS = DV + PAD;         // row stride of V               [C][VS]
  static constexpr int SS = DV + PAD;         // row stride of the state copy  [R][SS]
  static constexpr int KS = Op<OP>::K;
  static constexpr int PL = Op<OP>::PL;
  static constexpr int RB = C / 16;           // 16-token row blocks per chunk
  static constexpr int CT = DV / 16;          // 16-wide value-column tiles
  static constexpr int FT = R / 16;           // 16-wide feature tiles
  static constexpr int NTILE = CT * FT;       // 16x16 tiles of the state
  static constexpr int TPW = NTILE / kWaves;  // state tiles owned per wave
  static constexpr int ZPW = FT / kWaves;     // z tiles owned per wave
  static constexpr int VQ = C * D / EPL;      // 16-byte vectors of one Q/K chunk
  static constexpr int VV = C * DV / EPL;     // ... of one V chunk
  static constexpr int LQ = (VQ + kThreads - 1) / kThreads;
  static constexpr int LV = (VV + kThreads - 1) / kThreads;
  // causal output work split: waves per row block, row blocks per wave,
  // value-column tiles per wave
  static constexpr int WPR = RB >= kWaves ? 1 : kWaves / RB;
  static constexpr int RBW = RB >= kWaves ? RB / kWaves : 1;
  static constexpr int CTW = CT / WPR;
  static_assert(R == D, "pointwise feature maps keep the dimension");
  static_assert(NTILE % kWaves == 0 && FT % kWaves == 0, "state tiles must split evenly over waves");
  static_assert(C % 16 == 0 && C <= 128, "chunk must be 16, 32, 64 or 128");
  static_assert(CT % WPR == 0, "value tiles must split over the waves of a row block");
};

// ------------------------------------------------------------------ LDS fragments

__device__ __forceinline__ bf16x4 ds_read_tr4(const bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4*)(p));
}

// bf16 operand fragment whose 8 k-slots run down two groups of 4 rows of a
// row-major LDS tile (slots 0-3: rows ra..ra+3, slots 4-7: rows rb..rb+3) at
// this lane's column col_base + a_stride*(li/4) + li%4.
__device__ __forceinline__ bf16x8 tr_frag(const bf16* base, int stride, int ra, int rb, int col_base,
                                          int a_stride, int li) {
  const int off = (li >> 2) * stride + col_base + a_stride * (li & 3);
  const bf16x4 x = ds_read_tr4(base + ra * stride + off);
  const bf16x4 y = ds_read_tr4(base + rb * stride + off);
  return __builtin_shufflevector(x, y, 0, 1, 2, 3, 4, 5, 6, 7);
}

// The same fragment with the upper 4 slots zero (a 16-token chunk).
__device__ __forceinline__ bf16x8 tr_frag_lo(const bf16* base, int stride, int ra, int col_base, int a_stride,
                                             int li) {
  const int off = (li >> 2) * stride + col_base + a_stride * (li & 3);
  const bf16x4 x = ds_read_tr4(base + ra * stride + off);
  const bf16x4 z4 = bf16x4{0, 0, 0, 0};
  return __builtin_shufflevector(x, z4, 0, 1, 2, 3, 4, 5, 6, 7);
}

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
  const int tid = threadIdx.x;
  constexpr int QV = CF::D / CF::EPL;   // vectors per Q/K row
  constexpr int VVR = CF::DV / CF::EPL; // vectors per V row
#pragma unroll
  for (int i = 0; i < CF::LQ; ++i) {
    const int vi = tid + i * kThreads;
    u32x4 kq = u32x4{0, 0, 0, 0}, qq = u32x4{0, 0, 0, 0};
    const int t = t0 + vi / QV;
    const int col = (vi % QV) * CF::EPL;
    if ((CF::VQ % kThreads == 0 || vi < CF::VQ) && t < N) {
      kq = *reinterpret_cast<const u32x4*>(Kh + (size_t)t * CF::D + col);
      if constexpr (WITH_Q) qq = *reinterpret_cast<const u32x4*>(Qh + (size_t)t * CF::D + col);
    }
    cr.k[i] = kq;
    if constexpr (WITH_Q) cr.q[i] = qq;
  }
#pragma unroll
  for (int i = 0; i < CF::LV; ++i) {
    const int vi = tid + i * kThreads;
    u32x4 vv = u32x4{0, 0, 0, 0};
    const int t = t0 + vi / VVR;
    const int col = (vi % VVR) * CF::EPL;
    if ((CF::VV % kThreads == 0 || vi < CF::VV) && t < N)
      vv = *reinterpret_cast<const u32x4*>(Vh + (size_t)t * CF::DV + col);
    cr.v[i] = vv;
  }
}

// Registers -> LDS, all row-major with 16-byte stores.  phi is applied to Q
// and K in fp32 and rounded to the operand type; keys beyond N get zero
// features so that they add nothing to the state.  With a non-null sk_lo the
// rounding residual phi - round(phi) of the keys is stored too (a bf16 lo
// word), so that hi + lo carries phi(K) to ~2^-16 relative.
template <class CF, bool WITH_Q>
__device__ __forceinline__ void stage_chunk(const ChunkRegs<CF, WITH_Q>& cr, typename CF::OP* sq,
                                            typename CF::OP* sk, typename CF::OP* sk_lo,
                                            typename CF::OP* sv, int t0, int N) {
  using T = typename CF::IO;
  using OP = typename CF::OP;
  const int tid = threadIdx.x;
  constexpr int QV = CF::D / CF::EPL;
  constexpr int VVR = CF::DV / CF::EPL;
#pragma unroll
  for (int i = 0; i < CF::LQ; ++i) {
    const int vi = tid + i * kThreads;
    if (CF::VQ % kThreads == 0 || vi < CF::VQ) {
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
      *reinterpret_cast<u32x4*>(sk + tok * CF::QS + col) = pack16<OP>(f);
      if constexpr (sizeof(OP) == 2) {
        if (sk_lo) {
          float lo[CF::EPL];
#pragma unroll
          for (int e = 0; e < CF::EPL; ++e) lo[e] = f[e] - round_op<OP>(f[e]);
          *reinterpret_cast<u32x4*>(sk_lo + tok * CF::QS + col) = pack16<OP>(lo);
        }
      }
    }
  }
#pragma unroll
  for (int i = 0; i < CF::LV; ++i) {
    const int vi = tid + i * kThreads;
    if (CF::VV % kThreads == 0 || vi < CF::VV) {
      const int tok = vi / VVR;
      const int col = (vi % VVR) * CF::EPL;
      *reinterpret_cast<u32x4*>(sv + tok * CF::VS + col) = cr.v[i];
    }
  }
}

// ------------------------------------------------------------------ state update

// acc[i] += V_c^T phi(K_c) for the state tiles this wave owns, and
// zt[k] += 1^T phi(K_c) for its z tiles.  Tile i of wave w is t = w + 4 i
// with value tile ct = t % CT and feature tile ft = t / CT; lane (g, li)
// ends up holding S[f = 16 ft + li][c = 16 ct + 4 g + r].  z tile k of wave w
// covers features 16 (w + 4 k) + li (all four r hold the same sum).  With
// sk_lo, the lo words are contracted as well (hi + lo = phi to ~2^-16).
template <class CF>
__device__ __forceinline__ void state_mfma(f32x4 (&acc)[CF::TPW], f32x4 (&zt)[CF::ZPW],
                                           const typename CF::OP* sk, const typename CF::OP* sk_lo,
                                           const typename CF::OP* sv, int w, int g, int li) {
  using OP = typename CF::OP;
  if constexpr (sizeof(OP) == 2) {
    const bf16 one = static_cast<bf16>(1.0f);
    const bf16x8 ones = bf16x8{one, one, one, one, one, one, one, one};
    constexpr int NK = (CF::C + 31) / 32;  // k-steps of 32 tokens
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) {
      const int ra = ks * 32 + 8 * g, rb = ra + 4;
#pragma unroll
      for (int i = 0; i < CF::TPW; ++i) {
        const int t = w + kWaves * i;
        const int ct = t % CF::CT, ft = t / CF::CT;
        bf16x8 a, b;
        if constexpr (CF::C >= 32) {
          a = tr_frag(sv, CF::VS, ra, rb, 16 * ct, 4, li);
          b = tr_frag(sk, CF::QS, ra, rb, 16 * ft, 4, li);
        } else {  // 16 tokens: slots 0-3 = rows 4g..4g+3, upper half zero
          a = tr_frag_lo(sv, CF::VS, 4 * g, 16 * ct, 4, li);
          b = tr_frag_lo(sk, CF::QS, 4 * g, 16 * ft, 4, li);
        }
        acc[i] = mfma16(a, b, acc[i]);
        if (sk_lo) {
          const bf16x8 blo = CF::C >= 32 ? tr_frag(sk_lo, CF::QS, ra, rb, 16 * ft, 4, li)
                                         : tr_frag_lo(sk_lo, CF::QS, 4 * g, 16 * ft, 4, li);
          acc[i] = mfma16(a, blo, acc[i]);
        }
      }
#pragma unroll
      for (int k = 0; k < CF::ZPW; ++k) {
        const int ft = w + kWaves * k;
        const bf16x8 b = CF::C >= 32 ? tr_frag(sk, CF::QS, ra, rb, 16 * ft, 4, li)
                                     : tr_frag_lo(sk, CF::QS, 4 * g, 16 * ft, 4, li);
        zt[k] = mfma16(ones, b, zt[k]);
        if (sk_lo) {
          const bf16x8 blo = CF::C >= 32 ? tr_frag(sk_lo, CF::QS, ra, rb, 16 * ft, 4, li)
                                         : tr_frag_lo(sk_lo, CF::QS, 4 * g, 16 * ft, 4, li);
          zt[k] = mfma16(ones, blo, zt[k]);
        }
      }
    }
  } else {
#pragma unroll
    for (int ks = 0; ks < CF::C / 4; ++ks) {
      const int row = ks * 4 + g;
#pragma unroll
      for (int i = 0; i < CF::TPW; ++i) {
        const int t = w + kWaves * i;
        const int ct = t % CF::CT, ft = t / CF::CT;
        acc[i] = mfma16(sv[row * CF::VS + 16 * ct + li], sk[row * CF::QS + 16 * ft + li], acc[i]);
      }
#pragma unroll
      for (int k = 0; k < CF::ZPW; ++k) {
        const int ft = w + kWaves * k;
        zt[k] = mfma16(1.0f, sk[row * CF::QS + 16 * ft + li], zt[k]);
      }
    }
  }
}

// ------------------------------------------------------------------ outputs

// Output rows of one chunk.  For row block ib (query tokens 16 ib .. +15):
//  * weights: tiles a[jb] = phi(K_jb) phi(Q_ib)^T for key blocks jb <= ib;
//    lane (g, li) holds A[i = li][j = 16 jb + 4 g + r]; the diagonal block is
//    masked to j <= i by selection (never by multiplication, so non-finite
//    future keys cannot leak);
//  * numerator O^T = V^T A^T + S^T phi(Q)^T (MFMA), where the accumulator row
//    m of value tile ct maps to value column (DV/4)(m/4) + 4 ct + m%4, so that
//    every lane ends with 4*CTW consecutive columns of one row;
//  * denominator = rowsum(A) + phi(q_i).z  (fp32), then one divide per value.
// The weights and phi(Q) enter both sums exactly as rounded for the MFMA.
template <class CF, bool CAUSAL>
__device__ __forceinline__ void chunk_outputs(const typename CF::OP* sq, const typename CF::OP* sk,
                                              const typename CF::OP* sv, const typename CF::OP* ss,
                                              const float* sz, typename CF::IO* Oh, int t0, int N, int w,
                                              int g, int li) {
  using OP = typename CF::OP;
  using T = typename CF::IO;
  using frag = typename Op<OP>::frag;
  constexpr int KS = CF::KS, PL = CF::PL, RB = CF::RB, CTW = CF::CTW;
  constexpr int AST = CF::DV / 4;  // column step between lane quads (permuted value columns)
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
        if constexpr (PL == 8) {
#pragma unroll
          for (int jp = 0; jp < (RB + 1) / 2; ++jp) {
            const int jb0 = 2 * jp, jb1 = 2 * jp + 1;
            if (jb0 <= ib) {
              const bf16x4 blo = bf16x4{to_op<bf16>(a[jb0][0]), to_op<bf16>(a[jb0][1]),
                                        to_op<bf16>(a[jb0][2]), to_op<bf16>(a[jb0][3])};
              bf16x8 av, bv;
              if (jb1 < RB && jb1 <= ib) {
                av = tr_frag(sv, CF::VS, 16 * jb0 + 4 * g, 16 * jb1 + 4 * g, 4 * ct, AST, li);
                const bf16x4 bhi = bf16x4{to_op<bf16>(a[jb1][0]), to_op<bf16>(a[jb1][1]),
                                          to_op<bf16>(a[jb1][2]), to_op<bf16>(a[jb1][3])};
                bv = __builtin_shufflevector(blo, bhi, 0, 1, 2, 3, 4, 5, 6, 7);
              } else {
                av = tr_frag_lo(sv, CF::VS, 16 * jb0 + 4 * g, 4 * ct, AST, li);
                const bf16x4 z4 = bf16x4{0, 0, 0, 0};
                bv = __builtin_shufflevector(blo, z4, 0, 1, 2, 3, 4, 5, 6, 7);
              }
              o[cti] = mfma16(av, bv, o[cti]);
            }
          }
        } else {
          const int c = AST * (li >> 2) + 4 * ct + (li & 3);
#pragma unroll
          for (int jb = 0; jb < RB; ++jb) {
            if (jb <= ib) {
#pragma unroll
              for (int r = 0; r < 4; ++r) o[cti] = mfma16(sv[(16 * jb + 4 * g + r) * CF::VS + c], a[jb][r], o[cti]);
            }
          }
        }
      }
    }

    den = xor_sum16_32(den);

#pragma unroll
    for (int cti = 0; cti < CTW; ++cti) {
      const int ct = ct0 + cti;
      if constexpr (PL == 8) {
#pragma unroll
        for (int ks = 0; ks < CF::R / KS; ++ks)
          o[cti] = mfma16(tr_frag(ss, CF::SS, ks * 32 + 8 * g, ks * 32 + 8 * g + 4, 4 * ct, AST, li), qf[ks], o[cti]);
      } else {
        const int c = AST * (li >> 2) + 4 * ct + (li & 3);
#pragma unroll
        for (int ks = 0; ks < CF::R / KS; ++ks) o[cti] = mfma16(ss[(ks * 4 + g) * CF::SS + c], qf[ks], o[cti]);
      }
    }

    const int tok = t0 + 16 * ib + li;
    if (tok < N) {
      float vals[4 * CTW];
#pragma unroll
      for (int cti = 0; cti < CTW; ++cti)
#pragma unroll
        for (int r = 0; r < 4; ++r) vals[4 * cti + r] = o[cti][r] / den;
      T* dst = Oh + (size_t)tok * CF::DV + AST * g + 4 * ct0;
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

// Carried state -> LDS: S (operand type, row-major [R][DV]) and z (fp32).
template <class CF>
__device__ __forceinline__ void publish_state(const f32x4 (&sacc)[CF::TPW], const f32x4 (&zt)[CF::ZPW],
                                              typename CF::OP* ss, float* sz, int w, int g, int li) {
  using OP = typename CF::OP;
#pragma unroll
  for (int i = 0; i < CF::TPW; ++i) {
    const int t = w + kWaves * i;
    const int ct = t % CF::CT, ft = t / CF::CT;
    OP* dst = ss + (16 * ft + li) * CF::SS + 16 * ct + 4 * g;
    if constexpr (sizeof(OP) == 2) {
      *reinterpret_cast<bf16x4*>(dst) = bf16x4{to_op<bf16>(sacc[i][0]), to_op<bf16>(sacc[i][1]),
                                               to_op<bf16>(sacc[i][2]), to_op<bf16>(sacc[i][3])};
    } else {
      *reinterpret_cast<f32x4*>(dst) = sacc[i];
    }
  }
  if (g == 0) {
#pragma unroll
    for (int k = 0; k < CF::ZPW; ++k) sz[16 * (w + kWaves * k) + li] = zt[k][0];
  }
}

// ------------------------------------------------------------------ kernels

template <class CF>
struct SmemState {
  typename CF::OP k[CF::C * CF::QS];
  typename CF::OP k_lo[sizeof(typename CF::OP) == 2 ? CF::C * CF::QS : 1];
  typename CF::OP v[CF::C * CF::VS];
};

template <class CF>
struct SmemOut {
  typename CF::OP q[CF::C * CF::QS];
  typename CF::OP k[CF::C * CF::QS];
  typename CF::OP v[CF::C * CF::VS];
  typename CF::OP s[CF::R * CF::SS];
  float z[CF::R];
};

// Per-span state: dS = phi(K_span)^T V_span, dz = sum phi(K_span) -> ws slot s.
// Two chunks of loads are kept in flight (register double buffering).
template <class CF>
__global__ __launch_bounds__(kThreads) void la_state_kernel(const typename CF::IO* __restrict__ K,
                                                            const typename CF::IO* __restrict__ V,
                                                            float* __restrict__ ws, int N, int span,
                                                            int n_span) {
  using OP = typename CF::OP;
  __shared__ SmemState<CF> sm;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, g = l >> 4, li = l & 15;
  const int bh = blockIdx.x / n_span;
  const int s = blockIdx.x % n_span;
  const int t_begin = s * span;
  const int t_end = min(t_begin + span, N);
  const typename CF::IO* Kh = K + (size_t)bh * N * CF::D;
  const typename CF::IO* Vh = V + (size_t)bh * N * CF::DV;
  OP* klo = sizeof(OP) == 2 ? sm.k_lo : nullptr;

  f32x4 acc[CF::TPW];
#pragma unroll
  for (int i = 0; i < CF::TPW; ++i) acc[i] = zero4();
  f32x4 zt[CF::ZPW];
#pragma unroll
  for (int k = 0; k < CF::ZPW; ++k) zt[k] = zero4();

  ChunkRegs<CF, false> ca, cb;
  load_chunk<CF, false>(ca, nullptr, Kh, Vh, t_begin, N);
  if (t_begin + CF::C < t_end) load_chunk<CF, false>(cb, nullptr, Kh, Vh, t_begin + CF::C, N);
  for (int t0 = t_begin; t0 < t_end; t0 += 2 * CF::C) {
    __syncthreads();
    stage_chunk<CF, false>(ca, nullptr, sm.k, klo, sm.v, t0, N);
    __syncthreads();
    if (t0 + 2 * CF::C < t_end) load_chunk<CF, false>(ca, nullptr, Kh, Vh, t0 + 2 * CF::C, N);
    state_mfma<CF>(acc, zt, sm.k, klo, sm.v, w, g, li);
    const int t1 = t0 + CF::C;
    if (t1 >= t_end) break;
    __syncthreads();
    stage_chunk<CF, false>(cb, nullptr, sm.k, klo, sm.v, t1, N);
    __syncthreads();
    if (t1 + 2 * CF::C < t_end) load_chunk<CF, false>(cb, nullptr, Kh, Vh, t1 + 2 * CF::C, N);
    state_mfma<CF>(acc, zt, sm.k, klo, sm.v, w, g, li);
  }

  constexpr int E = CF::R * CF::DV + CF::R;
  float* slot = ws + ((size_t)bh * (n_span + 1) + s) * E;
#pragma unroll
  for (int i = 0; i < CF::TPW; ++i) {
    const int t = w + kWaves * i;
    const int ct = t % CF::CT, ft = t / CF::CT;
    *reinterpret_cast<f32x4*>(slot + (16 * ft + li) * CF::DV + 16 * ct + 4 * g) = acc[i];
  }
  if (g == 0) {
#pragma unroll
    for (int k = 0; k < CF::ZPW; ++k) slot[CF::R * CF::DV + 16 * (w + kWaves * k) + li] = zt[k][0];
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

  // carried state: this wave's tiles of S (fp32) and its z tiles
  constexpr int E = CF::R * CF::DV + CF::R;
  const float* pre = ws + ((size_t)bh * (n_span + 1) + (CAUSAL ? s : n_span)) * E;
  f32x4 sacc[CF::TPW];
#pragma unroll
  for (int i = 0; i < CF::TPW; ++i) {
    const int t = w + kWaves * i;
    const int ct = t % CF::CT, ft = t / CF::CT;
    sacc[i] = *reinterpret_cast<const f32x4*>(pre + (16 * ft + li) * CF::DV + 16 * ct + 4 * g);
  }
  f32x4 zt[CF::ZPW];
#pragma unroll
  for (int k = 0; k < CF::ZPW; ++k) {
    const float zv = pre[CF::R * CF::DV + 16 * (w + kWaves * k) + li];
    zt[k] = f32x4{zv, zv, zv, zv};
  }

  ChunkRegs<CF, true> cr;
  load_chunk<CF, true>(cr, Qh, Kh, Vh, t_begin, N);
  for (int t0 = t_begin; t0 < t_end; t0 += CF::C) {
    if (CAUSAL || t0 == t_begin) publish_state<CF>(sacc, zt, sm.s, sm.z, w, g, li);
    stage_chunk<CF, true>(cr, sm.q, sm.k, nullptr, sm.v, t0, N);
    __syncthreads();
    if (t0 + CF::C < t_end) load_chunk<CF, true>(cr, Qh, Kh, Vh, t0 + CF::C, N);
    chunk_outputs<CF, CAUSAL>(sm.q, sm.k, sm.v, sm.s, sm.z, Oh, t0, N, w, g, li);
    if constexpr (CAUSAL) state_mfma<CF>(sacc, zt, sm.k, nullptr, sm.v, w, g, li);
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

  (void)hipGetLastError();  // drop a stale error left by an unrelated earlier runtime call
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
