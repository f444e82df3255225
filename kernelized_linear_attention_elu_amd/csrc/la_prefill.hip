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
// col_start(o/4) + o%4.  bf16 tiles are unpadded and XOR-swizzled (see
// Tile) so that none of these access patterns has LDS bank conflicts.
//
// Global loads and stores go through buffer resources sized to the head, so
// tokens beyond N read as zero and their stores are dropped by the hardware:
// no branches guard memory operations, which lets the compiler wait for a
// prefetched chunk without draining the later ones.
//
// Data layout: Q, K [B*H][N][D], V, O [B*H][N][DV] (I/O type T), workspace
// fp32 [B*H][n_span+1][R*DV + R] holding S (row-major [R][DV]) then z.
#include <type_traits>

#include "la_common.h"
#include "la_prefill.h"
#include "la_tiles.h"

namespace la {

template <typename T, int D_, int R_, int DV_, int C_, int PHI_, int NW_ = kWaves>
struct Cfg {
  using IO = T;
  using OP = T;                               // MFMA operand type
  static constexpr int D = D_, R = R_, DV = DV_, C = C_, PHI = PHI_;
  static constexpr int NW = NW_;              // waves per workgroup
  static constexpr int NT = 64 * NW_;         // threads per workgroup
  // workgroups per CU the output kernel's registers are sized for
  static constexpr int MINB = (NW_ == 4 && D_ == 64) ? 3 : 1;
  // ... and with a decay (the weighted feature tile and the decay factors
  // need more registers than three workgroups per CU leave)
  static constexpr int MINB_DECAY = (NW_ == 4 && D_ == 64 && C_ <= 64) ? 2 : 1;
  static constexpr int EPL = Vec16<T>::N;     // elements per 16-byte vector
  static constexpr int KS = Op<OP>::K;
  static constexpr int PL = Op<OP>::PL;
  static constexpr int RB = C / 16;           // 16-token row blocks per chunk
  static constexpr int CT = DV / 16;          // 16-wide value-column tiles
  static constexpr int FT = R / 16;           // 16-wide feature tiles
  static constexpr int NTILE = CT * FT;       // 16x16 tiles of the state
  static constexpr int TPW = NTILE / NW;  // state tiles owned per wave
  static constexpr int ZPW = FT / NW;     // z tiles owned per wave
  static constexpr int VQ = C * D / EPL;      // 16-byte vectors of one Q/K chunk
  static constexpr int VV = C * DV / EPL;     // ... of one V chunk
  static constexpr int LQ = (VQ + NT - 1) / NT;
  static constexpr int LV = (VV + NT - 1) / NT;
  // causal output work split: waves per row block, row blocks per wave,
  // value-column tiles per wave
  static constexpr int WPR = RB >= NW ? 1 : NW / RB;
  static constexpr int RBW = RB >= NW ? RB / NW : 1;
  static constexpr int CTW = CT / WPR;
  // carried z as published in LDS: fp32 for fp32 operands; for bf16 three
  // rows of R bf16 (hi, lo = z - hi, zeros), read as an MFMA operand
  using ZT = typename std::conditional<sizeof(T) == 2, bf16, float>::type;
  static constexpr int ZE = sizeof(T) == 2 ? 3 * R : R;
  static_assert(R == D, "pointwise feature maps keep the dimension");
  static_assert(NTILE % NW == 0 && FT % NW == 0, "state tiles must split evenly over waves");
  static_assert(C % 16 == 0 && C <= 128, "chunk must be 16, 32, 64 or 128");
  static_assert(CT % WPR == 0, "value tiles must split over the waves of a row block");
};

// State tile i of wave w: feature tile ft = w (the wave's own), value tile
// ct = i.  Lane (g, li) of that tile holds S[f = 16 ft + li][c = 16 ct + 4 g
// + r]; the wave's z tile is its feature tile too.  With its feature tile
// fixed, a wave reads one phi(K) fragment per k-step and uses it for all of
// its value tiles and its z tile.
template <class CF>
__device__ __forceinline__ void state_tile(int w, int i, int& ct, int& ft) {
  static_assert(CF::NW == CF::FT && CF::TPW == CF::CT && CF::ZPW == 1, "one feature tile per wave");
  ft = w;
  ct = i;
}

// Row block (16 query tokens of the chunk) of wave w, its rbi-th.  With more
// waves than row blocks, wave w belongs to group p = w / RB (which takes
// value or feature tiles p CTW ..) and takes block w mod RB when p is even,
// RB - 1 - (w mod RB) when p is odd.  Waves w and w + 4 share a SIMD, so at
// eight waves and four row blocks each SIMD holds blocks b and 3 - b, and
// the causal weight tiles (b + 1 key blocks for block b) split evenly over
// the SIMDs.
template <class CF>
__device__ __forceinline__ int wave_row_block(int rbi, int w) {
  if constexpr (CF::RB >= CF::NW) {
    return w + CF::NW * rbi;
  } else {
    const int b = w % CF::RB;
    return ((w / CF::RB) & 1) ? CF::RB - 1 - b : b;
  }
}

// ------------------------------------------------------------------ decay kinds

// How the state decays from one token to the next.
constexpr int kNoDecay = 0;  // S_t = S_{t-1} + phi(k_t) v_t^T
constexpr int kFixed = 1;    // S_t = gamma S_{t-1} + ..., one gamma per head (lg = log2 gamma)
constexpr int kGated = 2;    // S_t = a_t S_{t-1} + ..., one gate per token (log a_t given)
constexpr int kChannel = 3;  // S_t = diag(a_t) S_{t-1} + ..., one gate per token and key channel

// A gate's log2 is clamped from below: a gate under 2^-126, zero included,
// acts as 2^-126 (far below what an fp32 sum of the outputs resolves), and
// differences of running sums stay finite (never -inf minus -inf).
constexpr float kMinLog2Gate = -126.f;
constexpr float kLog2e = 1.4426950408889634f;

// Inclusive prefix sum over the 64 lanes of a wave, in VALU data-parallel
// moves (DPP): shifts by 1, 2, 4 and 8 lanes inside each 16-lane row (lanes
// shifted in from outside the row read zero), then lane 15 of rows 0 and 2
// added into rows 1 and 3, then lane 31 into rows 2 and 3.
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ float dpp_add(float x) {
  const int y = __builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, ROW_MASK, 0xf, false);
  return x + __int_as_float(y);
}
__device__ __forceinline__ float wave_prefix_sum(float x) {
  x = dpp_add<0x111>(x);        // row_shr:1
  x = dpp_add<0x112>(x);        // row_shr:2
  x = dpp_add<0x114>(x);        // row_shr:4
  x = dpp_add<0x118>(x);        // row_shr:8
  x = dpp_add<0x142, 0xa>(x);   // row_bcast:15 into rows 1, 3
  x = dpp_add<0x143, 0xc>(x);   // row_bcast:31 into rows 2, 3
  return x;
}

// Running log2 gates of one chunk (kGated): lane l holds the sum of the
// clamped log2 gates of the chunk's tokens 0..l (lo) and, for 128-token
// chunks, 0..64+l (hi).  Gates past N load as log 0 (a gate of one), so the
// sum stays flat there.  Every wave forms its own copy from its own loads.
template <class CF>
struct GateCum {
  float lo = 0.f, hi = 0.f;
  __device__ __forceinline__ void init(const float (&a)[CF::C > 64 ? 2 : 1]) {
    lo = wave_prefix_sum(fmaxf(a[0] * kLog2e, kMinLog2Gate));
    if constexpr (CF::C > 64) hi = wave_prefix_sum(fmaxf(a[1] * kLog2e, kMinLog2Gate)) + lane_value(lo, 63);
  }
  // the value lane 'lane' holds, for a wave-uniform lane (a scalar read)
  __device__ static __forceinline__ float lane_value(float x, int lane) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), __builtin_amdgcn_readfirstlane(lane)));
  }
  // the running sum through chunk token tok, for a wave-uniform tok
  __device__ __forceinline__ float at_uniform(int tok) const {
    if constexpr (CF::C > 64) {
      if (tok >= 64) return lane_value(hi, tok - 64);
    }
    return lane_value(lo, tok);
  }
  // the running sum through chunk token tok (0 <= tok < C; tok may differ
  // between lanes)
  __device__ __forceinline__ float at(int tok) const {
    const float x = __shfl(lo, tok & 63);
    if constexpr (CF::C > 64) {
      const float y = __shfl(hi, tok & 63);
      return tok < 64 ? x : y;
    }
    return x;
  }
};

// ------------------------------------------------------------------ staging

template <class CF, bool WITH_Q>
struct ChunkRegs {
  u32x4 q[WITH_Q ? CF::LQ : 1];
  u32x4 k[CF::LQ];
  u32x4 v[CF::LV];
  float a[CF::C > 64 ? 2 : 1];  // natural log gates of tokens t0 + lane (+ 64) (kGated)
};

// Global -> registers for the chunk starting at token t0.  Rows beyond N
// read as zero (buffer bounds); no load is predicated.  GATED: the chunk's
// log gates first (staging needs them before the keys), one per lane.
template <class CF, bool WITH_Q, bool GATED = false>
__device__ __forceinline__ void load_chunk(ChunkRegs<CF, WITH_Q>& cr, const HeadBufs& hb, int t0) {
  const int tid = threadIdx.x;
  using T = typename CF::IO;
  constexpr int QV = CF::D / CF::EPL;   // vectors per Q/K row
  constexpr int VVR = CF::DV / CF::EPL; // vectors per V row
  if constexpr (GATED) {
    const int lane = tid & 63;
    cr.a[0] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(hb.a, (t0 + lane) * 4, 0, 0));
    if constexpr (CF::C > 64)
      cr.a[1] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(hb.a, (t0 + 64 + lane) * 4, 0, 0));
  }
  // (a chunk smaller than one vector per thread, 16 tokens at d = 64, is
  // the only case that needs the vi guard; it folds away otherwise)
#pragma unroll
  for (int i = 0; i < CF::LQ; ++i) {
    const int vi = tid + i * CF::NT;
    if (CF::VQ % CF::NT == 0 || vi < CF::VQ) {
      const int off = ((t0 + vi / QV) * CF::D + (vi % QV) * CF::EPL) * (int)sizeof(T);
      cr.k[i] = __builtin_amdgcn_raw_buffer_load_b128(hb.k, off, 0, 0);
      if constexpr (WITH_Q) cr.q[i] = __builtin_amdgcn_raw_buffer_load_b128(hb.q, off, 0, 0);
    }
  }
#pragma unroll
  for (int i = 0; i < CF::LV; ++i) {
    const int vi = tid + i * CF::NT;
    if (CF::VV % CF::NT == 0 || vi < CF::VV) {
      const int off = ((t0 + vi / VVR) * CF::DV + (vi % VVR) * CF::EPL) * (int)sizeof(T);
      cr.v[i] = __builtin_amdgcn_raw_buffer_load_b128(hb.v, off, 0, 0);
    }
  }
}

// Registers -> LDS, all row-major with 16-byte stores.  phi is applied to Q
// and K in fp32 and rounded to the operand type; keys beyond N get zero
// features so that they add nothing to the state.  With a non-null sk_lo the
// rounding residual phi - round(phi) of the keys is stored too (a bf16 lo
// word), so that hi + lo carries phi(K) to ~2^-16 relative.
// Decay (DK != kNoDecay): key j of the chunk (0-based) is weighted by its
// decay at the end of the chunk's len tokens, gamma^(len - 1 - j) (kFixed,
// lg = log2 gamma) or a_{j+1} ... a_{len-1} (kGated, from the running log2
// gates, which wave 0 also writes to scum[0 .. max(C, 64)) when scum is
// given).  The weighted features go to sk (and sk_lo) when skw is null,
// otherwise sk keeps the plain features and skw receives the weighted ones.
// A non-zero after (log2, at most 0) multiplies every key weight by 2^after:
// the decay from the chunk's end to a later reference token.
// Returns the log2 of the chunk's whole decay over its len tokens (what a
// state carried across the chunk is multiplied by), 0 without a decay.
template <class CF, bool WITH_Q, int DK = kNoDecay, bool WITH_V = true>
__device__ __forceinline__ float stage_chunk(const ChunkRegs<CF, WITH_Q>& cr, typename CF::OP* sq,
                                             typename CF::OP* sk, typename CF::OP* sk_lo,
                                             typename CF::OP* sv, int t0, int N, float lg = 0.f, int len = 0,
                                             typename CF::OP* skw = nullptr, float* scum = nullptr,
                                             float after = 0.f) {
  using T = typename CF::IO;
  using OP = typename CF::OP;
  using TQ = Tile<OP, CF::R>;
  using TV = Tile<OP, CF::DV>;
  const int tid = threadIdx.x;
  constexpr int QV = CF::D / CF::EPL;
  constexpr int VVR = CF::DV / CF::EPL;
  GateCum<CF> gc;
  float total = 0.f;
  if constexpr (DK == kGated) {
    gc.init(cr.a);
    total = gc.at_uniform(len - 1);
    if (scum && wave_id() == 0) {
      const int lane = tid & 63;
      scum[lane] = gc.lo;
      if constexpr (CF::C > 64) scum[64 + lane] = gc.hi;
    }
  } else if constexpr (DK == kFixed) {
    total = lg * (float)len;
  }
  // only a chunk that reaches past N has keys to mask (a uniform branch)
  auto keys = [&](auto tail) {
#pragma unroll
    for (int i = 0; i < CF::LQ; ++i) {
      const int vi = tid + i * CF::NT;
      if (!(CF::VQ % CF::NT == 0 || vi < CF::VQ)) continue;
      const int tok = vi / QV;
      const int col = (vi % QV) * CF::EPL;
      float f[CF::EPL];
      if constexpr (WITH_Q) {
        unpack16<T>(cr.q[i], f);
#pragma unroll
        for (int e = 0; e < CF::EPL; ++e) f[e] = phi_pointwise<CF::PHI>(f[e]);
        *reinterpret_cast<u32x4*>(sq + TQ::off(tok, col)) = pack16<OP>(f);
      }
      unpack16<T>(cr.k[i], f);
#pragma unroll
      for (int e = 0; e < CF::EPL; ++e) f[e] = phi_pointwise<CF::PHI>(f[e]);
      u32x4 hw = u32x4{0u, 0u, 0u, 0u};  // weighted features for skw
      if constexpr (DK != kNoDecay) {
        // (keys past len, beyond N, may get a weight above one; they are
        // zeroed below by selection, never by arithmetic)
        const float wgt =
            __builtin_amdgcn_exp2f((DK == kFixed ? lg * (float)(len - 1 - tok) : total - gc.at(tok)) + after);
        if (skw) {
          float fw[CF::EPL];
#pragma unroll
          for (int e = 0; e < CF::EPL; ++e) fw[e] = f[e] * wgt;
          hw = pack16<OP>(fw);
        } else {
#pragma unroll
          for (int e = 0; e < CF::EPL; ++e) f[e] *= wgt;
        }
      }
      u32x4 hi = pack16<OP>(f);
      u32x4 lo = u32x4{0u, 0u, 0u, 0u};
      if constexpr (sizeof(OP) == 2) {
        if (sk_lo) {
          float h[CF::EPL], r[CF::EPL];
          unpack16<bf16>(hi, h);
#pragma unroll
          for (int e = 0; e < CF::EPL; ++e) r[e] = f[e] - h[e];
          lo = pack16<OP>(r);
        }
      }
      if constexpr (decltype(tail)::value) {
        // keys at or beyond N get zero features (selected on the packed words)
        const bool valid = t0 + tok < N;
        hi = valid ? hi : u32x4{0u, 0u, 0u, 0u};
        lo = valid ? lo : u32x4{0u, 0u, 0u, 0u};
        hw = valid ? hw : u32x4{0u, 0u, 0u, 0u};
      }
      *reinterpret_cast<u32x4*>(sk + TQ::off(tok, col)) = hi;
      if constexpr (DK != kNoDecay) {
        if (skw) *reinterpret_cast<u32x4*>(skw + TQ::off(tok, col)) = hw;
      }
      if constexpr (sizeof(OP) == 2) {
        if (sk_lo) *reinterpret_cast<u32x4*>(sk_lo + TQ::off(tok, col)) = lo;
      }
    }
  };
  if (t0 + CF::C > N)
    keys(std::true_type{});
  else
    keys(std::false_type{});
  if constexpr (WITH_V) {  // (otherwise the keys only)
#pragma unroll
    for (int i = 0; i < CF::LV; ++i) {
      const int vi = tid + i * CF::NT;
      if (CF::VV % CF::NT == 0 || vi < CF::VV)
        *reinterpret_cast<u32x4*>(sv + TV::off(vi / VVR, (vi % VVR) * CF::EPL)) = cr.v[i];
    }
  }
  return total;
}

// V rows of the chunk -> LDS (the value half of stage_chunk).
template <class CF, bool WITH_Q>
__device__ __forceinline__ void stage_values(const ChunkRegs<CF, WITH_Q>& cr, typename CF::OP* sv) {
  using TV = Tile<typename CF::OP, CF::DV>;
  constexpr int VVR = CF::DV / CF::EPL;
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < CF::LV; ++i) {
    const int vi = tid + i * CF::NT;
    if (CF::VV % CF::NT == 0 || vi < CF::VV)
      *reinterpret_cast<u32x4*>(sv + TV::off(vi / VVR, (vi % VVR) * CF::EPL)) = cr.v[i];
  }
}

// ------------------------------------------------------------------ state update

// acc[i] += V_c^T phi(K_c) for the state tiles this wave owns (state_tile:
// feature tile w, value tile i), and zt[k] += 1^T phi(K_c) for its z tile
// (features 16 w + li; all four r hold the same sum).  With sk_lo, the lo
// words are contracted as well (hi + lo = phi to ~2^-16).
template <class CF>
__device__ __forceinline__ void state_mfma(f32x4 (&acc)[CF::TPW], f32x4 (&zt)[CF::ZPW],
                                           const typename CF::OP* sk, const typename CF::OP* sk_lo,
                                           const typename CF::OP* sv, int w, int g, int li) {
  using OP = typename CF::OP;
  constexpr int R = CF::R, DV = CF::DV;
  if constexpr (sizeof(OP) == 2) {
    const bf16 one = static_cast<bf16>(1.0f);
    const bf16x8 ones = bf16x8{one, one, one, one, one, one, one, one};
    constexpr int NK = (CF::C + 31) / 32;  // k-steps of 32 tokens
    auto kfrag = [&](const OP* base, int ra, int ft) {
      return CF::C >= 32 ? tr_frag<R>(base, ra, ra + 4, 16 * ft, li) : tr_frag_lo<R>(base, 4 * g, 16 * ft, li);
    };
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) {
      const int ra = ks * 32 + 8 * g;
      // the wave's feature tile (state_tile): one phi(K) fragment (and its
      // lo word) per k-step, shared by every value tile and the z tile
      const bf16x8 kh = kfrag(sk, ra, w);
      const bf16x8 kl = sk_lo ? kfrag(sk_lo, ra, w) : kh;
#pragma unroll
      for (int i = 0; i < CF::TPW; ++i) {
        int ct, ft;
        state_tile<CF>(w, i, ct, ft);
        const bf16x8 a = CF::C >= 32 ? tr_frag<DV>(sv, ra, ra + 4, 16 * ct, li) : tr_frag_lo<DV>(sv, 4 * g, 16 * ct, li);
        acc[i] = mfma16(a, kh, acc[i]);
        if (sk_lo) acc[i] = mfma16(a, kl, acc[i]);
      }
      zt[0] = mfma16(ones, kh, zt[0]);
      if (sk_lo) zt[0] = mfma16(ones, kl, zt[0]);
    }
  } else {
    using TQ = Tile<OP, R>;
    using TV = Tile<OP, DV>;
#pragma unroll
    for (int ks = 0; ks < CF::C / 4; ++ks) {
      const int row = ks * 4 + g;
#pragma unroll
      for (int i = 0; i < CF::TPW; ++i) {
        int ct, ft;
        state_tile<CF>(w, i, ct, ft);
        acc[i] = mfma16(sv[TV::off(row, 16 * ct + li)], sk[TQ::off(row, 16 * ft + li)], acc[i]);
      }
#pragma unroll
      for (int k = 0; k < CF::ZPW; ++k) {
        const int ft = w + CF::NW * k;
        zt[k] = mfma16(1.0f, sk[TQ::off(row, 16 * ft + li)], zt[k]);
      }
    }
  }
}

// ------------------------------------------------------------------ outputs

// phi(Q) MFMA fragments of this wave's query rows.  k-slot -> feature
// mapping: bf16 lane group g owns features 32 ks + 8 g .. +7 (one 16-byte
// vector per k-step); fp32 lane group g owns features 16 g .. 16 g + 15
// (k-step ks -> 16 g + ks).  The same mapping is used for every operand
// contracted against phi(Q).
//
// bf16 (kRows): the wave's query rows are loaded as whole 128/256-byte rows
// (consecutive lanes read consecutive 16 bytes, so every load instruction
// covers whole cache lines), written to the wave's own LDS scratch and read
// back in fragment layout.  A fragment-layout global load would touch 16
// partial lines per instruction, which streams about a third slower.  (Waves
// that share a row block each load it; the second read hits L2.)  fp32: the
// fragments are loaded from global memory directly.
template <class CF, bool ROWS = true>
struct QRegs {
  using OP = typename CF::OP;
  using frag = typename Op<OP>::frag;
  static constexpr bool kRows = ROWS && CF::PL == 8;
  // output rows leave whole when this wave's columns span 64 or 128 values
  static constexpr int OCOLS = CF::CTW * 16;
  static constexpr bool kRowsOut = kRows && (OCOLS == 64 || OCOLS == 128);
  static constexpr int NV = CF::PL == 8 ? CF::R / 32 : CF::R / 16;  // 16-byte vectors per lane per row block
  static constexpr int UPR = CF::D / 8;                              // 16-byte units per bf16 row
  u32x4 raw[CF::RBW][NV];
  __device__ static __forceinline__ int feature(int ks, int g) { return CF::PL == 8 ? 32 * ks + 8 * g : 16 * g + ks; }
  __device__ static __forceinline__ int row_block(int rbi, int w) {
    return wave_row_block<CF>(rbi, w);
  }
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t q, int t0, int w, int g, int li) {
    using T = typename CF::IO;
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int rbi = 0; rbi < CF::RBW; ++rbi) {
      const int ib = row_block(rbi, w);
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        int row, col;
        if constexpr (kRows) {
          const int qi = v * 64 + lane;
          row = t0 + 16 * ib + qi / UPR;
          col = 8 * (qi % UPR);
        } else {
          row = t0 + 16 * ib + li;
          col = CF::PL == 8 ? 32 * v + 8 * g : 16 * g + 4 * v;
        }
        raw[rbi][v] = __builtin_amdgcn_raw_buffer_load_b128(q, (row * CF::D + col) * (int)sizeof(T), 0, kStreamLoad);
      }
    }
  }
  // phi in fp32, kept in fp32 (the per-channel gated path scales it before
  // rounding): value n of a lane is feature 32 (n / 8) + 8 g + n % 8 (bf16)
  // or 16 g + n (fp32), the k-slot order of to_frags
  __device__ __forceinline__ void to_f32(float (&fq)[CF::RBW][CF::R / 4], OP* scr, int g, int li) const {
    using T = typename CF::IO;
    if constexpr (kRows) {
      using TS = Tile<OP, CF::D>;
      const int lane = threadIdx.x & 63;
#pragma unroll
      for (int rbi = 0; rbi < CF::RBW; ++rbi)
#pragma unroll
        for (int v = 0; v < NV; ++v) {
          const int qi = v * 64 + lane;
          *reinterpret_cast<u32x4*>(scr + TS::off(16 * rbi + qi / UPR, 8 * (qi % UPR))) = raw[rbi][v];
        }
#pragma unroll
      for (int rbi = 0; rbi < CF::RBW; ++rbi)
#pragma unroll
        for (int ks = 0; ks < NV; ++ks) {
          float f[8];
          unpack16<bf16>(*reinterpret_cast<const u32x4*>(scr + TS::off(16 * rbi + li, 32 * ks + 8 * g)), f);
#pragma unroll
          for (int e = 0; e < 8; ++e) fq[rbi][8 * ks + e] = phi_pointwise<CF::PHI>(f[e]);
        }
    } else {
      static_assert(CF::PL == 1, "fp32 operands read their fragments directly");
#pragma unroll
      for (int rbi = 0; rbi < CF::RBW; ++rbi) {
#pragma unroll
        for (int v = 0; v < NV; ++v) {
          float f[CF::EPL];
          unpack16<T>(raw[rbi][v], f);
#pragma unroll
          for (int e = 0; e < 4; ++e) fq[rbi][4 * v + e] = phi_pointwise<CF::PHI>(f[e]);
        }
      }
    }
  }
  // the rows as loaded, in fragment layout (no phi; bf16 rows only)
  __device__ __forceinline__ void to_raw(bf16x8 (&fr)[CF::RBW][CF::R / CF::KS], OP* scr, int g, int li) const {
    static_assert(kRows, "raw fragments of bf16 rows");
    using TS = Tile<OP, CF::D>;
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int rbi = 0; rbi < CF::RBW; ++rbi)
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        const int qi = v * 64 + lane;
        *reinterpret_cast<u32x4*>(scr + TS::off(16 * rbi + qi / UPR, 8 * (qi % UPR))) = raw[rbi][v];
      }
#pragma unroll
    for (int rbi = 0; rbi < CF::RBW; ++rbi)
#pragma unroll
      for (int ks = 0; ks < NV; ++ks)
        fr[rbi][ks] = *reinterpret_cast<const bf16x8*>(scr + TS::off(16 * rbi + li, 32 * ks + 8 * g));
  }
  // apply phi in fp32 and round to the operand type (scr: this wave's LDS
  // scratch of RBW x 16 rows, used when kRows)
  __device__ __forceinline__ void to_frags(frag (&qf)[CF::RBW][CF::R / CF::KS], OP* scr, int g, int li) const {
    using T = typename CF::IO;
    if constexpr (kRows) {
      using TS = Tile<OP, CF::D>;
      const int lane = threadIdx.x & 63;
#pragma unroll
      for (int rbi = 0; rbi < CF::RBW; ++rbi)
#pragma unroll
        for (int v = 0; v < NV; ++v) {
          const int qi = v * 64 + lane;
          *reinterpret_cast<u32x4*>(scr + TS::off(16 * rbi + qi / UPR, 8 * (qi % UPR))) = raw[rbi][v];
        }
#pragma unroll
      for (int rbi = 0; rbi < CF::RBW; ++rbi)
#pragma unroll
        for (int ks = 0; ks < NV; ++ks) {
          float f[8];
          unpack16<bf16>(*reinterpret_cast<const u32x4*>(scr + TS::off(16 * rbi + li, 32 * ks + 8 * g)), f);
#pragma unroll
          for (int e = 0; e < 8; ++e) f[e] = phi_pointwise<CF::PHI>(f[e]);
          qf[rbi][ks] = cvt_bf16x8(f);
        }
    } else {
#pragma unroll
      for (int rbi = 0; rbi < CF::RBW; ++rbi) {
#pragma unroll
        for (int v = 0; v < NV; ++v) {
          float f[CF::EPL];
          unpack16<T>(raw[rbi][v], f);
          if constexpr (CF::PL == 8) {
#pragma unroll
            for (int e = 0; e < 8; ++e) f[e] = phi_pointwise<CF::PHI>(f[e]);
            qf[rbi][v] = cvt_bf16x8(f);
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) qf[rbi][4 * v + e] = phi_pointwise<CF::PHI>(f[e]);
          }
        }
      }
    }
  }
};

// phi(Q) shared by the two waves of a row block (eight waves, chunk 64,
// bf16): each wave loads half of the block's Q columns, [64 h, 64 h + 64)
// for its group h = w / RB (128-byte half rows), applies phi to them and
// writes them as operand fragments (k-steps 2 h, 2 h + 1) into a phi(Q)
// tile of the chunk, from which both waves read all of them.  That halves
// the phi evaluations and the Q row traffic per wave against each wave
// forming the whole row block itself.
template <class CF>
struct SharedQ {
  static constexpr bool on = CF::NW == 8 && CF::RB == 4 && CF::RBW == 1 && sizeof(typename CF::OP) == 2 &&
                             CF::PL == 8 && CF::D == 128;
  static constexpr int HC = CF::D / 2;       // columns per half
  static constexpr int UPH = HC / 8;         // 16-byte units per half row
  static constexpr int NV = 16 * UPH / 64;   // vectors per lane
  u32x4 raw[NV];
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t q, int t0, int ib, int h) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const int qi = v * 64 + lane;
      const int row = t0 + 16 * ib + qi / UPH, col = HC * h + 8 * (qi % UPH);
      raw[v] = __builtin_amdgcn_raw_buffer_load_b128(q, (row * CF::D + col) * 2, 0, kStreamLoad);
    }
  }
  // the loaded half rows -> the wave's scratch -> phi -> tile sq (rows 16 ib
  // + li, the half's k-steps, in the layout of the key tiles)
  __device__ __forceinline__ void to_tile(bf16* scr, bf16* sq, int ib, int h, int g, int li) const {
    using TS = Tile<bf16, HC>;
    using TQ = Tile<bf16, CF::R>;
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const int qi = v * 64 + lane;
      *reinterpret_cast<u32x4*>(scr + TS::off(qi / UPH, 8 * (qi % UPH))) = raw[v];
    }
#pragma unroll
    for (int kk = 0; kk < HC / 32; ++kk) {
      float f[8];
      unpack16<bf16>(*reinterpret_cast<const u32x4*>(scr + TS::off(li, 32 * kk + 8 * g)), f);
#pragma unroll
      for (int e = 0; e < 8; ++e) f[e] = phi_pointwise<CF::PHI>(f[e]);
      *reinterpret_cast<bf16x8*>(sq + TQ::off(16 * ib + li, HC * h + 32 * kk + 8 * g)) = cvt_bf16x8(f);
    }
  }
};

// Per-wave LDS scratch of the output kernels (bf16 row staging of Q and O).
template <class CF>
struct Scratch {
  static constexpr int QE = CF::RBW * 16 * CF::D;
  static constexpr int OE = QRegs<CF>::kRowsOut ? CF::RBW * 16 * QRegs<CF>::OCOLS : 0;
  static constexpr int PER_WAVE = QRegs<CF>::kRows ? (QE > OE ? QE : OE) : 8;
  static constexpr int ELEMS = CF::NW * PER_WAVE;
};

// Finished output values of one lane for one chunk (row 16 ib + li, value
// columns 16 ct + 4 g .. +3 for each of its CTW value tiles), already rounded
// to the I/O type, kept in registers until they are stored.
template <class CF>
struct OutRegs {
  using vec = typename std::conditional<sizeof(typename CF::IO) == 2, bf16x4, f32x4>::type;
  vec v[CF::RBW][CF::CTW];
};

// Output rows of one chunk.  For row block ib (query tokens 16 ib .. +15):
//  * weights: tiles a[jb] = phi(K_jb) phi(Q_ib)^T for key blocks jb <= ib;
//    lane (g, li) holds A[i = li][j = 16 jb + 4 g + r]; the diagonal block is
//    masked to j <= i by selection (never by multiplication, so non-finite
//    future keys cannot leak);
//  * numerator O^T = V^T A^T + S^T phi(Q)^T (MFMA): lane (g, li) ends with
//    O[i = li][c = 16 ct + 4 g + r];
//  * denominator = rowsum(A) + phi(q_i).z, then one reciprocal per row.
//    bf16: both terms on the MFMA as well, into one accumulator dacc: an A
//    operand whose rows 4m hold z_hi and rows 4m+1 z_lo (the published z
//    rows; other rows read the zero row) against phi(Q), and an A operand
//    of ones on rows 4m against the weights, so that every lane ends with
//    dacc[0] = z_hi.phi(q) + rowsum(A) and dacc[1] = z_lo.phi(q).
//    fp32: in VALU.
// The weights and phi(Q) enter both sums exactly as rounded for the MFMA.
// Decay (DK != kNoDecay): for row i = 16 ib + li of the chunk the carried
// state's read-out and its z term are scaled by the decay over tokens
// 0..i, gamma^(i+1) (kFixed, lg = log2 gamma) or 2^cum[i] (kGated; cum: the
// chunk's running log2 gates in LDS), formed first; weight (i, j) by the
// decay over tokens j+1..i, gamma^(i-j) or 2^(cum[i] - cum[j]), before the
// diagonal mask.  normalize = 0 (with a decay only) skips the division.
template <class CF, bool CAUSAL, int DK = kNoDecay>
__device__ __forceinline__ void chunk_outputs(const typename QRegs<CF>::frag (&qf)[CF::RBW][CF::R / CF::KS],
                                              const typename CF::OP* sk, const typename CF::OP* sv,
                                              const typename CF::OP* ss, const typename CF::ZT* sz,
                                              OutRegs<CF>& out, int w, int g, int li, float lg = 0.f,
                                              int normalize = 1, const float* scum = nullptr) {
  constexpr bool DECAY = DK != kNoDecay;
  using OP = typename CF::OP;
  using TQ = Tile<OP, CF::R>;
  using TV = Tile<OP, CF::DV>;
  constexpr int KS = CF::KS, PL = CF::PL, RB = CF::RB, CTW = CF::CTW, R = CF::R, DV = CF::DV;
  const bf16 one = static_cast<bf16>(1.0f), zero = static_cast<bf16>(0.0f);
  const bf16 o1 = (li & 3) == 0 ? one : zero;
  const bf16x8 ones_rows = bf16x8{o1, o1, o1, o1, o1, o1, o1, o1};  // rows 4m of the ones operand
  const int zrow = min(li & 3, 2);                                    // z_hi, z_lo or zeros
#pragma unroll
  for (int rbi = 0; rbi < CF::RBW; ++rbi) {
    const int ib = wave_row_block<CF>(rbi, w);
    const int ct0 = (RB >= CF::NW) ? 0 : (w / RB) * CTW;

    float den = 0.f;
    f32x4 dacc = zero4();
#pragma unroll
    for (int ks = 0; ks < R / KS; ++ks) {
      if constexpr (PL == 1) {
        den += qf[rbi][ks] * sz[QRegs<CF>::feature(ks, g)];
      } else {
        dacc = mfma16(load_frag(sz + zrow * R + ks * KS + g * PL), qf[rbi][ks], dacc);
      }
    }

    f32x4 o[CTW];
#pragma unroll
    for (int c = 0; c < CTW; ++c) o[c] = zero4();
    // read-out of the carried state: o += S^T phi(Q)^T
    auto readout = [&]() {
#pragma unroll
      for (int cti = 0; cti < CTW; ++cti) {
        const int ct = ct0 + cti;
        if constexpr (PL == 8) {
#pragma unroll
          for (int ks = 0; ks < R / KS; ++ks)
            o[cti] = mfma16(tr_frag<DV>(ss, ks * 32 + 8 * g, ks * 32 + 8 * g + 4, 16 * ct, li), qf[rbi][ks], o[cti]);
        } else {
#pragma unroll
          for (int ks = 0; ks < R / KS; ++ks)
            o[cti] = mfma16(ss[TV::off(QRegs<CF>::feature(ks, g), 16 * ct + li)], qf[rbi][ks], o[cti]);
        }
      }
    };
    // running log2 decay through row i (kGated)
    const float crow = DK == kGated ? scum[16 * ib + li] : 0.f;
    if constexpr (DECAY) {
      const float rowdec = __builtin_amdgcn_exp2f(DK == kFixed ? lg * (float)(16 * ib + li + 1) : crow);
      readout();
#pragma unroll
      for (int cti = 0; cti < CTW; ++cti) o[cti] *= rowdec;
      if constexpr (PL == 8) {
        dacc *= rowdec;
      } else {
        den *= rowdec;
      }
    }

    if constexpr (CAUSAL) {
      // key blocks are taken in pairs (one K = 32 MFMA step for bf16); only
      // the pair's two weight tiles are live at a time
      auto weights = [&](int jb) {
        f32x4 t = zero4();
#pragma unroll
        for (int ks = 0; ks < R / KS; ++ks) {
          if constexpr (PL == 8) {
            t = mfma16(load_frag(sk + TQ::off(16 * jb + li, ks * KS + g * PL)), qf[rbi][ks], t);
          } else {
            t = mfma16(sk[TQ::off(16 * jb + li, QRegs<CF>::feature(ks, g))], qf[rbi][ks], t);
          }
        }
        if constexpr (DK == kFixed) {
          // gamma^(i-j); above the diagonal the factor exceeds one, and those
          // entries are then replaced by zero (selection below)
#pragma unroll
          for (int r = 0; r < 4; ++r) t[r] *= __builtin_amdgcn_exp2f(lg * (float)(16 * (ib - jb) + li - 4 * g - r));
        } else if constexpr (DK == kGated) {
          // 2^(cum[i] - cum[j]) (above the diagonal: replaced by selection)
          const f32x4 cj = *reinterpret_cast<const f32x4*>(scum + 16 * jb + 4 * g);
#pragma unroll
          for (int r = 0; r < 4; ++r) t[r] *= __builtin_amdgcn_exp2f(crow - cj[r]);
        }
        if constexpr (PL == 8) {
          if (jb == ib) {  // wave-uniform: only the diagonal block is masked
#pragma unroll
            for (int r = 0; r < 4; ++r) t[r] = 4 * g + r > li ? 0.f : t[r];
          }
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float x = (jb == ib && 4 * g + r > li) ? 0.f : t[r];
            t[r] = x;
            den += x;
          }
        }
        return t;
      };
#pragma unroll
      for (int jp = 0; jp < (RB + 1) / 2; ++jp) {
        const int jb0 = 2 * jp, jb1 = 2 * jp + 1;
        if (jb0 > ib) continue;
        const f32x4 a0 = weights(jb0);
        const bool two = jb1 < RB && jb1 <= ib;
        const f32x4 a1 = two ? weights(jb1) : zero4();
        if constexpr (PL == 8) {
          const float w8[8] = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
          const bf16x8 bv = cvt_bf16x8(w8);
          dacc = mfma16(ones_rows, bv, dacc);
#pragma unroll
          for (int cti = 0; cti < CTW; ++cti) {
            const int ct = ct0 + cti;
            const bf16x8 av = two ? tr_frag<DV>(sv, 16 * jb0 + 4 * g, 16 * jb1 + 4 * g, 16 * ct, li)
                                  : tr_frag_lo<DV>(sv, 16 * jb0 + 4 * g, 16 * ct, li);
            o[cti] = mfma16(av, bv, o[cti]);
          }
        } else {
#pragma unroll
          for (int cti = 0; cti < CTW; ++cti) {
            const int ct = ct0 + cti;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              o[cti] = mfma16(sv[TV::off(16 * jb0 + 4 * g + r, 16 * ct + li)], a0[r], o[cti]);
              if (two) o[cti] = mfma16(sv[TV::off(16 * jb1 + 4 * g + r, 16 * ct + li)], a1[r], o[cti]);
            }
          }
        }
      }
    }

    if constexpr (PL == 8) {
      den = dacc[0] + dacc[1];
    } else {
      den = xor_sum16_32(den);
    }

    if constexpr (!DECAY) readout();

    // one reciprocal per row (<= 1 ulp)
    const float rden = (DECAY && !normalize) ? 1.f : __builtin_amdgcn_rcpf(den);
#pragma unroll
    for (int cti = 0; cti < CTW; ++cti) {
      if constexpr (sizeof(typename CF::IO) == 2) {
        out.v[rbi][cti] = cvt_bf16x4(o[cti] * rden);
      } else {
        out.v[rbi][cti] = o[cti] * rden;
      }
    }
  }
}

// Store one chunk's outputs (rows beyond N are dropped by the buffer bounds).
// With drop set, every store gets an offset past the buffer and the hardware
// discards it: the store instructions are still issued, so that the memory
// counter waits of the surrounding loop stay exact.  bf16 with one wave per
// row block: the wave's finished rows go through its LDS scratch and leave as
// whole rows, 16 bytes per lane (consecutive lanes, consecutive addresses).
template <class CF, bool ROWS = true>
__device__ __forceinline__ void store_outputs(const OutRegs<CF>& out, __amdgpu_buffer_rsrc_t orsrc, int t0,
                                              int w, int g, int li, bool drop, typename CF::OP* scr) {
  using T = typename CF::IO;
  constexpr int RB = CF::RB, CTW = CF::CTW;
  if constexpr (QRegs<CF, ROWS>::kRowsOut) {
    // this wave's columns [16 ct0, 16 ct0 + OCOLS) of its rows
    constexpr int OC = QRegs<CF, ROWS>::OCOLS;
    using TS = Tile<typename CF::OP, OC>;
    constexpr int UPR = OC / 8;                   // 16-byte units per row piece
    constexpr int NVO = 16 * UPR / 64;            // units per lane per row block
    const int lane = threadIdx.x & 63;
    const int ct0 = (RB >= CF::NW) ? 0 : (w / RB) * CTW;
#pragma unroll
    for (int rbi = 0; rbi < CF::RBW; ++rbi)
#pragma unroll
      for (int cti = 0; cti < CTW; ++cti)
        *reinterpret_cast<bf16x4*>(scr + TS::off(16 * rbi + li, 16 * cti + 4 * g)) = out.v[rbi][cti];
#pragma unroll
    for (int rbi = 0; rbi < CF::RBW; ++rbi) {
      const int ib = QRegs<CF>::row_block(rbi, w);
#pragma unroll
      for (int v = 0; v < NVO; ++v) {
        const int qi = v * 64 + lane;
        const u32x4 x = *reinterpret_cast<const u32x4*>(scr + TS::off(16 * rbi + qi / UPR, 8 * (qi % UPR)));
        const int off =
            drop ? kDropOffset : ((t0 + 16 * ib + qi / UPR) * CF::DV + 16 * ct0 + 8 * (qi % UPR)) * 2;
        __builtin_amdgcn_raw_buffer_store_b128(x, orsrc, off, 0, kStreamStore);
      }
    }
  } else {
#pragma unroll
    for (int rbi = 0; rbi < CF::RBW; ++rbi) {
      const int ib = QRegs<CF>::row_block(rbi, w);
      const int ct0 = (RB >= CF::NW) ? 0 : (w / RB) * CTW;
      const int row = t0 + 16 * ib + li;
#pragma unroll
      for (int cti = 0; cti < CTW; ++cti) {
        const int off = drop ? kDropOffset : (row * CF::DV + 16 * (ct0 + cti) + 4 * g) * (int)sizeof(T);
        if constexpr (sizeof(T) == 2) {
          typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
          __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, out.v[rbi][cti]), orsrc, off, 0,
                                                kStreamStore);
        } else {
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, out.v[rbi][cti]), orsrc, off, 0,
                                                 kStreamStore);
        }
      }
    }
  }
}

// The store instructions of store_outputs<CF, ROWS> (same count, width and
// policy), all aimed past the buffer, where the hardware drops them.  Issued
// once ahead of a loop whose iterations end with store_outputs, they make
// the memory operations outstanding at the loop head the same on entry as
// on the back edge, so that the compiler's counter wait there covers only
// the prefetched loads and not the previous chunk's stores.
template <class CF, bool ROWS = true>
__device__ __forceinline__ void dummy_stores(__amdgpu_buffer_rsrc_t orsrc) {
  constexpr int CTW = CF::CTW;
  if constexpr (QRegs<CF, ROWS>::kRowsOut) {
    constexpr int NVO = 16 * (QRegs<CF, ROWS>::OCOLS / 8) / 64;
    static_assert(CF::RBW * NVO <= 4, "distinct drop offsets");
#pragma unroll
    for (int i = 0; i < CF::RBW * NVO; ++i)  // distinct offsets: no store is merged away
      __builtin_amdgcn_raw_buffer_store_b128(u32x4{0u, 0u, 0u, 0u}, orsrc, kDropOffset - 16 * i, 0, kStreamStore);
  } else {
    static_assert(CF::RBW * CTW <= 4, "distinct drop offsets");
#pragma unroll
    for (int i = 0; i < CF::RBW * CTW; ++i) {
      if constexpr (sizeof(typename CF::IO) == 2) {
        typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
        __builtin_amdgcn_raw_buffer_store_b64(u32x2{0u, 0u}, orsrc, kDropOffset - 16 * i, 0, kStreamStore);
      } else {
        __builtin_amdgcn_raw_buffer_store_b128(u32x4{0u, 0u, 0u, 0u}, orsrc, kDropOffset - 16 * i, 0, kStreamStore);
      }
    }
  }
}

// Carried state -> LDS: S (operand type, row-major [R][DV]) and z (fp32, or
// for bf16 the hi / lo / zero rows read by chunk_outputs).
template <class CF>
__device__ __forceinline__ void publish_state(const f32x4 (&sacc)[CF::TPW], const f32x4 (&zt)[CF::ZPW],
                                              typename CF::OP* ss, typename CF::ZT* sz, int w, int g, int li) {
  using OP = typename CF::OP;
  using TS = Tile<OP, CF::DV>;
#pragma unroll
  for (int i = 0; i < CF::TPW; ++i) {
    int ct, ft;
    state_tile<CF>(w, i, ct, ft);
    OP* dst = ss + TS::off(16 * ft + li, 16 * ct + 4 * g);
    if constexpr (sizeof(OP) == 2) {
      *reinterpret_cast<bf16x4*>(dst) = cvt_bf16x4(sacc[i]);
    } else {
      *reinterpret_cast<f32x4*>(dst) = sacc[i];
    }
  }
  if constexpr (sizeof(OP) == 2) {
    // lane group 0 writes z_hi, group 1 z_lo, group 2 the zero row
    if (g < 3) {
#pragma unroll
      for (int k = 0; k < CF::ZPW; ++k) {
        const float z = zt[k][0];
        const bf16 h = static_cast<bf16>(z);
        const bf16 v = g == 0 ? h : g == 1 ? static_cast<bf16>(z - static_cast<float>(h)) : static_cast<bf16>(0.f);
        sz[g * CF::R + 16 * (w + CF::NW * k) + li] = v;
      }
    }
  } else {
    if (g == 0) {
#pragma unroll
      for (int k = 0; k < CF::ZPW; ++k) sz[16 * (w + CF::NW * k) + li] = zt[k][0];
    }
  }
}

// ------------------------------------------------------------------ kernels

// LDS of the state kernel: two chunk buffers (staging of chunk c+1 overlaps
// the MFMA work on chunk c; one barrier per chunk).
template <class CF>
struct SmemState {
  using OP = typename CF::OP;
  static constexpr int KE = Tile<OP, CF::R>::elems(CF::C);
  static constexpr int VE = Tile<OP, CF::DV>::elems(CF::C);
  OP k[2][KE];
  OP k_lo[2][sizeof(OP) == 2 ? KE : 1];
  OP v[2][VE];
};

// LDS of the output kernel: phi(K) and V of the chunk, the carried state (S
// as an MFMA operand, z), and the per-wave row scratch.  The barrier at the
// top of each chunk orders every reuse; with EK the phi(K) tiles of two
// consecutive chunks (the next chunk's is formed during this chunk's
// outputs).
template <class CF, bool EK = false>
struct SmemOut {
  using OP = typename CF::OP;
  OP k[EK ? 2 : 1][Tile<OP, CF::R>::elems(CF::C)];
  OP v[Tile<OP, CF::DV>::elems(CF::C)];
  OP s[Tile<OP, CF::DV>::elems(CF::R)];
  alignas(16) typename CF::ZT z[CF::ZE];
  alignas(16) OP scr[Scratch<CF>::ELEMS];
  // phi(Q) tiles of two consecutive chunks (SharedQ)
  alignas(16) OP sq[SharedQ<CF>::on ? 2 : 1][SharedQ<CF>::on ? Tile<OP, CF::R>::elems(CF::C) : 8];
  __device__ OP* kt(int b) { return k[EK ? b : 0]; }
  __device__ OP* kw_tile() { return nullptr; }
  __device__ float* cum_tile() { return nullptr; }
};
// With a decay: also the keys' features weighted by their decay at the end
// of the chunk, which the state carry contracts (the weights use the plain
// features), and (gated) the chunk's running log2 gates.
template <class CF>
struct SmemOutDecay : SmemOut<CF, false> {
  using OP = typename CF::OP;
  alignas(16) OP kw[Tile<OP, CF::R>::elems(CF::C)];
  alignas(16) float cum[CF::C > 64 ? CF::C : 64];
  __device__ OP* kw_tile() { return kw; }
  __device__ float* cum_tile() { return cum; }
};

// LDS of the non-causal output kernel: the full-sequence sums only.
template <class CF>
struct SmemOutNC {
  using OP = typename CF::OP;
  OP s[Tile<OP, CF::DV>::elems(CF::R)];
  alignas(16) typename CF::ZT z[CF::ZE];
  alignas(16) OP scr[Scratch<CF>::ELEMS];
};

// First token of span s when a head's ceil(N/C) chunks are split as evenly as
// possible over n_span spans (span lengths differ by at most one chunk).
template <class CF>
__device__ __forceinline__ int span_begin(int s, int n_span, int N) {
  const long long n_chunks = (N + CF::C - 1) / CF::C;
  return (int)min((long long)N, CF::C * ((long long)s * n_chunks / n_span));
}

template <class CF>
__device__ __forceinline__ HeadBufs head_bufs(const typename CF::IO* Q, const typename CF::IO* K,
                                              const typename CF::IO* V, typename CF::IO* O, int bh, int N) {
  using T = typename CF::IO;
  const size_t qk = (size_t)N * CF::D, vo = (size_t)N * CF::DV;
  HeadBufs hb;
  hb.q = make_rsrc(Q ? Q + bh * qk : nullptr, (unsigned)(qk * sizeof(T)));
  hb.k = make_rsrc(K + bh * qk, (unsigned)(qk * sizeof(T)));
  hb.v = make_rsrc(V + bh * vo, (unsigned)(vo * sizeof(T)));
  hb.o = make_rsrc(O ? O + bh * vo : nullptr, (unsigned)(vo * sizeof(T)));
  return hb;
}

// Per-span state: dS = phi(K_span)^T V_span, dz = sum phi(K_span) -> ws slot s.
// With a decay (DK != kNoDecay: gamma[head], or the head's per-token log
// gates log_a[bh][N]), the span's sum is decayed to the span's end: key t
// enters with its decay over tokens t+1 .. t_end-1.  Per chunk the running
// sum is multiplied by the chunk's whole decay before the chunk's keys,
// weighted by their decay to the chunk's end, are added.  Gated: the span's
// total log2 gate goes to totals[bh][s] for the span scan.
template <class CF, int DK = kNoDecay>
__global__ __launch_bounds__(CF::NT) void la_state_kernel(const typename CF::IO* __restrict__ K,
                                                            const typename CF::IO* __restrict__ V,
                                                            float* __restrict__ ws, int N, int n_span,
                                                            const float* __restrict__ gamma, int H,
                                                            const float* __restrict__ log_a,
                                                            float* __restrict__ totals) {
  using OP = typename CF::OP;
  constexpr bool GATED = DK == kGated;
  __shared__ SmemState<CF> sm;
  const int tid = threadIdx.x, w = wave_id(), l = tid & 63, g = l >> 4, li = l & 15;
  const int bh = blockIdx.x / n_span;
  const int s = blockIdx.x % n_span;
  const int t_begin = span_begin<CF>(s, n_span, N);
  const int t_end = span_begin<CF>(s + 1, n_span, N);
  HeadBufs hb = head_bufs<CF>(nullptr, K, V, nullptr, bh, N);
  if constexpr (GATED) hb.a = make_rsrc(log_a + (size_t)bh * N, (unsigned)N * 4u);
  const float lg = DK == kFixed ? __builtin_amdgcn_logf(gamma[bh % H]) : 0.f;  // log2(gamma)
  // with a decay: the log2 decay from the end of the chunk being staged to
  // the span's end (the chunks already summed lie after it); at the loop's
  // end, the span's whole log2 decay
  float after = 0.f;

  f32x4 acc[CF::TPW];
#pragma unroll
  for (int i = 0; i < CF::TPW; ++i) acc[i] = zero4();
  f32x4 zt[CF::ZPW];
#pragma unroll
  for (int k = 0; k < CF::ZPW; ++k) zt[k] = zero4();

  // two chunks of loads in flight: chunk c+2 is requested as soon as chunk
  // c has been staged (LDS double buffering, one barrier per chunk).  Every
  // load is issued unconditionally (past the span's end it re-reads the
  // chunk read last, from L2), so that no loop path differs in the number
  // of memory operations and the counter waits stay exact.
  // Order: last chunk to first.  The chunks this kernel reads last are then
  // each span's first ones, which la_output_kernel, walking its spans
  // forward, reads first, while they are the likeliest to still sit in the
  // memory-side cache.  A decay is applied to each chunk's key weights (its
  // decay to the span's end, after), so no running sum is rescaled.
  const int nch = (t_end - t_begin + CF::C - 1) / CF::C;
  auto chunk_t0 = [&](int k) { return t_begin + max(nch - 1 - k, 0) * CF::C; };
  ChunkRegs<CF, false> ca, cb;
  load_chunk<CF, false, GATED>(ca, hb, chunk_t0(0));
  mem_order_fence();  // ca's loads first, as in the loop: exact counter waits
  load_chunk<CF, false, GATED>(cb, hb, chunk_t0(1));
  int buf = 0;
  for (int k = 0; k < nch; k += 2) {
    OP* lo = sizeof(OP) == 2 ? sm.k_lo[buf] : nullptr;
    const int ta = chunk_t0(k);
    after += stage_chunk<CF, false, DK>(ca, nullptr, sm.k[buf], lo, sm.v[buf], ta, N, lg, min(CF::C, t_end - ta),
                                        nullptr, nullptr, after);
    load_chunk<CF, false, GATED>(ca, hb, chunk_t0(k + 2));
    __syncthreads();
    state_mfma<CF>(acc, zt, sm.k[buf], lo, sm.v[buf], w, g, li);
    buf ^= 1;
    const bool second = k + 1 < nch;  // workgroup-uniform
    const int tb = chunk_t0(k + 1);
    lo = sizeof(OP) == 2 ? sm.k_lo[buf] : nullptr;
    if (second)
      after += stage_chunk<CF, false, DK>(cb, nullptr, sm.k[buf], lo, sm.v[buf], tb, N, lg, min(CF::C, t_end - tb),
                                          nullptr, nullptr, after);
    load_chunk<CF, false, GATED>(cb, hb, chunk_t0(k + 3));
    if (second) {
      __syncthreads();
      state_mfma<CF>(acc, zt, sm.k[buf], lo, sm.v[buf], w, g, li);
      buf ^= 1;
    }
  }
  if constexpr (GATED) {
    if (tid == 0) totals[(size_t)bh * n_span + s] = after;
  }

  constexpr int E = CF::R * CF::DV + CF::R;
  float* slot = ws + ((size_t)bh * (n_span + 1) + s) * E;
#pragma unroll
  for (int i = 0; i < CF::TPW; ++i) {
    int ct, ft;
    state_tile<CF>(w, i, ct, ft);
    *reinterpret_cast<f32x4*>(slot + (16 * ft + li) * CF::DV + 16 * ct + 4 * g) = acc[i];
  }
  if (g == 0) {
#pragma unroll
    for (int k = 0; k < CF::ZPW; ++k) slot[CF::R * CF::DV + 16 * (w + CF::NW * k) + li] = zt[k][0];
  }
}

// Exclusive fp32 prefix over spans, element-parallel: slot s becomes the
// state before span s (starting from S0/z0 or zero); slot n_span receives
// the total, which is also copied to S_out/z_out when given.  The summation
// order is fixed, so results are reproducible.  With a decay (DECAY) the
// running state is multiplied by gamma^L before a span of L tokens is added
// (each span's own sum is already decayed to the span's end); the span
// lengths are walked with an incremental quotient and remainder of
// s * n_chunks / n_span, the split span_begin uses.  With gates (kGated)
// the running state is multiplied by 2^totals[bh][s], the span's total log2
// gate, instead; with per-channel gates (kChannel) by 2^totals[bh][s][f]
// for state row f.  TOTAL (the non-causal form, which reads only the
// total): slot n_span alone is written; slots 0 .. n_span - 1 keep the span
// sums.
template <int DK, bool TOTAL = false>
__global__ __launch_bounds__(kThreads) void la_scan_kernel(float* __restrict__ ws, int R, int DV, int n_span,
                                                           const float* __restrict__ S0,
                                                           const float* __restrict__ z0,
                                                           float* __restrict__ S_out,
                                                           float* __restrict__ z_out,
                                                           const float* __restrict__ gamma, int H, int N,
                                                           int chunk, const float* __restrict__ totals,
                                                           const float* __restrict__ kappa) {
  constexpr bool DECAY = DK == kFixed;
  const int E = R * DV + R;
  const int e = blockIdx.x * kThreads + threadIdx.x;
  const int bh = blockIdx.y;
  if (e >= E) return;
  const bool is_s = e < R * DV;
  // states stored at 2^kappa times their value (kappa: log2 per head): the
  // initial state enters, and the final state leaves, rescaled
  const float kp = kappa ? kappa[bh] : 0.f;
  float acc = 0.f;
  if (is_s) {
    if (S0) acc = S0[(size_t)bh * R * DV + e];
  } else {
    if (z0) acc = z0[(size_t)bh * R + (e - R * DV)];
  }
  if (kappa) acc *= __builtin_amdgcn_exp2f(kp);
  float* p = ws + (size_t)bh * (n_span + 1) * E + e;
  float lg = 0.f;                    // log2(gamma)
  int q_ch = 0, r_ch = 0, rem = 0;   // n_chunks = q_ch n_span + r_ch; running remainder
  int t_beg = 0;                     // first token of the current span
  if constexpr (DECAY) {
    lg = __builtin_amdgcn_logf(gamma[bh % H]);
    const int n_chunks = (N + chunk - 1) / chunk;
    q_ch = n_chunks / n_span;
    r_ch = n_chunks % n_span;
  }
  // all loads of a batch are issued before the dependent adds, so a span
  // scan costs ceil(n_span / 16) memory round trips instead of n_span
  constexpr int kBatch = 16;
  for (int s0 = 0; s0 < n_span; s0 += kBatch) {
    float x[kBatch], tl[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) x[j] = s0 + j < n_span ? p[(size_t)(s0 + j) * E] : 0.f;
    if constexpr (DK == kGated) {
#pragma unroll
      for (int j = 0; j < kBatch; ++j) tl[j] = s0 + j < n_span ? totals[(size_t)bh * n_span + s0 + j] : 0.f;
    } else if constexpr (DK == kChannel) {
      // this element's state row (or z entry)
      const int f = is_s ? e / DV : e - R * DV;
#pragma unroll
      for (int j = 0; j < kBatch; ++j)
        tl[j] = s0 + j < n_span ? totals[((size_t)bh * n_span + s0 + j) * R + f] : 0.f;
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      if (s0 + j < n_span) {
        if constexpr (!TOTAL) p[(size_t)(s0 + j) * E] = acc;
        if constexpr (DK == kGated || DK == kChannel) acc *= __builtin_amdgcn_exp2f(tl[j]);
        if constexpr (DECAY) {
          rem += r_ch;
          const int step = q_ch + (rem >= n_span ? 1 : 0);
          rem -= rem >= n_span ? n_span : 0;
          // (32-bit: N < 2^24, as a head's rows fit a 32-bit byte range)
          const int t_e = min(N, t_beg + step * chunk);
          acc *= __builtin_amdgcn_exp2f(lg * (float)(t_e - t_beg));
          t_beg = t_e;
        }
      }
      acc += x[j];
    }
  }
  p[(size_t)n_span * E] = acc;
  if (kappa) acc *= __builtin_amdgcn_exp2f(-kp);
  if (is_s) {
    if (S_out) S_out[(size_t)bh * R * DV + e] = acc;
  } else {
    if (z_out) z_out[(size_t)bh * R + (e - R * DV)] = acc;
  }
}

// Outputs of one span, carrying (S, z) from the span's prefix (causal) or
// reading the full-sequence sums (non-causal: only Q is read).  Causal: chunk
// c+1 is loaded into registers while chunk c is computed; LDS holds one
// chunk, with a barrier before it is overwritten and one after it is written;
// chunk c's outputs are stored before the state update.
// With a decay (DK != kNoDecay, causal only): chunk_outputs applies it to
// the weights and to the carried state's read-out, and the carry is
// S <- D S + sum_j D_j phi(k_j) v_j^T (z likewise), from the weighted
// feature tile, with D the chunk's whole decay and D_j key j's decay to the
// chunk's end (gamma^C and gamma^(C-1-j), or products of the chunk's gates).
template <class CF, bool CAUSAL, int DK = kNoDecay>
__global__ __launch_bounds__(CF::NT, DK != kNoDecay ? CF::MINB_DECAY : CF::MINB) void la_output_kernel(
    const typename CF::IO* __restrict__ Q, const typename CF::IO* __restrict__ K,
    const typename CF::IO* __restrict__ V, typename CF::IO* __restrict__ O, const float* __restrict__ ws, int N,
    int n_span, const float* __restrict__ gamma, int H, int normalize, const float* __restrict__ log_a) {
  constexpr bool DECAY = DK != kNoDecay, GATED = DK == kGated;
  static_assert(CAUSAL || !DECAY, "the decay is defined for the causal form");
  __shared__ typename std::conditional<CAUSAL,
                                       typename std::conditional<DECAY, SmemOutDecay<CF>, SmemOut<CF, CF::NW == 8>>::type,
                                       SmemOutNC<CF>>::type sm;
  const int tid = threadIdx.x, w = wave_id(), l = tid & 63, g = l >> 4, li = l & 15;
  // heads in the reverse order of la_state_kernel: the keys and values
  // that kernel read last are the likeliest to still sit in the
  // memory-side cache
  const int bh = (int)(gridDim.x / n_span) - 1 - (int)(blockIdx.x / n_span);
  const int s = blockIdx.x % n_span;
  const int t_begin = span_begin<CF>(s, n_span, N);
  const int t_end = span_begin<CF>(s + 1, n_span, N);
  HeadBufs hb = head_bufs<CF>(Q, K, V, O, bh, N);
  if constexpr (GATED) hb.a = make_rsrc(log_a + (size_t)bh * N, (unsigned)N * 4u);
  const float lg = DK == kFixed ? __builtin_amdgcn_logf(gamma[bh % H]) : 0.f;  // log2(gamma)

  // carried state: this wave's tiles of S (fp32) and its z tiles
  constexpr int E = CF::R * CF::DV + CF::R;
  const float* pre = ws + ((size_t)bh * (n_span + 1) + (CAUSAL ? s : n_span)) * E;
  f32x4 sacc[CF::TPW];
#pragma unroll
  for (int i = 0; i < CF::TPW; ++i) {
    int ct, ft;
    state_tile<CF>(w, i, ct, ft);
    sacc[i] = *reinterpret_cast<const f32x4*>(pre + (16 * ft + li) * CF::DV + 16 * ct + 4 * g);
  }
  f32x4 zt[CF::ZPW];
#pragma unroll
  for (int k = 0; k < CF::ZPW; ++k) {
    const float zv = pre[CF::R * CF::DV + 16 * (w + CF::NW * k) + li];
    zt[k] = f32x4{zv, zv, zv, zv};
  }

  OutRegs<CF> out;
  if constexpr (!CAUSAL) {
    // non-causal: the full-sequence sums serve every row; only Q is read,
    // two chunks ahead, and each chunk's outputs are stored right away
    publish_state<CF>(sacc, zt, sm.s, sm.z, w, g, li);
    __syncthreads();
    // every step issues its load (past the span's last chunk it re-reads
    // that chunk, from L2), so that the counter wait before each step's
    // phi(Q) waits for that chunk's rows and not for the stores issued
    // after them
    if (t_begin >= t_end) return;
    const int last = t_begin + ((t_end - t_begin - 1) / CF::C) * CF::C;
    QRegs<CF> qa, qb;
    qa.load(hb.q, t_begin, w, g, li);
    qb.load(hb.q, min(t_begin + CF::C, last), w, g, li);
    typename CF::OP* scr = sm.scr + w * Scratch<CF>::PER_WAVE;
    auto step = [&](QRegs<CF>& q, int t0) {
      typename QRegs<CF>::frag qf[CF::RBW][CF::R / CF::KS];
      q.to_frags(qf, scr, g, li);
      q.load(hb.q, min(t0 + 2 * CF::C, last), w, g, li);
      chunk_outputs<CF, false>(qf, nullptr, nullptr, sm.s, sm.z, out, w, g, li);
      store_outputs<CF>(out, hb.o, t0, w, g, li, false, scr);
    };
    for (int t0 = t_begin; t0 < t_end; t0 += 2 * CF::C) {
      step(qa, t0);
      if (t0 + CF::C < t_end) step(qb, t0 + CF::C);
    }
  } else {
    // every memory operation is issued on every iteration (loads past the
    // span re-read its last chunk from L2), and the prologue ends with the
    // loop's memory operations in the loop's order (K and V, then the
    // stores, dropped, then the next chunk's Q), so the counter wait at the
    // loop head is exact: it waits for the prefetched chunk, not for the
    // previous chunk's stores or the Q rows loaded after them
    // (an empty span returns here, so that the prologue and the loop entry
    // are one block and the compiler keeps the prologue's issue order)
    if (t_begin >= t_end) return;
    const int last = t_begin + ((t_end - t_begin - 1) / CF::C) * CF::C;
    constexpr bool SQ = SharedQ<CF>::on;
    const int qib = wave_row_block<CF>(0, w), qh = w / CF::RB;  // (SQ) row block and column half
    ChunkRegs<CF, false> cr;
    QRegs<CF> qr;
    SharedQ<CF> qs;
    auto q_load = [&](int t) {
      if constexpr (SQ)
        qs.load(hb.q, t, qib, qh);
      else
        qr.load(hb.q, t, w, g, li);
    };
    load_chunk<CF, false, GATED>(cr, hb, t_begin);
    mem_order_fence();
    q_load(t_begin);
    mem_order_fence();
    dummy_stores<CF>(hb.o);
    typename CF::OP* scr = sm.scr + w * Scratch<CF>::PER_WAVE;
    int t0 = t_begin;
    // phi(Q) of a chunk is formed at the end of the previous chunk's
    // outputs, in the wave's own scratch (no barrier involved), where its
    // VALU work can issue beside the carry's MFMAs; its Q rows are loaded
    // one chunk ahead of that.  SQ: into the chunk's phi(Q) tile, which
    // both waves of the row block read after the chunk's second barrier
    // (the tile of chunk c + 1 is written after the second barrier of
    // chunk c, by which every wave has read the tile of chunk c - 1)
    typename QRegs<CF>::frag qf[CF::RBW][CF::R / CF::KS];
    int qbuf = 0;
    if constexpr (SQ)
      qs.to_tile(scr, sm.sq[0], qib, qh, g, li);
    else
      qr.to_frags(qf, scr, g, li);
    q_load(min(t0 + CF::C, last));
    // Without a decay, phi(K) of a chunk is likewise formed during the
    // previous chunk's outputs (from the raw rows loaded in its staging
    // phase), into the other of two phi(K) tiles, and the staging phase
    // only publishes the state and copies V: the feature map's VALU work
    // then issues beside MFMAs instead of in a phase of its own.  The tile
    // of chunk c + 1 is written after the second barrier of chunk c, by
    // which every wave is done with the tile of chunk c - 1.  (Eight waves:
    // at four, where two workgroups share a CU and the kernel is bound by
    // its memory stream, back-to-back steps measured slower with it.)
    constexpr bool EK = !DECAY && CF::NW == 8;
    int kb = 0;
    if constexpr (EK) stage_chunk<CF, false, kNoDecay, false>(cr, nullptr, sm.kt(0), nullptr, nullptr, t0, N);
    do {
      __syncthreads();  // every wave is done with the previous chunk's S, z, phi(K), V
      publish_state<CF>(sacc, zt, sm.s, sm.z, w, g, li);
      float l2 = 0.f;
      if constexpr (EK)
        stage_values<CF>(cr, sm.v);
      else
        l2 = stage_chunk<CF, false, DK>(cr, nullptr, sm.kt(0), nullptr, sm.v, t0, N, lg, CF::C, sm.kw_tile(),
                                        sm.cum_tile());
      load_chunk<CF, false, GATED>(cr, hb, min(t0 + CF::C, last));
      __syncthreads();
      if constexpr (SQ) {
        using TQ = Tile<typename CF::OP, CF::R>;
#pragma unroll
        for (int ks = 0; ks < CF::R / CF::KS; ++ks)
          qf[0][ks] = load_frag(sm.sq[qbuf] + TQ::off(16 * qib + li, ks * CF::KS + g * 8));
      }
      chunk_outputs<CF, true, DK>(qf, sm.kt(kb), sm.v, sm.s, sm.z, out, w, g, li, lg, normalize, sm.cum_tile());
      store_outputs<CF>(out, hb.o, t0, w, g, li, false, scr);
      if constexpr (SQ) {
        qbuf ^= 1;
        qs.to_tile(scr, sm.sq[qbuf], qib, qh, g, li);
      } else {
        qr.to_frags(qf, scr, g, li);
      }
      q_load(min(t0 + 2 * CF::C, last));
      // (past the span's last chunk the rows re-read are staged and unused)
      if constexpr (EK)
        stage_chunk<CF, false, kNoDecay, false>(cr, nullptr, sm.kt(kb ^ 1), nullptr, nullptr, t0 + CF::C, N);
      if constexpr (DECAY) {
        // the carry past this chunk (unused after a span's last chunk, so a
        // partial last chunk needs no other length; gates past N are one)
        const float dg = __builtin_amdgcn_exp2f(l2);
#pragma unroll
        for (int i = 0; i < CF::TPW; ++i) sacc[i] *= dg;
#pragma unroll
        for (int k = 0; k < CF::ZPW; ++k) zt[k] *= dg;
        state_mfma<CF>(sacc, zt, sm.kw_tile(), nullptr, sm.v, w, g, li);
      } else {
        state_mfma<CF>(sacc, zt, sm.kt(kb), nullptr, sm.v, w, g, li);
      }
      kb ^= 1;
      t0 += CF::C;
    } while (t0 < t_end);
  }
}


// ------------------------------------------------------------------ per-channel gates

// Causal prefill with a gate per key channel (the GLA form):
//   S_t = diag(a_t) S_{t-1} + phi(k_t) v_t^T,  z_t = a_t z_{t-1} + phi(k_t),
// a_t in (0, 1]^R given as natural logs [B*H][N][R].  Per chunk and channel,
// with lg = max(log2 a, kGlaMinLog2):
//   P_i  the sum of lg over the tokens of i's 16-token block up to i
//        (block-local running sums, an fp32 [C][R] LDS tile);
//   M_b  P at token 7 of block b, T_b P at its token 15 (the block's total).
// Every gate product of the chunk is 2^x with x a short sum of these, and
// each factor goes on one MFMA operand:
//   weight (i, j), j in an earlier block jb:
//       2^(P_i + sum_{jb<b<ib} T_b) on phi(q_i), 2^(T_jb - P_j) on phi(k_j);
//   weight (i, j), same block b, row i among the block's tokens 0..7:
//       2^(P_i) on phi(q_i), 2^(-P_j) on phi(k_j);
//   ... row i among tokens 8..15:  2^(P_i - M_b) on phi(q_i), 2^(M_b - P_j) on phi(k_j);
//   read-out of the carried state, row i:  2^(P_i + sum_{b<ib} T_b);
//   key j's decay to the chunk's end:  2^(T_jb - P_j + sum_{b>jb} T_b);
//   the carried state over the chunk:  2^(sum_b T_b) per state row.
// Row i's factors use gates of tokens up to i only, so no later token can
// change an earlier output, not even in rounding.  Every query factor is at
// most one, and so is every key factor except the same-block ones, which
// lie below 2^(8 |kGlaMinLog2|) = 2^112 on the entries that are kept (at
// most 8 tokens between j and the reference): with features below 2^16 in
// magnitude they stay finite in fp32 and bf16 (largest 2^128), which is
// what the floor is for.  The entries above the diagonal, whose factors may
// overflow, are replaced by selection.
constexpr float kGlaMinLog2 = -14.f;

template <class CF>
struct GlaCfg {
  static constexpr int GV = CF::C * CF::R / 4;   // fp32 gate vectors (4 channels) per chunk
  static constexpr int NU = GV / 64;             // units of 64 vectors: one block x 16 channels
  static constexpr int GPW = NU / CF::NW;        // units per wave
  static constexpr int NQ = CF::R / 4;           // phi(q) values per lane and row block
  static_assert(CF::R % 16 == 0 && NU % CF::NW == 0, "gate units must split evenly over waves");
};

template <class CF>
struct GateRegsGla {
  f32x4 g[GlaCfg<CF>::GPW];
};

// Unit k of the calling wave: block b = u % RB and channels 16 (u / RB) ..
// +15 with u = wave + NW k; lane l holds token 16 b + l % 16 and channels
// 4 (4 (u / RB) + l / 16) .. +3, so each 16-lane row of the wave holds one
// block's tokens of 4 channels, in token order.
template <class CF>
__device__ __forceinline__ void gla_unit(int k, int w, int lane, int& tok, int& ch) {
  const int u = w + CF::NW * k;
  tok = 16 * (u % CF::RB) + (lane & 15);
  ch = 4 * (4 * (u / CF::RB) + (lane >> 4));
}

template <class CF>
__device__ __forceinline__ void load_gates_gla(GateRegsGla<CF>& gr, __amdgpu_buffer_rsrc_t a, int t0) {
  const int w = wave_id(), lane = threadIdx.x & 63;
#pragma unroll
  for (int k = 0; k < GlaCfg<CF>::GPW; ++k) {
    int tok, ch;
    gla_unit<CF>(k, w, lane, tok, ch);
    gr.g[k] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(a, ((t0 + tok) * CF::R + ch) * 4, 0, 0));
  }
}

// Clamped log2 gates -> block-local running sums (a prefix over each 16-lane
// row, in DPP moves) -> the P tile.
template <class CF>
__device__ __forceinline__ void gla_prefix_to_lds(const GateRegsGla<CF>& gr, float* sp) {
  using TP = Tile<float, CF::R>;
  const int w = wave_id(), lane = threadIdx.x & 63;
#pragma unroll
  for (int k = 0; k < GlaCfg<CF>::GPW; ++k) {
    f32x4 x = gr.g[k];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float y = fmaxf(x[e] * kLog2e, kGlaMinLog2);
      y = dpp_add<0x111>(y);  // row_shr:1
      y = dpp_add<0x112>(y);  // row_shr:2
      y = dpp_add<0x114>(y);  // row_shr:4
      y = dpp_add<0x118>(y);  // row_shr:8
      x[e] = y;
    }
    int tok, ch;
    gla_unit<CF>(k, w, lane, tok, ch);
    *reinterpret_cast<f32x4*>(sp + TP::off(tok, ch)) = x;
  }
}

// phi(K) of the chunk, weighted, -> LDS (reads the P tile):
//   skw   phi(k_j) 2^(T_jb - P_j + sum_{b>jb} T_b)  (decay to the chunk's end;
//         with skw_lo its bf16 rounding residual too)
//   OUT:  skd0 phi(k_j) 2^(-P_j), skd1 phi(k_j) 2^(M_jb - P_j) (same-block
//         weights of rows 0..7 and 8..15), skb phi(k_j) 2^(T_jb - P_j).
// With base given, skw's weights also carry 2^base[e] for this thread's
// channels col + e (its channels are the same for every unit it stages): a
// decay from the chunk's end to a later reference token, per channel.
// Keys at or beyond N get zero features.
template <class CF, bool OUT>
__device__ __forceinline__ void gla_stage_keys(const ChunkRegs<CF, false>& cr, const float* sp,
                                               typename CF::OP* skd0, typename CF::OP* skd1, typename CF::OP* skb,
                                               typename CF::OP* skw, typename CF::OP* skw_lo, int t0, int N,
                                               const float* base = nullptr) {
  using T = typename CF::IO;
  using OP = typename CF::OP;
  using TQ = Tile<OP, CF::R>;
  using TP = Tile<float, CF::R>;
  constexpr int QV = CF::D / CF::EPL, EPL = CF::EPL, RB = CF::RB;
  const int tid = threadIdx.x;
  auto row = [&](int r, int col, float* x) {
#pragma unroll
    for (int e4 = 0; e4 < EPL / 4; ++e4) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(sp + TP::off(r, col + 4 * e4));
#pragma unroll
      for (int e = 0; e < 4; ++e) x[4 * e4 + e] = v[e];
    }
  };
#pragma unroll
  for (int i = 0; i < CF::LQ; ++i) {
    const int vi = tid + i * CF::NT;
    if (!(CF::VQ % CF::NT == 0 || vi < CF::VQ)) continue;
    const int tok = vi / QV;
    const int col = (vi % QV) * EPL;
    const int jb = tok >> 4;
    float f[EPL], pj[EPL], tj[EPL], after[EPL];
    unpack16<T>(cr.k[i], f);
#pragma unroll
    for (int e = 0; e < EPL; ++e) f[e] = phi_pointwise<CF::PHI>(f[e]);
    row(tok, col, pj);
    row(16 * jb + 15, col, tj);
#pragma unroll
    for (int e = 0; e < EPL; ++e) after[e] = base ? base[e] : 0.f;
#pragma unroll
    for (int b = 1; b < RB; ++b) {
      if (b > jb) {
        float tb[EPL];
        row(16 * b + 15, col, tb);
#pragma unroll
        for (int e = 0; e < EPL; ++e) after[e] += tb[e];
      }
    }
    const bool valid = t0 + tok < N;
    const u32x4 zero = u32x4{0u, 0u, 0u, 0u};
    float kw[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) kw[e] = f[e] * __builtin_amdgcn_exp2f(tj[e] - pj[e] + after[e]);
    const u32x4 hw = pack16<OP>(kw);
    *reinterpret_cast<u32x4*>(skw + TQ::off(tok, col)) = valid ? hw : zero;
    if constexpr (sizeof(OP) == 2) {
      if (skw_lo) {
        float h[EPL], r[EPL];
        unpack16<bf16>(hw, h);
#pragma unroll
        for (int e = 0; e < EPL; ++e) r[e] = kw[e] - h[e];
        const u32x4 lo = pack16<OP>(r);
        *reinterpret_cast<u32x4*>(skw_lo + TQ::off(tok, col)) = valid ? lo : zero;
      }
    }
    if constexpr (OUT) {
      float mj[EPL], kd0[EPL], kd1[EPL], kb[EPL];
      row(16 * jb + 7, col, mj);
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        kd0[e] = f[e] * __builtin_amdgcn_exp2f(-pj[e]);
        kd1[e] = f[e] * __builtin_amdgcn_exp2f(mj[e] - pj[e]);
        kb[e] = f[e] * __builtin_amdgcn_exp2f(tj[e] - pj[e]);
      }
      const u32x4 x0 = pack16<OP>(kd0), x1 = pack16<OP>(kd1), xb = pack16<OP>(kb);
      *reinterpret_cast<u32x4*>(skd0 + TQ::off(tok, col)) = valid ? x0 : zero;
      *reinterpret_cast<u32x4*>(skd1 + TQ::off(tok, col)) = valid ? x1 : zero;
      *reinterpret_cast<u32x4*>(skb + TQ::off(tok, col)) = valid ? xb : zero;
    }
  }
}

// Output rows of one chunk with per-channel gates: chunk_outputs' causal
// product with the operand scalings listed above.  fq: this wave's phi(q)
// values in fp32 (QRegs::to_f32 order).  Key blocks are taken from the
// diagonal down, so that the query scaling for block jb is the one for jb+1
// plus T_{jb+1}.
template <class CF>
__device__ __forceinline__ void chunk_outputs_gla(const float (&fq)[CF::RBW][CF::R / 4], const typename CF::OP* skd0,
                                                  const typename CF::OP* skd1, const typename CF::OP* skb,
                                                  const typename CF::OP* sv,
                                                  const typename CF::OP* ss, const typename CF::ZT* sz,
                                                  const float* sp, OutRegs<CF>& out, int w, int g, int li,
                                                  int normalize) {
  using OP = typename CF::OP;
  using frag = typename Op<OP>::frag;
  using TQ = Tile<OP, CF::R>;
  using TV = Tile<OP, CF::DV>;
  using TP = Tile<float, CF::R>;
  constexpr int KS = CF::KS, PL = CF::PL, RB = CF::RB, CTW = CF::CTW, R = CF::R, DV = CF::DV;
  constexpr int NQ = GlaCfg<CF>::NQ;
  const bf16 one = static_cast<bf16>(1.0f), zero = static_cast<bf16>(0.0f);
  const bf16 o1 = (li & 3) == 0 ? one : zero;
  const bf16x8 ones_rows = bf16x8{o1, o1, o1, o1, o1, o1, o1, o1};
  const int zrow = min(li & 3, 2);
  // feature of value n of this lane (QRegs::to_f32 order); groups of 4
  // consecutive n are consecutive features
  auto chan = [&](int n) { return PL == 8 ? 32 * (n >> 3) + 8 * g + (n & 7) : 16 * g + n; };
  auto row_vals = [&](int r, float (&x)[NQ]) {
#pragma unroll
    for (int n4 = 0; n4 < NQ / 4; ++n4) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(sp + TP::off(r, chan(4 * n4)));
#pragma unroll
      for (int e = 0; e < 4; ++e) x[4 * n4 + e] = v[e];
    }
  };
#pragma unroll
  for (int rbi = 0; rbi < CF::RBW; ++rbi) {
    const int ib = wave_row_block<CF>(rbi, w);
    const int ct0 = (RB >= CF::NW) ? 0 : (w / RB) * CTW;
    // phi(q_i) scaled by 2^x, rounded to MFMA operands
    auto scaled = [&](const float (&x)[NQ], frag (&qs)[R / KS]) {
      if constexpr (PL == 8) {
#pragma unroll
        for (int ks = 0; ks < R / KS; ++ks) {
          float f8[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) f8[e] = fq[rbi][8 * ks + e] * __builtin_amdgcn_exp2f(x[8 * ks + e]);
          qs[ks] = cvt_bf16x8(f8);
        }
      } else {
#pragma unroll
        for (int ks = 0; ks < R / KS; ++ks) qs[ks] = fq[rbi][ks] * __builtin_amdgcn_exp2f(x[ks]);
      }
    };
    // x = P_i + sum_{jb < b < ib} T_b: the query scaling for key block jb.
    // The key blocks are visited in descending order (the diagonal first,
    // which reads x while it is still P_i); advance(jb) adds the block totals
    // T_b for jb < b < ib not yet in x, advance(-1) those for b < ib.
    float x[NQ];
    row_vals(16 * ib + li, x);
    auto add_block = [&](int b) {
      float tb[NQ];
      row_vals(16 * b + 15, tb);
#pragma unroll
      for (int n = 0; n < NQ; ++n) x[n] += tb[n];
    };
    int x_at = ib - 1;  // loop form: x holds the totals of the blocks above x_at
    auto advance = [&](int jb) {
      if constexpr (NQ <= 16) {
        // each descending step adds exactly one block, T_{jb+1}: a
        // wave-uniform branch and no loop, so x stays in its registers
        // (the loop form's merges copied it: 2 % slower at d = 64)
        if (jb + 1 < RB && jb + 1 < ib) add_block(jb + 1);
      } else {
        // at d = 128 the unrolled steps need more registers than the kernel
        // has (it spilled and ran 1.5x slower); the loop form stays
        while (x_at > jb) add_block(x_at--);
      }
    };

    float den = 0.f;
    f32x4 dacc = zero4();
    f32x4 o[CTW];
#pragma unroll
    for (int c = 0; c < CTW; ++c) o[c] = zero4();

    auto contract = [&](const OP* kt, int jb, const frag (&qs)[R / KS]) {
      f32x4 t = zero4();
#pragma unroll
      for (int ks = 0; ks < R / KS; ++ks) {
        if constexpr (PL == 8) {
          t = mfma16(load_frag(kt + TQ::off(16 * jb + li, ks * KS + g * PL)), qs[ks], t);
        } else {
          t = mfma16(kt[TQ::off(16 * jb + li, QRegs<CF>::feature(ks, g))], qs[ks], t);
        }
      }
      return t;
    };
    auto weights = [&](int jb) {
      frag qs[R / KS];
      f32x4 t;
      if (jb == ib) {
        // rows 0..7 of the block: reference at the block's start; rows
        // 8..15: at its token 7.  Each lane scales its own row's phi(q);
        // both contractions cover all 16 rows and each lane keeps its own.
        float xd[NQ];
        row_vals(16 * ib + 7, xd);
#pragma unroll
        for (int n = 0; n < NQ; ++n) xd[n] = li < 8 ? x[n] : x[n] - xd[n];
        scaled(xd, qs);
        const f32x4 t0 = contract(skd0, jb, qs);
        const f32x4 t1 = contract(skd1, jb, qs);
#pragma unroll
        for (int r = 0; r < 4; ++r) t[r] = li < 8 ? t0[r] : t1[r];
      } else {
        advance(jb);
        scaled(x, qs);
        t = contract(skb, jb, qs);
      }
      if constexpr (PL == 8) {
        if (jb == ib) {
#pragma unroll
          for (int r = 0; r < 4; ++r) t[r] = 4 * g + r > li ? 0.f : t[r];
        }
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float xv = (jb == ib && 4 * g + r > li) ? 0.f : t[r];
          t[r] = xv;
          den += xv;
        }
      }
      return t;
    };
#pragma unroll
    for (int jp = (RB + 1) / 2 - 1; jp >= 0; --jp) {
      const int jb0 = 2 * jp, jb1 = 2 * jp + 1;
      if (jb0 > ib) continue;
      const bool two = jb1 < RB && jb1 <= ib;
      const f32x4 a1 = two ? weights(jb1) : zero4();
      const f32x4 a0 = weights(jb0);
      if constexpr (PL == 8) {
        const float w8[8] = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
        const bf16x8 bv = cvt_bf16x8(w8);
        dacc = mfma16(ones_rows, bv, dacc);
#pragma unroll
        for (int cti = 0; cti < CTW; ++cti) {
          const int ct = ct0 + cti;
          const bf16x8 av = two ? tr_frag<DV>(sv, 16 * jb0 + 4 * g, 16 * jb1 + 4 * g, 16 * ct, li)
                                : tr_frag_lo<DV>(sv, 16 * jb0 + 4 * g, 16 * ct, li);
          o[cti] = mfma16(av, bv, o[cti]);
        }
      } else {
#pragma unroll
        for (int cti = 0; cti < CTW; ++cti) {
          const int ct = ct0 + cti;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            o[cti] = mfma16(sv[TV::off(16 * jb0 + 4 * g + r, 16 * ct + li)], a0[r], o[cti]);
            if (two) o[cti] = mfma16(sv[TV::off(16 * jb1 + 4 * g + r, 16 * ct + li)], a1[r], o[cti]);
          }
        }
      }
    }

    // read-out of the carried state and its z term: phi(q_i) 2^(P_i + sum_{b<ib} T_b)
    advance(-1);
    {
      frag qs[R / KS];
      scaled(x, qs);
#pragma unroll
      for (int ks = 0; ks < R / KS; ++ks) {
        if constexpr (PL == 1) {
          den += qs[ks] * sz[QRegs<CF>::feature(ks, g)];
        } else {
          dacc = mfma16(load_frag(sz + zrow * R + ks * KS + g * PL), qs[ks], dacc);
        }
      }
#pragma unroll
      for (int cti = 0; cti < CTW; ++cti) {
        const int ct = ct0 + cti;
#pragma unroll
        for (int ks = 0; ks < R / KS; ++ks) {
          if constexpr (PL == 8) {
            o[cti] = mfma16(tr_frag<DV>(ss, ks * 32 + 8 * g, ks * 32 + 8 * g + 4, 16 * ct, li), qs[ks], o[cti]);
          } else {
            o[cti] = mfma16(ss[TV::off(QRegs<CF>::feature(ks, g), 16 * ct + li)], qs[ks], o[cti]);
          }
        }
      }
    }

    if constexpr (PL == 8) {
      den = dacc[0] + dacc[1];
    } else {
      den = xor_sum16_32(den);
    }
    const float rden = normalize ? __builtin_amdgcn_rcpf(den) : 1.f;
#pragma unroll
    for (int cti = 0; cti < CTW; ++cti) {
      if constexpr (sizeof(typename CF::IO) == 2) {
        out.v[rbi][cti] = cvt_bf16x4(o[cti] * rden);
      } else {
        out.v[rbi][cti] = o[cti] * rden;
      }
    }
  }
}

// This lane's state row f = 16 w + li: the log2 of its decay over the chunk,
// sum_b T_b.
template <class CF>
__device__ __forceinline__ float gla_chunk_l2(const float* sp, int w, int li) {
  using TP = Tile<float, CF::R>;
  float c = 0.f;
#pragma unroll
  for (int b = 0; b < CF::RB; ++b) c += sp[TP::off(16 * b + 15, 16 * w + li)];
  return c;
}

template <class CF>
struct SmemStateGla {
  using OP = typename CF::OP;
  OP kw[Tile<OP, CF::R>::elems(CF::C)];
  OP kw_lo[sizeof(OP) == 2 ? Tile<OP, CF::R>::elems(CF::C) : 1];
  OP v[Tile<OP, CF::DV>::elems(CF::C)];
  alignas(16) float p[Tile<float, CF::R>::elems(CF::C)];
};

template <class CF>
struct SmemOutGla {
  using OP = typename CF::OP;
  OP kd0[Tile<OP, CF::R>::elems(CF::C)];
  OP kd1[Tile<OP, CF::R>::elems(CF::C)];
  OP kb[Tile<OP, CF::R>::elems(CF::C)];
  OP kw[Tile<OP, CF::R>::elems(CF::C)];
  OP v[Tile<OP, CF::DV>::elems(CF::C)];
  OP s[Tile<OP, CF::DV>::elems(CF::R)];
  alignas(16) typename CF::ZT z[CF::ZE];
  alignas(16) OP scr[Scratch<CF>::ELEMS];
  alignas(16) float p[Tile<float, CF::R>::elems(CF::C)];
};

// Whether the per-channel gated kernels of this configuration fit the LDS.
template <class CF>
constexpr bool gla_fits() {
  return sizeof(SmemOutGla<CF>) <= 160 * 1024 && sizeof(SmemStateGla<CF>) <= 160 * 1024;
}

// Per-span state with per-channel gates: the span's sum decayed to its end.
// The chunks go last to first (as in la_state_kernel), and key j of a chunk
// is weighted by its decay to the span's end: to the chunk's end, times the
// decay of the chunks already summed, per channel (the thread's running sum
// of their totals sum_b T_b).  The span's total log2 gate per channel goes
// to totals[bh][s][R].  One LDS buffer, three barriers per chunk (the P tile
// is complete before the keys are weighted).
template <class CF>
__global__ __launch_bounds__(CF::NT) void la_state_kernel_gla(const typename CF::IO* __restrict__ K,
                                                                const typename CF::IO* __restrict__ V,
                                                                float* __restrict__ ws, int N, int n_span,
                                                                const float* __restrict__ log_a,
                                                                float* __restrict__ totals) {
  using OP = typename CF::OP;
  __shared__ SmemStateGla<CF> sm;
  const int tid = threadIdx.x, w = wave_id(), l = tid & 63, g = l >> 4, li = l & 15;
  const int bh = blockIdx.x / n_span;
  const int s = blockIdx.x % n_span;
  const int t_begin = span_begin<CF>(s, n_span, N);
  const int t_end = span_begin<CF>(s + 1, n_span, N);
  HeadBufs hb = head_bufs<CF>(nullptr, K, V, nullptr, bh, N);
  hb.a = make_rsrc(log_a + (size_t)bh * N * CF::R, (unsigned)N * CF::R * 4u);

  f32x4 acc[CF::TPW];
#pragma unroll
  for (int i = 0; i < CF::TPW; ++i) acc[i] = zero4();
  f32x4 zt[CF::ZPW];
#pragma unroll
  for (int k = 0; k < CF::ZPW; ++k) zt[k] = zero4();
  float span_l2 = 0.f;  // row 16 w + li: the span's total log2 gate so far
  // this thread's staging channels col .. col + EPL - 1: the log2 decay of
  // the chunks already summed (the decay from the next chunk's end to the
  // span's end)
  using TP = Tile<float, CF::R>;
  static_assert(CF::NT % (CF::D / CF::EPL) == 0, "a thread stages the same channels in every unit");
  const int col = (tid % (CF::D / CF::EPL)) * CF::EPL;
  float base[CF::EPL];
#pragma unroll
  for (int e = 0; e < CF::EPL; ++e) base[e] = 0.f;

  const int nch = (t_end - t_begin + CF::C - 1) / CF::C;
  auto chunk_t0 = [&](int k) { return t_begin + max(nch - 1 - k, 0) * CF::C; };
  ChunkRegs<CF, false> cr;
  GateRegsGla<CF> gr;
  load_gates_gla<CF>(gr, hb.a, chunk_t0(0));
  load_chunk<CF, false>(cr, hb, chunk_t0(0));
  OP* lo = sizeof(OP) == 2 ? sm.kw_lo : nullptr;
  for (int k = 0; k < nch; ++k) {
    const int t0 = chunk_t0(k);
    __syncthreads();  // the previous chunk's MFMA work is done with kw, v
    gla_prefix_to_lds<CF>(gr, sm.p);
    stage_values<CF>(cr, sm.v);
    __syncthreads();
    gla_stage_keys<CF, false>(cr, sm.p, nullptr, nullptr, nullptr, sm.kw, lo, t0, N, base);
    span_l2 += gla_chunk_l2<CF>(sm.p, w, li);
#pragma unroll
    for (int b = 0; b < CF::RB; ++b) {
#pragma unroll
      for (int e4 = 0; e4 < CF::EPL / 4; ++e4) {
        const f32x4 tb = *reinterpret_cast<const f32x4*>(sm.p + TP::off(16 * b + 15, col + 4 * e4));
#pragma unroll
        for (int e = 0; e < 4; ++e) base[4 * e4 + e] += tb[e];
      }
    }
    const int tn = chunk_t0(k + 1);
    load_gates_gla<CF>(gr, hb.a, tn);
    load_chunk<CF, false>(cr, hb, tn);
    __syncthreads();
    state_mfma<CF>(acc, zt, sm.kw, lo, sm.v, w, g, li);
  }

  constexpr int E = CF::R * CF::DV + CF::R;
  float* slot = ws + ((size_t)bh * (n_span + 1) + s) * E;
#pragma unroll
  for (int i = 0; i < CF::TPW; ++i) {
    int ct, ft;
    state_tile<CF>(w, i, ct, ft);
    *reinterpret_cast<f32x4*>(slot + (16 * ft + li) * CF::DV + 16 * ct + 4 * g) = acc[i];
  }
  if (g == 0) {
    slot[CF::R * CF::DV + 16 * w + li] = zt[0][0];
    totals[((size_t)bh * n_span + s) * CF::R + 16 * w + li] = span_l2;
  }
}

// Outputs of one span with per-channel gates (causal): la_output_kernel's
// chunk walk with the P tile, four weighted key tiles and one more barrier
// per chunk (the keys are weighted once the P tile is complete).
template <class CF>
__global__ __launch_bounds__(CF::NT, CF::MINB_DECAY) void la_output_kernel_gla(
    const typename CF::IO* __restrict__ Q, const typename CF::IO* __restrict__ K,
    const typename CF::IO* __restrict__ V, typename CF::IO* __restrict__ O, const float* __restrict__ ws, int N,
    int n_span, const float* __restrict__ log_a, int normalize) {
  __shared__ SmemOutGla<CF> sm;
  const int tid = threadIdx.x, w = wave_id(), l = tid & 63, g = l >> 4, li = l & 15;
  const int bh = (int)(gridDim.x / n_span) - 1 - (int)(blockIdx.x / n_span);
  const int s = blockIdx.x % n_span;
  const int t_begin = span_begin<CF>(s, n_span, N);
  const int t_end = span_begin<CF>(s + 1, n_span, N);
  HeadBufs hb = head_bufs<CF>(Q, K, V, O, bh, N);
  hb.a = make_rsrc(log_a + (size_t)bh * N * CF::R, (unsigned)N * CF::R * 4u);

  constexpr int E = CF::R * CF::DV + CF::R;
  const float* pre = ws + ((size_t)bh * (n_span + 1) + s) * E;
  f32x4 sacc[CF::TPW];
#pragma unroll
  for (int i = 0; i < CF::TPW; ++i) {
    int ct, ft;
    state_tile<CF>(w, i, ct, ft);
    sacc[i] = *reinterpret_cast<const f32x4*>(pre + (16 * ft + li) * CF::DV + 16 * ct + 4 * g);
  }
  f32x4 zt[CF::ZPW];
  {
    const float zv = pre[CF::R * CF::DV + 16 * w + li];
    zt[0] = f32x4{zv, zv, zv, zv};
  }

  // the same exact counter waits as la_output_kernel: the prologue issues
  // the loop's memory operations in the loop's order (gates, K and V, Q,
  // then the stores, dropped)
  if (t_begin >= t_end) return;
  const int last = t_begin + ((t_end - t_begin - 1) / CF::C) * CF::C;
  ChunkRegs<CF, false> cr;
  GateRegsGla<CF> gr;
  QRegs<CF> qr;
  load_gates_gla<CF>(gr, hb.a, t_begin);
  load_chunk<CF, false>(cr, hb, t_begin);
  mem_order_fence();
  qr.load(hb.q, t_begin, w, g, li);
  mem_order_fence();
  dummy_stores<CF>(hb.o);
  typename CF::OP* scr = sm.scr + w * Scratch<CF>::PER_WAVE;
  OutRegs<CF> out;
  int t0 = t_begin;
  do {
    __syncthreads();  // every wave is done with the previous chunk's tiles
    publish_state<CF>(sacc, zt, sm.s, sm.z, w, g, li);
    gla_prefix_to_lds<CF>(gr, sm.p);
    stage_values<CF>(cr, sm.v);
    float fq[CF::RBW][GlaCfg<CF>::NQ];
    qr.to_f32(fq, scr, g, li);
    __syncthreads();  // the P tile is complete
    gla_stage_keys<CF, true>(cr, sm.p, sm.kd0, sm.kd1, sm.kb, sm.kw, nullptr, t0, N);
    const int tn = min(t0 + CF::C, last);
    load_gates_gla<CF>(gr, hb.a, tn);
    load_chunk<CF, false>(cr, hb, tn);
    qr.load(hb.q, tn, w, g, li);
    __syncthreads();
    chunk_outputs_gla<CF>(fq, sm.kd0, sm.kd1, sm.kb, sm.v, sm.s, sm.z, sm.p, out, w, g, li, normalize);
    store_outputs<CF>(out, hb.o, t0, w, g, li, false, scr);
    // the carry past this chunk (gates past N are one)
    const float dg = __builtin_amdgcn_exp2f(gla_chunk_l2<CF>(sm.p, w, li));
#pragma unroll
    for (int i = 0; i < CF::TPW; ++i) sacc[i] *= dg;
    zt[0] *= dg;
    state_mfma<CF>(sacc, zt, sm.kw, nullptr, sm.v, w, g, li);
    t0 += CF::C;
  } while (t0 < t_end);
}


// ------------------------------------------------------------------ backward

// Gradients of the causal, normalised output (no initial state) for an
// upstream gradient dO.  With A_ij = phi(q_i).phi(k_j) (j <= i), D_i =
// sum_j A_ij, O_i = sum_j A_ij v_j / D_i, g_i = dO_i / D_i and h_i =
// -(dO_i . O_i) / D_i:
//   dphi(q_i) = sum_{j<=i} (v_j.g_i + h_i) phi(k_j) = S_i g_i + h_i z_i
//   dphi(k_j) = sum_{i>=j} (v_j.g_i + h_i) phi(q_i) = R_j v_j + u_j
//   dv_j      = sum_{i>=j} A_ij g_i                  = R_j^T phi(k_j)
// with the prefix state S_i, z_i of the forward and the suffix state
// R_j = sum_{i>=j} phi(q_i) g_i^T, u_j = sum_{i>=j} phi(q_i) h_i; then
// dq = dphi(q) * phi'(q), and phi' = min(1, phi) for ELU+1 (1 for x > 0,
// e^x = phi(x) otherwise), 1 for the identity.  Chunkwise like the forward:
//   pass A (la_bwd_dq_kernel), spans walked forward from the forward's span
//     prefix: per chunk the masked weights give D_i (as the forward does),
//     then g, h, W_ij = v_j.g_i + h_i (MFMA, masked) and dphi(q) = W phi(K)
//     + S g + h z; D_i and h_i go to the workspace, and the span's own
//     reverse sums dR = phi(Q)^T G, du = sum phi(q) h to a second set of
//     span slots;
//   a reverse scan of those slots gives each span the suffix (R, u) of the
//     later spans;
//   pass B (la_bwd_dkv_kernel), spans walked backward: per chunk
//     A^T, W^T (MFMA, masked i >= j), dv = A^T G + R^T phi(K), dphi(k) =
//     W^T phi(Q) + R v + u, then R += phi(Q)^T G, u += sum phi(q) h.
// Arithmetic as in the forward: bf16 operands (phi, V, g, the weights), fp32
// accumulation and states.

// phi'(x) from phi(x) for the pointwise maps.
template <int PHI>
__device__ __forceinline__ float phi_deriv_from_phi(float p) {
  if constexpr (PHI == PHI_ELU1) return fminf(p, 1.f);
  return 1.f;
}

// acc += X^T Y over the chunk's tokens, as state_mfma but with the tiles
// named (sx: the row operand, [C][R] phi(Q) or phi(K); sy: [C][DV] G or V),
// and the z-like row weighted per token by sw[token] (fp32, or all ones
// when sw is null).
template <class CF>
__device__ __forceinline__ void state_mfma_w(f32x4 (&acc)[CF::TPW], f32x4 (&zt)[CF::ZPW], const bf16* sx,
                                             const bf16* sy, const float* sw, int w, int g, int li) {
  constexpr int R = CF::R, DV = CF::DV;
  static_assert(CF::C >= 32, "k-steps of 32 tokens");
  const bf16 one = static_cast<bf16>(1.0f);
#pragma unroll
  for (int ks = 0; ks < CF::C / 32; ++ks) {
    const int ra = ks * 32 + 8 * g;
    const bf16x8 kh = tr_frag<R>(sx, ra, ra + 4, 16 * w, li);
#pragma unroll
    for (int i = 0; i < CF::TPW; ++i) {
      const bf16x8 a = tr_frag<DV>(sy, ra, ra + 4, 16 * i, li);
      acc[i] = mfma16(a, kh, acc[i]);
    }
    bf16x8 wv;
    if (sw) {
      // k-slots of this lane: tokens ra .. ra + 3, ra + 4 .. ra + 7
      const f32x4 w0 = *reinterpret_cast<const f32x4*>(sw + ra);
      const f32x4 w1 = *reinterpret_cast<const f32x4*>(sw + ra + 4);
      const float w8[8] = {w0[0], w0[1], w0[2], w0[3], w1[0], w1[1], w1[2], w1[3]};
      wv = cvt_bf16x8(w8);
    } else {
      wv = bf16x8{one, one, one, one, one, one, one, one};
    }
    zt[0] = mfma16(wv, kh, zt[0]);
  }
}

template <class CF>
struct SmemBwdA {
  using OP = typename CF::OP;
  OP k[Tile<OP, CF::R>::elems(CF::C)];
  OP v[Tile<OP, CF::DV>::elems(CF::C)];
  OP s[Tile<OP, CF::DV>::elems(CF::R)];
  OP q[Tile<OP, CF::R>::elems(CF::C)];     // phi(Q) rows of the chunk
  OP gt[Tile<OP, CF::DV>::elems(CF::C)];   // g rows of the chunk
  alignas(16) float h[CF::C];
  alignas(16) typename CF::ZT z[CF::ZE];
  alignas(16) OP scr[Scratch<CF>::ELEMS];
};

// Pass A: dQ, and per token (D_i, h_i) -> dh[bh][N][2]; per span the reverse
// sums -> wsb slot s.  O and dO are read in the layout of Q.
template <class CF>
__global__ __launch_bounds__(CF::NT, CF::NW == 8 ? 1 : 2) void la_bwd_dq_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V, const bf16* __restrict__ O,
    const bf16* __restrict__ dO, bf16* __restrict__ dQ, const float* __restrict__ ws, float* __restrict__ wsb,
    float* __restrict__ dh, int N, int n_span) {
  using OP = typename CF::OP;
  static_assert(sizeof(OP) == 2 && CF::RBW == 1 && CF::R == CF::DV && CF::CTW * CF::WPR == CF::CT,
                "one 16-row block per wave (WPR waves share it, each with its share of the column tiles), d = d_v");
  constexpr int R = CF::R, DV = CF::DV, KS = CF::KS, RB = CF::RB, FT = CF::FT;
  using TQ = Tile<OP, R>;
  using TV = Tile<OP, DV>;
  __shared__ SmemBwdA<CF> sm;
  const int tid = threadIdx.x, w = wave_id(), l = tid & 63, g = l >> 4, li = l & 15;
  const int bh = blockIdx.x / n_span;
  const int s = blockIdx.x % n_span;
  const int t_begin = span_begin<CF>(s, n_span, N);
  const int t_end = span_begin<CF>(s + 1, n_span, N);
  const HeadBufs hb = head_bufs<CF>(Q, K, V, dQ, bh, N);
  const size_t qk = (size_t)N * CF::D;
  const __amdgpu_buffer_rsrc_t r_o = make_rsrc(O + bh * qk, (unsigned)(qk * 2));
  const __amdgpu_buffer_rsrc_t r_do = make_rsrc(dO + bh * qk, (unsigned)(qk * 2));
  const __amdgpu_buffer_rsrc_t r_dh = make_rsrc(dh + (size_t)bh * N * 2, (unsigned)N * 8u);

  constexpr int E = R * DV + R;
  const float* pre = ws + ((size_t)bh * (n_span + 1) + s) * E;
  f32x4 sacc[CF::TPW], racc[CF::TPW];
#pragma unroll
  for (int i = 0; i < CF::TPW; ++i) {
    int ct, ft;
    state_tile<CF>(w, i, ct, ft);
    sacc[i] = *reinterpret_cast<const f32x4*>(pre + (16 * ft + li) * DV + 16 * ct + 4 * g);
    racc[i] = zero4();
  }
  f32x4 zt[1], ut[1];
  {
    const float zv = pre[R * DV + 16 * w + li];
    zt[0] = f32x4{zv, zv, zv, zv};
    ut[0] = zero4();
  }
  const bf16 one = static_cast<bf16>(1.0f), zero = static_cast<bf16>(0.0f);
  const bf16 o1 = (li & 3) == 0 ? one : zero;
  const bf16x8 ones_rows = bf16x8{o1, o1, o1, o1, o1, o1, o1, o1};
  const int zrow = min(li & 3, 2);
  // this wave's row block; with eight waves two share a block and each
  // takes half of the feature tiles of dQ
  constexpr int FTW = FT / CF::WPR;
  // four waves form the span's reverse sums here; eight (d = 128) leave
  // them to la_bwd_rsum_kernel (no registers for a second 128 x 128 state)
  constexpr bool RSUM = CF::NW == 4;
  const int ib = wave_row_block<CF>(0, w), half = w / RB, ft0 = half * FTW;
  OP* scr = sm.scr + w * Scratch<CF>::PER_WAVE;

  // four waves: chunk c+1 is loaded into registers while chunk c is
  // computed; eight (d = 128) have registers to spare for chunk c+1's K and
  // V only, and load its Q, O and dO rows at the top of its iteration
  constexpr bool PREFETCH = CF::NW == 4;
  const int last = t_end > t_begin ? t_begin + ((t_end - t_begin - 1) / CF::C) * CF::C : t_begin;
  ChunkRegs<CF, false> cr;
  QRegs<CF> qr, orr, dor;
  auto load_rows = [&](int tc) {
    qr.load(hb.q, tc, w, g, li);
    orr.load(r_o, tc, w, g, li);
    dor.load(r_do, tc, w, g, li);
  };
  auto load_all = [&](int tc) {
    load_chunk<CF, false>(cr, hb, tc);
    load_rows(tc);
  };
  if constexpr (PREFETCH)
    load_all(t_begin);
  else
    load_chunk<CF, false>(cr, hb, t_begin);
  for (int t0 = t_begin; t0 < t_end; t0 += CF::C) {
    if constexpr (!PREFETCH) load_rows(t0);
    __syncthreads();  // every wave is done with the previous chunk's tiles
    publish_state<CF>(sacc, zt, sm.s, sm.z, w, g, li);
    stage_chunk<CF, false>(cr, nullptr, sm.k, nullptr, sm.v, t0, N);
    typename QRegs<CF>::frag qf[1][R / KS];
    qr.to_frags(qf, scr, g, li);
    bf16x8 of[1][R / KS], df[1][R / KS];
    orr.to_raw(of, scr, g, li);
    dor.to_raw(df, scr, g, li);
    // phi(q) rows of this wave's block -> the chunk's phi(Q) tile
    if (half == 0) {
#pragma unroll
      for (int ks = 0; ks < R / KS; ++ks)
        *reinterpret_cast<bf16x8*>(sm.q + TQ::off(16 * ib + li, 32 * ks + 8 * g)) = qf[0][ks];
    }
    // (past the span's last chunk: re-read, unused)
    if constexpr (PREFETCH)
      load_all(min(t0 + CF::C, last));
    else
      load_chunk<CF, false>(cr, hb, min(t0 + CF::C, last));
    __syncthreads();

    // 1. D_i: the masked weights' row sums (bf16 weights, as the forward)
    //    plus phi(q_i).z
    f32x4 dacc = zero4();
#pragma unroll
    for (int ks = 0; ks < R / KS; ++ks) dacc = mfma16(load_frag(sm.z + zrow * R + ks * KS + g * 8), qf[0][ks], dacc);
    auto masked = [&](f32x4 t, int jb) {
      if (jb == ib) {
#pragma unroll
        for (int r = 0; r < 4; ++r) t[r] = 4 * g + r > li ? 0.f : t[r];
      }
      return t;
    };
#pragma unroll
    for (int jp = 0; jp < (RB + 1) / 2; ++jp) {
      const int jb0 = 2 * jp, jb1 = 2 * jp + 1;
      if (jb0 > ib) continue;
      const bool two = jb1 < RB && jb1 <= ib;
      f32x4 a0 = zero4(), a1 = zero4();
#pragma unroll
      for (int ks = 0; ks < R / KS; ++ks) {
        a0 = mfma16(load_frag(sm.k + TQ::off(16 * jb0 + li, ks * KS + g * 8)), qf[0][ks], a0);
        if (two) a1 = mfma16(load_frag(sm.k + TQ::off(16 * jb1 + li, ks * KS + g * 8)), qf[0][ks], a1);
      }
      a0 = masked(a0, jb0);
      a1 = two ? masked(a1, jb1) : zero4();
      const float w8[8] = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
      dacc = mfma16(ones_rows, cvt_bf16x8(w8), dacc);
    }
    const float den = dacc[0] + dacc[1];
    // rows beyond N get g = 0, h = 0 (their denominator may be zero, and
    // their g enters the span's reverse sums)
    const float rden = t0 + 16 * ib + li < N ? __builtin_amdgcn_rcpf(den) : 0.f;

    // 2. g_i = dO_i / D_i (operand), h_i = -(dO_i . O_i) / D_i
    bf16x8 gf[R / KS];
    float dot = 0.f;
#pragma unroll
    for (int ks = 0; ks < R / KS; ++ks) {
      float fd[8], fo[8], fg[8];
      unpack16<bf16>(__builtin_bit_cast(u32x4, df[0][ks]), fd);
      unpack16<bf16>(__builtin_bit_cast(u32x4, of[0][ks]), fo);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        dot += fd[e] * fo[e];
        fg[e] = fd[e] * rden;
      }
      gf[ks] = cvt_bf16x8(fg);
    }
    const float hv = -xor_sum16_32(dot) * rden;
    // g rows and h -> LDS for the reverse sums; (D_i, h_i) -> dh
    if (RSUM && half == 0) {
#pragma unroll
      for (int ks = 0; ks < R / KS; ++ks)
        *reinterpret_cast<bf16x8*>(sm.gt + TV::off(16 * ib + li, 32 * ks + 8 * g)) = gf[ks];
    }
    if (half == 0 && g == 0) {
      if constexpr (RSUM) sm.h[16 * ib + li] = hv;
      typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
      __builtin_amdgcn_raw_buffer_store_b64(u32x2{__float_as_uint(den), __float_as_uint(hv)}, r_dh,
                                            (t0 + 16 * ib + li) * 8, 0, 0);
    }

    // 3. W_ij = v_j.g_i + h_i (masked), and dphi(q_i) = sum_j W_ij phi(k_j)
    f32x4 dq[FTW];
#pragma unroll
    for (int fi = 0; fi < FTW; ++fi) dq[fi] = zero4();
#pragma unroll
    for (int jp = 0; jp < (RB + 1) / 2; ++jp) {
      const int jb0 = 2 * jp, jb1 = 2 * jp + 1;
      if (jb0 > ib) continue;
      const bool two = jb1 < RB && jb1 <= ib;
      f32x4 w0 = zero4(), w1 = zero4();
#pragma unroll
      for (int ks = 0; ks < DV / KS; ++ks) {
        w0 = mfma16(load_frag(sm.v + TV::off(16 * jb0 + li, ks * KS + g * 8)), gf[ks], w0);
        if (two) w1 = mfma16(load_frag(sm.v + TV::off(16 * jb1 + li, ks * KS + g * 8)), gf[ks], w1);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        w0[r] += hv;
        w1[r] += hv;
      }
      w0 = masked(w0, jb0);
      w1 = two ? masked(w1, jb1) : zero4();
      const float w8[8] = {w0[0], w0[1], w0[2], w0[3], w1[0], w1[1], w1[2], w1[3]};
      const bf16x8 bv = cvt_bf16x8(w8);
#pragma unroll
      for (int fi = 0; fi < FTW; ++fi) {
        const int ft = ft0 + fi;
        const bf16x8 av = two ? tr_frag<R>(sm.k, 16 * jb0 + 4 * g, 16 * jb1 + 4 * g, 16 * ft, li)
                              : tr_frag_lo<R>(sm.k, 16 * jb0 + 4 * g, 16 * ft, li);
        dq[fi] = mfma16(av, bv, dq[fi]);
      }
    }
    // 4. + S g_i + h_i z, then phi'(q)
#pragma unroll
    for (int fi = 0; fi < FTW; ++fi) {
      const int ft = ft0 + fi;
#pragma unroll
      for (int ks = 0; ks < DV / KS; ++ks)
        dq[fi] = mfma16(load_frag(sm.s + TV::off(16 * ft + li, ks * KS + g * 8)), gf[ks], dq[fi]);
      const bf16x4 fq4 = *reinterpret_cast<const bf16x4*>(sm.q + TQ::off(16 * ib + li, 16 * ft + 4 * g));
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int f = 16 * ft + 4 * g + r;
        const float zf = static_cast<float>(sm.z[f]) + static_cast<float>(sm.z[R + f]);
        dq[fi][r] = (dq[fi][r] + hv * zf) * phi_deriv_from_phi<CF::PHI>(static_cast<float>(fq4[r]));
      }
    }
    OutRegs<CF> out;
#pragma unroll
    for (int fi = 0; fi < FTW; ++fi) out.v[0][fi] = cvt_bf16x4(dq[fi]);
    store_outputs<CF>(out, hb.o, t0, w, g, li, false, scr);
    if constexpr (RSUM) {
      __syncthreads();  // the chunk's phi(Q), G and h tiles are complete
      // 5. reverse sums of the span
      state_mfma_w<CF>(racc, ut, sm.q, sm.gt, sm.h, w, g, li);
    }
    // the forward carry
    state_mfma<CF>(sacc, zt, sm.k, nullptr, sm.v, w, g, li);
  }

  if constexpr (!RSUM) return;
  float* slot = wsb + ((size_t)bh * (n_span + 1) + s) * E;
#pragma unroll
  for (int i = 0; i < CF::TPW; ++i) {
    int ct, ft;
    state_tile<CF>(w, i, ct, ft);
    *reinterpret_cast<f32x4*>(slot + (16 * ft + li) * DV + 16 * ct + 4 * g) = racc[i];
  }
  if (g == 0) slot[R * DV + 16 * w + li] = ut[0][0];
}


// The span's reverse sums dR = phi(Q)^T G, du = sum phi(q) h -> wsb slot s,
// for the eight-wave (d = 128) backward, whose dQ pass has no registers for
// them: per chunk phi(Q) and G = dO / D (from the (D, h) the dQ pass wrote)
// staged in LDS, then state_mfma_w.
template <class CF>
__global__ __launch_bounds__(CF::NT) void la_bwd_rsum_kernel(const bf16* __restrict__ Q,
                                                            const bf16* __restrict__ dO,
                                                            const float* __restrict__ dh,
                                                            float* __restrict__ wsb, int N, int n_span) {
  using OP = typename CF::OP;
  constexpr int R = CF::R, DV = CF::DV, E = R * DV + R, VVR = DV / 8;
  using TV = Tile<OP, DV>;
  struct Smem {
    OP q[Tile<OP, R>::elems(CF::C)];
    OP gt[Tile<OP, DV>::elems(CF::C)];
    alignas(16) float h[CF::C];
  };
  __shared__ Smem sm;
  const int tid = threadIdx.x, w = wave_id(), l = tid & 63, g = l >> 4, li = l & 15;
  const int bh = blockIdx.x / n_span;
  const int s = blockIdx.x % n_span;
  const int t_begin = span_begin<CF>(s, n_span, N);
  const int t_end = span_begin<CF>(s + 1, n_span, N);
  const size_t qk = (size_t)N * CF::D;
  HeadBufs hb;
  hb.k = make_rsrc(Q + bh * qk, (unsigned)(qk * 2));      // Q rows staged as keys are
  hb.v = make_rsrc(dO + bh * qk, (unsigned)(qk * 2));     // dO rows staged as values are
  const __amdgpu_buffer_rsrc_t r_dh = make_rsrc(dh + (size_t)bh * N * 2, (unsigned)N * 8u);
  f32x4 racc[CF::TPW];
#pragma unroll
  for (int i = 0; i < CF::TPW; ++i) racc[i] = zero4();
  f32x4 ut[1] = {zero4()};
  // one chunk ahead: chunk c+1's Q, dO and (D, h) loads are issued once
  // chunk c is staged and run under its MFMA work
  const int nch = (t_end - t_begin + CF::C - 1) / CF::C;
  auto chunk_t0 = [&](int k) { return t_begin + k * CF::C; };
  ChunkRegs<CF, false> cr;
  float rd[CF::LV], hl = 0.f;
  auto load = [&](int t0) {
    load_chunk<CF, false>(cr, hb, t0);
#pragma unroll
    for (int i = 0; i < CF::LV; ++i) {
      const int tok = (tid + i * CF::NT) / VVR;
      rd[i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r_dh, (t0 + tok) * 8, 0, 0));
    }
    hl = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r_dh, (t0 + l) * 8 + 4, 0, 0));
  };
  if (nch > 0) load(chunk_t0(0));
  for (int k = 0; k < nch; ++k) {
    const int t0 = chunk_t0(k);
    __syncthreads();  // the previous chunk's MFMA work is done with the tiles
    // phi(Q) (zero beyond N, as keys are) and G = dO / D
    stage_chunk<CF, false>(cr, nullptr, sm.q, nullptr, sm.gt, t0, N);
#pragma unroll
    for (int i = 0; i < CF::LV; ++i) {
      const int vi = tid + i * CF::NT;
      const int tok = vi / VVR;
      float f[8];
      unpack16<bf16>(cr.v[i], f);
      const float r = t0 + tok < N ? __builtin_amdgcn_rcpf(rd[i]) : 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) f[e] *= r;
      *reinterpret_cast<u32x4*>(sm.gt + TV::off(tok, (vi % VVR) * 8)) = pack16<bf16>(f);
    }
    if (w == 0 && l < CF::C) sm.h[l] = t0 + l < N ? hl : 0.f;
    if (k + 1 < nch) load(chunk_t0(k + 1));
    __syncthreads();
    state_mfma_w<CF>(racc, ut, sm.q, sm.gt, sm.h, w, g, li);
  }
  float* slot = wsb + ((size_t)bh * (n_span + 1) + s) * E;
#pragma unroll
  for (int i = 0; i < CF::TPW; ++i) {
    int ct, ft;
    state_tile<CF>(w, i, ct, ft);
    *reinterpret_cast<f32x4*>(slot + (16 * ft + li) * DV + 16 * ct + 4 * g) = racc[i];
  }
  if (g == 0) slot[R * DV + 16 * w + li] = ut[0][0];
}

// Exclusive suffix over spans: slot s becomes the sum of the slots after it.
__global__ __launch_bounds__(kThreads) void la_suffix_scan_kernel(float* __restrict__ ws, int E, int n_span) {
  const int e = blockIdx.x * kThreads + threadIdx.x;
  const int bh = blockIdx.y;
  if (e >= E) return;
  float* p = ws + (size_t)bh * (n_span + 1) * E + e;
  float acc = 0.f;
  // a batch's loads are issued before its dependent adds (as la_scan_kernel)
  constexpr int kBatch = 16;
  for (int s1 = n_span; s1 > 0; s1 -= kBatch) {   // spans s1 - kBatch .. s1 - 1, from the top
    float x[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) x[j] = s1 - 1 - j >= 0 ? p[(size_t)(s1 - 1 - j) * E] : 0.f;
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      if (s1 - 1 - j >= 0) {
        p[(size_t)(s1 - 1 - j) * E] = acc;
        acc += x[j];
      }
    }
  }
  p[(size_t)n_span * E] = acc;
}

template <class CF>
struct SmemBwdB {
  using OP = typename CF::OP;
  OP q[Tile<OP, CF::R>::elems(CF::C)];
  OP k[Tile<OP, CF::R>::elems(CF::C)];
  OP v[Tile<OP, CF::DV>::elems(CF::C)];
  OP gt[Tile<OP, CF::DV>::elems(CF::C)];
  OP rs[Tile<OP, CF::DV>::elems(CF::R)];   // the carried R, bf16
  alignas(16) float h[CF::C];
  alignas(16) float u[CF::R];
  alignas(16) OP scr[Scratch<CF>::ELEMS];
};

// Pass B: dK, dV, spans walked backward from the suffix (R, u) of the
// later spans (wsb slot s after the suffix scan).
template <class CF>
__global__ __launch_bounds__(CF::NT, CF::NW == 8 ? 1 : 2) void la_bwd_dkv_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    const bf16* __restrict__ dO, const float* __restrict__ dh, bf16* __restrict__ dK, bf16* __restrict__ dV,
    const float* __restrict__ wsb, int N, int n_span) {
  using OP = typename CF::OP;
  static_assert(sizeof(OP) == 2 && CF::RBW == 1 && CF::R == CF::DV && CF::CTW * CF::WPR == CF::CT,
                "one 16-row block per wave (WPR waves share it, each with its share of the column tiles), d = d_v");
  constexpr int R = CF::R, DV = CF::DV, KS = CF::KS, RB = CF::RB, FT = CF::FT, CT = CF::CT;
  using TQ = Tile<OP, R>;
  using TV = Tile<OP, DV>;
  __shared__ SmemBwdB<CF> sm;
  const int tid = threadIdx.x, w = wave_id(), l = tid & 63, g = l >> 4, li = l & 15;
  const int bh = blockIdx.x / n_span;
  const int s = blockIdx.x % n_span;
  const int t_begin = span_begin<CF>(s, n_span, N);
  const int t_end = span_begin<CF>(s + 1, n_span, N);
  const HeadBufs hb = head_bufs<CF>(Q, K, V, dK, bh, N);
  const size_t qk = (size_t)N * CF::D;
  const __amdgpu_buffer_rsrc_t r_do = make_rsrc(dO + bh * qk, (unsigned)(qk * 2));
  const __amdgpu_buffer_rsrc_t r_dv = make_rsrc(dV + bh * qk, (unsigned)(qk * 2));
  const __amdgpu_buffer_rsrc_t r_dh = make_rsrc(dh + (size_t)bh * N * 2, (unsigned)N * 8u);

  constexpr int E = R * DV + R;
  const float* suf = wsb + ((size_t)bh * (n_span + 1) + s) * E;
  f32x4 racc[CF::TPW];
#pragma unroll
  for (int i = 0; i < CF::TPW; ++i) {
    int ct, ft;
    state_tile<CF>(w, i, ct, ft);
    racc[i] = *reinterpret_cast<const f32x4*>(suf + (16 * ft + li) * DV + 16 * ct + 4 * g);
  }
  f32x4 ut[1];
  {
    const float uv = suf[R * DV + 16 * w + li];
    ut[0] = f32x4{uv, uv, uv, uv};
  }
  // this wave's key block; with eight waves two share a block and each
  // takes half of the value tiles of dV and half of the feature tiles of dK
  constexpr int FTW = FT / CF::WPR, CTW = CT / CF::WPR;
  const int jb = wave_row_block<CF>(0, w), half = w / RB, ft0 = half * FTW, ct0 = half * CTW;
  OP* scr = sm.scr + w * Scratch<CF>::PER_WAVE;
  constexpr int VVR = DV / 8;
  if (t_begin >= t_end) return;
  const int last = t_begin + ((t_end - t_begin - 1) / CF::C) * CF::C;

  // chunk c-1 is loaded into registers while chunk c is computed (four
  // waves; eight load each chunk at the top of its iteration): Q, K, V, the
  // dO rows (V's layout), each row's D and the chunk's h
  constexpr bool PREFETCH = CF::NW == 4;
  ChunkRegs<CF, true> cr;
  u32x4 dov[CF::LV];
  float rd[CF::LV];
  float hl;
  auto load_all = [&](int tc) {
    load_chunk<CF, true>(cr, hb, tc);
#pragma unroll
    for (int i = 0; i < CF::LV; ++i) {
      const int vi = tid + i * CF::NT;
      const int tok = vi / VVR;
      dov[i] = __builtin_amdgcn_raw_buffer_load_b128(r_do, ((tc + tok) * DV + (vi % VVR) * 8) * 2, 0, 0);
      rd[i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r_dh, (tc + tok) * 8, 0, 0));
    }
    hl = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r_dh, (tc + (tid & 63)) * 8 + 4, 0, 0));
  };
  if constexpr (PREFETCH) load_all(last);
  for (int t0 = last; t0 >= t_begin; t0 -= CF::C) {
    // eight waves: the lane indices pass through an empty asm statement on
    // every chunk, so that the swizzled LDS offsets derived from them are
    // formed inside the loop instead of being kept live across it (which
    // spilled about ten VGPRs)
    int g_in = g, li_in = li;
    if constexpr (!PREFETCH) asm volatile("" : "+v"(g_in), "+v"(li_in));
    const int g = g_in, li = li_in;
    if constexpr (!PREFETCH) load_all(t0);
    __syncthreads();  // every wave is done with the previous chunk's tiles
    // the carried R (bf16) and u
#pragma unroll
    for (int i = 0; i < CF::TPW; ++i) {
      int ct, ft;
      state_tile<CF>(w, i, ct, ft);
      *reinterpret_cast<bf16x4*>(sm.rs + TV::off(16 * ft + li, 16 * ct + 4 * g)) = cvt_bf16x4(racc[i]);
    }
    if (g == 0) sm.u[16 * w + li] = ut[0][0];
    stage_chunk<CF, true>(cr, sm.q, sm.k, nullptr, sm.v, t0, N);
#pragma unroll
    for (int i = 0; i < CF::LV; ++i) {
      const int vi = tid + i * CF::NT;
      const int tok = vi / VVR;
      float f[8];
      unpack16<bf16>(dov[i], f);
      const float r = t0 + tok < N ? __builtin_amdgcn_rcpf(rd[i]) : 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) f[e] *= r;
      *reinterpret_cast<u32x4*>(sm.gt + TV::off(tok, (vi % VVR) * 8)) = pack16<bf16>(f);
    }
    if (w == 0 && (tid & 63) < CF::C) sm.h[tid & 63] = t0 + (tid & 63) < N ? hl : 0.f;
    if constexpr (PREFETCH) load_all(max(t0 - CF::C, t_begin));  // (before the span's first chunk: re-read, unused)
    __syncthreads();

    // this wave's key rows j = 16 jb + li: phi(k_j), v_j as B operands
    bf16x8 kf[R / KS], vf[DV / KS];
#pragma unroll
    for (int ks = 0; ks < R / KS; ++ks) kf[ks] = load_frag(sm.k + TQ::off(16 * jb + li, ks * KS + g * 8));
#pragma unroll
    for (int ks = 0; ks < DV / KS; ++ks) vf[ks] = load_frag(sm.v + TV::off(16 * jb + li, ks * KS + g * 8));
    auto masked = [&](f32x4 t, int ib) {
      if (ib == jb) {
#pragma unroll
        for (int r = 0; r < 4; ++r) t[r] = 4 * g + r < li ? 0.f : t[r];
      }
      return t;
    };
    f32x4 dv[CTW], dk[FTW];
#pragma unroll
    for (int ci = 0; ci < CTW; ++ci) dv[ci] = zero4();
#pragma unroll
    for (int fi = 0; fi < FTW; ++fi) dk[fi] = zero4();
    // query blocks ib >= jb, in pairs (one 32-token MFMA step)
#pragma unroll
    for (int ip = 0; ip < (RB + 1) / 2; ++ip) {
      const int ib0 = 2 * ip, ib1 = 2 * ip + 1;
      if (ib1 < jb || (ib1 >= RB && ib0 < jb)) continue;
      const bool has0 = ib0 >= jb, has1 = ib1 < RB && ib1 >= jb;
      f32x4 a0 = zero4(), a1 = zero4(), w0 = zero4(), w1 = zero4();
#pragma unroll
      for (int ks = 0; ks < R / KS; ++ks) {
        if (has0) a0 = mfma16(load_frag(sm.q + TQ::off(16 * ib0 + li, ks * KS + g * 8)), kf[ks], a0);
        if (has1) a1 = mfma16(load_frag(sm.q + TQ::off(16 * ib1 + li, ks * KS + g * 8)), kf[ks], a1);
      }
#pragma unroll
      for (int ks = 0; ks < DV / KS; ++ks) {
        if (has0) w0 = mfma16(load_frag(sm.gt + TV::off(16 * ib0 + li, ks * KS + g * 8)), vf[ks], w0);
        if (has1) w1 = mfma16(load_frag(sm.gt + TV::off(16 * ib1 + li, ks * KS + g * 8)), vf[ks], w1);
      }
      // lane (g, li): entry [i = 16 ib + 4 g + r][j = 16 jb + li]; W^T adds h_i
      const f32x4 h0 = *reinterpret_cast<const f32x4*>(sm.h + 16 * ib0 + 4 * g);
      const f32x4 h1 = has1 ? *reinterpret_cast<const f32x4*>(sm.h + 16 * ib1 + 4 * g) : zero4();
      w0 += h0;
      w1 += h1;
      a0 = has0 ? masked(a0, ib0) : zero4();
      a1 = has1 ? masked(a1, ib1) : zero4();
      w0 = has0 ? masked(w0, ib0) : zero4();
      w1 = has1 ? masked(w1, ib1) : zero4();
      const float a8[8] = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
      const float w8[8] = {w0[0], w0[1], w0[2], w0[3], w1[0], w1[1], w1[2], w1[3]};
      const bf16x8 ab = cvt_bf16x8(a8), wb = cvt_bf16x8(w8);
#pragma unroll
      for (int ci = 0; ci < CTW; ++ci)
        dv[ci] = mfma16(tr_frag<DV>(sm.gt, 16 * ib0 + 4 * g, 16 * ib1 + 4 * g, 16 * (ct0 + ci), li), ab, dv[ci]);
#pragma unroll
      for (int fi = 0; fi < FTW; ++fi)
        dk[fi] = mfma16(tr_frag<R>(sm.q, 16 * ib0 + 4 * g, 16 * ib1 + 4 * g, 16 * (ft0 + fi), li), wb, dk[fi]);
    }
    // + the later chunks: dv_j += R^T phi(k_j), dphi(k_j) += R v_j + u
#pragma unroll
    for (int ci = 0; ci < CTW; ++ci)
#pragma unroll
      for (int ks = 0; ks < R / KS; ++ks)
        dv[ci] = mfma16(tr_frag<DV>(sm.rs, ks * 32 + 8 * g, ks * 32 + 8 * g + 4, 16 * (ct0 + ci), li), kf[ks], dv[ci]);
#pragma unroll
    for (int fi = 0; fi < FTW; ++fi) {
      const int f = ft0 + fi;
#pragma unroll
      for (int ks = 0; ks < DV / KS; ++ks)
        dk[fi] = mfma16(load_frag(sm.rs + TV::off(16 * f + li, ks * KS + g * 8)), vf[ks], dk[fi]);
      const f32x4 uf = *reinterpret_cast<const f32x4*>(sm.u + 16 * f + 4 * g);
      const bf16x4 fk4 = *reinterpret_cast<const bf16x4*>(sm.k + TQ::off(16 * jb + li, 16 * f + 4 * g));
#pragma unroll
      for (int r = 0; r < 4; ++r) dk[fi][r] = (dk[fi][r] + uf[r]) * phi_deriv_from_phi<CF::PHI>(static_cast<float>(fk4[r]));
    }
    OutRegs<CF> ok, ov;
#pragma unroll
    for (int ci = 0; ci < CTW; ++ci) {
      ov.v[0][ci] = cvt_bf16x4(dv[ci]);
      ok.v[0][ci] = cvt_bf16x4(dk[ci]);
    }
    store_outputs<CF>(ok, hb.o, t0, w, g, li, false, scr);
    store_outputs<CF>(ov, r_dv, t0, w, g, li, false, scr);
    // the carry toward earlier chunks
    state_mfma_w<CF>(racc, ut, sm.q, sm.gt, sm.h, w, g, li);
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

  (void)hipGetLastError();  // drop a stale error left by an unrelated earlier runtime call
  auto rec = [&](int i) {
    if (a.events && a.events[i]) (void)hipEventRecord(static_cast<hipEvent_t>(a.events[i]), st);
  };
  if (a.log_a_ch) {
    if constexpr (gla_fits<CF>()) {
      if (!a.causal) return hipErrorInvalidValue;
      float* tot = ws + (size_t)BH * (n_span + 1) * (CF::R * CF::DV + CF::R);
      const dim3 grid(BH * n_span), block(CF::NT);
      rec(0);
      if (n_span > 0 && BH > 0)
        hipLaunchKernelGGL((la_state_kernel_gla<CF>), grid, block, 0, st, K, V, ws, a.N, n_span, a.log_a_ch, tot);
      rec(1);
      rec(2);
      hipError_t e = scan_launch(ws, BH, CF::R, CF::DV, n_span, a.S0, a.z0, a.S_out, a.z_out, st, nullptr, a.H,
                                 a.N, CF::C, tot, 1);
      if (e != hipSuccess) return e;
      rec(3);
      rec(4);
      if (n_span > 0 && BH > 0)
        hipLaunchKernelGGL((la_output_kernel_gla<CF>), grid, block, 0, st, Q, K, V, O, ws, a.N, n_span,
                           a.log_a_ch, a.normalize);
      rec(5);
      return hipGetLastError();
    } else {
      return hipErrorInvalidValue;
    }
  }
  const int dk = !a.causal ? kNoDecay : a.log_a ? kGated : a.gamma ? kFixed : kNoDecay;
  // gated: the spans' total log2 gates follow the span states
  float* totals = dk == kGated ? ws + (size_t)BH * (n_span + 1) * (CF::R * CF::DV + CF::R) : nullptr;
  const dim3 grid(BH * n_span), block(CF::NT);
  rec(0);
  if (n_span > 0 && BH > 0) {
    if (dk == kGated)
      hipLaunchKernelGGL((la_state_kernel<CF, kGated>), grid, block, 0, st, K, V, ws, a.N, n_span, nullptr, 1,
                         a.log_a, totals);
    else if (dk == kFixed)
      hipLaunchKernelGGL((la_state_kernel<CF, kFixed>), grid, block, 0, st, K, V, ws, a.N, n_span, a.gamma, a.H,
                         nullptr, nullptr);
    else
      hipLaunchKernelGGL((la_state_kernel<CF, kNoDecay>), grid, block, 0, st, K, V, ws, a.N, n_span, nullptr, 1,
                         nullptr, nullptr);
  }
  rec(1);
  rec(2);
  hipError_t e = scan_launch(ws, BH, CF::R, CF::DV, n_span, a.S0, a.z0, a.S_out, a.z_out, st,
                             dk == kFixed ? a.gamma : nullptr, a.H, a.N, CF::C, totals, 0, !a.causal);
  if (e != hipSuccess) return e;
  rec(3);
  rec(4);
  if (n_span > 0 && BH > 0) {
    if (dk == kGated)
      hipLaunchKernelGGL((la_output_kernel<CF, true, kGated>), grid, block, 0, st, Q, K, V, O, ws, a.N, n_span,
                         nullptr, 1, a.normalize, a.log_a);
    else if (dk == kFixed)
      hipLaunchKernelGGL((la_output_kernel<CF, true, kFixed>), grid, block, 0, st, Q, K, V, O, ws, a.N, n_span,
                         a.gamma, a.H, a.normalize, nullptr);
    else if (a.causal)
      hipLaunchKernelGGL((la_output_kernel<CF, true>), grid, block, 0, st, Q, K, V, O, ws, a.N, n_span, nullptr, 1,
                         1, nullptr);
    else
      hipLaunchKernelGGL((la_output_kernel<CF, false>), grid, block, 0, st, Q, K, V, O, ws, a.N, n_span, nullptr,
                         1, 1, nullptr);
  }
  rec(5);
  return hipGetLastError();
}

template <typename T, int D, int PHI>
static hipError_t dispatch_chunk(const PrefillArgs& a) {
  // wide heads run eight waves per workgroup: half the state tiles and
  // registers per wave, and twice the waves per CU
  constexpr int NW = D == 128 ? 8 : kWaves;
  switch (a.chunk) {
    case 16: return launch_prefill<Cfg<T, D, D, D, 16, PHI, NW>>(a);
    case 32: return launch_prefill<Cfg<T, D, D, D, 32, PHI, NW>>(a);
    case 64: return launch_prefill<Cfg<T, D, D, D, 64, PHI, NW>>(a);
    case 128:
      if constexpr (sizeof(T) == 2 && D == 64) return launch_prefill<Cfg<T, D, D, D, 128, PHI>>(a);
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
}

hipError_t scan_launch(float* ws, int BH, int R, int DV, int n_span, const float* S0, const float* z0,
                       float* S_out, float* z_out, hipStream_t stream, const float* gamma, int H, int N, int chunk,
                       const float* totals, int per_channel, int total_only, const float* kappa) {
  const int E = R * DV + R;
  if (BH > 0) {
    const dim3 grid((E + kThreads - 1) / kThreads, BH);
    if (totals && per_channel)
      hipLaunchKernelGGL(la_scan_kernel<kChannel>, grid, dim3(kThreads), 0, stream, ws, R, DV, n_span, S0, z0,
                         S_out, z_out, nullptr, 1, N, chunk > 0 ? chunk : 64, totals, nullptr);
    else if (totals)
      hipLaunchKernelGGL(la_scan_kernel<kGated>, grid, dim3(kThreads), 0, stream, ws, R, DV, n_span, S0, z0, S_out,
                         z_out, nullptr, 1, N, chunk > 0 ? chunk : 64, totals, nullptr);
    else if (gamma)
      hipLaunchKernelGGL(la_scan_kernel<kFixed>, grid, dim3(kThreads), 0, stream, ws, R, DV, n_span, S0, z0, S_out,
                         z_out, gamma, H > 0 ? H : 1, N, chunk > 0 ? chunk : 64, nullptr, nullptr);
    else if (total_only)
      hipLaunchKernelGGL((la_scan_kernel<kNoDecay, true>), grid, dim3(kThreads), 0, stream, ws, R, DV, n_span, S0,
                         z0, S_out, z_out, nullptr, 1, N, chunk > 0 ? chunk : 64, nullptr, kappa);
    else
      hipLaunchKernelGGL(la_scan_kernel<kNoDecay>, grid, dim3(kThreads), 0, stream, ws, R, DV, n_span, S0, z0,
                         S_out, z_out, nullptr, 1, N, chunk > 0 ? chunk : 64, nullptr, kappa);
  }
  return hipGetLastError();
}

bool prefill_supported(int io, int phi, int d, int dv, int r, int chunk) {
  if (phi == PHI_FAVOR) return favor_prefill_supported(io, d, dv, r, chunk);
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

template <class CF>
static hipError_t launch_backward(const BackwardArgs& a) {
  const int BH = a.B * a.H, n_span = a.n_span;
  hipStream_t st = static_cast<hipStream_t>(a.stream);
  constexpr int E = CF::R * CF::DV + CF::R;
  float* wsf = static_cast<float*>(a.workspace);
  float* wsb = wsf + (size_t)BH * (n_span + 1) * E;
  float* dh = wsb + (size_t)BH * (n_span + 1) * E;
  const bf16* Q = static_cast<const bf16*>(a.Q);
  const bf16* K = static_cast<const bf16*>(a.K);
  const bf16* V = static_cast<const bf16*>(a.V);
  (void)hipGetLastError();
  auto rec = [&](int i) {
    if (a.events && a.events[i]) (void)hipEventRecord(static_cast<hipEvent_t>(a.events[i]), st);
  };
  const dim3 grid(BH * n_span), block(CF::NT);
  rec(0);
  hipLaunchKernelGGL((la_state_kernel<CF, kNoDecay>), grid, block, 0, st, K, V, wsf, a.N, n_span, nullptr, 1, nullptr,
                     nullptr);
  rec(1);
  rec(2);
  hipError_t e = scan_launch(wsf, BH, CF::R, CF::DV, n_span, nullptr, nullptr, nullptr, nullptr, st);
  if (e != hipSuccess) return e;
  rec(3);
  rec(4);
  hipLaunchKernelGGL((la_bwd_dq_kernel<CF>), grid, block, 0, st, Q, K, V, static_cast<const bf16*>(a.O),
                     static_cast<const bf16*>(a.dO), static_cast<bf16*>(a.dQ), wsf, wsb, dh, a.N, n_span);
  if constexpr (CF::NW != 4)  // (inside the dQ pass's event interval)
    hipLaunchKernelGGL((la_bwd_rsum_kernel<CF>), grid, block, 0, st, Q, static_cast<const bf16*>(a.dO), dh, wsb,
                       a.N, n_span);
  rec(5);
  rec(6);
  hipLaunchKernelGGL(la_suffix_scan_kernel, dim3((E + kThreads - 1) / kThreads, BH), dim3(kThreads), 0, st, wsb, E,
                     n_span);
  rec(7);
  rec(8);
  hipLaunchKernelGGL((la_bwd_dkv_kernel<CF>), grid, block, 0, st, Q, K, V, static_cast<const bf16*>(a.dO), dh,
                     static_cast<bf16*>(a.dK), static_cast<bf16*>(a.dV), wsb, a.N, n_span);
  rec(9);
  return hipGetLastError();
}

bool backward_supported(int io, int phi, int d, int dv, int r, int chunk) {
  return io == 1 && (phi == PHI_ELU1 || phi == PHI_IDENTITY) && (d == 64 || d == 128) && dv == d && r == d &&
         chunk == 64;
}

hipError_t backward_launch(const BackwardArgs& a) {
  if (!backward_supported(a.io, a.phi, a.d, a.dv, a.r, a.chunk)) return hipErrorInvalidValue;
  if (a.B * a.H == 0 || a.N == 0) return hipSuccess;
  if (a.d == 128)
    return a.phi == PHI_ELU1 ? launch_backward<Cfg<bf16, 128, 128, 128, 64, PHI_ELU1, 8>>(a)
                             : launch_backward<Cfg<bf16, 128, 128, 128, 64, PHI_IDENTITY, 8>>(a);
  return a.phi == PHI_ELU1 ? launch_backward<Cfg<bf16, 64, 64, 64, 64, PHI_ELU1>>(a)
                           : launch_backward<Cfg<bf16, 64, 64, 64, 64, PHI_IDENTITY>>(a);
}

bool gla_supported(int io, int d, int dv, int r, int chunk) {
  if (r != d || dv != d) return false;
  if (chunk != 16 && chunk != 32 && chunk != 64 && chunk != 128) return false;
  if (io == 1) return d == 64 || (d == 128 && chunk <= 32);  // (d = 128, chunk 64: the tiles exceed the LDS)
  if (io == 0) return d == 64 && chunk <= 64;
  return false;
}

hipError_t prefill_launch(const PrefillArgs& a) {
  if (a.phi == PHI_FAVOR) return favor_prefill_launch(a);
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
