// Chunked prefill with FAVOR+ positive random features fused in (gfx950).
//
// FAVOR+ ("Efficient attention variants", sec. 6): with x = u / d^(1/4),
//   phi(u)_f = exp(w_f . x - |x|^2 / 2) / sqrt(r),   f = 0 .. r-1,
// where w_f is row f of the projection omega [r][d].  The method is the
// chunked causal linear attention of the pointwise feature maps (same span
// state / span scan / output split, same workspace layout); only the
// features change: they come from a projection instead of a pointwise map.
// Supported: bf16 I/O, d = d_v = 64, r = 256, chunk 64.
//
// The projection X omega^T is a bf16 MFMA.  X is exact in bf16.  For the span
// state, omega (fp32) enters as a bf16 hi + lo pair, so the projection is
// accurate to ~2^-16 relative and the fp32 state that later spans read is
// accurate; the output kernel rounds its feature tiles to bf16 anyway and
// uses omega's hi part only.  Eight waves per workgroup (two per SIMD); each
// wave owns 32 of the 256 features and keeps its omega fragments in
// registers for the whole kernel.  The squared norm |u|^2 of
// every token is summed in fp32 while the chunk is staged.  phi itself is
// evaluated in fp32 as one exp2; features of tokens beyond N are zero.
//
//   la_state_favor_kernel  - per span: dS = phi(K)^T V, dz = sum phi(K).
//                            The projection tiles come out of the MFMA with
//                            tokens along the k-slot direction, so they feed
//                            the state MFMA directly as bf16 hi + lo
//                            operands (no LDS round trip); dz comes from a
//                            ones operand against the same fragments.
//   la_output_favor_kernel - per span, chunk by chunk: phi(Q), phi(K) tiles
//                            -> LDS and the state carry (from phi(K) in
//                            registers, as in the span-state kernel), then
//                            the masked intra-chunk product, read-out of the
//                            carried state and divide.  phi(Q) and phi(K)
//                            are contracted over features in a permuted
//                            order: k-slot e of lane group g at k-step ks is
//                            feature 32 ks + 16 (e / 4) + 4 g + e % 4, which
//                            is how the projection accumulators lay them
//                            out.  S and z are read in the same order.
#include "la_common.h"
#include "la_prefill.h"
#include "la_tiles.h"

namespace la {
namespace {

constexpr int FD = 64;                    // head dimension d
constexpr int FR = 256;                   // random features r
constexpr int FDV = 64;                   // value dimension
constexpr int FC = 64;                    // chunk
constexpr int FFT = FR / 16;              // feature tiles
constexpr int FCT = FDV / 16;             // value tiles
constexpr int FNW = 8;                    // waves per workgroup (two per SIMD)
constexpr int FNT = 64 * FNW;             // threads per workgroup
constexpr int FPW = FFT / FNW;            // feature tiles owned by a wave in the projections
constexpr int FE = FR * FDV + FR;         // floats per workspace slot
constexpr int FVQ = FC * FD / 8;          // 16-byte vectors per raw chunk
constexpr int FLQ = FVQ / FNT;            // ... per thread
static_assert(FVQ % FNT == 0 && FDV == FD, "raw chunk tiles are 64 x 64 bf16");

using T64 = Tile<bf16, 64>;

// exp2 argument constants of phi: log2(e) d^(-1/4), log2(e) / (2 sqrt(d)),
// and log2(sqrt(r)).
struct FavorConsts {
  float a1, a2, a3;
};
__device__ __forceinline__ FavorConsts favor_consts() {
  const float log2e = 1.4426950408889634f;
  return FavorConsts{log2e * 0.35355339059327373f /* 64^(-1/4) */, log2e / 16.0f /* 1 / (2 sqrt(64)) */,
                     4.0f /* log2(sqrt(256)) */};
}
// Per-token part of the exponent of a key: -(|u|^2 log2(e) / (2 sqrt(d)) +
// log2(sqrt(r))), plus the head's shift kappa; -inf for a token past the
// end of the sequence, whose features are then exp2(-inf) = 0.
__device__ __forceinline__ float favor_bias(const FavorConsts& c, float norm2) { return -(norm2 * c.a2 + c.a3); }
__device__ __forceinline__ float favor_kbias(const FavorConsts& c, float norm2, float kappa, bool valid) {
  return valid ? favor_bias(c, norm2) + kappa : -__builtin_inff();
}

// Numeric range ("Efficient attention variants", sec. 6 asks for a stable
// estimator).  Each feature of a query carries the factor exp(-|x|^2 / 2),
// each feature of a key as well; for |x| beyond about 12 their products
// leave the fp32 range and the ratio becomes 0/0.  A constant factor per
// query row cancels in num/den, and so does one per (batch, head) on all
// keys, so the kernels evaluate
//   queries:  exp(w . x - 4 |x|) / sqrt(r)        (the row's factor
//             exp(4 |x| - |x|^2 / 2) taken out; 4 |x| is about the largest
//             w . x over 256 features, so the row's largest feature stays
//             near 1 for any |x|),
//   keys:     exp(w . x - |x|^2 / 2 + kappa_h) / sqrt(r),
//             kappa_h = |x_0|^2 / 2 - 4 |x_0|, x_0 the head's first key
//             (its own largest feature near 1; the first key enters every
//             output, so no later token changes a result).
// The span states carry the factor 2^kappa_h (log2 units below); the scan
// takes it out of the returned S_N, z_N and puts it into a given S0, z0.
// Key norms that differ from the first key's by much more than the first
// key's own norm can still leave the range.
constexpr float kQueryShift = 4.0f;
__device__ __forceinline__ float favor_qbias(const FavorConsts& c, float norm2) {
  return -(c.a1 * kQueryShift * __builtin_sqrtf(norm2) + c.a3);
}
// (the same in every lane: kept in a scalar register)
__device__ __forceinline__ float favor_kappa(const FavorConsts& c, float norm2_first) {
  const float k = norm2_first * c.a2 - c.a1 * kQueryShift * __builtin_sqrtf(norm2_first);
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(k)));
}
// |u|^2 of the head's first key, in every thread (8 threads per 16-byte
// piece of the row, a 3-step butterfly); 0 for an empty head.
__device__ __forceinline__ float favor_first_norm2(__amdgpu_buffer_rsrc_t k) {
  float f[8];
  unpack16<bf16>(__builtin_amdgcn_raw_buffer_load_b128(k, (threadIdx.x & 7) * 16, 0, 0), f);
  float n2 = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) n2 += f[e] * f[e];
  n2 += __shfl_xor(n2, 1);
  n2 += __shfl_xor(n2, 2);
  n2 += __shfl_xor(n2, 4);
  return n2;
}
// Precision of the output pass's projections.  By default they use omega's
// bf16 hi part only: omega's rounding (2^-9 relative) puts an error of about
// 2^-9 |w . x| into the exponent of each feature, which at the workload's
// norms (|x| near 1) is below the bf16 rounding of the features themselves,
// but at |x| of 2 and more shows in the outputs (about 1.5e-2 relative per
// row at |x| = 2, 5e-2 at 8).  The precise form (LA_PHI_FAVOR_PRECISE) adds
// the lo part, as the span state pass always does, at about 1.4 times the
// output pass's time.  Selecting the form per token inside the pass would
// keep the fast form's speed only if it cost no registers, which it does
// not (the lo fragments of the projections are live across the feature
// phase), so the caller chooses.
// phi for one feature: exp2(proj log2(e) d^(-1/4) + bias) - one FMA and one exp2
// (0 for the bias -inf of a masked token, whose projection is 0).
__device__ __forceinline__ float favor_phi(const FavorConsts& c, float proj, float bias) {
  return __builtin_amdgcn_exp2f(__builtin_fmaf(proj, c.a1, bias));
}

// omega fragments of the 4 feature tiles a wave owns (features 64 w + 16 j +
// li), for the two 32-wide k-steps over d: lane (g, li) holds
// omega[f][32 ks + 8 g .. +7] as bf16 hi and lo = round(x - hi).  The same
// fragment serves as an A operand (features along M) or a B operand
// (features along N).
template <bool LO>
struct OmegaFrags {
  bf16x8 hi[FPW][2], lo[LO ? FPW : 1][2];
  __device__ __forceinline__ void load(const float* __restrict__ omega, int w, int g, int li) {
#pragma unroll
    for (int j = 0; j < FPW; ++j) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const float* p = omega + (size_t)(16 * (FPW * w + j) + li) * FD + 32 * ks + 8 * g;
        const f32x4 a = *reinterpret_cast<const f32x4*>(p);
        const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x = e < 4 ? a[e] : b[e - 4];
          const bf16 h = static_cast<bf16>(x);
          hi[j][ks][e] = h;
          if constexpr (LO) lo[j][ks][e] = static_cast<bf16>(x - static_cast<float>(h));
        }
      }
    }
  }
};

// omega's lo fragment (round(x - hi)) for feature tile j, k-step ks of wave
// w, read from memory where needed (the output pass keeps only hi in
// registers).  The lane's byte offset is formed here, behind an empty asm
// statement, so that it is not kept live across the chunk loop.
__device__ __forceinline__ bf16x8 omega_lo_frag(__amdgpu_buffer_rsrc_t om, int w, int j, int ks) {
  int lane = threadIdx.x & 63;
  asm volatile("" : "+v"(lane));
  const int off = (((16 * (FPW * w + j) + (lane & 15)) * FD + 32 * ks + 8 * (lane >> 4)) * 4);
  const f32x4 a = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(om, off, 0, 0));
  const f32x4 b = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(om, off + 16, 0, 0));
  bf16x8 lo;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float x = e < 4 ? a[e] : b[e - 4];
    lo[e] = static_cast<bf16>(x - static_cast<float>(static_cast<bf16>(x)));
  }
  return lo;
}

// Raw (unmapped) chunk rows held in registers between load and staging.
template <int NS>
struct RawRegs {
  u32x4 x[NS][FLQ];
};

// Global -> registers: raw rows of the given streams for the chunk at t0
// (rows beyond N read as zero through the buffer bounds).
template <int NS>
__device__ __forceinline__ void load_raw(RawRegs<NS>& rr, const __amdgpu_buffer_rsrc_t (&src)[NS], int t0) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < FLQ; ++i) {
    const int vi = tid + i * FNT;
    const int off = ((t0 + vi / 8) * FD + (vi % 8) * 8) * 2;
#pragma unroll
    for (int s = 0; s < NS; ++s) rr.x[s][i] = __builtin_amdgcn_raw_buffer_load_b128(src[s], off, 0, 0);
  }
}

// Registers -> LDS (row-major swizzled 64 x 64 tiles).  For the streams
// flagged in `norms`, the squared norm |u|^2 of each token row is summed in
// fp32 (8 threads hold one row: a 3-step butterfly) and its exponent bias
// is written to nrm: the query form for the streams flagged in `queries`,
// otherwise the key form with the head's shift kappa, and -inf for rows at
// or beyond `live` (tokens past the end of the sequence; their raw rows
// read as zero), so that every feature of theirs is exp2(-inf) = 0.
template <int NS>
__device__ __forceinline__ void stage_raw(const RawRegs<NS>& rr, bf16* const (&dst)[NS], float* const (&nrm)[NS],
                                          int norms, int queries, float kappa, int live) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < FLQ; ++i) {
    const int vi = tid + i * FNT;
    const int tok = vi / 8, col = (vi % 8) * 8;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      *reinterpret_cast<u32x4*>(dst[s] + T64::off(tok, col)) = rr.x[s][i];
      if (norms & (1 << s)) {
        float f[8];
        unpack16<bf16>(rr.x[s][i], f);
        float n2 = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) n2 += f[e] * f[e];
        n2 += __shfl_xor(n2, 1);
        n2 += __shfl_xor(n2, 2);
        n2 += __shfl_xor(n2, 4);
        if ((tid & 7) == 0) {
          const FavorConsts c = favor_consts();
          nrm[s][tok] = (queries & (1 << s)) ? favor_qbias(c, n2) : favor_kbias(c, n2, kappa, tok < live);
        }
      }
    }
  }
}

// Projection tile of 16 tokens (block tb of a staged raw chunk) against the
// feature tile j of this wave: acc += X_tb omega_j^T in one of two
// orientations.  TOKENS_ON_M: lane (g, li) ends with tokens 16 tb + 4 g + r
// of feature li; otherwise features 4 g + r of token 16 tb + li.
template <bool TOKENS_ON_M, bool LO>
__device__ __forceinline__ f32x4 project(const bf16* raw, const OmegaFrags<LO>& om, int j, int tb, int g, int li) {
  f32x4 acc = zero4();
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    const bf16x8 x = load_frag(raw + T64::off(16 * tb + li, 32 * ks + 8 * g));
    if constexpr (TOKENS_ON_M) {
      acc = mfma16(x, om.hi[j][ks], acc);
      if constexpr (LO) acc = mfma16(x, om.lo[j][ks], acc);
    } else {
      acc = mfma16(om.hi[j][ks], x, acc);
      if constexpr (LO) acc = mfma16(om.lo[j][ks], x, acc);
    }
  }
  return acc;
}

__device__ __forceinline__ int span_begin64(int s, int n_span, int N) {
  const long long n_chunks = (N + FC - 1) / FC;
  return (int)min((long long)N, FC * ((long long)s * n_chunks / n_span));
}

__device__ __forceinline__ bf16x8 cat4(bf16x4 a, bf16x4 b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// ------------------------------------------------------------------ span state

// dS = phi(K_span)^T V_span, dz = sum phi(K_span) -> workspace slot s.  Wave w
// owns features 32 w .. 32 w + 31 (tiles j = 0, 1) for all value tiles ct:
// acc[j][ct] lane (g, li) holds S[f = 32 w + 16 j + li][c = 16 ct + 4 g + r].
__global__ __launch_bounds__(FNT, 1) void la_state_favor_kernel(const bf16* __restrict__ K,
                                                                     const bf16* __restrict__ V,
                                                                     const float* __restrict__ omega,
                                                                     float* __restrict__ ws,
                                                                     float* __restrict__ kappa_out, int N,
                                                                     int n_span) {
  __shared__ bf16 kraw[2][FC * FD];
  __shared__ bf16 vt[2][FC * FDV];
  __shared__ float kn[2][FC];
  const int tid = threadIdx.x, w = wave_id(), l = tid & 63, g = l >> 4, li = l & 15;
  const int bh = blockIdx.x / n_span;
  const int s = blockIdx.x % n_span;
  const int t_begin = span_begin64(s, n_span, N);
  const int t_end = span_begin64(s + 1, n_span, N);
  const size_t head = (size_t)N * FD;
  const __amdgpu_buffer_rsrc_t src[2] = {make_rsrc(K + bh * head, (unsigned)(head * 2)),
                                         make_rsrc(V + bh * head, (unsigned)(head * 2))};
  const FavorConsts fc = favor_consts();
  OmegaFrags<true> om;
  om.load(omega, w, g, li);
  const float kappa = favor_kappa(fc, favor_first_norm2(src[0]));
  if (s == 0 && tid == 0) kappa_out[bh] = kappa;

  // dz on the MFMA as well (a ones operand against the same hi + lo feature
  // fragments), off the VALU, which the features keep busy: lane (g, li) of
  // zt[j] ends with the sum over the span of feature 16 (FPW w + j) + li
  f32x4 acc[FPW][FCT], zt[FPW];
#pragma unroll
  for (int j = 0; j < FPW; ++j) {
    zt[j] = zero4();
#pragma unroll
    for (int ct = 0; ct < FCT; ++ct) acc[j][ct] = zero4();
  }
  const bf16 one = static_cast<bf16>(1.0f);
  const bf16x8 ones = bf16x8{one, one, one, one, one, one, one, one};

  // the span's chunks last to first: the output pass, walking its spans
  // forward, then starts on the chunks read last, the likeliest to still
  // sit in the memory-side cache
  const int nch = (t_end - t_begin + FC - 1) / FC;
  RawRegs<2> rr;
  load_raw<2>(rr, src, t_begin + max(nch - 1, 0) * FC);
  int buf = 0;
  for (int k = 0; k < nch; ++k, buf ^= 1) {
    const int t0 = t_begin + (nch - 1 - k) * FC;
    {
      bf16* const dst[2] = {kraw[buf], vt[buf]};
      float* const nrm[2] = {kn[buf], nullptr};
      stage_raw<2>(rr, dst, nrm, 1, 0, kappa, N - t0);
    }
    if (k + 1 < nch) load_raw<2>(rr, src, t0 - FC);
    __syncthreads();

    // V^T fragments (A operands): k-slots 0-3 = tokens 32 kp + 4 g + r,
    // 4-7 = tokens 32 kp + 16 + 4 g + r, matching the projection tiles of
    // token blocks 2 kp and 2 kp + 1.
    bf16x8 va[2][FCT];
#pragma unroll
    for (int kp = 0; kp < 2; ++kp)
#pragma unroll
      for (int ct = 0; ct < FCT; ++ct) va[kp][ct] = tr_frag<64>(vt[buf], 32 * kp + 4 * g, 32 * kp + 16 + 4 * g, 16 * ct, li);

#pragma unroll
    for (int j = 0; j < FPW; ++j) {
      bf16x4 ph[4], pl[4];
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
        const f32x4 p = project<true, true>(kraw[buf], om, j, tb, g, li);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int tok = 16 * tb + 4 * g + r;
          const float f = favor_phi(fc, p[r], kn[buf][tok]);  // 0 past the end (bias -inf)
          const bf16 h = static_cast<bf16>(f);
          ph[tb][r] = h;
          pl[tb][r] = static_cast<bf16>(f - static_cast<float>(h));
        }
      }
#pragma unroll
      for (int kp = 0; kp < 2; ++kp) {
        const bf16x8 bh8 = cat4(ph[2 * kp], ph[2 * kp + 1]);
        const bf16x8 bl8 = cat4(pl[2 * kp], pl[2 * kp + 1]);
#pragma unroll
        for (int ct = 0; ct < FCT; ++ct) {
          acc[j][ct] = mfma16(va[kp][ct], bh8, acc[j][ct]);
          acc[j][ct] = mfma16(va[kp][ct], bl8, acc[j][ct]);
        }
        zt[j] = mfma16(ones, bh8, zt[j]);
        zt[j] = mfma16(ones, bl8, zt[j]);
      }
    }
  }

  float* slot = ws + ((size_t)bh * (n_span + 1) + s) * FE;
#pragma unroll
  for (int j = 0; j < FPW; ++j) {
    const int f = 16 * (FPW * w + j) + li;
#pragma unroll
    for (int ct = 0; ct < FCT; ++ct) *reinterpret_cast<f32x4*>(slot + f * FDV + 16 * ct + 4 * g) = acc[j][ct];
    if (g == 0) slot[FR * FDV + f] = zt[j][0];
  }
}

// ------------------------------------------------------------------ outputs

// The phi(Q)/phi(K) tiles ([token][feature], 256 features) and the carried
// state tile ([feature][value]) of the output pass are only ever accessed in
// 8-byte pieces (4 bf16 starting at a multiple of 4), so their rows are
// swizzled at that granularity: piece p of row r is stored at p ^ hash(r mod 16).
// gfx950 serves 8-byte LDS reads (plain and transposing) 32 lanes at a time
// from 64 four-byte banks, and 8-byte writes 16 lanes at a time from a
// 128-byte window (measured with the bank-conflict counter).  With
//   phi tiles:  hash bits (0..4) = (r3, r2, r0, r1, r3),
//   state tile: hash bits (0..3) = (r0, r3, r1, r2),
// every access pattern of the pass is conflict-free:
//   phi writes (16 consecutive rows, one piece): hash bits 0-3 are a
//     bijection of r, so the rows hit 16 distinct pieces of the window;
//   phi row reads (16 rows x pieces p, p + 1, p even): bits 1-4 are a
//     bijection of r, so the 16 pairs are distinct;
//   phi transposing reads (rows {b..b+3, b+8..b+11} x 4 pieces): bits 2-4
//     are a bijection of (r0, r1, r3), so the 8 aligned groups are distinct;
//   state writes (16 rows, one piece; a row is 128 bytes): the hash is a
//     bijection of r;
//   state transposing reads (8 consecutive rows x 4 pieces): r0 picks the
//     half of the 256-byte bank space, bits 2-3 are a bijection of (r1, r2).
__device__ __forceinline__ int phi_hash(int r) {
  return ((r >> 3) & 1) | (((r >> 2) & 1) << 1) | ((r & 1) << 2) | (((r >> 1) & 1) << 3) | (((r >> 3) & 1) << 4);
}
__device__ __forceinline__ int phi_off(int row, int col) {
  return row * FR + ((((col >> 2) ^ phi_hash(row & 15)) << 2) | (col & 3));
}
__device__ __forceinline__ int st_hash(int r) {
  return (r & 1) | (((r >> 3) & 1) << 1) | (((r >> 1) & 1) << 2) | (((r >> 2) & 1) << 3);
}
__device__ __forceinline__ int st_off(int row, int col) {
  return row * FDV + ((((col >> 2) ^ st_hash(row & 15)) << 2) | (col & 3));
}

constexpr int FZS = FR + 8;  // z row stride: the three rows start 16 bytes apart in bank space

struct SmemOutFavor {
  bf16 qraw[2][FC * FD];
  bf16 kraw[2][FC * FD];
  bf16 v[2][FC * FDV];
  float qn[2][FC];
  float kn[2][FC];
  bf16 sq[FC * FR];   // phi(Q) of the chunk, [token][feature] (phi_off)
  bf16 sk[FC * FR];   // phi(K) of the chunk
  bf16 ss[FR * FDV];  // carried S, [feature][value] (st_off)
  bf16 sz[3 * FZS];   // carried z as rows: bf16 hi, lo = z - hi, zeros
  bf16 so[FC * FDV];  // the chunk's outputs, [token][value] (T64), for whole-row stores
};

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ bf16x4 lds4(const bf16* p) { return *reinterpret_cast<const bf16x4*>(p); }
// 8-byte LDS store as one ds_write_b64 (a bf16x4 store is split in two dword writes)
__device__ __forceinline__ void sts4(bf16* p, bf16x4 v) { *reinterpret_cast<u32x2*>(p) = __builtin_bit_cast(u32x2, v); }
// Transposing operand fragment from two 4-row groups (k-slots 0-3 at p0, 4-7 at p1).
__device__ __forceinline__ bf16x8 tr2(const bf16* p0, const bf16* p1) { return cat4(ds_read_tr4(p0), ds_read_tr4(p1)); }

// Outputs of one span (carried state from the scanned slot when causal, the
// full-sequence sums otherwise).  Per chunk: stage raw Q, K, V (double
// buffered) -> barrier -> the carried state -> LDS, feature tiles of phi(Q),
// phi(K) (wave w: features 32 w .. +31 of every token) -> LDS, and the state
// carry -> barrier -> outputs.  Outputs: the two waves w and 7 - w share row
// block ib = min(w, 7 - w) (query tokens 16 ib + li); each forms the row
// block's weights and denominator and produces value tiles 2 (w / 4) and
// 2 (w / 4) + 1.  Carried state: wave w owns the features it projects,
// 32 w .. +31 (feature tiles 2 w, 2 w + 1), for all four value tiles, and
// their z tiles, so that it carries the state from its own phi(K) values in
// registers, beside the exponentials of the feature phase, where the matrix
// cores would otherwise idle.  phi(K) goes to LDS feature-major ([feature]
// [token], in the state tile's layout), which is what the weights' operand
// reads take, like the state read-out.
template <bool CAUSAL, bool PRECISE>
__global__ __launch_bounds__(FNT, 1) void la_output_favor_kernel(const bf16* __restrict__ Q,
                                                                 const bf16* __restrict__ K,
                                                                 const bf16* __restrict__ V,
                                                                 bf16* __restrict__ O,
                                                                 const float* __restrict__ omega,
                                                                 const float* __restrict__ ws, int N,
                                                                 int n_span) {
  __shared__ SmemOutFavor sm;
  const int tid = threadIdx.x, w = wave_id(), l = tid & 63;
  const int g = l >> 4, li = l & 15, q4 = li >> 2, r4 = li & 3;
  const int bh = blockIdx.x / n_span;
  const int s = blockIdx.x % n_span;
  const int t_begin = span_begin64(s, n_span, N);
  const int t_end = span_begin64(s + 1, n_span, N);
  const size_t head = (size_t)N * FD;
  const unsigned hbytes = (unsigned)(head * 2);
  const __amdgpu_buffer_rsrc_t src[3] = {make_rsrc(Q + bh * head, hbytes), make_rsrc(K + bh * head, hbytes),
                                         make_rsrc(V + bh * head, hbytes)};
  const __amdgpu_buffer_rsrc_t orsrc = make_rsrc(O + bh * head, hbytes);
  const FavorConsts fc = favor_consts();
  OmegaFrags<false> om;  // phi tiles are rounded to bf16 here: omega hi (lo in the precise form)
  om.load(omega, w, g, li);
  const float kappa = CAUSAL ? favor_kappa(fc, favor_first_norm2(src[1])) : 0.f;

  constexpr int TPW = FFT * FCT / FNW;  // carried state tiles per wave (8): [FCT j + ct]
  constexpr int ZPW = FFT / FNW;        // z tiles per wave (2)
  static_assert(TPW == FPW * FCT && ZPW == FPW, "a wave carries the features it projects");
  constexpr int OCT = FCT / 2;          // value tiles per wave in the outputs (2)
  // output row block: waves w and w + 4 run on one SIMD, so they take row
  // blocks b and 3 - b, which balances the causal weight tiles per SIMD
  const int ib = w < 4 ? w : 7 - w;
  const int oct0 = OCT * (w / 4);       // first output value tile

  // Lane offsets (elements) into the LDS tiles, formed once.  Rows 16 apart
  // share a hash, so every access of the chunk loop is one of these plus a
  // compile-time constant.  In the 64-element rows of the state-layout
  // tiles (S and phi(K)^T), piece 4 c + x (c < 4) of a row r sits at
  // 16 (c ^ (H >> 2)) + 4 (x ^ (H & 3)), H = st_hash(r mod 16): a base per
  // row and lane plus 16 (c ^ hh), formed where used.
  int o_raw[2];      // raw Q/K rows (projection operands): row li, columns 32 ks + 8 g
  int o_phw[FPW];    // phi(Q) writes: row li, features 16 (FPW w + j) + 4 g
  int o_prow[4][2];  // phi(Q) row reads: row li, features 32 kq + 16 h + 4 g (k-step kq + 4: + 128)
  int o_vo[OCT];     // V transposing reads (outputs): row 4 g + li / 4, values 16 (oct0 + c) + 4 (li % 4)
  int o_so[OCT];     // S transposing reads: the same rows and columns of the state tile
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    o_raw[h] = T64::off(li, 32 * h + 8 * g);
    o_phw[h] = phi_off(li, 16 * (FPW * w + h) + 4 * g);
    o_vo[h] = T64::off(4 * g + q4, 16 * (oct0 + h) + 4 * r4);
    o_so[h] = st_off(4 * g + q4, 16 * (oct0 + h) + 4 * r4);
#pragma unroll
    for (int kq = 0; kq < 4; ++kq) o_prow[kq][h] = phi_off(li, 32 * kq + 16 * h + 4 * g);
  }
  // S and phi(K)^T writes: row 16 FPW w + li (+ 16 j), piece 4 c + g
  int b_sw = (16 * FPW * w + li) * FDV + 4 * ((g ^ st_hash(li)) & 3), h_sw = st_hash(li) >> 2;
  // phi(K)^T transposing reads (weights): rows 4 g + li / 4 (+ 32 ks, + 16), piece 4 jb + li % 4
  const int h_tr = st_hash((4 * g + q4) & 15);
  int b_kw = (4 * g + q4) * FC + 4 * ((r4 ^ h_tr) & 3), hh_kw = h_tr >> 2;
  const int zrow = min(r4, 2);                                 // z_hi, z_lo or zeros
  const int o_z = zrow * FZS + 4 * g;                          // z row reads (+ 32 ks, + 16)
  // phi operand fragment of row `row` (a multiple of 16 plus li) at k-step ks
  auto prow = [&](const bf16* t, int ks) {
    const bf16* p = t + 128 * (ks >> 2);
    return cat4(lds4(p + o_prow[ks & 3][0]), lds4(p + o_prow[ks & 3][1]));
  };

  const float* pre = ws + ((size_t)bh * (n_span + 1) + (CAUSAL ? s : n_span)) * FE;
  f32x4 sacc[TPW];
#pragma unroll
  for (int j = 0; j < FPW; ++j)
#pragma unroll
    for (int ct = 0; ct < FCT; ++ct)
      sacc[FCT * j + ct] = *reinterpret_cast<const f32x4*>(pre + (16 * (FPW * w + j) + li) * FDV + 16 * ct + 4 * g);
  f32x4 zt[ZPW];
#pragma unroll
  for (int j = 0; j < ZPW; ++j) {
    const float zv = pre[FR * FDV + 16 * (FPW * w + j) + li];
    zt[j] = f32x4{zv, zv, zv, zv};
  }
  const bf16 one = static_cast<bf16>(1.0f), zero = static_cast<bf16>(0.0f);
  const bf16x8 ones = bf16x8{one, one, one, one, one, one, one, one};
  const bf16 o1 = r4 == 0 ? one : zero;
  const bf16x8 ones_rows = bf16x8{o1, o1, o1, o1, o1, o1, o1, o1};  // rows 4m of the ones operand

  // A chunk's outputs go through the LDS tile so and leave, after the next
  // chunk's first barrier, as whole rows: thread t stores 16 bytes of row
  // t / 8 (two waves produce each row).  One store per thread and iteration
  // (the first one, and one in the prologue, aimed past the buffer, where the
  // hardware drops them), issued after the prefetch, so that at the loop
  // head the memory operations outstanding are the same on every path and
  // the staging's counter wait covers the prefetched loads only.
  const int srow = tid >> 3, scol = 8 * (tid & 7);
  int o_or = T64::off(srow, scol);                             // row reads of so
  int o_ow = T64::off(16 * ib + li, 16 * oct0 + 4 * g);         // writes of so (value tile oct0 + c: XOR 16 c)
  auto store_rows = [&](int t, bool real) {
    const u32x4 x = *reinterpret_cast<const u32x4*>(sm.so + o_or);
    __builtin_amdgcn_raw_buffer_store_b128(x, orsrc, real ? ((t + srow) * FDV + scol) * 2 : kDropOffset, 0,
                                           kStreamStore);
  };
  RawRegs<3> rr;
  load_raw<3>(rr, src, t_begin);
  mem_order_fence();
  __builtin_amdgcn_raw_buffer_store_b128(u32x4{0u, 0u, 0u, 0u}, orsrc, kDropOffset, 0, kStreamStore);
  int buf = 0;
  for (int t0 = t_begin; t0 < t_end; t0 += FC, buf ^= 1) {
    // the XORed offsets of the state-layout tiles and the output tile are
    // formed in the loop rather than kept live across it (registers are
    // tight at two waves per SIMD)
    asm volatile("" : "+v"(b_sw), "+v"(h_sw), "+v"(b_kw), "+v"(hh_kw), "+v"(o_or), "+v"(o_ow));
    {
      bf16* const dst[3] = {sm.qraw[buf], sm.kraw[buf], sm.v[buf]};
      float* const nrm[3] = {sm.qn[buf], sm.kn[buf], nullptr};
      stage_raw<3>(rr, dst, nrm, CAUSAL ? 3 : 1, 1, kappa, N - t0);
    }
    if (t0 + FC < t_end) load_raw<3>(rr, src, t0 + FC);
    __syncthreads();
    store_rows(t0 - FC, t0 != t_begin);  // the previous chunk's outputs (rows past N are dropped)

    // the carried state before this chunk -> LDS (the carry below then
    // updates the registers)
    if (CAUSAL || t0 == t_begin) {
#pragma unroll
      for (int j = 0; j < FPW; ++j)
#pragma unroll
        for (int ct = 0; ct < FCT; ++ct)
          sts4(sm.ss + 16 * j * FDV + b_sw + 16 * (ct ^ h_sw), cvt_bf16x4(sacc[FCT * j + ct]));
      // lane group 0 writes z_hi, group 1 z_lo, group 2 the zero row
      if (g < 3) {
#pragma unroll
        for (int j = 0; j < ZPW; ++j) {
          const float z = zt[j][0];
          const bf16 h = static_cast<bf16>(z);
          const bf16 v = g == 0 ? h : g == 1 ? static_cast<bf16>(z - static_cast<float>(h)) : zero;
          sm.sz[g * FZS + 16 * (FPW * w + j) + li] = v;
        }
      }
    }

    // feature tiles (features of tokens past the end are 0 through their
    // -inf bias).  phi(Q): lane (g, li) gets features 16 ft + 4 g + r of
    // token 16 tb + li; phi(K), projected the other way round: tokens
    // 16 tb + 4 g + r of feature 16 ft + li, kept in registers for the carry.
    // Token block by token block, both feature tiles of the wave from one
    // read of the raw rows; the raw rows of block tb + 1 are read before the
    // tiles of block tb are written, so that the reads do not wait behind
    // the writes.
    {
      constexpr int NST = CAUSAL ? 2 : 1;  // streams with features: Q, and K when causal
      const bf16* const raw[2] = {sm.qraw[buf], sm.kraw[buf]};
      bf16x8 xf[2][NST][2];  // [token block parity][stream][k-step]
      float nb[2];           // phi(Q) biases of token 16 tb + li
      f32x4 kb[2];           // phi(K) biases of tokens 16 tb + 4 g + r
      auto read_block = [&](int tb, int p) {
#pragma unroll
        for (int st = 0; st < NST; ++st) {
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) xf[p][st][ks] = load_frag(raw[st] + 16 * tb * FD + o_raw[ks]);
        }
        nb[p] = sm.qn[buf][16 * tb + li];
        if constexpr (CAUSAL) kb[p] = *reinterpret_cast<const f32x4*>(&sm.kn[buf][16 * tb + 4 * g]);
      };
      bf16x4 kh[FPW][4];  // phi(K) of the wave's features, [j][tb]
      // the precise form: omega's lo fragments, read once per chunk (from cache)
      bf16x8 olo[PRECISE ? FPW : 1][2];
      if constexpr (PRECISE) {
        const __amdgpu_buffer_rsrc_t omrsrc = make_rsrc(omega, FR * FD * 4);
#pragma unroll
        for (int j = 0; j < FPW; ++j)
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) olo[j][ks] = omega_lo_frag(omrsrc, w, j, ks);
      }
      read_block(0, 0);
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
        const int p = tb & 1;
        if (tb < 3) read_block(tb + 1, p ^ 1);
        f32x4 pr[NST][FPW];
#pragma unroll
        for (int st = 0; st < NST; ++st)
#pragma unroll
          for (int j = 0; j < FPW; ++j) {
            pr[st][j] = zero4();
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
              if (st == 0) {
                pr[st][j] = mfma16(om.hi[j][ks], xf[p][st][ks], pr[st][j]);
                if constexpr (PRECISE) pr[st][j] = mfma16(olo[j][ks], xf[p][st][ks], pr[st][j]);
              } else {
                pr[st][j] = mfma16(xf[p][st][ks], om.hi[j][ks], pr[st][j]);
                if constexpr (PRECISE) pr[st][j] = mfma16(xf[p][st][ks], olo[j][ks], pr[st][j]);
              }
            }
          }
#pragma unroll
        for (int j = 0; j < FPW; ++j) {
          bf16x4 h;
#pragma unroll
          for (int r = 0; r < 4; ++r) h[r] = static_cast<bf16>(favor_phi(fc, pr[0][j][r], nb[p]));
          sts4(sm.sq + 16 * tb * FR + o_phw[j], h);
        }
        if constexpr (CAUSAL) {
#pragma unroll
          for (int j = 0; j < FPW; ++j) {
#pragma unroll
            for (int r = 0; r < 4; ++r) kh[j][tb][r] = static_cast<bf16>(favor_phi(fc, pr[NST - 1][j][r], kb[p][r]));
            sts4(sm.sk + 16 * j * FC + b_sw + 16 * (tb ^ h_sw), kh[j][tb]);
          }
        }
      }
      // ---- state carry: S += phi(K_c)^T V_c, z += phi(K_c)^T 1, from the
      // wave's own phi(K) values (bf16, as the weights use them).  V^T
      // fragments: k-slots 0-3 = tokens 32 kp + 4 g + r, 4-7 = tokens
      // 32 kp + 16 + 4 g + r, the token order of token blocks 2 kp, 2 kp + 1.
      if constexpr (CAUSAL) {
#pragma unroll
        for (int kp = 0; kp < 2; ++kp) {
          bf16x8 bk[FPW];
#pragma unroll
          for (int j = 0; j < FPW; ++j) bk[j] = cat4(kh[j][2 * kp], kh[j][2 * kp + 1]);
#pragma unroll
          for (int ct = 0; ct < FCT; ++ct) {
            const bf16x8 va = tr_frag<64>(sm.v[buf], 32 * kp + 4 * g, 32 * kp + 16 + 4 * g, 16 * ct, li);
#pragma unroll
            for (int j = 0; j < FPW; ++j) sacc[FCT * j + ct] = mfma16(va, bk[j], sacc[FCT * j + ct]);
          }
#pragma unroll
          for (int j = 0; j < FPW; ++j) zt[j] = mfma16(ones, bk[j], zt[j]);
        }
      }
    }
    __syncthreads();

    // ---- outputs of row block ib, value tiles oct0, oct0 + 1
    const bf16* vb = sm.v[buf];
    const bf16* sq_ib = sm.sq + 16 * ib * FR;
    bf16x8 qf[FR / 32];
    f32x4 dacc = zero4();  // [0] = z_hi . phi(q) + rowsum(weights), [1] = z_lo . phi(q)
#pragma unroll
    for (int ks = 0; ks < FR / 32; ++ks) {
      qf[ks] = prow(sq_ib, ks);
      const bf16* zp = sm.sz + o_z + 32 * ks;
      dacc = mfma16(cat4(lds4(zp), lds4(zp + 16)), qf[ks], dacc);
    }
    f32x4 o[OCT];
#pragma unroll
    for (int c = 0; c < OCT; ++c) o[c] = zero4();
    if constexpr (CAUSAL) {
      // weights of key block jb: lane (g, li) holds A[i = li][j = 16 jb + 4 g + r];
      // the diagonal block is masked to j <= i by selection
      auto weights = [&](int jb) {
        f32x4 t = zero4();
        const bf16* kbase = sm.sk + b_kw + 16 * (jb ^ hh_kw);
#pragma unroll
        for (int ks = 0; ks < FR / 32; ++ks) {
          const bf16* p0 = kbase + 32 * ks * FC;
          t = mfma16(tr2(p0, p0 + 16 * FC), qf[ks], t);
        }
        if (jb == ib) {  // wave-uniform: only the diagonal block is masked
#pragma unroll
          for (int r = 0; r < 4; ++r) t[r] = 4 * g + r > li ? 0.f : t[r];
        }
        return t;
      };
#pragma unroll
      for (int jp = 0; jp < 2; ++jp) {
        const int jb0 = 2 * jp, jb1 = 2 * jp + 1;
        if (jb0 > ib) continue;
        const f32x4 a0 = weights(jb0);
        const bool two = jb1 <= ib;
        const f32x4 a1 = two ? weights(jb1) : zero4();
        const float w8[8] = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
        const bf16x8 bv = cvt_bf16x8(w8);
        dacc = mfma16(ones_rows, bv, dacc);
#pragma unroll
        for (int c = 0; c < OCT; ++c) {
          const bf16* p0 = vb + o_vo[c] + 16 * jb0 * FDV;
          const bf16x8 av = two ? tr2(p0, p0 + 16 * FDV) : cat4(ds_read_tr4(p0), bf16x4{0, 0, 0, 0});
          o[c] = mfma16(av, bv, o[c]);
        }
      }
    }
#pragma unroll
    for (int c = 0; c < OCT; ++c)
#pragma unroll
      for (int ks = 0; ks < FR / 32; ++ks) {
        const bf16* p0 = sm.ss + o_so[c] + 32 * ks * FDV;
        o[c] = mfma16(tr2(p0, p0 + 16 * FDV), qf[ks], o[c]);
      }
    const float rden = __builtin_amdgcn_rcpf(dacc[0] + dacc[1]);
#pragma unroll
    for (int c = 0; c < OCT; ++c) sts4(sm.so + (o_ow ^ (16 * c)), cvt_bf16x4(o[c] * rden));

  }
  if (t_end > t_begin) {
    __syncthreads();
    store_rows(t_begin + ((t_end - t_begin - 1) / FC) * FC, true);
  }
}

}  // namespace

bool favor_prefill_supported(int io, int d, int dv, int r, int chunk) {
  return io == 1 && d == FD && dv == FDV && r == FR && chunk == FC;
}

hipError_t favor_prefill_launch(const PrefillArgs& a) {
  const bf16* Q = static_cast<const bf16*>(a.Q);
  const bf16* K = static_cast<const bf16*>(a.K);
  const bf16* V = static_cast<const bf16*>(a.V);
  bf16* O = static_cast<bf16*>(a.O);
  float* ws = static_cast<float*>(a.workspace);
  const int BH = a.B * a.H;
  hipStream_t st = static_cast<hipStream_t>(a.stream);
  const int n_span = a.n_span;
  (void)hipGetLastError();
  auto rec = [&](int i) {
    if (a.events && a.events[i]) (void)hipEventRecord(static_cast<hipEvent_t>(a.events[i]), st);
  };
  // one log2 state scale per head after the span states (written by the
  // state pass; with no spans, none is applied)
  float* kappa = reinterpret_cast<float*>(static_cast<char*>(a.workspace) + favor_kappa_offset(BH, n_span, FR, FDV));
  rec(0);
  if (n_span > 0 && BH > 0)
    hipLaunchKernelGGL(la_state_favor_kernel, dim3(BH * n_span), dim3(FNT), 0, st, K, V, a.omega, ws, kappa, a.N,
                       n_span);
  rec(1);
  rec(2);
  hipError_t e = scan_launch(ws, BH, FR, FDV, n_span, a.S0, a.z0, a.S_out, a.z_out, st, nullptr, 1, 0, 64, nullptr,
                             0, !a.causal, n_span > 0 ? kappa : nullptr);
  if (e != hipSuccess) return e;
  rec(3);
  rec(4);
  if (n_span > 0 && BH > 0) {
    const dim3 grid(BH * n_span), block(FNT);
    if (a.causal && a.favor_precise)
      hipLaunchKernelGGL((la_output_favor_kernel<true, true>), grid, block, 0, st, Q, K, V, O, a.omega, ws, a.N,
                         n_span);
    else if (a.causal)
      hipLaunchKernelGGL((la_output_favor_kernel<true, false>), grid, block, 0, st, Q, K, V, O, a.omega, ws, a.N,
                         n_span);
    else if (a.favor_precise)
      hipLaunchKernelGGL((la_output_favor_kernel<false, true>), grid, block, 0, st, Q, K, V, O, a.omega, ws, a.N,
                         n_span);
    else
      hipLaunchKernelGGL((la_output_favor_kernel<false, false>), grid, block, 0, st, Q, K, V, O, a.omega, ws, a.N,
                         n_span);
  }
  rec(5);
  return hipGetLastError();
}

}  // namespace la
