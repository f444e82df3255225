// Internal (C++) interface between the C-ABI layer and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace la {

struct PrefillArgs {
  const void* Q;
  const void* K;
  const void* V;
  void* O;
  int B, H, N, d, dv, r;
  int io;      // 0 = fp32, 1 = bf16
  int phi;     // PhiKind
  const float* omega;
  int causal;
  int chunk;
  int n_span;  // spans per head (a head's chunks split evenly over them)
  const float* S0;
  const float* z0;
  float* S_out;
  float* z_out;
  void* workspace;
  void* stream;
  void* const* events;  // optional: 6 hipEvent_t recorded around the three kernels
  int favor_precise = 0;  // FAVOR+: output-pass projections with omega hi + lo
  // fixed per-head decay (device [H] fp32 in (0, 1]; null: none), causal
  // pointwise maps only: S_t = gamma S_{t-1} + phi(k_t) v_t^T, z likewise
  const float* gamma = nullptr;
  int normalize = 1;    // 0: o_t = phi(q_t)^T S_t (no division by phi(q_t)^T z_t)
  // per-token gate (device [B*H][N] fp32, natural log of a_t <= 0; null:
  // none), causal pointwise maps only: S_t = a_t S_{t-1} + phi(k_t) v_t^T,
  // z likewise; excludes gamma.  The workspace then also holds one fp32
  // total log2 gate per (head, span) after the span states.
  const float* log_a = nullptr;
  // per-token, per-key-channel gate (device [B*H][N][r] fp32, natural logs;
  // null: none), causal pointwise maps only: S_t = diag(a_t) S_{t-1} +
  // phi(k_t) v_t^T; excludes gamma and log_a.  The workspace then also holds
  // r fp32 total log2 gates per (head, span) after the span states.
  const float* log_a_ch = nullptr;
};

// Workspace of the three-kernel path: fp32 span states [B*H][n_span+1][R*DV+R],
// then (gated decay) the spans' total log2 gates [B*H][n_span].
inline size_t prefill_workspace_bytes(long long BH, int n_span, int r, int dv, bool gated, bool per_channel = false) {
  const size_t E = (size_t)r * dv + r;
  const size_t tot = per_channel ? (size_t)BH * n_span * r : gated ? (size_t)BH * n_span : 0;
  return (size_t)BH * ((size_t)n_span + 1) * E * sizeof(float) + tot * sizeof(float);
}
// FAVOR+ workspace: the span states, then one fp32 per head (the log2
// scale kappa of its stored states), at a 256-byte boundary.
inline size_t favor_workspace_bytes(long long BH, int n_span, int r, int dv) {
  const size_t states = ((prefill_workspace_bytes(BH, n_span, r, dv, false) + 255) / 256) * 256;
  return states + (size_t)BH * sizeof(float);
}
inline size_t favor_kappa_offset(long long BH, int n_span, int r, int dv) {
  return ((prefill_workspace_bytes(BH, n_span, r, dv, false) + 255) / 256) * 256;
}
// Shapes the per-channel gated prefill supports (causal, ELU+1 / identity).
bool gla_supported(int io, int d, int dv, int r, int chunk);

bool prefill_supported(int io, int phi, int d, int dv, int r, int chunk);
hipError_t prefill_launch(const PrefillArgs& a);

// FAVOR+ prefill (la_prefill_favor.hip).
bool favor_prefill_supported(int io, int d, int dv, int r, int chunk);
hipError_t favor_prefill_launch(const PrefillArgs& a);

// Span scan over a workspace of R x DV states (la_prefill.hip).  With a decay
// (gamma, H heads), a span of L tokens multiplies the running state by
// gamma^L; span lengths follow from N, the chunk and n_span.  With gates
// (totals: [BH][n_span] total log2 gate of each span), span s multiplies it
// by 2^totals[s].  total_only (no decay or gates): only the total, slot
// n_span, is written (what the non-causal form reads).  kappa (no decay or
// gates; device [BH] fp32, null: none): the span states are stored at
// 2^kappa[bh] times their value, so S0/z0 are multiplied by 2^kappa on entry
// and S_out/z_out by 2^-kappa.
hipError_t scan_launch(float* ws, int BH, int R, int DV, int n_span, const float* S0, const float* z0,
                       float* S_out, float* z_out, hipStream_t stream, const float* gamma = nullptr, int H = 1,
                       int N = 0, int chunk = 64, const float* totals = nullptr, int per_channel = 0,
                       int total_only = 0, const float* kappa = nullptr);

// Gradients of the causal normalised output (la_prefill.hip).
struct BackwardArgs {
  const void* Q;
  const void* K;
  const void* V;
  const void* O;
  const void* dO;
  void* dQ;
  void* dK;
  void* dV;
  int B, H, N, d, dv, r;
  int io, phi, chunk, n_span;
  void* workspace;
  void* stream;
  void* const* events;  // optional: 10 hipEvent_t around the five kernels
};
// Workspace: forward span states, reverse span sums (both [B*H][n_span+1]
// [r*d_v + r] fp32), then (D_i, h_i) per token ([B*H][N][2] fp32).
inline size_t backward_workspace_bytes(long long BH, int n_span, int N, int r, int dv) {
  const size_t E = (size_t)r * dv + r;
  return (2 * (size_t)BH * ((size_t)n_span + 1) * E + (size_t)BH * N * 2) * sizeof(float);
}
bool backward_supported(int io, int phi, int d, int dv, int r, int chunk);
hipError_t backward_launch(const BackwardArgs& a);

struct DecodeArgs {
  const float* S;
  const float* z;
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* S_new;
  float* z_new;
  int B, H, d, dv, r;
  int io;
  int phi;
  const float* omega;
  void* stream;
  const float* gamma = nullptr;  // per-head decay (device [H]); null: none
  int normalize = 1;
  const float* log_a = nullptr;  // this token's gate per (batch, head), natural log (device [B*H]); null: none
  const float* log_a_ch = nullptr;  // this token's per-channel gates, natural logs (device [B*H][r]); null: none
};

bool decode_supported(int io, int phi, int d, int dv, int r);
hipError_t decode_launch(const DecodeArgs& a);

struct FeatureArgs {
  const void* X;
  float* Y;
  long long rows;
  int d, r;
  int io;
  int phi;
  const float* omega;
  void* stream;
};

bool feature_supported(int io, int phi, int d, int r);
hipError_t feature_launch(const FeatureArgs& a);

}  // namespace la
