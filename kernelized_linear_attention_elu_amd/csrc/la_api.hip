// C-ABI layer: argument validation, span choice, workspace sizing, dispatch.
// Validation makes no device calls, so every error path can be exercised on
// a machine without a GPU (the span choice asks the runtime for the current
// device's compute-unit count and falls back to 256 when there is none).
#include <stdint.h>
#include <stdlib.h>

#include <algorithm>
#include <atomic>
#include <mutex>

#include <hip/hip_runtime.h>

#include "la.h"
#include "la_prefill.h"

namespace {

constexpr int kMaxDim = 1 << 20;

// Text of the most recent HIP failure seen by a call on this thread.
thread_local const char* t_last_hip_error = "";

la_status hip_status(hipError_t e) {
  if (e == hipSuccess) return LA_OK;
  t_last_hip_error = hipGetErrorString(e);
  return LA_ERR_HIP;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// The precise FAVOR+ form computes the same features as LA_PHI_FAVOR (only
// the prefill output pass differs): everything but that pass sees FAVOR.
int canon_phi(int phi) { return phi == LA_PHI_FAVOR_PRECISE ? LA_PHI_FAVOR : phi; }

int norm_r(int phi, int d, int r) {
  if (phi == LA_PHI_ELU1 || phi == LA_PHI_IDENTITY) return r == 0 ? d : r;
  return r;
}

int norm_chunk(int chunk) { return chunk == 0 ? 64 : chunk; }

// Spans per head.  Both prefill kernels run one workgroup per (head, span)
// and a span's chunks are contiguous; spans of a head differ by at most one
// chunk.  The default fills one round of workgroup slots of the output
// kernel (the device's compute units x workgroups per CU at its occupancy
// for this configuration) so that no CU runs a partial second round, but
// keeps at least 4 chunks per span so that the per-span state traffic
// (r*d_v*4 bytes written, scanned and read back) stays small next to the
// span's data.  la_set_span_tokens sets a process-wide span length instead
// (tests use it to force several spans per head).

// Span length set by la_set_span_tokens (0: the default choice).
std::atomic<int> g_span_tokens{0};

// Compute units of the calling thread's current device, queried once per
// device (256 on MI355X; also the answer when no device can be queried, so
// that shape queries work on a host without a GPU).
constexpr int kDefaultCUs = 256;
constexpr int kMaxDevices = 64;
std::atomic<int> g_cus[kMaxDevices];

int device_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return kDefaultCUs;
  }
  int n = g_cus[dev].load(std::memory_order_relaxed);
  if (n > 0) return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
    (void)hipGetLastError();
    n = kDefaultCUs;
  }
  g_cus[dev].store(n, std::memory_order_relaxed);
  return n;
}

int output_occupancy(int io, int phi, int d, int chunk, int causal, int decay) {
  if (phi == LA_PHI_FAVOR) return 1;
  // per-channel gates: three weighted key tiles and the gate tile in LDS
  if (decay == 2) return (io == LA_BF16 && d == 64 && chunk <= 64) ? 2 : 1;
  // with a decay the output kernel runs two workgroups per CU at d = 64
  if (decay) return (d == 64 && chunk <= 64) ? 2 : 1;
  // the non-causal output kernel holds only Q chunks and the shared sums
  if (!causal && io == LA_BF16 && d == 64) return 6;
  if (d == 64) {
    if (io == LA_BF16) return chunk <= 32 ? 4 : (chunk == 64 ? 3 : 1);
    return chunk <= 32 ? 4 : 3;
  }
  return 1;  // d = 128: one workgroup of eight waves per CU
}

int choose_n_span(long long BH, int N, int chunk, int d, int io, int phi, int causal, int decay) {
  if (N <= 0) return 0;
  const long long n_chunks = (static_cast<long long>(N) + chunk - 1) / chunk;
  const int v = g_span_tokens.load(std::memory_order_relaxed);
  if (v >= chunk && v % chunk == 0) return static_cast<int>((static_cast<long long>(N) + v - 1) / v);
  // Spans fill two workgroups per CU, or the output kernel's occupancy when
  // that is lower: an even two per CU (every CU holds two state and two
  // output workgroups for the whole kernel) measured faster than filling
  // the kernel's three (causal) or six (non-causal) workgroups per CU with
  // shorter spans - long causal 151 -> 148 us, prefill B4 H16 N4096 51 ->
  // 48 us, long non-causal 119 -> 110 us - and counts that do not divide
  // over the CUs were slower than either.
  const int per_cu = std::min(output_occupancy(io, phi, d, chunk, causal, decay), 2);
  const long long slots = static_cast<long long>(device_cus()) * per_cu;
  long long n = (slots + BH - 1) / (BH > 0 ? BH : 1);
  const long long cap = n_chunks / 4 > 0 ? n_chunks / 4 : 1;
  if (n > cap) n = cap;
  if (n < 1) n = 1;
  return static_cast<int>(n);
}

struct Shape {
  int B, H, N, d, dv, r, phi, causal, chunk, n_span;
  long long BH;
};

// decay: 1 for a fixed per-head decay or per-token gates, 2 for per-channel
// gates (causal, pointwise maps only).
la_status check_forward_shape(int B, int H, int N, int d, int d_v, int io, int phi, int r, int causal, int chunk,
                              Shape* sh, int decay = 0) {
  if (B < 0 || H < 0 || N < 0 || d <= 0 || d_v <= 0 || r < 0 || chunk < 0) return LA_ERR_SHAPE;
  if (d > kMaxDim || d_v > kMaxDim || r > kMaxDim) return LA_ERR_SHAPE;
  if (io != LA_F32 && io != LA_BF16) return LA_ERR_UNSUPPORTED;
  if (phi != LA_PHI_ELU1 && phi != LA_PHI_FAVOR && phi != LA_PHI_IDENTITY) return LA_ERR_UNSUPPORTED;
  if (causal != 0 && causal != 1) return LA_ERR_UNSUPPORTED;
  if (decay && (phi == LA_PHI_FAVOR || !causal)) return LA_ERR_UNSUPPORTED;
  const int rr = norm_r(phi, d, r);
  const int ch = decay == 2 && chunk == 0 && d == 128 ? 32 : norm_chunk(chunk);
  if (!la::prefill_supported(io, phi, d, d_v, rr, ch)) return LA_ERR_UNSUPPORTED;
  if (decay == 2 && !la::gla_supported(io, d, d_v, rr, ch)) return LA_ERR_UNSUPPORTED;
  const long long BH = static_cast<long long>(B) * H;
  if (BH > (1LL << 30)) return LA_ERR_SHAPE;
  // a head's Q/K/V/O must fit a 32-bit buffer range (the kernels address
  // each head through a buffer resource), and the grid (B*H*n_span
  // workgroups) must fit a 32-bit launch
  const long long row = static_cast<long long>(d > d_v ? d : d_v) * (io == LA_BF16 ? 2 : 4);
  if (static_cast<long long>(N) * row >= (1LL << 31)) return LA_ERR_SHAPE;
  // per-channel gates: a head's [N][r] fp32 gates, one chunk past N included
  if (decay == 2 && (static_cast<long long>(N) + 128) * rr * 4 >= (1LL << 31)) return LA_ERR_SHAPE;
  const int n_span = choose_n_span(BH, N, ch, d, io, phi, causal, decay);
  if (BH * n_span > 0x7fffffffLL) return LA_ERR_SHAPE;
  sh->B = B; sh->H = H; sh->N = N; sh->d = d; sh->dv = d_v; sh->r = rr; sh->phi = phi;
  sh->causal = causal; sh->chunk = ch; sh->n_span = n_span; sh->BH = BH;
  return LA_OK;
}

size_t workspace_for(const Shape& sh, bool gated = false, bool per_channel = false) {
  if (sh.phi == LA_PHI_FAVOR) return la::favor_workspace_bytes(sh.BH, sh.n_span, sh.r, sh.dv);
  return la::prefill_workspace_bytes(sh.BH, sh.n_span, sh.r, sh.dv, gated, per_channel);
}

// gamma: fixed per-head decay; log_a: per-token gates; log_a_ch: per-token,
// per-channel gates (at most one of the three).
la_status forward_impl(const void* Q, const void* K, const void* V, void* O, int B, int H, int N, int d,
                       int d_v, int io, int phi, int r, const float* omega, int causal, int chunk, const float* S0,
                       const float* z0, float* S_out, float* z_out, void* workspace, size_t workspace_bytes,
                       void* stream, void* const* events, const float* gamma = nullptr, int normalize = 1,
                       const float* log_a = nullptr, const float* log_a_ch = nullptr) {
  const bool precise = phi == LA_PHI_FAVOR_PRECISE;
  phi = canon_phi(phi);
  Shape sh;
  const int decay = log_a_ch != nullptr ? 2 : (gamma != nullptr || log_a != nullptr) ? 1 : 0;
  la_status st = check_forward_shape(B, H, N, d, d_v, io, phi, r, causal, chunk, &sh, decay);
  if (st != LA_OK) return st;
  const bool have_tokens = sh.BH > 0 && N > 0;
  if (have_tokens && (!Q || !K || !V || !O)) return LA_ERR_NULL;
  if (phi == LA_PHI_FAVOR && !omega) return LA_ERR_NULL;
  if ((S0 == nullptr) != (z0 == nullptr)) return LA_ERR_NULL;
  if ((S_out == nullptr) != (z_out == nullptr)) return LA_ERR_NULL;
  const void* ptrs[] = {Q, K, V, O, omega, S0, z0, S_out, z_out, workspace, gamma, log_a, log_a_ch};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return LA_ERR_ALIGN;
  const size_t need = workspace_for(sh, log_a != nullptr, log_a_ch != nullptr);
  if (sh.BH > 0 && (!workspace || workspace_bytes < need)) return LA_ERR_WORKSPACE;
  if (sh.BH == 0) return LA_OK;

  la::PrefillArgs a;
  a.Q = Q; a.K = K; a.V = V; a.O = O;
  a.B = B; a.H = H; a.N = N; a.d = d; a.dv = d_v; a.r = sh.r;
  a.io = io; a.phi = phi; a.omega = omega; a.causal = causal;
  a.chunk = sh.chunk; a.n_span = sh.n_span;
  a.S0 = S0; a.z0 = z0; a.S_out = S_out; a.z_out = z_out;
  a.workspace = workspace; a.stream = stream; a.events = events;
  a.gamma = gamma; a.normalize = normalize; a.log_a = log_a; a.log_a_ch = log_a_ch;
  a.favor_precise = precise ? 1 : 0;
  return hip_status(la::prefill_launch(a));
}

// ------------------------------------------------------------------ fixed scratch

// Device memory of la_forward_noalloc, for callers that cannot allocate: the
// span states of the three-kernel path live in this file-scope array, of
// which every GPU the library runs on holds its own copy until the process
// ends.  Host code never passes the array's name to a kernel: its device
// address on the current GPU comes from hipGetSymbolAddress, looked up once
// per device on that device's first call and kept below.
constexpr size_t kScratchBytes = LA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

la_status scratch_address(void** out) {
  int dev = 0;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e);
  if (dev < 0 || dev >= kMaxDevices) return LA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t es = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (es != hipSuccess) return hip_status(es);
    if (!p) return LA_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return LA_OK;
}

}  // namespace

extern "C" {

la_status la_set_span_tokens(int tokens) {
  if (tokens < 0 || tokens > (1 << 24) || tokens % 16 != 0) return LA_ERR_SHAPE;
  g_span_tokens.store(tokens, std::memory_order_relaxed);
  return LA_OK;
}

int la_get_span_tokens(void) { return g_span_tokens.load(std::memory_order_relaxed); }

size_t la_forward_workspace_bytes(int B, int H, int N, int d, int d_v, int io_dtype, int phi, int r, int causal,
                                  int chunk) {
  Shape sh;
  if (check_forward_shape(B, H, N, d, d_v, io_dtype, canon_phi(phi), r, causal, chunk, &sh) != LA_OK) return 0;
  return workspace_for(sh);
}

la_status la_forward_config(int B, int H, int N, int d, int d_v, int io_dtype, int phi, int r, int causal, int chunk,
                            int* n_span, int* single_pass) {
  Shape sh;
  const la_status st = check_forward_shape(B, H, N, d, d_v, io_dtype, canon_phi(phi), r, causal, chunk, &sh);
  if (st != LA_OK) return st;
  if (n_span) *n_span = sh.n_span;
  if (single_pass) *single_pass = 0;
  return LA_OK;
}

la_status la_forward_decay_config(int B, int H, int N, int d, int d_v, int io_dtype, int phi, int r, int chunk,
                                  int* n_span) {
  Shape sh;
  const la_status st = check_forward_shape(B, H, N, d, d_v, io_dtype, phi, r, 1, chunk, &sh, 1);
  if (st != LA_OK) return st;
  if (n_span) *n_span = sh.n_span;
  return LA_OK;
}

la_status la_forward(const void* Q, const void* K, const void* V, void* O, int B, int H, int N, int d, int d_v,
                     int io_dtype, int phi, int r, const float* omega, int causal, int chunk, const float* S0,
                     const float* z0, float* S_out, float* z_out, void* workspace, size_t workspace_bytes,
                     void* stream) {
  return forward_impl(Q, K, V, O, B, H, N, d, d_v, io_dtype, phi, r, omega, causal, chunk, S0, z0, S_out, z_out,
                      workspace, workspace_bytes, stream, nullptr);
}

la_status la_forward_timed(const void* Q, const void* K, const void* V, void* O, int B, int H, int N, int d,
                           int d_v, int io_dtype, int phi, int r, const float* omega, int causal, int chunk,
                           const float* S0, const float* z0, float* S_out, float* z_out, void* workspace,
                           size_t workspace_bytes, void* stream, void* const* events) {
  return forward_impl(Q, K, V, O, B, H, N, d, d_v, io_dtype, phi, r, omega, causal, chunk, S0, z0, S_out, z_out,
                      workspace, workspace_bytes, stream, events);
}

la_status la_forward_noalloc(const void* Q, const void* K, const void* V, void* O, int B, int H, int N, int d,
                             int d_v, int io_dtype, int phi, int r, const float* omega, int causal, int chunk,
                             const float* S0, const float* z0, float* S_out, float* z_out, void* stream) {
  // the size limit is checked before any runtime call
  Shape sh;
  const la_status st = check_forward_shape(B, H, N, d, d_v, io_dtype, canon_phi(phi), r, causal, chunk, &sh);
  if (st != LA_OK) return st;
  if (workspace_for(sh) > kScratchBytes) return LA_ERR_SCRATCH;
  if (sh.BH == 0) return LA_OK;
  void* ws = nullptr;
  const la_status sa = scratch_address(&ws);
  if (sa != LA_OK) return sa;
  return forward_impl(Q, K, V, O, B, H, N, d, d_v, io_dtype, phi, r, omega, causal, chunk, S0, z0, S_out, z_out,
                      ws, kScratchBytes, stream, nullptr);
}

namespace {

la_status decode_impl(const float* S, const float* z, const void* q, const void* k, const void* v, void* o,
                      float* S_new, float* z_new, int B, int H, int d, int d_v, int io_dtype, int phi, int r,
                      const float* omega, void* stream, const float* gamma, int normalize,
                      const float* log_a = nullptr, const float* log_a_ch = nullptr) {
  if (!gamma && !log_a && !log_a_ch) phi = canon_phi(phi);
  if (B < 0 || H < 0 || d <= 0 || d_v <= 0 || r < 0) return LA_ERR_SHAPE;
  if (static_cast<long long>(B) * H > 0x7fffffffLL) return LA_ERR_SHAPE;
  if (io_dtype != LA_F32 && io_dtype != LA_BF16) return LA_ERR_UNSUPPORTED;
  if (phi != LA_PHI_ELU1 && phi != LA_PHI_FAVOR && phi != LA_PHI_IDENTITY) return LA_ERR_UNSUPPORTED;
  const int rr = norm_r(phi, d, r);
  if (!la::decode_supported(io_dtype, phi, d, d_v, rr)) return LA_ERR_UNSUPPORTED;
  const long long BH = static_cast<long long>(B) * H;
  if (BH > 0 && (!S || !z || !q || !k || !v || !o || !S_new || !z_new)) return LA_ERR_NULL;
  if (phi == LA_PHI_FAVOR && !omega) return LA_ERR_NULL;
  const void* ptrs[] = {S, z, q, k, v, o, S_new, z_new, omega, gamma, log_a, log_a_ch};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return LA_ERR_ALIGN;
  if (BH == 0) return LA_OK;
  la::DecodeArgs a;
  a.S = S; a.z = z; a.q = q; a.k = k; a.v = v; a.o = o; a.S_new = S_new; a.z_new = z_new;
  a.B = B; a.H = H; a.d = d; a.dv = d_v; a.r = rr; a.io = io_dtype; a.phi = phi; a.omega = omega;
  a.stream = stream; a.gamma = gamma; a.normalize = normalize; a.log_a = log_a; a.log_a_ch = log_a_ch;
  return hip_status(la::decode_launch(a));
}

}  // namespace

la_status la_decode_step(const float* S, const float* z, const void* q, const void* k, const void* v, void* o,
                         float* S_new, float* z_new, int B, int H, int d, int d_v, int io_dtype, int phi, int r,
                         const float* omega, void* stream) {
  return decode_impl(S, z, q, k, v, o, S_new, z_new, B, H, d, d_v, io_dtype, phi, r, omega, stream, nullptr, 1);
}

la_status la_forward_decay(const void* Q, const void* K, const void* V, void* O, int B, int H, int N, int d,
                           int d_v, int io_dtype, int phi, int r, const float* gamma, int normalize, int chunk,
                           const float* S0, const float* z0, float* S_out, float* z_out, void* workspace,
                           size_t workspace_bytes, void* stream) {
  if (!gamma) return LA_ERR_NULL;
  if (normalize != 0 && normalize != 1) return LA_ERR_UNSUPPORTED;
  return forward_impl(Q, K, V, O, B, H, N, d, d_v, io_dtype, phi, r, nullptr, 1, chunk, S0, z0, S_out, z_out,
                      workspace, workspace_bytes, stream, nullptr, gamma, normalize);
}

la_status la_forward_decay_timed(const void* Q, const void* K, const void* V, void* O, int B, int H, int N, int d,
                                 int d_v, int io_dtype, int phi, int r, const float* gamma, int normalize, int chunk,
                                 const float* S0, const float* z0, float* S_out, float* z_out, void* workspace,
                                 size_t workspace_bytes, void* stream, void* const* events) {
  if (!gamma) return LA_ERR_NULL;
  if (normalize != 0 && normalize != 1) return LA_ERR_UNSUPPORTED;
  return forward_impl(Q, K, V, O, B, H, N, d, d_v, io_dtype, phi, r, nullptr, 1, chunk, S0, z0, S_out, z_out,
                      workspace, workspace_bytes, stream, events, gamma, normalize);
}

la_status la_decode_step_decay(const float* S, const float* z, const void* q, const void* k, const void* v,
                               void* o, float* S_new, float* z_new, int B, int H, int d, int d_v, int io_dtype,
                               int phi, int r, const float* gamma, int normalize, void* stream) {
  if (!gamma) return LA_ERR_NULL;
  if (normalize != 0 && normalize != 1) return LA_ERR_UNSUPPORTED;
  if (phi == LA_PHI_FAVOR) return LA_ERR_UNSUPPORTED;
  return decode_impl(S, z, q, k, v, o, S_new, z_new, B, H, d, d_v, io_dtype, phi, r, nullptr, stream, gamma,
                     normalize);
}

size_t la_forward_gated_workspace_bytes(int B, int H, int N, int d, int d_v, int io_dtype, int phi, int r,
                                        int chunk) {
  Shape sh;
  if (check_forward_shape(B, H, N, d, d_v, io_dtype, phi, r, 1, chunk, &sh, 1) != LA_OK) return 0;
  return workspace_for(sh, true);
}

la_status la_forward_gated_config(int B, int H, int N, int d, int d_v, int io_dtype, int phi, int r, int chunk,
                                  int* n_span) {
  return la_forward_decay_config(B, H, N, d, d_v, io_dtype, phi, r, chunk, n_span);
}

la_status la_forward_gated(const void* Q, const void* K, const void* V, void* O, int B, int H, int N, int d,
                           int d_v, int io_dtype, int phi, int r, const float* log_a, int normalize, int chunk,
                           const float* S0, const float* z0, float* S_out, float* z_out, void* workspace,
                           size_t workspace_bytes, void* stream) {
  if (!log_a) return LA_ERR_NULL;
  if (normalize != 0 && normalize != 1) return LA_ERR_UNSUPPORTED;
  return forward_impl(Q, K, V, O, B, H, N, d, d_v, io_dtype, phi, r, nullptr, 1, chunk, S0, z0, S_out, z_out,
                      workspace, workspace_bytes, stream, nullptr, nullptr, normalize, log_a);
}

la_status la_forward_gated_timed(const void* Q, const void* K, const void* V, void* O, int B, int H, int N, int d,
                                 int d_v, int io_dtype, int phi, int r, const float* log_a, int normalize, int chunk,
                                 const float* S0, const float* z0, float* S_out, float* z_out, void* workspace,
                                 size_t workspace_bytes, void* stream, void* const* events) {
  if (!log_a) return LA_ERR_NULL;
  if (normalize != 0 && normalize != 1) return LA_ERR_UNSUPPORTED;
  return forward_impl(Q, K, V, O, B, H, N, d, d_v, io_dtype, phi, r, nullptr, 1, chunk, S0, z0, S_out, z_out,
                      workspace, workspace_bytes, stream, events, nullptr, normalize, log_a);
}

la_status la_decode_step_gated(const float* S, const float* z, const void* q, const void* k, const void* v,
                               void* o, float* S_new, float* z_new, int B, int H, int d, int d_v, int io_dtype,
                               int phi, int r, const float* log_a, int normalize, void* stream) {
  if (!log_a) return LA_ERR_NULL;
  if (normalize != 0 && normalize != 1) return LA_ERR_UNSUPPORTED;
  if (phi == LA_PHI_FAVOR) return LA_ERR_UNSUPPORTED;
  return decode_impl(S, z, q, k, v, o, S_new, z_new, B, H, d, d_v, io_dtype, phi, r, nullptr, stream, nullptr,
                     normalize, log_a);
}

size_t la_forward_gla_workspace_bytes(int B, int H, int N, int d, int d_v, int io_dtype, int phi, int r,
                                      int chunk) {
  Shape sh;
  if (check_forward_shape(B, H, N, d, d_v, io_dtype, phi, r, 1, chunk, &sh, 2) != LA_OK) return 0;
  return workspace_for(sh, false, true);
}

la_status la_forward_gla_config(int B, int H, int N, int d, int d_v, int io_dtype, int phi, int r, int chunk,
                                int* n_span, int* chunk_used) {
  Shape sh;
  const la_status st = check_forward_shape(B, H, N, d, d_v, io_dtype, phi, r, 1, chunk, &sh, 2);
  if (st != LA_OK) return st;
  if (n_span) *n_span = sh.n_span;
  if (chunk_used) *chunk_used = sh.chunk;
  return LA_OK;
}

la_status la_forward_gla(const void* Q, const void* K, const void* V, void* O, int B, int H, int N, int d,
                         int d_v, int io_dtype, int phi, int r, const float* log_a, int normalize, int chunk,
                         const float* S0, const float* z0, float* S_out, float* z_out, void* workspace,
                         size_t workspace_bytes, void* stream) {
  if (!log_a) return LA_ERR_NULL;
  if (normalize != 0 && normalize != 1) return LA_ERR_UNSUPPORTED;
  return forward_impl(Q, K, V, O, B, H, N, d, d_v, io_dtype, phi, r, nullptr, 1, chunk, S0, z0, S_out, z_out,
                      workspace, workspace_bytes, stream, nullptr, nullptr, normalize, nullptr, log_a);
}

la_status la_forward_gla_timed(const void* Q, const void* K, const void* V, void* O, int B, int H, int N, int d,
                               int d_v, int io_dtype, int phi, int r, const float* log_a, int normalize, int chunk,
                               const float* S0, const float* z0, float* S_out, float* z_out, void* workspace,
                               size_t workspace_bytes, void* stream, void* const* events) {
  if (!log_a) return LA_ERR_NULL;
  if (normalize != 0 && normalize != 1) return LA_ERR_UNSUPPORTED;
  return forward_impl(Q, K, V, O, B, H, N, d, d_v, io_dtype, phi, r, nullptr, 1, chunk, S0, z0, S_out, z_out,
                      workspace, workspace_bytes, stream, events, nullptr, normalize, nullptr, log_a);
}

la_status la_decode_step_gla(const float* S, const float* z, const void* q, const void* k, const void* v, void* o,
                             float* S_new, float* z_new, int B, int H, int d, int d_v, int io_dtype, int phi, int r,
                             const float* log_a, int normalize, void* stream) {
  if (!log_a) return LA_ERR_NULL;
  if (normalize != 0 && normalize != 1) return LA_ERR_UNSUPPORTED;
  if (phi == LA_PHI_FAVOR) return LA_ERR_UNSUPPORTED;
  return decode_impl(S, z, q, k, v, o, S_new, z_new, B, H, d, d_v, io_dtype, phi, r, nullptr, stream, nullptr,
                     normalize, nullptr, log_a);
}

namespace {

la_status backward_shape(int B, int H, int N, int d, int d_v, int io_dtype, int phi, int r, int chunk, Shape* sh) {
  if (B < 0 || H < 0 || N < 0 || d <= 0 || d_v <= 0 || r < 0 || chunk < 0) return LA_ERR_SHAPE;
  if (io_dtype != LA_F32 && io_dtype != LA_BF16) return LA_ERR_UNSUPPORTED;
  if (phi != LA_PHI_ELU1 && phi != LA_PHI_FAVOR && phi != LA_PHI_IDENTITY) return LA_ERR_UNSUPPORTED;
  const int rr = norm_r(phi, d, r);
  const int ch = norm_chunk(chunk);
  if (!la::backward_supported(io_dtype, phi, d, d_v, rr, ch)) return LA_ERR_UNSUPPORTED;
  return check_forward_shape(B, H, N, d, d_v, io_dtype, phi, r, 1, chunk, sh, 1);
}

la_status backward_impl(const void* Q, const void* K, const void* V, const void* O, const void* dO, void* dQ,
                        void* dK, void* dV, int B, int H, int N, int d, int d_v, int io_dtype, int phi, int r,
                        int chunk, void* workspace, size_t workspace_bytes, void* stream, void* const* events) {
  Shape sh;
  const la_status st = backward_shape(B, H, N, d, d_v, io_dtype, phi, r, chunk, &sh);
  if (st != LA_OK) return st;
  const bool have_tokens = sh.BH > 0 && N > 0;
  if (have_tokens && (!Q || !K || !V || !O || !dO || !dQ || !dK || !dV)) return LA_ERR_NULL;
  const void* ptrs[] = {Q, K, V, O, dO, dQ, dK, dV, workspace};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return LA_ERR_ALIGN;
  const size_t need = la::backward_workspace_bytes(sh.BH, sh.n_span, N, sh.r, sh.dv);
  if (have_tokens && (!workspace || workspace_bytes < need)) return LA_ERR_WORKSPACE;
  if (!have_tokens) return LA_OK;
  la::BackwardArgs a;
  a.Q = Q; a.K = K; a.V = V; a.O = O; a.dO = dO; a.dQ = dQ; a.dK = dK; a.dV = dV;
  a.B = B; a.H = H; a.N = N; a.d = d; a.dv = d_v; a.r = sh.r;
  a.io = io_dtype; a.phi = phi; a.chunk = sh.chunk; a.n_span = sh.n_span;
  a.workspace = workspace; a.stream = stream; a.events = events;
  return hip_status(la::backward_launch(a));
}

}  // namespace

size_t la_backward_workspace_bytes(int B, int H, int N, int d, int d_v, int io_dtype, int phi, int r, int chunk) {
  Shape sh;
  if (backward_shape(B, H, N, d, d_v, io_dtype, phi, r, chunk, &sh) != LA_OK) return 0;
  return la::backward_workspace_bytes(sh.BH, sh.n_span, N, sh.r, sh.dv);
}

la_status la_backward_config(int B, int H, int N, int d, int d_v, int io_dtype, int phi, int r, int chunk,
                             int* n_span) {
  Shape sh;
  const la_status st = backward_shape(B, H, N, d, d_v, io_dtype, phi, r, chunk, &sh);
  if (st != LA_OK) return st;
  if (n_span) *n_span = sh.n_span;
  return LA_OK;
}

la_status la_backward(const void* Q, const void* K, const void* V, const void* O, const void* dO, void* dQ, void* dK,
                      void* dV, int B, int H, int N, int d, int d_v, int io_dtype, int phi, int r, int chunk,
                      void* workspace, size_t workspace_bytes, void* stream) {
  return backward_impl(Q, K, V, O, dO, dQ, dK, dV, B, H, N, d, d_v, io_dtype, phi, r, chunk, workspace,
                       workspace_bytes, stream, nullptr);
}

la_status la_backward_timed(const void* Q, const void* K, const void* V, const void* O, const void* dO, void* dQ,
                            void* dK, void* dV, int B, int H, int N, int d, int d_v, int io_dtype, int phi, int r,
                            int chunk, void* workspace, size_t workspace_bytes, void* stream, void* const* events) {
  return backward_impl(Q, K, V, O, dO, dQ, dK, dV, B, H, N, d, d_v, io_dtype, phi, r, chunk, workspace,
                       workspace_bytes, stream, events);
}

la_status la_feature_map(const void* X, float* Y, long long rows, int d, int io_dtype, int phi, int r,
                         const float* omega, void* stream) {
  phi = canon_phi(phi);
  if (rows < 0 || d <= 0 || r < 0 || d > kMaxDim) return LA_ERR_SHAPE;
  if (io_dtype != LA_F32 && io_dtype != LA_BF16) return LA_ERR_UNSUPPORTED;
  if (phi != LA_PHI_ELU1 && phi != LA_PHI_FAVOR && phi != LA_PHI_IDENTITY) return LA_ERR_UNSUPPORTED;
  const int rr = norm_r(phi, d, r);
  if (!la::feature_supported(io_dtype, phi, d, rr)) return LA_ERR_UNSUPPORTED;
  if (rows > (1LL << 40) / (rr > d ? rr : d)) return LA_ERR_SHAPE;
  if (rows > 0 && (!X || !Y)) return LA_ERR_NULL;
  if (phi == LA_PHI_FAVOR && !omega) return LA_ERR_NULL;
  const void* ptrs[] = {X, Y, omega};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return LA_ERR_ALIGN;
  if (rows == 0) return LA_OK;
  la::FeatureArgs a;
  a.X = X; a.Y = Y; a.rows = rows; a.d = d; a.r = rr; a.io = io_dtype; a.phi = phi; a.omega = omega;
  a.stream = stream;
  return hip_status(la::feature_launch(a));
}

const char* la_status_string(int status) {
  switch (status) {
    case LA_OK: return "ok";
    case LA_ERR_NULL: return "a required pointer is NULL";
    case LA_ERR_SHAPE: return "invalid size or shape";
    case LA_ERR_UNSUPPORTED: return "unsupported dtype, feature map, dimension or chunk";
    case LA_ERR_ALIGN: return "pointer not 16-byte aligned";
    case LA_ERR_WORKSPACE: return "workspace missing or too small";
    case LA_ERR_HIP: return "HIP runtime error";
    case LA_ERR_SCRATCH: return "the call needs more device memory than the fixed scratch of la_forward_noalloc holds";
    default: return "unknown status";
  }
}

int la_version(void) { return 100; }

const char* la_hip_error_string(void) { return t_last_hip_error; }

la_status la_event_create(void** event) {
  if (!event) return LA_ERR_NULL;
  hipEvent_t e;
  // timing only: no system-scope fence (cache write-back and invalidate)
  // when the event is recorded, so that recording it does not slow the
  // kernels that follow; elapsed times stay valid after a device sync
  if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return hip_status(hipErrorUnknown);
  *event = e;
  return LA_OK;
}

la_status la_event_destroy(void* event) {
  if (!event) return LA_ERR_NULL;
  return hipEventDestroy(static_cast<hipEvent_t>(event)) == hipSuccess ? LA_OK : LA_ERR_HIP;
}

la_status la_event_elapsed_ms(void* start, void* end, float* ms) {
  if (!start || !end || !ms) return LA_ERR_NULL;
  return hipEventElapsedTime(ms, static_cast<hipEvent_t>(start), static_cast<hipEvent_t>(end)) == hipSuccess
             ? LA_OK
             : LA_ERR_HIP;
}

}  // extern "C"
