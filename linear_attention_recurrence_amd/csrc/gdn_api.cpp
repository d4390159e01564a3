// gdn_api.cpp -- the C ABI of libgdn.so: host-side validation and dispatch.
//
// Every entry point validates its arguments before touching the HIP runtime, so a rejected
// call launches nothing and writes nothing. Launch errors are reported as GDN_ERR_HIP.
#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <vector>
#include "gdn.h"

#include <hip/hip_runtime.h>

#include "gdn_launch.h"

namespace {

constexpr int32_t kHead = 128;

bool heads_ok(int32_t h_qk, int32_t h_v) { return h_qk > 0 && h_v > 0 && h_v % h_qk == 0; }

gdn_status check_common(int32_t h_qk, int32_t h_v, int32_t d_k, int32_t d_v) {
  if (h_qk <= 0 || h_v <= 0 || d_k <= 0 || d_v <= 0) return GDN_ERR_SHAPE;
  if (!heads_ok(h_qk, h_v)) return GDN_ERR_SHAPE;
  if (d_k != kHead || d_v != kHead) return GDN_ERR_UNSUPPORTED;
  return GDN_OK;
}

gdn_status from_hip(hipError_t e) { return e == hipSuccess ? GDN_OK : GDN_ERR_HIP; }

// Opt-in checks of the device-side contracts, for debugging a caller: with the environment
// variable GDN_CHECK_CONTRACTS set to 1, the index arrays are copied to the host on the
// call's stream and waited for (so such a call synchronises its stream), and a violation
// returns GDN_ERR_SHAPE before anything is launched. Off, nothing is read.
bool contract_checks() {
  const char* e = std::getenv("GDN_CHECK_CONTRACTS");
  return e && e[0] == '1' && e[1] == '\0';
}

gdn_status fetch_ints(const int32_t* src, int32_t n, void* stream, std::vector<int32_t>& out) {
  out.resize((size_t)n);
  if (n == 0) return GDN_OK;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (hipMemcpyAsync(out.data(), src, sizeof(int32_t) * (size_t)n, hipMemcpyDeviceToHost, st) != hipSuccess)
    return GDN_ERR_HIP;
  return hipStreamSynchronize(st) == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

// cu_seqlens[0] = 0, nondecreasing, cu_seqlens[num_seqs] = total_tokens.
gdn_status check_seqlens(const int32_t* cu, int32_t num_seqs, int32_t total_tokens, void* stream) {
  if (!contract_checks()) return GDN_OK;
  std::vector<int32_t> h;
  const gdn_status st = fetch_ints(cu, num_seqs + 1, stream, h);
  if (st != GDN_OK) return st;
  if (h[0] != 0 || h[(size_t)num_seqs] != total_tokens) return GDN_ERR_SHAPE;
  for (int32_t i = 0; i < num_seqs; ++i)
    if (h[(size_t)i + 1] < h[(size_t)i]) return GDN_ERR_SHAPE;
  return GDN_OK;
}

// Slot indices non-negative and distinct (the pool size is not passed, so the upper bound
// stays the caller's).
gdn_status check_slots(const int32_t* slots, int32_t num_seqs, void* stream) {
  if (!slots || !contract_checks()) return GDN_OK;
  std::vector<int32_t> h;
  const gdn_status st = fetch_ints(slots, num_seqs, stream, h);
  if (st != GDN_OK) return st;
  std::sort(h.begin(), h.end());
  for (size_t i = 0; i < h.size(); ++i)
    if (h[i] < 0 || (i > 0 && h[i] == h[i - 1])) return GDN_ERR_SHAPE;
  return GDN_OK;
}

// Every log-decay finite and <= 0 (alpha = exp(g) in (0, 1]).
gdn_status check_log_decay(const float* g, size_t count, void* stream) {
  if (!g || count == 0 || !contract_checks()) return GDN_OK;
  std::vector<float> h(count);
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (hipMemcpyAsync(h.data(), g, sizeof(float) * count, hipMemcpyDeviceToHost, st) != hipSuccess)
    return GDN_ERR_HIP;
  if (hipStreamSynchronize(st) != hipSuccess) return GDN_ERR_HIP;
  for (const float x : h)
    if (!(x <= 0.f) || !std::isfinite(x)) return GDN_ERR_SHAPE;
  return GDN_OK;
}

#define GDN_TRY(expr)                      \
  do {                                     \
    const gdn_status gdn_st_ = (expr);     \
    if (gdn_st_ != GDN_OK) return gdn_st_; \
  } while (0)

// The integer a caller passed for an enum argument. A C caller may pass any int, and in C++
// loading an enum object that holds a value outside the enum's range is undefined, so the
// bits are copied out rather than loaded as the enum.
template <typename E>
int enum_code(const E* e) {
  static_assert(sizeof(E) == sizeof(int), "enum arguments are int-sized");
  int v;
  std::memcpy(&v, e, sizeof v);
  return v;
}

}  // namespace

extern "C" {

const char* gdn_status_string(gdn_status s) {
  switch (enum_code(&s)) {
    case GDN_OK: return "GDN_OK";
    case GDN_ERR_NULL: return "GDN_ERR_NULL: a required pointer is NULL";
    case GDN_ERR_SHAPE: return "GDN_ERR_SHAPE: a size is negative or inconsistent";
    case GDN_ERR_UNSUPPORTED: return "GDN_ERR_UNSUPPORTED: valid but not implemented";
    case GDN_ERR_WORKSPACE: return "GDN_ERR_WORKSPACE: workspace missing or too small";
    case GDN_ERR_HIP: return "GDN_ERR_HIP: the HIP runtime reported an error";
  }
  return "unknown gdn_status";
}

size_t gdn_chunk_prefill_workspace_bytes(int32_t total_tokens, int32_t num_seqs, int32_t h_qk,
                                         int32_t h_v, int32_t d_k, int32_t d_v) {
  if (total_tokens < 0 || num_seqs <= 0 || check_common(h_qk, h_v, d_k, d_v) != GDN_OK) return 0;
  return gdn::chunk_prefill_workspace_bytes(total_tokens, num_seqs, h_qk, h_v);
}

gdn_status gdn_chunk_prefill(const void* q, const void* k, const void* v, gdn_dtype io_dtype,
                             const float* g, const float* beta,
                             const int32_t* cu_seqlens, int32_t num_seqs, int32_t total_tokens,
                             int32_t h_qk, int32_t h_v, int32_t d_k, int32_t d_v, float scale,
                             const float* initial_state, float* final_state,
                             void* o, void* workspace, size_t workspace_bytes, void* stream) {
  if (num_seqs < 0 || total_tokens < 0) return GDN_ERR_SHAPE;
  const gdn_status st = check_common(h_qk, h_v, d_k, d_v);
  if (st != GDN_OK) return st;
  if (enum_code(&io_dtype) != GDN_BF16 && enum_code(&io_dtype) != GDN_F32) return GDN_ERR_UNSUPPORTED;
  if (num_seqs == 0) return total_tokens == 0 ? GDN_OK : GDN_ERR_SHAPE;
  if (!cu_seqlens) return GDN_ERR_NULL;
  if (total_tokens > 0 && (!q || !k || !v || !g || !beta || !o)) return GDN_ERR_NULL;
  if (!final_state && total_tokens == 0) return GDN_OK;   // nothing observable to do
  GDN_TRY(check_seqlens(cu_seqlens, num_seqs, total_tokens, stream));
  GDN_TRY(check_log_decay(g, (size_t)total_tokens * h_v, stream));
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (enum_code(&io_dtype) == GDN_F32)
    return from_hip(gdn::launch_recurrent_prefill(q, k, v, false, g, beta, cu_seqlens, num_seqs,
                                                  h_qk, h_v, scale, initial_state, final_state,
                                                  o, s));
  const size_t need = gdn_chunk_prefill_workspace_bytes(total_tokens, num_seqs, h_qk, h_v, d_k, d_v);
  if (need > 0 && (!workspace || workspace_bytes < need)) return GDN_ERR_WORKSPACE;
  return from_hip(gdn::launch_chunk_prefill(q, k, v, g, beta, cu_seqlens, num_seqs, total_tokens,
                                            h_qk, h_v, scale, initial_state, final_state, o,
                                            workspace, s));
}

size_t gdn_chunk_prefill_conv_workspace_bytes(int32_t total_tokens, int32_t num_seqs, int32_t h_qk,
                                              int32_t h_v, int32_t d_k, int32_t d_v) {
  if (total_tokens < 0 || num_seqs <= 0 || check_common(h_qk, h_v, d_k, d_v) != GDN_OK) return 0;
  return gdn::chunk_prefill_conv_workspace_bytes(total_tokens, num_seqs, h_qk, h_v);
}

gdn_status gdn_chunk_prefill_conv(const void* mixed_qkv, const float* conv_weight, int32_t conv_kernel,
                                  float q_scale, const float* g, const float* beta,
                                  const int32_t* cu_seqlens, int32_t num_seqs, int32_t total_tokens,
                                  int32_t h_qk, int32_t h_v, int32_t d_k, int32_t d_v, float scale,
                                  const float* initial_state, float* final_state, void* o,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  if (num_seqs < 0 || total_tokens < 0) return GDN_ERR_SHAPE;
  const gdn_status st = check_common(h_qk, h_v, d_k, d_v);
  if (st != GDN_OK) return st;
  if (conv_kernel < 1) return GDN_ERR_SHAPE;
  if (conv_kernel > 4) return GDN_ERR_UNSUPPORTED;
  if (num_seqs == 0) return total_tokens == 0 ? GDN_OK : GDN_ERR_SHAPE;
  if (!cu_seqlens) return GDN_ERR_NULL;
  if (total_tokens > 0 && (!mixed_qkv || !conv_weight || !g || !beta || !o)) return GDN_ERR_NULL;
  if (!final_state && total_tokens == 0) return GDN_OK;   // nothing observable to do
  const size_t need = gdn_chunk_prefill_conv_workspace_bytes(total_tokens, num_seqs, h_qk, h_v, d_k, d_v);
  if (need > 0 && (!workspace || workspace_bytes < need)) return GDN_ERR_WORKSPACE;
  GDN_TRY(check_seqlens(cu_seqlens, num_seqs, total_tokens, stream));
  GDN_TRY(check_log_decay(g, (size_t)total_tokens * h_v, stream));
  return from_hip(gdn::launch_chunk_prefill_conv(mixed_qkv, conv_weight, conv_kernel, q_scale, g, beta,
                                                 cu_seqlens, num_seqs, total_tokens, h_qk, h_v, scale,
                                                 initial_state, final_state, o, workspace,
                                                 static_cast<hipStream_t>(stream)));
}

gdn_status gdn_chunk_prefill_noalloc(const void* q, const void* k, const void* v, gdn_dtype io_dtype,
                                     const float* g, const float* beta,
                                     const int32_t* cu_seqlens, int32_t num_seqs,
                                     int32_t total_tokens, int32_t h_qk, int32_t h_v, int32_t d_k,
                                     int32_t d_v, float scale, const float* initial_state,
                                     float* final_state, void* o, void* stream) {
  static_assert(GDN_NOALLOC_SCRATCH_BYTES == gdn::kNoAllocScratchBytes, "header and library agree");
  if (num_seqs < 0 || total_tokens < 0) return GDN_ERR_SHAPE;
  const gdn_status st = check_common(h_qk, h_v, d_k, d_v);
  if (st != GDN_OK) return st;
  if (enum_code(&io_dtype) != GDN_BF16 && enum_code(&io_dtype) != GDN_F32) return GDN_ERR_UNSUPPORTED;
  if (num_seqs == 0) return total_tokens == 0 ? GDN_OK : GDN_ERR_SHAPE;
  if (!cu_seqlens) return GDN_ERR_NULL;
  if (total_tokens > 0 && (!q || !k || !v || !g || !beta || !o)) return GDN_ERR_NULL;
  if (!final_state && total_tokens == 0) return GDN_OK;   // nothing observable to do
  if (enum_code(&io_dtype) == GDN_BF16 &&
      gdn_chunk_prefill_workspace_bytes(total_tokens, num_seqs, h_qk, h_v, d_k, d_v) > GDN_NOALLOC_SCRATCH_BYTES)
    return GDN_ERR_WORKSPACE;
  GDN_TRY(check_seqlens(cu_seqlens, num_seqs, total_tokens, stream));
  GDN_TRY(check_log_decay(g, (size_t)total_tokens * h_v, stream));
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (enum_code(&io_dtype) == GDN_F32)
    return from_hip(gdn::launch_recurrent_prefill(q, k, v, false, g, beta, cu_seqlens, num_seqs,
                                                  h_qk, h_v, scale, initial_state, final_state,
                                                  o, s));
  void* ws = nullptr;
  if (gdn::noalloc_scratch(&ws) != hipSuccess) return GDN_ERR_HIP;
  return from_hip(gdn::launch_chunk_prefill(q, k, v, g, beta, cu_seqlens, num_seqs, total_tokens,
                                            h_qk, h_v, scale, initial_state, final_state, o, ws, s));
}

gdn_status gdn_decode_step(const void* q, const void* k, const void* v, gdn_dtype io_dtype,
                           const float* g, const float* beta,
                           float* state_pool, const int32_t* state_slots,
                           int32_t num_seqs, int32_t h_qk, int32_t h_v, int32_t d_k, int32_t d_v,
                           float scale, void* o, void* stream) {
  if (num_seqs < 0) return GDN_ERR_SHAPE;
  const gdn_status st = check_common(h_qk, h_v, d_k, d_v);
  if (st != GDN_OK) return st;
  if (enum_code(&io_dtype) != GDN_BF16 && enum_code(&io_dtype) != GDN_F32) return GDN_ERR_UNSUPPORTED;
  if (num_seqs == 0) return GDN_OK;
  if (!q || !k || !v || !g || !beta || !state_pool || !o) return GDN_ERR_NULL;
  GDN_TRY(check_slots(state_slots, num_seqs, stream));
  GDN_TRY(check_log_decay(g, (size_t)num_seqs * h_v, stream));
  return from_hip(gdn::launch_decode(q, k, v, enum_code(&io_dtype) == GDN_BF16, g, beta, state_pool,
                                     state_slots, num_seqs, h_qk, h_v, scale, o,
                                     static_cast<hipStream_t>(stream)));
}

gdn_status gdn_verify_step(const void* q, const void* k, const void* v, gdn_dtype io_dtype,
                           const float* g, const float* beta,
                           float* state_pool, const int32_t* state_slots, float* snapshots,
                           int32_t num_seqs, int32_t num_tokens, int32_t h_qk, int32_t h_v,
                           int32_t d_k, int32_t d_v, float scale, void* o, void* stream) {
  if (num_seqs < 0 || num_tokens < 0) return GDN_ERR_SHAPE;
  const gdn_status st = check_common(h_qk, h_v, d_k, d_v);
  if (st != GDN_OK) return st;
  if (enum_code(&io_dtype) != GDN_BF16 && enum_code(&io_dtype) != GDN_F32) return GDN_ERR_UNSUPPORTED;
  if (num_seqs == 0 || num_tokens == 0) return GDN_OK;
  if (!q || !k || !v || !g || !beta || !state_pool || !o) return GDN_ERR_NULL;
  GDN_TRY(check_slots(state_slots, num_seqs, stream));
  GDN_TRY(check_log_decay(g, (size_t)num_seqs * num_tokens * h_v, stream));
  return from_hip(gdn::launch_verify(q, k, v, enum_code(&io_dtype) == GDN_BF16, g, beta, state_pool,
                                     state_slots, snapshots, num_seqs, num_tokens, h_qk, h_v,
                                     scale, o, static_cast<hipStream_t>(stream)));
}

gdn_status gdn_channel_decay_prefill(const void* q, const void* k, const void* v, gdn_dtype io_dtype,
                                     const float* g, const float* beta,
                                     const int32_t* cu_seqlens, int32_t num_seqs, int32_t total_tokens,
                                     int32_t h_qk, int32_t h_v, int32_t d_k, int32_t d_v, float scale,
                                     const float* initial_state, float* final_state, void* o,
                                     void* stream) {
  if (num_seqs < 0 || total_tokens < 0) return GDN_ERR_SHAPE;
  const gdn_status st = check_common(h_qk, h_v, d_k, d_v);
  if (st != GDN_OK) return st;
  if (enum_code(&io_dtype) != GDN_BF16 && enum_code(&io_dtype) != GDN_F32) return GDN_ERR_UNSUPPORTED;
  if (num_seqs == 0) return total_tokens == 0 ? GDN_OK : GDN_ERR_SHAPE;
  if (!cu_seqlens) return GDN_ERR_NULL;
  if (total_tokens > 0 && (!q || !k || !v || !g || !beta || !o)) return GDN_ERR_NULL;
  if (!final_state && total_tokens == 0) return GDN_OK;   // nothing observable to do
  GDN_TRY(check_seqlens(cu_seqlens, num_seqs, total_tokens, stream));
  GDN_TRY(check_log_decay(g, (size_t)total_tokens * h_v * d_v, stream));
  return from_hip(gdn::launch_channel_prefill(q, k, v, enum_code(&io_dtype) == GDN_BF16, g, beta, cu_seqlens,
                                              num_seqs, h_qk, h_v, scale, initial_state,
                                              final_state, o, static_cast<hipStream_t>(stream)));
}

gdn_status gdn_channel_decay_decode_step(const void* q, const void* k, const void* v, gdn_dtype io_dtype,
                                         const float* g, const float* beta,
                                         float* state_pool, const int32_t* state_slots,
                                         int32_t num_seqs, int32_t h_qk, int32_t h_v, int32_t d_k,
                                         int32_t d_v, float scale, void* o, void* stream) {
  if (num_seqs < 0) return GDN_ERR_SHAPE;
  const gdn_status st = check_common(h_qk, h_v, d_k, d_v);
  if (st != GDN_OK) return st;
  if (enum_code(&io_dtype) != GDN_BF16 && enum_code(&io_dtype) != GDN_F32) return GDN_ERR_UNSUPPORTED;
  if (num_seqs == 0) return GDN_OK;
  if (!q || !k || !v || !g || !beta || !state_pool || !o) return GDN_ERR_NULL;
  GDN_TRY(check_slots(state_slots, num_seqs, stream));
  GDN_TRY(check_log_decay(g, (size_t)num_seqs * h_v * d_v, stream));
  return from_hip(gdn::launch_channel_decode(q, k, v, enum_code(&io_dtype) == GDN_BF16, g, beta, state_pool,
                                             state_slots, num_seqs, h_qk, h_v, scale, o,
                                             static_cast<hipStream_t>(stream)));
}

gdn_status gdn_conv_prep(const void* mixed_qkv, const float* conv_weight, int32_t conv_kernel,
                         const int32_t* cu_seqlens, int32_t num_seqs, int32_t total_tokens,
                         int32_t h_qk, int32_t h_v, int32_t d_k, int32_t d_v, float q_scale,
                         void* q, void* k, void* v, void* stream) {
  if (num_seqs < 0 || total_tokens < 0) return GDN_ERR_SHAPE;
  const gdn_status st = check_common(h_qk, h_v, d_k, d_v);
  if (st != GDN_OK) return st;
  if (conv_kernel < 1) return GDN_ERR_SHAPE;
  if (conv_kernel > 4) return GDN_ERR_UNSUPPORTED;
  if (num_seqs == 0) return total_tokens == 0 ? GDN_OK : GDN_ERR_SHAPE;
  if (total_tokens == 0) return GDN_OK;
  if (!mixed_qkv || !conv_weight || !cu_seqlens || !q || !k || !v) return GDN_ERR_NULL;
  GDN_TRY(check_seqlens(cu_seqlens, num_seqs, total_tokens, stream));
  return from_hip(gdn::launch_conv_prep(mixed_qkv, conv_weight, conv_kernel, cu_seqlens, num_seqs,
                                        total_tokens, h_qk, h_v, q_scale, q, k, v,
                                        static_cast<hipStream_t>(stream)));
}

gdn_status gdn_conv_decode_step(const void* mixed_qkv, const float* conv_weight, int32_t conv_kernel,
                                void* conv_window, const int32_t* window_slots, int32_t num_seqs,
                                int32_t h_qk, int32_t h_v, int32_t d_k, int32_t d_v, float q_scale,
                                void* q, void* k, void* v, void* stream) {
  if (num_seqs < 0) return GDN_ERR_SHAPE;
  const gdn_status st = check_common(h_qk, h_v, d_k, d_v);
  if (st != GDN_OK) return st;
  if (conv_kernel < 1) return GDN_ERR_SHAPE;
  if (conv_kernel > 4) return GDN_ERR_UNSUPPORTED;
  if (num_seqs == 0) return GDN_OK;
  if (!mixed_qkv || !conv_weight || !q || !k || !v) return GDN_ERR_NULL;
  if (conv_kernel > 1 && !conv_window) return GDN_ERR_NULL;
  GDN_TRY(check_slots(window_slots, num_seqs, stream));
  return from_hip(gdn::launch_conv_decode(mixed_qkv, conv_weight, conv_kernel, conv_window,
                                          window_slots, num_seqs, h_qk, h_v, q_scale, q, k, v,
                                          static_cast<hipStream_t>(stream)));
}

gdn_status gdn_decode_step_with_conv(const void* mixed_qkv, const float* conv_weight,
                                     int32_t conv_kernel, void* conv_window,
                                     const int32_t* window_slots, float q_scale, const float* g,
                                     const float* beta, float* state_pool,
                                     const int32_t* state_slots, int32_t num_seqs, int32_t h_qk,
                                     int32_t h_v, int32_t d_k, int32_t d_v, float scale, void* o,
                                     void* stream) {
  if (num_seqs < 0) return GDN_ERR_SHAPE;
  const gdn_status st = check_common(h_qk, h_v, d_k, d_v);
  if (st != GDN_OK) return st;
  if (conv_kernel < 1) return GDN_ERR_SHAPE;
  if (conv_kernel > 4) return GDN_ERR_UNSUPPORTED;
  if (h_v != h_qk && h_v != 2 * h_qk) return GDN_ERR_UNSUPPORTED;
  if (num_seqs == 0) return GDN_OK;
  if (!mixed_qkv || !conv_weight || !g || !beta || !state_pool || !o) return GDN_ERR_NULL;
  if (conv_kernel > 1 && !conv_window) return GDN_ERR_NULL;
  GDN_TRY(check_slots(window_slots, num_seqs, stream));
  GDN_TRY(check_slots(state_slots, num_seqs, stream));
  GDN_TRY(check_log_decay(g, (size_t)num_seqs * h_v, stream));
  return from_hip(gdn::launch_decode_with_conv(mixed_qkv, conv_weight, conv_kernel, conv_window,
                                               window_slots, q_scale, g, beta, state_pool,
                                               state_slots, num_seqs, h_qk, h_v, scale, o,
                                               static_cast<hipStream_t>(stream)));
}

gdn_status gdn_conv_window_from_prefill(const void* mixed_qkv, int32_t conv_kernel,
                                        const int32_t* cu_seqlens, int32_t num_seqs,
                                        int32_t total_tokens, int32_t h_qk, int32_t h_v,
                                        int32_t d_k, int32_t d_v, void* conv_window,
                                        const int32_t* window_slots, void* stream) {
  if (num_seqs < 0 || total_tokens < 0) return GDN_ERR_SHAPE;
  const gdn_status st = check_common(h_qk, h_v, d_k, d_v);
  if (st != GDN_OK) return st;
  if (conv_kernel < 1) return GDN_ERR_SHAPE;
  if (conv_kernel > 4) return GDN_ERR_UNSUPPORTED;
  if (num_seqs == 0) return total_tokens == 0 ? GDN_OK : GDN_ERR_SHAPE;
  if (conv_kernel == 1) return GDN_OK;   // no window
  if (!cu_seqlens || !conv_window || (total_tokens > 0 && !mixed_qkv)) return GDN_ERR_NULL;
  GDN_TRY(check_seqlens(cu_seqlens, num_seqs, total_tokens, stream));
  GDN_TRY(check_slots(window_slots, num_seqs, stream));
  return from_hip(gdn::launch_conv_window(mixed_qkv, conv_kernel, cu_seqlens, num_seqs, h_qk, h_v,
                                          conv_window, window_slots,
                                          static_cast<hipStream_t>(stream)));
}

gdn_status gdn_gated_rmsnorm(const void* o, const void* z, gdn_dtype io_dtype, const float* weight,
                             int32_t rows, int32_t h_v, int32_t d_v, float eps, gdn_gate gate,
                             void* out, void* stream) {
  if (rows < 0 || h_v < 1 || d_v < 1) return GDN_ERR_SHAPE;
  if (!(eps >= 0.f) || !std::isfinite(eps)) return GDN_ERR_SHAPE;
  if (d_v != 128) return GDN_ERR_UNSUPPORTED;
  if (enum_code(&io_dtype) != GDN_BF16 && enum_code(&io_dtype) != GDN_F32) return GDN_ERR_UNSUPPORTED;
  if (enum_code(&gate) != GDN_GATE_SIGMOID && enum_code(&gate) != GDN_GATE_SILU) return GDN_ERR_UNSUPPORTED;
  const long long n_vec = (long long)rows * h_v;
  if (n_vec > (1LL << 34)) return GDN_ERR_UNSUPPORTED;
  if (rows == 0) return GDN_OK;
  if (!o || !z || !weight || !out) return GDN_ERR_NULL;
  return from_hip(gdn::launch_gated_rmsnorm(o, z, enum_code(&io_dtype) == GDN_BF16, weight, n_vec, eps,
                                            enum_code(&gate) == GDN_GATE_SILU,
                                            out, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
