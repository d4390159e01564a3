// gdn_launch.h -- internal launchers behind the C ABI (arguments already validated).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

// One decode step over an fp32 state pool, in place (recurrent.hip).
hipError_t launch_decode(const void* q, const void* k, const void* v, bool io_bf16,
                         const float* g, const float* beta, float* pool, const int32_t* slots,
                         int num_seqs, int h_qk, int h_v, float scale, void* o,
                         hipStream_t stream);

// The decode-time front end and the decode step in one launch (recurrent.hip): one
// workgroup per (sequence, QK head); h_v / h_qk must be 1 or 2.
hipError_t launch_decode_with_conv(const void* mixed_qkv, const float* conv_weight, int conv_kernel,
                                  void* conv_window, const int32_t* window_slots, float q_scale,
                                  const float* g, const float* beta, float* pool,
                                  const int32_t* slots, int num_seqs, int h_qk, int h_v,
                                  float scale, void* o, hipStream_t stream);

// Several decode steps per sequence, the state read and written once, per-token states
// optionally written out (recurrent.hip).
hipError_t launch_verify(const void* q, const void* k, const void* v, bool io_bf16, const float* g,
                         const float* beta, float* pool, const int32_t* slots, float* snapshots,
                         int num_seqs, int num_tokens, int h_qk, int h_v, float scale, void* o,
                         hipStream_t stream);

// The per-channel form (one decay per value row, the correction from the state before the
// decay): token-sequential prefill over a packed batch, and one decode step over a pool
// (recurrent.hip).
hipError_t launch_channel_prefill(const void* q, const void* k, const void* v, bool io_bf16,
                                  const float* g, const float* beta, const int32_t* cu_seqlens,
                                  int num_seqs, int h_qk, int h_v, float scale, const float* s0,
                                  float* s_final, void* o, hipStream_t stream);
hipError_t launch_channel_decode(const void* q, const void* k, const void* v, bool io_bf16,
                                 const float* g, const float* beta, float* pool, const int32_t* slots,
                                 int num_seqs, int h_qk, int h_v, float scale, void* o,
                                 hipStream_t stream);

// Output epilogue: per-head RMS norm with the zero-centred scale, then the output gate, over
// n_vec vectors of 128 channels (epilogue.hip).
hipError_t launch_gated_rmsnorm(const void* o, const void* z, bool io_bf16, const float* weight,
                                long long n_vec, float eps, bool silu, void* out,
                                hipStream_t stream);

// Token-sequential prefill with the state on chip (recurrent.hip); used for fp32 I/O.
hipError_t launch_recurrent_prefill(const void* q, const void* k, const void* v, bool io_bf16,
                                    const float* g, const float* beta, const int32_t* cu_seqlens,
                                    int num_seqs, int h_qk, int h_v, float scale,
                                    const float* s0, float* s_final, void* o, hipStream_t stream);

// Chunked bf16 prefill on the matrix cores (chunk_prefill.hip): a chunk table, a
// chunk-parallel prep launch and the sequential state pass, all on `stream`.
size_t chunk_prefill_workspace_bytes(int total_tokens, int num_seqs, int h_qk, int h_v);
hipError_t launch_chunk_prefill(const void* q, const void* k, const void* v, const float* g,
                                const float* beta, const int32_t* cu_seqlens, int num_seqs,
                                int total_tokens, int h_qk, int h_v, float scale,
                                const float* s0, float* s_final, void* o, void* workspace,
                                hipStream_t stream);

// The chunked prefill with the front end in front of it (chunk_prefill.hip): from the mixed
// q | k | v input and the conv taps. The front end runs as its own pass into the workspace
// (whose size the query includes), then the prefill.
size_t chunk_prefill_conv_workspace_bytes(int total_tokens, int num_seqs, int h_qk, int h_v);
hipError_t launch_chunk_prefill_conv(const void* mixed, const float* conv_weight, int conv_kernel,
                                     float q_scale, const float* g, const float* beta,
                                     const int32_t* cu_seqlens, int num_seqs, int total_tokens,
                                     int h_qk, int h_v, float scale, const float* s0, float* s_final,
                                     void* o, void* workspace, hipStream_t stream);

// The prefill workspace of gdn_chunk_prefill_noalloc: the device address of this GPU's
// copy of a static device array of kNoAllocScratchBytes, looked up once per device
// (chunk_prefill.hip).
constexpr size_t kNoAllocScratchBytes = (size_t)64 << 20;
hipError_t noalloc_scratch(void** ptr);

// Causal depthwise conv + SiLU + q/k L2 norm + q scale (conv_prep.hip).
hipError_t launch_conv_prep(const void* mixed, const float* w, int K, const int32_t* cu,
                            int num_seqs, int total_tokens, int h_qk, int h_v, float q_scale,
                            void* q, void* k, void* v, hipStream_t stream);

// Decode-side front end: one token per sequence against a window pool of the last K - 1
// inputs, updated in place (conv_prep.hip).
hipError_t launch_conv_decode(const void* mixed, const float* w, int K, void* window,
                              const int32_t* slots, int num_seqs, int h_qk, int h_v, float q_scale,
                              void* q, void* k, void* v, hipStream_t stream);

// The window a prefill over packed sequences leaves for decode (conv_prep.hip).
hipError_t launch_conv_window(const void* mixed, int K, const int32_t* cu, int num_seqs, int h_qk,
                              int h_v, void* window, const int32_t* slots, hipStream_t stream);

}  // namespace gdn
