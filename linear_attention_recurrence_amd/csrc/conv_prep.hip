// conv_prep.hip -- front end of the Gated DeltaNet mixer on gfx950.
//
// Per token t and channel c of the projected q|k|v activations (section
// "01 . GatedDeltaNet(config)" of page "Qwen3-Next 80B-A3B -- The Evolving Transformer":
// a short 1-D convolution gives local context; keys are L2-normalised):
//
//   y[t,c] = sum_i w[c,i] * x[t-(K-1)+i, c]     (x = 0 before the sequence start)
//   z      = y * sigmoid(y)                      (SiLU)
//   q head = z / max(||z||_2, 1e-12) * q_scale,  k head = z / max(||z||_2, 1e-12),  v = z
//
// HBM-bound (16 KB read + 16 KB written per token at the model's 8192 channels). Each
// thread owns 8 adjacent channels (one 16-byte load/store) and walks R = 128 consecutive
// tokens, keeping the last K-1 inputs of its channels in registers, so every input row is
// read once (plus K-1 halo rows per block, 2 %). The rows are loaded in groups of 4 tokens,
// the next group in flight while the current one is computed, so each thread keeps up to 8
// loads outstanding; the input is read once, so its loads are non-temporal. Four-token groups
// and a bound of 128 registers fit four waves per SIMD (eight-token groups need 163, three
// waves): 1.99 -> 1.90 ms on 64 packed sequences. Sixteen threads
// cover one 128-channel head, so the head norm is a 16-lane reduction. A block covers 2048
// channels x R tokens. (R = 32 with cached loads ran at 4.0 TB/s; R = 128 with
// non-temporal loads at 4.7 TB/s, on 64 packed sequences of 128..8192 tokens.)
#include "conv_device.h"
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {
namespace {

constexpr int kTokensPerBlock = 128;
constexpr int kGroup = 4;                                   // tokens per load group
constexpr int kChanPerThread = 8;
constexpr int kThreads = 256;
constexpr int kChanPerBlock = kThreads * kChanPerThread;   // 2048

struct ConvArgs {
  const bf16* x;
  const float* w;
  const int32_t* cu;
  bf16* q;
  bf16* k;
  bf16* v;
  int K, num_seqs, total_tokens, h_qk, h_v, C;
  float q_scale;
};

__device__ __forceinline__ void load8(const bf16* p, float (&x)[8]) {
  const bf16x8 r = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = (float)r[e];
}

// Rows t0 .. t0 + kGroup - 1 of this thread's channels; rows at or past t_end repeat row
// t_end - 1 (those tokens are never processed). The loads are unconditional: loads under a
// branch made the compiler wait for every load in flight, the next group's included, before
// each token.
__device__ __forceinline__ void load_group(const bf16* x, size_t C, int t0, int t_end,
                                           bf16x8 (&raw)[kGroup]) {
#pragma unroll
  for (int u = 0; u < kGroup; ++u)
    raw[u] = __builtin_bit_cast(bf16x8, __builtin_nontemporal_load(
                 reinterpret_cast<const u32x4*>(x + (size_t)min(t0 + u, t_end - 1) * C)));
}

// Largest n with cu[n] <= t < cu[n+1] (t < total_tokens, so such n exists).
__device__ int find_sequence(const int32_t* cu, int num_seqs, int t) {
  int lo = 0, hi = num_seqs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= t) lo = mid;
    else hi = mid - 1;
  }
  // zero-length sequences share their start with the next one; cu[lo] <= t holds and the
  // search picked the last such n, whose end lies beyond t
  return lo;
}

__global__ __launch_bounds__(kThreads, 4) void conv_prep_kernel(ConvArgs a) {
  const int c0 = blockIdx.x * kChanPerBlock + threadIdx.x * kChanPerThread;
  const int t_begin = blockIdx.y * kTokensPerBlock;
  if (t_begin >= a.total_tokens) return;
  const int t_end = min(a.total_tokens, t_begin + kTokensPerBlock);
  if (c0 >= a.C) return;          // whole 16-lane groups leave together (C % 128 == 0)

  const int nq = a.h_qk * kHeadDim;
  const int nv = a.h_v * kHeadDim;
  const bool is_q = c0 < nq;
  const bool is_k = !is_q && c0 < 2 * nq;

  float wt[4][8];
  load_taps(a.w, a.K, c0, wt);

  const int n = find_sequence(a.cu, a.num_seqs, t_begin);
  const int seq_start = a.cu[n];
  // the tokens of this block that start a sequence (offsets from t_begin, never 0: the first
  // token's history comes from the rows before it), one bit each; found once here so the
  // token loop reads nothing but its rows
  uint64_t starts_lo = 0, starts_hi = 0;
  for (int m = n + 1; m <= a.num_seqs && a.cu[m] < t_end; ++m) {
    const int off = a.cu[m] - t_begin;
    if (off < 64) starts_lo |= 1ull << off;
    else starts_hi |= 1ull << (off - 64);
  }

  float h1[8], h2[8], h3[8];     // inputs at t-1, t-2, t-3 (zero before the sequence start)
  {
    float r1[8], r2[8], r3[8];
    load8(a.x + (size_t)max(t_begin - 1, 0) * a.C + c0, r1);
    load8(a.x + (size_t)max(t_begin - 2, 0) * a.C + c0, r2);
    load8(a.x + (size_t)max(t_begin - 3, 0) * a.C + c0, r3);
    const bool k1 = a.K > 1 && t_begin - 1 >= seq_start;
    const bool k2 = a.K > 2 && t_begin - 2 >= seq_start;
    const bool k3 = a.K > 3 && t_begin - 3 >= seq_start;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      h1[e] = k1 ? r1[e] : 0.f;
      h2[e] = k2 ? r2[e] : 0.f;
      h3[e] = k3 ? r3[e] : 0.f;
    }
  }

  const bf16* xc = a.x + c0;
  // One group of kGroup tokens from its loaded rows. Returns false once the block's tokens
  // are done.
  auto process = [&](const bf16x8 (&raw)[kGroup], int gi) {
#pragma unroll
    for (int u = 0; u < kGroup; ++u) {
      const int t = t_begin + gi * kGroup + u;
      if (t >= t_end) return false;
      const int off = gi * kGroup + u;
      if (((off < 64 ? starts_lo >> off : starts_hi >> (off - 64)) & 1) != 0) {   // a new sequence: no history
#pragma unroll
        for (int e = 0; e < 8; ++e) h1[e] = h2[e] = h3[e] = 0.f;
      }
      float x0[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) x0[e] = (float)raw[u][e];
      const bf16x8 out = conv_token(wt, x0, h1, h2, h3, is_q, is_k, a.q_scale);
      bf16* dst = is_q ? a.q + (size_t)t * nq + c0
                : is_k ? a.k + (size_t)t * nq + (c0 - nq)
                       : a.v + (size_t)t * nv + (c0 - 2 * nq);
      *reinterpret_cast<bf16x8*>(dst) = out;
      // inputs more than K - 1 tokens back stay zero (as in the decode window), so every
      // tap past the kernel multiplies zero by zero in both
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        h3[e] = a.K > 3 ? h2[e] : 0.f;
        h2[e] = a.K > 2 ? h1[e] : 0.f;
        h1[e] = a.K > 1 ? x0[e] : 0.f;
      }
    }
    return true;
  };
  // two buffers named apart (every index static, so neither lands in scratch memory), the
  // next group's rows in flight while a group computes
  bf16x8 ra[kGroup], rb[kGroup];
  load_group(xc, a.C, t_begin, t_end, ra);
#pragma unroll
  for (int gi = 0; gi < kTokensPerBlock / kGroup; gi += 2) {
    load_group(xc, a.C, t_begin + (gi + 1) * kGroup, t_end, rb);
    asm volatile("" ::: "memory");   // the refill stays here
    if (!process(ra, gi)) break;
    if (gi + 2 < kTokensPerBlock / kGroup) load_group(xc, a.C, t_begin + (gi + 2) * kGroup, t_end, ra);
    asm volatile("" ::: "memory");
    if (!process(rb, gi + 1)) break;
  }
}

// ---- Decode side: one token per sequence, the last K - 1 inputs of each sequence in a
// window pool [pool][K - 1][C] bf16 (row r holds the input K - 1 - r tokens back).

struct ConvDecodeArgs {
  const bf16* x;            // [num_seqs][C], this step's inputs
  const float* w;
  bf16* win;                // window pool, updated in place
  const int32_t* slots;     // sequence n uses window slots[n] (n when null)
  bf16* q;
  bf16* k;
  bf16* v;
  int K, num_seqs, h_qk, h_v, C;
  float q_scale;
};

// One block per (2048 channels, kSeqPerBlock sequences), 8 channels per thread: the taps are
// loaded once for the block's sequences, and every sequence's loads are issued before any is
// computed. The current input and the window give the same conv_token inputs as the prefill
// kernel at that token; the window then moves one token on (row r takes row r + 1, the last
// row the current input).
constexpr int kSeqPerBlock = 4;

__global__ __launch_bounds__(kThreads) void conv_decode_kernel(ConvDecodeArgs a) {
  const int c0 = blockIdx.x * kChanPerBlock + threadIdx.x * kChanPerThread;
  if (c0 >= a.C) return;          // whole 16-lane groups leave together (C % 128 == 0)
  const int nq = a.h_qk * kHeadDim;
  const int nv = a.h_v * kHeadDim;
  const bool is_q = c0 < nq;
  const bool is_k = !is_q && c0 < 2 * nq;
  const int n0 = blockIdx.y * kSeqPerBlock;
  const int ns = min(kSeqPerBlock, a.num_seqs - n0);
  int slot[kSeqPerBlock];
#pragma unroll
  for (int s = 0; s < kSeqPerBlock; ++s)
    slot[s] = s < ns ? (a.slots ? a.slots[n0 + s] : n0 + s) : 0;
  bf16x8 xr[kSeqPerBlock], hr[kSeqPerBlock][3];   // hr[s][d - 1]: input d tokens back
#pragma unroll
  for (int s = 0; s < kSeqPerBlock; ++s) {
    xr[s] = bf16x8{};
    hr[s][0] = hr[s][1] = hr[s][2] = bf16x8{};
    if (s < ns) {
      xr[s] = *reinterpret_cast<const bf16x8*>(a.x + (size_t)(n0 + s) * a.C + c0);
      const bf16* wrow = a.win + (size_t)slot[s] * (a.K - 1) * a.C + c0;
#pragma unroll
      for (int d = 1; d < 4; ++d)
        if (d < a.K) hr[s][d - 1] = *reinterpret_cast<const bf16x8*>(wrow + (size_t)(a.K - 1 - d) * a.C);
    }
  }
  float wt[4][8];
  load_taps(a.w, a.K, c0, wt);
#pragma unroll
  for (int s = 0; s < kSeqPerBlock; ++s) {
    if (s >= ns) break;
    const int n = n0 + s;
    float x0[8], h1[8], h2[8], h3[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      x0[e] = (float)xr[s][e];
      h1[e] = (float)hr[s][0][e];
      h2[e] = (float)hr[s][1][e];
      h3[e] = (float)hr[s][2][e];
    }
    const bf16x8 out = conv_token(wt, x0, h1, h2, h3, is_q, is_k, a.q_scale);
    bf16* dst = is_q ? a.q + (size_t)n * nq + c0
              : is_k ? a.k + (size_t)n * nq + (c0 - nq)
                     : a.v + (size_t)n * nv + (c0 - 2 * nq);
    *reinterpret_cast<bf16x8*>(dst) = out;
    // row K - 1 - d now holds the input d - 1 tokens back (the current one for d = 1)
    bf16* wrow = a.win + (size_t)slot[s] * (a.K - 1) * a.C + c0;
#pragma unroll
    for (int d = 1; d < 4; ++d)
      if (d < a.K) *reinterpret_cast<bf16x8*>(wrow + (size_t)(a.K - 1 - d) * a.C) = d == 1 ? xr[s] : hr[s][d - 2];
  }
}

struct ConvWindowArgs {
  const bf16* x;            // [total_tokens][C] prefill inputs
  const int32_t* cu;
  bf16* win;
  const int32_t* slots;
  int K, C;
};

// The window each sequence of a prefill leaves for decode: its last K - 1 inputs, zero where
// the sequence is shorter (the zero history the prefill started from).
__global__ __launch_bounds__(kThreads) void conv_window_kernel(ConvWindowArgs a) {
  const int c0 = blockIdx.x * kChanPerBlock + threadIdx.x * kChanPerThread;
  const int n = blockIdx.y;
  if (c0 >= a.C) return;
  const int s0 = a.cu[n], s1 = a.cu[n + 1];
  const int slot = a.slots ? a.slots[n] : n;
  bf16* wrow = a.win + (size_t)slot * (a.K - 1) * a.C + c0;
  for (int r = 0; r < a.K - 1; ++r) {
    const int t = s1 - (a.K - 1) + r;
    const bf16x8 val = t >= s0 ? *reinterpret_cast<const bf16x8*>(a.x + (size_t)t * a.C + c0) : bf16x8{};
    *reinterpret_cast<bf16x8*>(wrow + (size_t)r * a.C) = val;
  }
}

}  // namespace

hipError_t launch_conv_prep(const void* mixed, const float* w, int K, const int32_t* cu,
                            int num_seqs, int total_tokens, int h_qk, int h_v, float q_scale,
                            void* q, void* k, void* v, hipStream_t stream) {
  if (total_tokens == 0) return hipSuccess;
  ConvArgs a;
  a.x = static_cast<const bf16*>(mixed);
  a.w = w;
  a.cu = cu;
  a.q = static_cast<bf16*>(q);
  a.k = static_cast<bf16*>(k);
  a.v = static_cast<bf16*>(v);
  a.K = K;
  a.num_seqs = num_seqs;
  a.total_tokens = total_tokens;
  a.h_qk = h_qk;
  a.h_v = h_v;
  a.C = (2 * h_qk + h_v) * kHeadDim;
  a.q_scale = q_scale;
  const dim3 grid((a.C + kChanPerBlock - 1) / kChanPerBlock,
                  (total_tokens + kTokensPerBlock - 1) / kTokensPerBlock);
  hipLaunchKernelGGL(conv_prep_kernel, grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace gdn

namespace gdn {

hipError_t launch_conv_decode(const void* mixed, const float* w, int K, void* window,
                              const int32_t* slots, int num_seqs, int h_qk, int h_v, float q_scale,
                              void* q, void* k, void* v, hipStream_t stream) {
  if (num_seqs == 0) return hipSuccess;
  ConvDecodeArgs a;
  a.x = static_cast<const bf16*>(mixed);
  a.w = w;
  a.win = static_cast<bf16*>(window);
  a.slots = slots;
  a.q = static_cast<bf16*>(q);
  a.k = static_cast<bf16*>(k);
  a.v = static_cast<bf16*>(v);
  a.K = K;
  a.num_seqs = num_seqs;
  a.h_qk = h_qk;
  a.h_v = h_v;
  a.C = (2 * h_qk + h_v) * kHeadDim;
  a.q_scale = q_scale;
  const dim3 grid((a.C + kChanPerBlock - 1) / kChanPerBlock, (num_seqs + kSeqPerBlock - 1) / kSeqPerBlock);
  hipLaunchKernelGGL(conv_decode_kernel, grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_conv_window(const void* mixed, int K, const int32_t* cu, int num_seqs, int h_qk,
                              int h_v, void* window, const int32_t* slots, hipStream_t stream) {
  if (num_seqs == 0 || K == 1) return hipSuccess;
  ConvWindowArgs a;
  a.x = static_cast<const bf16*>(mixed);
  a.cu = cu;
  a.win = static_cast<bf16*>(window);
  a.slots = slots;
  a.K = K;
  a.C = (2 * h_qk + h_v) * kHeadDim;
  const dim3 grid((a.C + kChanPerBlock - 1) / kChanPerBlock, num_seqs);
  hipLaunchKernelGGL(conv_window_kernel, grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace gdn
