// recurrent.hip -- token-sequential gated delta rule on gfx950, no matrix cores.
//
// One workgroup of 256 threads owns one (sequence, V head) state of 128 x 128 fp32 (64 KB)
// and keeps it in registers: thread (wave w, lane l) holds columns 4*(l%32) .. +3 of the
// 16 rows i*8 + 2*w + l/32, i = 0..15, so each load or store instruction of a wave covers
// two whole rows (1 KB, fully coalesced). Per token (page "Qwen3-Next -- How a running
// memory and a searchable history cooperate", section "Correcting a memory instead of
// adding to it", with the read-out after the update of the "01 . GatedDeltaNet(config)"
// token loop on page "Qwen3-Next 80B-A3B -- The Evolving Transformer"):
//
//   u = S k,  r = S q                      (row dot products, reduced over 32 lanes)
//   c = beta * (v - alpha * u)             (the correction of the decayed memory)
//   S <- alpha * S + c k^T
//   o = scale * S q = scale * (alpha * r + c * (k . q))
//
// Three kernels:
//  * decode_kernel: one token per sequence, the state streamed from and back to an fp32
//    pool in HBM (64 KB read + 64 KB written per head; bound by HBM bandwidth). 512 threads
//    per head, 8 rows each: the layout that streams fastest on this chip.
//  * seq_kernel: decode_kernel's layout and arithmetic (decode_token) over several tokens per
//    sequence with the state in registers between them: the verify step (draft tokens
//    checked at once, the state optionally written out after each token).
//  * rows_kernel: token-sequential prefill, 16 value rows per one-wave workgroup: the fp32
//    I/O prefill and the per-channel form.
// The per-channel form is the code panel of section "01 . GatedDeltaNet(config)" on the
// Evolving Transformer page: one decay per value row, the correction taken from the state
// before the decay (decode_kernel and rows_kernel with CH = true).
#include "conv_device.h"
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {
namespace {


struct RecArgs {
  int n_tok;                   // verify: tokens per sequence
  float* snap;                 // verify: per-token states, or NULL
  const void* q;
  const void* k;
  const void* v;
  const float* g;
  const float* beta;
  const int32_t* cu_seqlens;   // prefill: sequence spans; decode: unused
  const int32_t* slots;        // decode: pool entry per sequence (NULL = identity)
  const float* s_in;           // prefill: initial states or NULL; decode: the pool
  float* s_out;                // prefill: final states or NULL; decode: the pool
  void* o;
  int num_seqs, h_qk, h_v;
  float scale;
};

// Value of lane `src` (a constant below 32) of this lane's half-wave: two lane reads into
// scalars and a select, instead of a crossbar permute.
__device__ __forceinline__ float half_lane(float x, int src, bool upper) {
  const float lo = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), src));
  const float hi = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), src + 32));
  return upper ? hi : lo;
}

// Sum over the 32 lanes of each half-wave; every lane receives its half's total.
__device__ __forceinline__ float half_sum(float x) {
  x += xor_lane(x, 16);
  x += xor_lane(x, 8);
  x += xor_lane(x, 4);
  x += xor_lane(x, 2);
  x += xor_lane(x, 1);
  return x;
}

// One level of a half-wave reduce-scatter over n partial sums: lanes with bit m set keep
// the upper half of the indices and send the lower half to their partner l ^ m, the others
// the reverse, so each half of the lanes ends with n/2 partial sums of twice as many lanes.
// Sizes are template constants so every index is static (a runtime index would turn the
// array into select chains).
template <int M, int N, int L>
__device__ __forceinline__ void rs_level(float (&vals)[L], int lane32) {
  const bool upper = (lane32 & M) != 0;
#pragma unroll
  for (int idx = 0; idx < N / 2; ++idx) {
    const float send = upper ? vals[idx] : vals[idx + N / 2];
    const float keep = upper ? vals[idx + N / 2] : vals[idx];
    vals[idx] = keep + xor_lane(send, M);
  }
}

// Reduce-scatter of 16 partial sums over the 32 lanes of a half-wave: afterwards lanes
// 2c and 2c + 1 both hold the half-wave total of index c.
__device__ __forceinline__ float reduce_scatter16(float (&vals)[16], int lane32) {
  rs_level<16, 16>(vals, lane32);
  rs_level<8, 8>(vals, lane32);
  rs_level<4, 4>(vals, lane32);
  rs_level<2, 2>(vals, lane32);
  return vals[0] + xor_lane(vals[0], 1);
}

// One token of the decode layout (8 rows per thread, rows row_base + 16 i): u = S k and r = S q
// on the rows, c = beta (v - alpha u) and the rank-one update of S in place. Returns
// scale (alpha r + c (k . q)), this lane's output when (c4 & 3) == 2 (for row my_row).
__device__ __forceinline__ float decode_token(f32x4 (&S)[8], f32x4 k4, f32x4 q4, float alpha, float beta,
                                              float vrow, float scale, int c4) {
  // Every operation is spelled out (explicit fused multiply-adds, no contraction left to the
  // compiler): the decode, verify and fused decode kernels all run this and must agree bit
  // for bit, and the compiler's own contraction choices can differ between them.
#pragma clang fp contract(off)
  const bool my_is_r = (c4 & 2) != 0;
  const bool upper = (__lane_id() & 32) != 0;   // which half-wave (rows of this lane)
  float vals[16];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    vals[2 * i] = __builtin_fmaf(S[i][3], k4[3], __builtin_fmaf(S[i][2], k4[2],
                  __builtin_fmaf(S[i][1], k4[1], S[i][0] * k4[0])));
    vals[2 * i + 1] = __builtin_fmaf(S[i][3], q4[3], __builtin_fmaf(S[i][2], q4[2],
                      __builtin_fmaf(S[i][1], q4[1], S[i][0] * q4[0])));
  }
  const float mine = reduce_scatter16(vals, c4);
  const float other = xor_lane(mine, 2);
  const float u = my_is_r ? other : mine;
  const float r = my_is_r ? mine : other;
  const float kq = half_sum(__builtin_fmaf(k4[3], q4[3], __builtin_fmaf(k4[2], q4[2],
                            __builtin_fmaf(k4[1], q4[1], k4[0] * q4[0]))));
  const float c = beta * __builtin_fmaf(-alpha, u, vrow);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float ci = half_lane(c, 4 * i, upper);
#pragma unroll
    for (int e = 0; e < 4; ++e) S[i][e] = __builtin_fmaf(ci, k4[e], alpha * S[i][e]);
  }
  return scale * __builtin_fmaf(c, kq, alpha * r);
}

// The per-channel form at one token, decode layout: each value row i has its own decay
// alpha_i and the correction comes from the state before the decay,
// c_i = beta (v_i - u_i), S_i <- alpha_i S_i + c_i k^T. arow[i] is the decay of row
// row_base + 16 i, a_mine that of this lane's output row. Returns
// scale (a_mine r + c (k . q)), the output on lanes with (c4 & 3) == 2.
__device__ __forceinline__ float decode_token_channel(f32x4 (&S)[8], f32x4 k4, f32x4 q4, const float (&arow)[8],
                                                      float a_mine, float beta, float vrow, float scale, int c4) {
  const bool my_is_r = (c4 & 2) != 0;
  const bool upper = (__lane_id() & 32) != 0;   // which half-wave (rows of this lane)
  float vals[16];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    vals[2 * i] = S[i][0] * k4[0] + S[i][1] * k4[1] + S[i][2] * k4[2] + S[i][3] * k4[3];
    vals[2 * i + 1] = S[i][0] * q4[0] + S[i][1] * q4[1] + S[i][2] * q4[2] + S[i][3] * q4[3];
  }
  const float mine = reduce_scatter16(vals, c4);
  const float other = xor_lane(mine, 2);
  const float u = my_is_r ? other : mine;
  const float r = my_is_r ? mine : other;
  const float kq = half_sum(k4[0] * q4[0] + k4[1] * q4[1] + k4[2] * q4[2] + k4[3] * q4[3]);
  const float c = beta * (vrow - u);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float ci = half_lane(c, 4 * i, upper);
    S[i][0] = arow[i] * S[i][0] + ci * k4[0];
    S[i][1] = arow[i] * S[i][1] + ci * k4[1];
    S[i][2] = arow[i] * S[i][2] + ci * k4[2];
    S[i][3] = arow[i] * S[i][3] + ci * k4[3];
  }
  return scale * (a_mine * r + c * kq);
}

// One decode step. Thread (wave w of 8, lane l) holds columns 4*(l%32) .. +3 of the 8 rows
// i*16 + 2*w + l/32, i = 0..7: each load or store instruction of a wave covers two whole
// rows (1 KB). CH selects the
// per-channel form (g [seq][h_v][128], one log-decay per value row, decode_token_channel).
template <typename IO, bool CH>
__global__ __launch_bounds__(512) void decode_kernel(RecArgs a) {
  constexpr int kRows = 8;
  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int half = lane >> 5;
  const int c4 = lane & 31;
  const int n = blockIdx.x / a.h_v;
  const int h = blockIdx.x % a.h_v;
  const int j = h / (a.h_v / a.h_qk);
  const IO* q = static_cast<const IO*>(a.q);
  const IO* k = static_cast<const IO*>(a.k);
  const IO* v = static_cast<const IO*>(a.v);
  IO* o = static_cast<IO*>(a.o);
  const int slot = a.slots ? a.slots[n] : n;
  const size_t state = ((size_t)slot * a.h_v + h) * kHeadDim * kHeadDim;
  const int row_base = w * 2 + half;        // rows row_base + 16*i

  float* sp = a.s_out + state + (size_t)row_base * kHeadDim + 4 * c4;
  f32x4 S[kRows];
#pragma unroll
  for (int i = 0; i < kRows; ++i)
    S[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(sp + (size_t)i * 16 * kHeadDim));

  // lanes 4i, 4i+1 finish u of row slot i; lanes 4i+2, 4i+3 finish r
  const int my_row = row_base + 16 * (c4 >> 2);

  const size_t qk_off = ((size_t)n * a.h_qk + j) * kHeadDim + 4 * c4;
  const f32x4 k4 = load4(k + qk_off);
  const f32x4 q4 = load4(q + qk_off);
  const float beta = a.beta[(size_t)n * a.h_v + h];
  const float vrow = load1(v + ((size_t)n * a.h_v + h) * kHeadDim + my_row);

  float out;
  if constexpr (CH) {
    const float* gh = a.g + ((size_t)n * a.h_v + h) * kHeadDim;
    float arow[kRows];
#pragma unroll
    for (int i = 0; i < kRows; ++i) arow[i] = __expf(gh[row_base + 16 * i]);
    out = decode_token_channel(S, k4, q4, arow, __expf(gh[my_row]), beta, vrow, a.scale, c4);
  } else {
    out = decode_token(S, k4, q4, __expf(a.g[(size_t)n * a.h_v + h]), beta, vrow, a.scale, c4);
  }
  if ((c4 & 3) == 2) store1(o + ((size_t)n * a.h_v + h) * kHeadDim + my_row, out);
#pragma unroll
  for (int i = 0; i < kRows; ++i)
    __builtin_nontemporal_store(S[i], reinterpret_cast<f32x4*>(sp + (size_t)i * 16 * kHeadDim));
}

// The decode step with the decode-time front end in front of it, one launch: one workgroup
// per (sequence, QK head) covers the G = h_v / h_qk V heads that share the QK head (512
// threads each, decode_kernel's layout), so the q and k channels of the window are read and
// shifted by a single workgroup. Every wave first requests its share of the states; wave 0
// then runs the front end for the workgroup's 256 + 128 G channels (8 per lane, one 16-lane
// group per head: lanes 0-15 q, 16-31 k, then the V heads) with the same conv_token as the
// front-end kernels, shifts the window and leaves the bf16 q, k and v in LDS; after a
// barrier every half runs decode_token on its V head. Outputs, states and window are bit for
// bit those of the front-end call followed by the decode step.
struct DecConvArgs {
  const bf16* x;          // [num_seqs][C] this step's projected inputs
  const float* w;         // [C][K] taps
  bf16* win;              // [pool][K - 1][C], in place
  const int32_t* wslots;  // window slot per sequence (NULL = identity)
  const float* g;
  const float* beta;
  const int32_t* slots;   // state slot per sequence (NULL = identity)
  float* pool;
  bf16* o;
  int num_seqs, h_qk, h_v, K, C;
  float q_scale, scale;
};

template <int G>
__global__ __launch_bounds__(512 * G) void decode_conv_kernel(DecConvArgs a) {
  constexpr int kRows = 8;
  __shared__ float qkv[(2 + G) * kHeadDim];   // q | k | v of the G heads, bf16 values
  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int half = lane >> 5;
  const int c4 = lane & 31;
  const int n = blockIdx.x / a.h_qk;
  const int j = blockIdx.x % a.h_qk;
  const int hl = w >> 3;                      // V head within the group
  const int h = j * G + hl;
  const int slot = a.slots ? a.slots[n] : n;
  const size_t state = ((size_t)slot * a.h_v + h) * kHeadDim * kHeadDim;
  const int row_base = (w & 7) * 2 + half;
  float* sp = a.pool + state + (size_t)row_base * kHeadDim + 4 * c4;
  f32x4 S[kRows];
#pragma unroll
  for (int i = 0; i < kRows; ++i)
    S[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(sp + (size_t)i * 16 * kHeadDim));

  if (w == 0) {
    const int grp = lane >> 4;                // 0: q, 1: k, 2..: V head grp - 2
    const int nq = a.h_qk * kHeadDim;
    const int c0 = grp == 0 ? j * kHeadDim + 8 * (lane & 15)
                 : grp == 1 ? nq + j * kHeadDim + 8 * (lane & 15)
                            : 2 * nq + (j * G + grp - 2) * kHeadDim + 8 * (lane & 15);
    const bool live = grp < 2 + G;            // G = 1 leaves the last 16 lanes idle
    if (live) {
      const bf16x8 xr = *reinterpret_cast<const bf16x8*>(a.x + (size_t)n * a.C + c0);
      const int wslot = a.wslots ? a.wslots[n] : n;
      bf16* wrow = a.win + (size_t)wslot * (a.K - 1) * a.C + c0;
      bf16x8 hr[3] = {bf16x8{}, bf16x8{}, bf16x8{}};
#pragma unroll
      for (int d = 1; d < 4; ++d)
        if (d < a.K) hr[d - 1] = *reinterpret_cast<const bf16x8*>(wrow + (size_t)(a.K - 1 - d) * a.C);
      float wt[4][8];
      load_taps(a.w, a.K, c0, wt);
      float x0[8], h1[8], h2[8], h3[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        x0[e] = (float)xr[e];
        h1[e] = (float)hr[0][e];
        h2[e] = (float)hr[1][e];
        h3[e] = (float)hr[2][e];
      }
      const bf16x8 out = conv_token(wt, x0, h1, h2, h3, grp == 0, grp == 1, a.q_scale);
#pragma unroll
      for (int e = 0; e < 8; ++e) qkv[grp * kHeadDim + 8 * (lane & 15) + e] = (float)out[e];
#pragma unroll
      for (int d = 1; d < 4; ++d)
        if (d < a.K) *reinterpret_cast<bf16x8*>(wrow + (size_t)(a.K - 1 - d) * a.C) = d == 1 ? xr : hr[d - 2];
    }
  }
  __syncthreads();

  const int my_row = row_base + 16 * (c4 >> 2);
  const f32x4 k4 = *reinterpret_cast<const f32x4*>(&qkv[kHeadDim + 4 * c4]);
  const f32x4 q4 = *reinterpret_cast<const f32x4*>(&qkv[4 * c4]);
  const float vrow = qkv[(2 + hl) * kHeadDim + my_row];
  const float beta = a.beta[(size_t)n * a.h_v + h];
  const float out = decode_token(S, k4, q4, __expf(a.g[(size_t)n * a.h_v + h]), beta, vrow, a.scale, c4);
  if ((c4 & 3) == 2) a.o[((size_t)n * a.h_v + h) * kHeadDim + my_row] = to_bf16(out);
#pragma unroll
  for (int i = 0; i < kRows; ++i)
    __builtin_nontemporal_store(S[i], reinterpret_cast<f32x4*>(sp + (size_t)i * 16 * kHeadDim));
}

// The verify step: tokens t = 0 .. n_tok - 1 of sequence n are rows n * n_tok + t of the
// inputs; the state comes from the pool, stays in registers across the tokens (decode
// layout, decode_token's arithmetic, so the bits of n_tok decode steps) and goes back to the
// pool, and the state after each token goes to snap[n][t] when snap is set.
template <typename IO>
__global__ __launch_bounds__(512) void seq_kernel(RecArgs a) {
  constexpr int kRows = 8;
  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int half = lane >> 5;
  const int c4 = lane & 31;
  const int n = blockIdx.x / a.h_v;
  const int h = blockIdx.x % a.h_v;
  const int j = h / (a.h_v / a.h_qk);
  const IO* q = static_cast<const IO*>(a.q);
  const IO* k = static_cast<const IO*>(a.k);
  const IO* v = static_cast<const IO*>(a.v);
  IO* o = static_cast<IO*>(a.o);
  const int row0 = n * a.n_tok;
  const int n_tok = a.n_tok;
  const int slot = a.slots ? a.slots[n] : n;
  const size_t state = ((size_t)slot * a.h_v + h) * kHeadDim * kHeadDim;
  const int row_base = w * 2 + half;        // rows row_base + 16*i
  const size_t lane_off = (size_t)row_base * kHeadDim + 4 * c4;

  f32x4 S[kRows];
  if (a.s_in) {
    const float* src = a.s_in + state + lane_off;
#pragma unroll
    for (int i = 0; i < kRows; ++i)
      S[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(src + (size_t)i * 16 * kHeadDim));
  } else {
#pragma unroll
    for (int i = 0; i < kRows; ++i) S[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const int my_row = row_base + 16 * (c4 >> 2);

  // token t's inputs are requested during token t - 1 (before its stores, so waiting for
  // them never waits for a store)
  struct Tok {
    f32x4 k4, q4;
    float g, beta, vrow;
  };
  auto fetch = [&](int t) {
    const size_t tok = (size_t)row0 + t;
    const size_t qk_off = (tok * a.h_qk + j) * kHeadDim + 4 * c4;
    Tok x;
    x.k4 = load4(k + qk_off);
    x.q4 = load4(q + qk_off);
    x.beta = a.beta[tok * a.h_v + h];
    x.vrow = load1(v + (tok * a.h_v + h) * kHeadDim + my_row);
    x.g = a.g[tok * a.h_v + h];
    return x;
  };
  // one token: the read-out and update, the output, and the snapshot when asked
  auto step = [&](Tok& x, int t) {
    const size_t tok = (size_t)row0 + t;
    const float out = decode_token(S, x.k4, x.q4, __expf(x.g), x.beta, x.vrow, a.scale, c4);
    if ((c4 & 3) == 2) store1(o + (tok * a.h_v + h) * kHeadDim + my_row, out);
    if (a.snap) {
      float* dst = a.snap + (tok * a.h_v + h) * kHeadDim * kHeadDim + lane_off;
#pragma unroll
      for (int i = 0; i < kRows; ++i)
        __builtin_nontemporal_store(S[i], reinterpret_cast<f32x4*>(dst + (size_t)i * 16 * kHeadDim));
    }
  };
  // Two alternating input sets (no copy from one to the other, so a load never has to wait
  // for the register it overwrites); past the last token the loads repeat it, unused.
  if (n_tok > 0) {
    Tok ta = fetch(0), tb;
    for (int t = 0; t < n_tok; t += 2) {
      tb = fetch(min(t + 1, n_tok - 1));
      // the next token's loads are issued here: this token's k and q pass through the asm,
      // so no product that uses them moves above it
      asm volatile("" : "+v"(ta.k4), "+v"(ta.q4) :: "memory");
      step(ta, t);
      if (t + 1 < n_tok) {
        ta = fetch(min(t + 2, n_tok - 1));
        asm volatile("" : "+v"(tb.k4), "+v"(tb.q4) :: "memory");
        step(tb, t + 1);
      }
    }
  }
  if (a.s_out) {
    float* dst = a.s_out + state + lane_off;
#pragma unroll
    for (int i = 0; i < kRows; ++i)
      __builtin_nontemporal_store(S[i], reinterpret_cast<f32x4*>(dst + (size_t)i * 16 * kHeadDim));
  }
}

// CPL consecutive inputs (k or q columns) of one token as the 32-bit words a load returns,
// converted to fp32 only where they are used: a ring of tokens in flight then carries loaded
// registers across the loop, and the compiler waits for each set by its own count instead
// of draining every load to convert it before the loop's back edge.
template <typename IO, int CPL>
struct RawCols {
  static constexpr int NW = CPL * (int)sizeof(IO) / 4;
  uint32_t w[NW];
};

template <typename IO, int CPL>
__device__ __forceinline__ RawCols<IO, CPL> load_cols(const IO* p) {
  RawCols<IO, CPL> r;
  constexpr int NW = RawCols<IO, CPL>::NW;
  const uint32_t* src = reinterpret_cast<const uint32_t*>(p);
  if constexpr (NW % 4 == 0) {
#pragma unroll
    for (int i = 0; i < NW / 4; ++i) {
      const u32x4 x = *reinterpret_cast<const u32x4*>(src + 4 * i);
      r.w[4 * i] = x[0]; r.w[4 * i + 1] = x[1]; r.w[4 * i + 2] = x[2]; r.w[4 * i + 3] = x[3];
    }
  } else {
    static_assert(NW == 2, "column group of 8 bytes or a multiple of 16");
    const u32x2 x = *reinterpret_cast<const u32x2*>(src);
    r.w[0] = x[0]; r.w[1] = x[1];
  }
  return r;
}

// Column e as fp32: a bf16 is the upper half of the fp32 with the same bits (element 2i sits
// in the low half of word i).
template <typename IO, int CPL>
__device__ __forceinline__ float col(const RawCols<IO, CPL>& r, int e) {
  if constexpr (sizeof(IO) == 2)
    return __builtin_bit_cast(float, (e & 1) ? (r.w[e / 2] & 0xffff0000u) : (r.w[e / 2] << 16));
  else
    return __builtin_bit_cast(float, r.w[e]);
}

// Token-sequential prefill with value rows split over workgroups: rows evolve independently
// in both forms, so each workgroup of one wave takes R rows of one (sequence, V head) and
// walks the sequence's tokens with its rows in registers. Lane (r = lane / L, p = lane % L,
// L = 64 / R lanes per row) holds columns 2R p .. 2R p + 2R - 1 of row R rb + r, so every
// per-row sum (S k, S q) and k . q is a partial over 2R columns and log2(L) lane exchanges
// inside a 16-lane DPP row (plus one swizzle when L = 32). Fewer rows per wave mean fewer
// columns, so less arithmetic per token on the chain, and more waves to spread over the
// chip's SIMDs; more rows per wave cost less in total when the grid is full anyway. The
// inputs of the next D tokens are in flight while a token computes. CH selects the
// per-channel form (g [row][h_v][128]: one log-decay per value row, the correction from the
// state before the decay); otherwise the main form (one decay per V head).
template <typename IO, bool CH, int R, int D>
__global__ __launch_bounds__(64) void rows_kernel(RecArgs a) {
  constexpr int L = 64 / R;          // lanes per row
  constexpr int CPL = 128 / L;       // columns per lane
  constexpr int NV = CPL / 4;        // f32x4 per lane
  constexpr int NB = 128 / R;        // workgroups per (sequence, V head)
  const int lane = threadIdx.x;
  const int rb = blockIdx.x % NB;
  const int nh = blockIdx.x / NB;
  const int n = nh / a.h_v;
  const int h = nh % a.h_v;
  const int j = h / (a.h_v / a.h_qk);
  const int row = R * rb + lane / L;
  const int c0 = CPL * (lane % L);
  const IO* q = static_cast<const IO*>(a.q);
  const IO* k = static_cast<const IO*>(a.k);
  const IO* v = static_cast<const IO*>(a.v);
  IO* o = static_cast<IO*>(a.o);
  const int t0 = a.cu_seqlens[n];
  const int n_tok = a.cu_seqlens[n + 1] - t0;
  const size_t state = (((size_t)n * a.h_v + h) * kHeadDim + row) * kHeadDim + c0;

  f32x4 S[NV];
  if (a.s_in) {
#pragma unroll
    for (int i = 0; i < NV; ++i) S[i] = *reinterpret_cast<const f32x4*>(a.s_in + state + 4 * i);
  } else {
#pragma unroll
    for (int i = 0; i < NV; ++i) S[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  struct Tok {
    RawCols<IO, CPL> k, q;
    float g, beta;
    IO vrow;
  };
  // Inputs are addressed from uniform per-token bases (scalar registers, advanced by one
  // token at a time) plus this lane's zero-extended offset, so each load is one instruction
  // with no per-lane address arithmetic. f is the next token to fetch, held at the last one
  // once the sequence is exhausted (the ring then refills with copies it never uses).
  const unsigned urow = (unsigned)row, uc0 = (unsigned)c0;
  const size_t s_qk = (size_t)a.h_qk * kHeadDim;
  int f = 0;
  size_t f_qk = ((size_t)t0 * a.h_qk + j) * kHeadDim;
  size_t f_vh = (size_t)t0 * a.h_v + h;
  auto fetch = [&]() {
    Tok x;
    x.k = load_cols<IO, CPL>(k + f_qk + uc0);
    x.q = load_cols<IO, CPL>(q + f_qk + uc0);
    x.g = CH ? a.g[f_vh * kHeadDim + urow] : a.g[f_vh];
    x.beta = a.beta[f_vh];
    x.vrow = v[f_vh * kHeadDim + urow];
    if (f < n_tok - 1) {
      ++f;
      f_qk += s_qk;
      f_vh += a.h_v;
    }
    return x;
  };
  size_t o_vh = (size_t)t0 * a.h_v + h;
  // The read-out is taken from the updated state (o = S_t q): its sum is off the chain that
  // carries the state to the next token, and k . q is not needed. Every lane of a row holds
  // the row's sums after the exchanges, so all of them store the same value (no branch, so
  // one token's read-out can overlap the next token's chain).
  auto step = [&](const Tok& x) {
    float kc[CPL];
#pragma unroll
    for (int e = 0; e < CPL; ++e) kc[e] = col(x.k, e);
    float u = 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) u += S[i][e] * kc[4 * i + e];
#pragma unroll
    for (int m = 1; m < L; m *= 2) u += xor_lane(u, m);
    const float alpha = __expf(x.g);
    const float vrow = (float)x.vrow;
    // main form: the correction of the decayed memory; per-channel form: of the memory before
    // this row's decay
    const float c = CH ? x.beta * (vrow - u) : x.beta * (vrow - alpha * u);
    float r = 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        S[i][e] = alpha * S[i][e] + c * kc[4 * i + e];
        r += S[i][e] * col(x.q, 4 * i + e);
      }
#pragma unroll
    for (int m = 1; m < L; m *= 2) r += xor_lane(r, m);
    store1(o + o_vh * kHeadDim + urow, a.scale * r);
    o_vh += a.h_v;
  };
  // A token's inputs pass through an empty asm just before its step: what is computed from
  // them (the bf16 widening, exp of the decay) cannot be hoisted above it, so no earlier
  // token waits for a later token's loads.
  auto pin = [&](Tok& x) {
#pragma unroll
    for (int i = 0; i < RawCols<IO, CPL>::NW; ++i) asm volatile("" : "+v"(x.k.w[i]), "+v"(x.q.w[i]));
    if constexpr (sizeof(IO) == 2) {
      unsigned short vb = __builtin_bit_cast(unsigned short, x.vrow);
      asm volatile("" : "+v"(x.g), "+v"(x.beta), "+v"(vb));
      x.vrow = __builtin_bit_cast(IO, vb);
    } else {
      asm volatile("" : "+v"(x.g), "+v"(x.beta), "+v"(x.vrow));
    }
  };
  if (n_tok > 0) {
    // ring of D token input sets; the loads are unconditional (see fetch), so the compiler
    // waits for each set by its own count
    Tok buf[D];
#pragma unroll
    for (int d = 0; d < D; ++d) buf[d] = fetch();
    int t = 0;
    for (; t + D <= n_tok; t += D) {
#pragma unroll
      for (int d = 0; d < D; ++d) {
        // the refill goes into the registers this token has just used, so nothing is copied
        // around the loop (a copy of a load in flight would have to wait for it)
        pin(buf[d]);
        step(buf[d]);
        buf[d] = fetch();
        // keeps the refill's loads here: left free, the scheduler sinks them towards their
        // use a whole ring later, and the wait for them lands on the next token
        asm volatile("" ::: "memory");
      }
    }
#pragma unroll
    for (int d = 0; d < D; ++d)
      if (t + d < n_tok) step(buf[d]);
  }
  if (a.s_out) {
#pragma unroll
    for (int i = 0; i < NV; ++i) *reinterpret_cast<f32x4*>(a.s_out + state + 4 * i) = S[i];
  }
}

// Shape of the token-sequential prefill by the number of (sequence, V head) pairs: up to 64
// pairs (two sequences of 32 V heads) the chain of one wave is the limit and 4 rows per wave
// (32 waves per pair, 8 tokens in flight) spread it over the most SIMDs; beyond that the
// chip is full and arithmetic per row is the limit, which 8 rows per wave (4 in flight)
// keeps lower.
template <typename IO, bool CH>
hipError_t launch_rows(const RecArgs& a, hipStream_t stream) {
  const unsigned pairs = (unsigned)a.num_seqs * (unsigned)a.h_v;
  if (pairs <= 64)
    hipLaunchKernelGGL((rows_kernel<IO, CH, 4, 8>), dim3(pairs * 32), dim3(64), 0, stream, a);
  else
    hipLaunchKernelGGL((rows_kernel<IO, CH, 8, 4>), dim3(pairs * 16), dim3(64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const void* q, const void* k, const void* v, bool io_bf16,
                         const float* g, const float* beta, float* pool, const int32_t* slots,
                         int num_seqs, int h_qk, int h_v, float scale, void* o,
                         hipStream_t stream) {
  RecArgs a{1, nullptr, q, k, v, g, beta, nullptr, slots, pool, pool, o, num_seqs, h_qk, h_v, scale};
  const dim3 grid((unsigned)num_seqs * (unsigned)h_v), block(512);
  if (io_bf16)
    hipLaunchKernelGGL((decode_kernel<bf16, false>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((decode_kernel<float, false>), grid, block, 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_decode_with_conv(const void* mixed_qkv, const float* conv_weight, int conv_kernel,
                                  void* conv_window, const int32_t* window_slots, float q_scale,
                                  const float* g, const float* beta, float* pool,
                                  const int32_t* slots, int num_seqs, int h_qk, int h_v,
                                  float scale, void* o, hipStream_t stream) {
  DecConvArgs a{static_cast<const bf16*>(mixed_qkv), conv_weight, static_cast<bf16*>(conv_window),
                window_slots, g, beta, slots, pool, static_cast<bf16*>(o), num_seqs, h_qk, h_v,
                conv_kernel, (2 * h_qk + h_v) * kHeadDim, q_scale, scale};
  const dim3 grid((unsigned)num_seqs * (unsigned)h_qk);
  if (h_v == h_qk)
    hipLaunchKernelGGL((decode_conv_kernel<1>), grid, dim3(512), 0, stream, a);
  else
    hipLaunchKernelGGL((decode_conv_kernel<2>), grid, dim3(1024), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_recurrent_prefill(const void* q, const void* k, const void* v, bool io_bf16,
                                    const float* g, const float* beta, const int32_t* cu_seqlens,
                                    int num_seqs, int h_qk, int h_v, float scale,
                                    const float* s0, float* s_final, void* o, hipStream_t stream) {
  RecArgs a{0, nullptr, q, k, v, g, beta, cu_seqlens, nullptr, s0, s_final, o, num_seqs, h_qk, h_v, scale};
  return io_bf16 ? launch_rows<bf16, false>(a, stream) : launch_rows<float, false>(a, stream);
}

hipError_t launch_verify(const void* q, const void* k, const void* v, bool io_bf16, const float* g,
                         const float* beta, float* pool, const int32_t* slots, float* snapshots,
                         int num_seqs, int num_tokens, int h_qk, int h_v, float scale, void* o,
                         hipStream_t stream) {
  RecArgs a{num_tokens, snapshots, q, k, v, g, beta, nullptr, slots, pool, pool, o, num_seqs, h_qk, h_v, scale};
  const dim3 grid((unsigned)num_seqs * (unsigned)h_v), block(512);
  if (io_bf16)
    hipLaunchKernelGGL((seq_kernel<bf16>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((seq_kernel<float>), grid, block, 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_channel_prefill(const void* q, const void* k, const void* v, bool io_bf16,
                                  const float* g, const float* beta, const int32_t* cu_seqlens,
                                  int num_seqs, int h_qk, int h_v, float scale, const float* s0,
                                  float* s_final, void* o, hipStream_t stream) {
  RecArgs a{0, nullptr, q, k, v, g, beta, cu_seqlens, nullptr, s0, s_final, o, num_seqs, h_qk, h_v, scale};
  return io_bf16 ? launch_rows<bf16, true>(a, stream) : launch_rows<float, true>(a, stream);
}

hipError_t launch_channel_decode(const void* q, const void* k, const void* v, bool io_bf16,
                                 const float* g, const float* beta, float* pool, const int32_t* slots,
                                 int num_seqs, int h_qk, int h_v, float scale, void* o,
                                 hipStream_t stream) {
  RecArgs a{1, nullptr, q, k, v, g, beta, nullptr, slots, pool, pool, o, num_seqs, h_qk, h_v, scale};
  const dim3 grid((unsigned)num_seqs * (unsigned)h_v), block(512);
  if (io_bf16)
    hipLaunchKernelGGL((decode_kernel<bf16, true>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((decode_kernel<float, true>), grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace gdn
