// chunk_prefill.hip -- chunked gated delta rule prefill on gfx950 matrix cores.
//
// The rule (page "Qwen3-Next -- How a running memory and a searchable history cooperate",
// section "Correcting a memory instead of adding to it"; read-out after the update as in the
// token loop of section "01 . GatedDeltaNet(config)" of page "Qwen3-Next 80B-A3B -- The
// Evolving Transformer") is applied to chunks of C = 64 tokens at once. For one V head and a
// chunk with entering state S (d_v x d_k), keys K, queries Q (C x d_k), values V (C x d_v),
// log-decays g and strengths beta, unrolling the per-token update gives:
//
//   G_r = g_1 + ... + g_r,  gam_r = exp(G_r),  Gam_rs = exp(G_r - G_s) (s <= r, never > 1)
//   A   = strictly-lower(diag(beta) (K K^T) o Gam),     T = (I + A)^-1
//   W   = T diag(beta gam) K,     U~ = T diag(beta) V,     U = U~ - W S^T
//   O   = scale * [ diag(gam) Q S^T + (Q K^T o Gam o lower-incl) U ]
//   S'  = gam_C S + (diag(gam_C / gam) U)^T K
//
// Everything that does not involve S depends on one chunk only, so the work splits in two
// launches that share a workspace:
//
//  * prep_kernel, one workgroup per (chunk, V head), all chunks in parallel: K K^T and Q K^T
//    on the bf16 matrix cores, the prefix sums, the unit-lower-triangular inverse T in fp32
//    (16 x 16 diagonal blocks by substitution, off-diagonal blocks on the fp32 matrix
//    cores), then U~ (T diag(beta) split into hi + lo bf16) and -W on the bf16 matrix cores.
//    Writes -W, U~ (fp32, in the accumulator layout of the state pass),
//    P = scale (Q K^T o Gam o lower-incl), gam, gam_C / gam and K^T.
//  * state_kernel, one workgroup per (sequence, V head, 64 value rows), walking the
//    sequence's chunks in order with its slice of S in fp32 registers (value rows evolve
//    independently). Per chunk: U = U~ - W S^T, Q S^T, O = scale gam (Q S^T) + P U and the
//    state update on the bf16 matrix cores. The next chunk's -W, Q, K^T, P and U~ stream
//    into a second LDS buffer with direct global-to-LDS loads while the current chunk
//    computes.
//
// Precision: every product keeps one exact bf16 operand (K, Q, V as given); T diag(beta)
// and the decayed U that feeds the state are split into hi + lo bf16 pairs so they keep
// ~16 mantissa bits; S stays in fp32 and is rounded to bf16 only as a product operand.
//
// Matrix-core layout (v_mfma_f32_16x16x32_bf16): lane l holds A[l%16][8*(l/16)+s],
// B[8*(l/16)+s][l%16] for s = 0..7, and C[4*(l/16)+i][l%16] for i = 0..3. A product is
// unchanged when the same permutation is applied to the K index of A and B, so a
// C-layout accumulator pair covering K rows k0..k0+15 and k0+16..k0+31 is a valid B
// operand once its A partner reads K entries {4g..4g+3, 16+4g..16+4g+3} (g = l/16).
// The fp32 16x16x4 instruction has lane l holding A[l%16][l/16], B[l/16][l%16] and the
// same C layout; the same permutation argument lets a C-layout tile feed it as B.
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {
namespace {

constexpr int kC = 64;          // chunk length
constexpr int kD = 128;         // head dim
constexpr int kThreads = 256;
constexpr int kTokPad = kC + 8;     // [x][token] LDS rows, bf16
constexpr int kRowPad = kD + 8;     // [token][d_k] LDS rows, bf16
constexpr int kF32Pad = kC + 4;     // [token][token] LDS rows, fp32

// Workspace: one block per (chunk, V head), then K^T per (chunk, QK head).
constexpr size_t kWsW = 0;                          // bf16 [64][128]: -W
constexpr size_t kWsP = kWsW + kC * kD * 2;         // bf16 [64][64]: P
constexpr size_t kWsGam = kWsP + kC * kC * 2;       // fp32 [64]: gam_r
constexpr size_t kWsLam = kWsGam + kC * 4;          // fp32 [64]: gam_C / gam_r
constexpr size_t kWsU = kWsLam + kC * 4;            // fp32 U~ in C layout: [8 col tiles][4 row tiles][64 lanes][4]
constexpr size_t kWsHead = kWsU + kC * kD * 4;      // 57856 bytes
constexpr size_t kWsKT = kD * kC * 2;               // bf16 [128][64] per (chunk, QK head)

__host__ __device__ inline size_t max_chunks(int total_tokens, int num_seqs) {
  return (size_t)(total_tokens + kC - 1) / kC + (size_t)num_seqs;
}

struct PrefillArgs {
  const bf16* q;
  const bf16* k;
  const bf16* v;
  const float* g;
  const float* beta;
  const int32_t* cu;
  const float* s0;
  float* s_final;
  bf16* o;
  uint8_t* ws_heads;        // per (chunk, V head) blocks
  uint8_t* ws_kt;           // per (chunk, QK head) K^T
  int num_seqs, h_qk, h_v, group, n_chunks_max;
  float scale;
};

typedef __attribute__((address_space(3))) void* lds_void_ptr;

__device__ __forceinline__ bf16x8 lds8(const bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }
__device__ __forceinline__ bf16x4 lds4(const bf16* p) { return *reinterpret_cast<const bf16x4*>(p); }
__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Chunks of a sequence: ceil(len / 64).
__device__ __forceinline__ int seq_chunks(const int32_t* cu, int m) {
  return (cu[m + 1] - cu[m] + kC - 1) / kC;
}

__device__ __forceinline__ int wave_incl_scan(int x, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  return x;
}

// Global chunk c -> (sequence n, chunk index within n). Chunks are numbered sequence by
// sequence. Whole-wave cooperative; every lane gets the answer. n = -1 past the last chunk.
__device__ void locate_chunk(const int32_t* cu, int num_seqs, int c, int lane, int& n_out,
                             int& local_out) {
  int base = 0;
  for (int s0 = 0; s0 < num_seqs; s0 += 64) {
    const int m = s0 + lane;
    const int cnt = m < num_seqs ? seq_chunks(cu, m) : 0;
    const int inc = wave_incl_scan(cnt, lane);
    const int excl = inc - cnt;
    const unsigned long long hit = __ballot(c >= base + excl && c < base + inc);
    if (hit) {
      const int src = __ffsll((long long)hit) - 1;
      n_out = s0 + src;
      local_out = c - base - __shfl(excl, src, 64);
      return;
    }
    base += __shfl(inc, 63, 64);
  }
  n_out = -1;
  local_out = 0;
}

// Index of sequence n's first chunk. Whole-wave cooperative.
__device__ int first_chunk(const int32_t* cu, int n, int lane) {
  int base = 0;
  for (int s0 = 0; s0 < n; s0 += 64) {
    const int m = s0 + lane;
    int cnt = m < n ? seq_chunks(cu, m) : 0;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) cnt += __shfl_xor(cnt, off, 64);
    base += cnt;
  }
  return base;
}

// ------------------------------------------------------------------------------------------
// prep_kernel: one workgroup per (chunk, V head)
// ------------------------------------------------------------------------------------------
struct PrepSmem {
  bf16 KT[kD][kTokPad];         // K^T of the chunk
  bf16 VT[kD][kTokPad];         // V^T of the chunk for this V head; later stages -W
  union {
    struct {
      float A[kC][kF32Pad];
      float T[kC][kF32Pad];     // T = (I + A)^-1
    } s;
    struct {
      bf16 Th[kC][kTokPad];     // T diag(beta), hi
      bf16 Tl[kC][kTokPad];     // T diag(beta), lo
      bf16 Tbg[kC][kTokPad];    // -T diag(beta gam)
    } o;
  } u;
  float G[kC];
  float beta[kC];
  float gam[kC];
};

__global__ __launch_bounds__(kThreads, 2) void prep_kernel(PrefillArgs a) {
  __shared__ PrepSmem sm;
  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int g4 = lane >> 4;
  const int l16 = lane & 15;

  // workgroups of the V heads sharing one QK head sit on the same XCD (blockIdx % 8)
  const int bid = blockIdx.x;
  const int grp = bid / (8 * a.group), rem = bid % (8 * a.group);
  const int p = grp * 8 + rem % 8;            // (chunk, QK head) pair
  const int gi = rem / 8;                     // V head within the QK group
  const int c = p / a.h_qk, j = p % a.h_qk;
  if (c >= a.n_chunks_max) return;
  int n, local;
  locate_chunk(a.cu, a.num_seqs, c, lane, n, local);
  if (n < 0) return;
  const int h = j * a.group + gi;
  const int t0 = a.cu[n] + local * kC;
  const int nv = min(kC, a.cu[n + 1] - t0);
  uint8_t* wsh = a.ws_heads + ((size_t)c * a.h_v + h) * kWsHead;

  // ---- loads: K^T and V^T into LDS, g, beta ----
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int pc = tid + kThreads * i;          // 1024 pieces of 8 bf16
    const int row = pc >> 4, cb = pc & 15;
    bf16x8 kv = {}, vv = {};
    if (row < nv) {
      kv = *reinterpret_cast<const bf16x8*>(a.k + ((size_t)(t0 + row) * a.h_qk + j) * kD + cb * 8);
      vv = *reinterpret_cast<const bf16x8*>(a.v + ((size_t)(t0 + row) * a.h_v + h) * kD + cb * 8);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      sm.KT[cb * 8 + e][row] = kv[e];
      sm.VT[cb * 8 + e][row] = vv[e];
    }
  }
  if (tid < kC) {
    float gg = 0.f, bb = 0.f;
    if (tid < nv) {
      gg = a.g[(size_t)(t0 + tid) * a.h_v + h];
      bb = a.beta[(size_t)(t0 + tid) * a.h_v + h];
    }
    sm.G[tid] = gg;
    sm.beta[tid] = bb;
  }
  __syncthreads();
  if (gi == 0) {   // K^T for the state pass, rows of 64 tokens
    uint8_t* kt = a.ws_kt + ((size_t)c * a.h_qk + j) * kWsKT;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int pc = tid + kThreads * i;        // 1024 pieces: row = d_k, 8 tokens each
      const int row = pc >> 3, cb = pc & 7;
      *reinterpret_cast<bf16x8*>(kt + ((size_t)row * kC + cb * 8) * 2) = lds8(&sm.KT[row][cb * 8]);
    }
  }
  // ---- prefix sum of log-decays ----
  if (w == 0) {
    float x = sm.G[lane];
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float y = __shfl_up(x, off, 64);
      if (lane >= off) x += y;
    }
    const float GC = __shfl(x, 63, 64);
    sm.G[lane] = x;
    const float gm = __expf(x);
    sm.gam[lane] = gm;
    reinterpret_cast<float*>(wsh + kWsGam)[lane] = gm;
    reinterpret_cast<float*>(wsh + kWsLam)[lane] = __expf(GC - x);
  }
  __syncthreads();

  // ---- K K^T -> A, Q K^T -> P: 10 lower tiles each, operands straight from memory ----
  bf16* P = reinterpret_cast<bf16*>(wsh + kWsP);
  for (int job = w; job < 20; job += 4) {
    const bool isq = job >= 10;
    const int t = isq ? job - 10 : job;
    const int rt = t < 1 ? 0 : t < 3 ? 1 : t < 6 ? 2 : 3;
    const int ct = t - rt * (rt + 1) / 2;
    const int ra = 16 * rt + l16, rb = 16 * ct + l16;
    const bf16* arow = (isq ? a.q : a.k) + ((size_t)(t0 + ra) * a.h_qk + j) * kD;
    const bf16* brow = a.k + ((size_t)(t0 + rb) * a.h_qk + j) * kD;
    bf16x8 av[4], bv[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      av[ks] = ra < nv ? lds8(arow + 32 * ks + 8 * g4) : bf16x8{};
      bv[ks] = rb < nv ? lds8(brow + 32 * ks + 8 * g4) : bf16x8{};
    }
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) acc = mfma16x16x32(av[ks], bv[ks], acc);
    const int s = 16 * ct + l16;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * rt + 4 * g4 + i;
      const float decay = __expf(fminf(sm.G[r] - sm.G[s], 0.f));
      if (isq) P[r * kC + s] = to_bf16(s <= r ? a.scale * decay * acc[i] : 0.f);
      else sm.u.s.A[r][s] = s < r ? sm.beta[r] * decay * acc[i] : 0.f;
    }
  }
  for (int e = tid; e < 6 * 256; e += kThreads) {   // strictly upper tiles are zero
    const int t = e >> 8;
    const int rt = t < 3 ? 0 : t < 5 ? 1 : 2;
    const int ct = t < 3 ? t + 1 : t < 5 ? t - 1 : 3;
    const int r = 16 * rt + ((e & 255) >> 4), s = 16 * ct + (e & 15);
    P[r * kC + s] = to_bf16(0.f);
    sm.u.s.T[r][s] = 0.f;
  }
  __syncthreads();

  // ---- T = (I + A)^-1 --------------------------------------------------------------------
  // diagonal 16 x 16 blocks: wave b inverts block b by forward substitution, lane = column
  if (lane < 16) {
    const int b0 = 16 * w, col = lane;
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) x[r] = (r == col) ? 1.f : 0.f;
#pragma unroll
    for (int r = 1; r < 16; ++r) {
      float s = 0.f;
#pragma unroll
      for (int m = 0; m < r; ++m) s += sm.u.s.A[b0 + r][b0 + m] * x[m];
      if (r > col) x[r] = -s;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) sm.u.s.T[b0 + r][b0 + col] = x[r];
  }
  __syncthreads();
  // off-diagonal block (i, b), i = b + d:  T_ib = -T_ii * sum_{k=b}^{i-1} A_ik T_kb,
  // level by level on the fp32 matrix cores (wave b handles block (b + d, b))
#pragma unroll 1
  for (int d = 1; d < 4; ++d) {
    if (w < 4 - d) {
      const int b = w, i = b + d;
      f32x4 X = {0.f, 0.f, 0.f, 0.f};
      for (int kb = b; kb < i; ++kb) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          X = mfma_f32(sm.u.s.A[16 * i + l16][16 * kb + 4 * ks + g4],
                       sm.u.s.T[16 * kb + 4 * ks + g4][16 * b + l16], X);
      }
      // X in the C layout feeds the next product as B with K order {4g + ks}
      f32x4 Y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) Y = mfma_f32(-sm.u.s.T[16 * i + l16][16 * i + 4 * g4 + ks], X[ks], Y);
#pragma unroll
      for (int r = 0; r < 4; ++r) sm.u.s.T[16 * i + 4 * g4 + r][16 * b + l16] = Y[r];
    }
    __syncthreads();
  }

  // ---- operands from T: T diag(beta) as hi + lo, -T diag(beta gam) ---------------------------
  bf16x8 hv[2], lv[2], gv[2];
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int pc = tid + kThreads * it;         // 512 pieces of 8 elements
    const int r = pc >> 3, s0 = (pc & 7) * 8;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float tb = sm.u.s.T[r][s0 + e] * sm.beta[s0 + e];
      const bf16 hh = to_bf16(tb);
      hv[it][e] = hh;
      lv[it][e] = to_bf16(tb - (float)hh);
      gv[it][e] = to_bf16(-tb * sm.gam[s0 + e]);
    }
  }
  __syncthreads();   // T is read; its space now holds the bf16 operands
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int pc = tid + kThreads * it;
    const int r = pc >> 3, s0 = (pc & 7) * 8;
    *reinterpret_cast<bf16x8*>(&sm.u.o.Th[r][s0]) = hv[it];
    *reinterpret_cast<bf16x8*>(&sm.u.o.Tl[r][s0]) = lv[it];
    *reinterpret_cast<bf16x8*>(&sm.u.o.Tbg[r][s0]) = gv[it];
  }
  __syncthreads();

  // ---- U~ = T diag(beta) V (hi + lo); wave w: column tiles 2w, 2w+1 -------------------------
  f32x4* Uw = reinterpret_cast<f32x4*>(wsh + kWsU);
#pragma unroll
  for (int cc = 0; cc < 2; ++cc) {
    const int ct = 2 * w + cc;
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks <= rt / 2; ++ks) {   // T is lower triangular
        const bf16x8 bv = lds8(&sm.VT[16 * ct + l16][32 * ks + 8 * g4]);
        acc = mfma16x16x32(lds8(&sm.u.o.Th[16 * rt + l16][32 * ks + 8 * g4]), bv, acc);
        acc = mfma16x16x32(lds8(&sm.u.o.Tl[16 * rt + l16][32 * ks + 8 * g4]), bv, acc);
      }
      Uw[(ct * 4 + rt) * 64 + lane] = acc;      // the state pass loads this lane's tile as is
    }
  }
  __syncthreads();   // V^T is read; its space now stages -W

  // ---- -W = (-T diag(beta gam)) K; wave w: column tiles 2w, 2w+1 ----------------------------
  bf16(*Wst)[kRowPad] = reinterpret_cast<bf16(*)[kRowPad]>(&sm.VT[0][0]);
#pragma unroll
  for (int cc = 0; cc < 2; ++cc) {
    const int ct = 2 * w + cc;
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks <= rt / 2; ++ks)
        acc = mfma16x16x32(lds8(&sm.u.o.Tbg[16 * rt + l16][32 * ks + 8 * g4]),
                           lds8(&sm.KT[16 * ct + l16][32 * ks + 8 * g4]), acc);
#pragma unroll
      for (int i = 0; i < 4; ++i) Wst[16 * rt + 4 * g4 + i][16 * ct + l16] = to_bf16(acc[i]);
    }
  }
  __syncthreads();
  bf16* Wg = reinterpret_cast<bf16*>(wsh + kWsW);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int pc = tid + kThreads * i;          // 1024 pieces of 8
    const int row = pc >> 4, cb = pc & 15;
    *reinterpret_cast<bf16x8*>(Wg + row * kD + cb * 8) = lds8(&Wst[row][cb * 8]);
  }
}

// ------------------------------------------------------------------------------------------
// state_kernel: one workgroup per (sequence, V head, 64 * NT value rows)
// ------------------------------------------------------------------------------------------
// LDS image of one chunk's shared operands. Rows are unpadded; 16-byte pieces are XOR
// swizzled so the operand reads below hit distinct banks: in a 256-byte row (W, Q) piece p
// of row r sits at slot p ^ (r & 15); in a 128-byte row (K^T, P) at slot p ^ ((r >> 1) & 7).
struct StateBuf {
  bf16 W[kC * kD];      // -W
  bf16 Q[kC * kD];
  bf16 KT[kD * kC];
  bf16 P[kC * kC];
  f32x4 U[4][4][64];    // U~ of the 64 value rows: [wave's column tile][row tile][lane]
  float gam[kC];
  float lam[kC];
};

__device__ __forceinline__ int sw256(int r, int piece) { return r * 128 + ((piece ^ (r & 15)) << 3); }
__device__ __forceinline__ int sw128(int r, int piece) { return r * 64 + ((piece ^ ((r >> 1) & 7)) << 3); }

// A operand, K order {4g..4g+3, 16+4g..16+4g+3} + k0, from a swizzled 256-byte-row image
__device__ __forceinline__ bf16x8 perm256(const bf16* img, int r, int k0, int g4) {
  const int k1 = k0 + 4 * g4, k2 = k1 + 16;
  return join8(lds4(img + sw256(r, k1 >> 3) + (k1 & 7)), lds4(img + sw256(r, k2 >> 3) + (k2 & 7)));
}
__device__ __forceinline__ bf16x8 perm128(const bf16* img, int r, int k0, int g4) {
  const int k1 = k0 + 4 * g4, k2 = k1 + 16;
  return join8(lds4(img + sw128(r, k1 >> 3) + (k1 & 7)), lds4(img + sw128(r, k2 >> 3) + (k2 & 7)));
}

// Direct global -> LDS loads of chunk c's operands into `buf`; every wave issues its share,
// in four parts (part 0..3) so they can be spread over the math of the current chunk.
struct DmaSrc {
  const bf16* W;
  const bf16* P;
  const float* G;
  const bf16* K;
  const f32x4* U;
  int t0, nv;
};

__device__ __forceinline__ DmaSrc dma_src(const PrefillArgs& a, int c, int t0, int nv, int h, int j,
                                          int dvb, int w) {
  const uint8_t* head = a.ws_heads + ((size_t)c * a.h_v + h) * kWsHead;
  DmaSrc d;
  d.W = reinterpret_cast<const bf16*>(head + kWsW);
  d.P = reinterpret_cast<const bf16*>(head + kWsP);
  d.G = reinterpret_cast<const float*>(head + kWsGam);
  d.U = reinterpret_cast<const f32x4*>(head + kWsU) + (size_t)(4 * dvb + w) * 4 * 64;
  d.K = reinterpret_cast<const bf16*>(a.ws_kt + ((size_t)c * a.h_qk + j) * kWsKT);
  d.t0 = t0;
  d.nv = nv;
  return d;
}

__device__ __forceinline__ void dma_part(const PrefillArgs& a, const DmaSrc& d, StateBuf& buf, int part,
                                         int j, int w, int lane) {
  // part i: W and Q rows of instruction i, K^T rows of instruction i, P (parts 0-1) or U~
  // (parts 2-3), and gam/lam with part 0
  const int i = part;
  {
    // 256-byte rows: one instruction fills 4 rows
    const int r = 4 * (4 * w + i) + (lane >> 4), slot = lane & 15, piece = slot ^ (r & 15);
    __builtin_amdgcn_global_load_lds(d.W + r * kD + piece * 8, (lds_void_ptr)&buf.W[16 * kD * w + 4 * kD * i], 16, 0, 0);
    const int rq = min(r, d.nv - 1);   // rows past the chunk end only feed unstored outputs
    __builtin_amdgcn_global_load_lds(a.q + ((size_t)(d.t0 + rq) * a.h_qk + j) * kD + piece * 8,
                                     (lds_void_ptr)&buf.Q[16 * kD * w + 4 * kD * i], 16, 0, 0);
    // 128-byte rows: one instruction fills 8 rows
    const int rk = 8 * (4 * w + i) + (lane >> 3), sk = lane & 7, pk = sk ^ ((rk >> 1) & 7);
    __builtin_amdgcn_global_load_lds(d.K + rk * kC + pk * 8, (lds_void_ptr)&buf.KT[32 * kC * w + 8 * kC * i], 16, 0, 0);
  }
  if (i < 2) {
    const int rp = 8 * (2 * w + i) + (lane >> 3), sp = lane & 7, pp = sp ^ ((rp >> 1) & 7);
    __builtin_amdgcn_global_load_lds(d.P + rp * kC + pp * 8, (lds_void_ptr)&buf.P[16 * kC * w + 8 * kC * i], 16, 0, 0);
  } else {
    // this wave's U~ column tile: 4 row tiles of 64 lanes x 16 bytes, already in lane order
    const int rt = 2 * (i - 2);
    __builtin_amdgcn_global_load_lds(d.U + rt * 64 + lane, (lds_void_ptr)&buf.U[w][rt][0], 16, 0, 0);
    __builtin_amdgcn_global_load_lds(d.U + (rt + 1) * 64 + lane, (lds_void_ptr)&buf.U[w][rt + 1][0], 16, 0, 0);
  }
  if (i == 0 && w == 0 && lane < 32)   // gam then lam, 512 contiguous bytes
    __builtin_amdgcn_global_load_lds(d.G + lane * 4, (lds_void_ptr)&buf.gam[0], 16, 0, 0);
}

__device__ __forceinline__ void dma_chunk(const PrefillArgs& a, StateBuf& buf, int c, int t0, int nv,
                                          int h, int j, int dvb, int w, int lane) {
  const DmaSrc d = dma_src(a, c, t0, nv, h, j, dvb, w);
#pragma unroll
  for (int part = 0; part < 4; ++part) dma_part(a, d, buf, part, j, w, lane);
}

// One chunk of the state pass for this wave's 16 value rows, reading `B` and streaming the
// next chunk into `Bn`. The outputs are formed transposed (value rows x tokens) so each lane
// ends up with four adjacent value rows of one token: 8-byte stores.
__device__ __forceinline__ void state_chunk(const PrefillArgs& a, const StateBuf& B, StateBuf& Bn,
                                            f32x4 (&St)[8], int c, int t0, int nv, int t_seq1,
                                            bool has_next, int h, int j, int dvb, int col0, int w,
                                            int lane) {
  const int g4 = lane >> 4;
  const int l16 = lane & 15;
  __builtin_amdgcn_s_waitcnt(0);   // this chunk's direct loads have landed (own share)
  __syncthreads();                 // ... everyone's; and the other buffer is free
  DmaSrc dn;
  if (has_next) dn = dma_src(a, c + 1, t0 + kC, min(kC, t_seq1 - t0 - kC), h, j, dvb, w);

  // S^T as bf16 operands (B operand of U, A operand of the transposed read-out)
  bf16x8 Sb[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) Sb[ks] = pack8(St[2 * ks], St[2 * ks + 1]);
  // U = U~ - W S^T  (token rows x value rows);  QSt = (Q S^T)^T (value rows x tokens)
  f32x4 U[4], QSt[4];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    U[rt] = B.U[w][rt][lane];
    QSt[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    bf16x8 aw[4], aq[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      aw[rt] = perm256(B.W, 16 * rt + l16, 32 * ks, g4);
      aq[rt] = perm256(B.Q, 16 * rt + l16, 32 * ks, g4);
    }
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      U[rt] = mfma16x16x32(aw[rt], Sb[ks], U[rt]);
      QSt[rt] = mfma16x16x32(Sb[ks], aq[rt], QSt[rt]);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (has_next) dma_part(a, dn, Bn, ks, j, w, lane);   // spread the next chunk's loads
    __builtin_amdgcn_sched_barrier(0);
  }
  // U as bf16 for the read-out; the decayed U as a hi + lo pair for the state update
  bf16x8 Ub[2], Bh[2], Bl[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    Ub[ks] = pack8(U[2 * ks], U[2 * ks + 1]);
    f32x4 hi[2], lo[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float u = U[2 * ks + hh][i] * B.lam[16 * (2 * ks + hh) + 4 * g4 + i];
        const float uh = (float)to_bf16(u);
        hi[hh][i] = uh;
        lo[hh][i] = u - uh;
      }
    Bh[ks] = pack8(hi[0], hi[1]);
    Bl[ks] = pack8(lo[0], lo[1]);
  }
  // O^T = scale gam (Q S^T)^T + (P U)^T = ... + U^T P^T, stored as 8-byte pieces
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    f32x4 acc = QSt[nt] * (a.scale * B.gam[16 * nt + l16]);
#pragma unroll
    for (int ks = 0; ks <= nt / 2; ++ks) acc = mfma16x16x32(Ub[ks], perm128(B.P, 16 * nt + l16, 32 * ks, g4), acc);
    const int tok = 16 * nt + l16;
    if (tok < nv) {
      bf16x4 ov;
      ov[0] = to_bf16(acc[0]); ov[1] = to_bf16(acc[1]); ov[2] = to_bf16(acc[2]); ov[3] = to_bf16(acc[3]);
      *reinterpret_cast<bf16x4*>(a.o + ((size_t)(t0 + tok) * a.h_v + h) * kD + col0 + 4 * g4) = ov;
    }
  }
  // S^T <- gam_C S^T + K^T (diag(gam_C / gam) U)
  const float gC = B.gam[kC - 1];
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) {
    const bf16x8 ak0 = perm128(B.KT, 16 * mt + l16, 0, g4);
    const bf16x8 ak1 = perm128(B.KT, 16 * mt + l16, 32, g4);
    f32x4 s = St[mt] * gC;
    s = mfma16x16x32(ak0, Bh[0], s);
    s = mfma16x16x32(ak0, Bl[0], s);
    s = mfma16x16x32(ak1, Bh[1], s);
    St[mt] = mfma16x16x32(ak1, Bl[1], s);
  }
}

// One workgroup per (sequence, V head, 64 value rows); wave w owns 16 of them.
__global__ __launch_bounds__(kThreads) void state_kernel(PrefillArgs a) {
  // two separately declared buffers so each half of the loop reads one while the other fills
  __shared__ StateBuf buf0;
  __shared__ StateBuf buf1;
  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int g4 = lane >> 4;
  const int l16 = lane & 15;

  // the two value-row blocks of one (sequence, V head) sit on the same XCD (blockIdx % 8)
  const int bid = blockIdx.x;
  const int grp = bid / 16, rem = bid % 16;
  const int pair = grp * 8 + rem % 8;
  const int dvb = rem / 8;
  if (pair >= a.num_seqs * a.h_v) return;
  const int n = pair / a.h_v, h = pair % a.h_v;
  const int j = h / a.group;
  const int col0 = dvb * 64 + 16 * w;              // this wave's first value row
  const int col = col0 + l16;                      // this lane's value row in S
  const int t_seq0 = a.cu[n], t_seq1 = a.cu[n + 1];
  const int n_chunks = (t_seq1 - t_seq0 + kC - 1) / kC;
  const int c_begin = first_chunk(a.cu, n, lane);
  const size_t state_off = (((size_t)n * a.h_v + h) * kD + col) * kD;

  // St[mt][i] = S[col][16 mt + 4 g4 + i]
  f32x4 St[8];
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) {
    if (a.s0) St[mt] = *reinterpret_cast<const f32x4*>(a.s0 + state_off + 16 * mt + 4 * g4);
    else St[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  if (n_chunks > 0) dma_chunk(a, buf0, c_begin, t_seq0, min(kC, t_seq1 - t_seq0), h, j, dvb, w, lane);
  for (int ci = 0; ci < n_chunks; ci += 2) {
    const int t0 = t_seq0 + ci * kC;
    state_chunk(a, buf0, buf1, St, c_begin + ci, t0, min(kC, t_seq1 - t0), t_seq1,
                ci + 1 < n_chunks, h, j, dvb, col0, w, lane);
    if (ci + 1 < n_chunks) {
      const int t1 = t0 + kC;
      state_chunk(a, buf1, buf0, St, c_begin + ci + 1, t1, min(kC, t_seq1 - t1), t_seq1,
                  ci + 2 < n_chunks, h, j, dvb, col0, w, lane);
    }
  }

  if (a.s_final) {
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
      *reinterpret_cast<f32x4*>(a.s_final + state_off + 16 * mt + 4 * g4) = St[mt];
  }
}

}  // namespace

size_t chunk_prefill_workspace_bytes(int total_tokens, int num_seqs, int h_qk, int h_v) {
  const size_t nc = max_chunks(total_tokens, num_seqs);
  return nc * (size_t)h_v * kWsHead + nc * (size_t)h_qk * kWsKT;
}

hipError_t launch_chunk_prefill(const void* q, const void* k, const void* v, const float* g,
                                const float* beta, const int32_t* cu_seqlens, int num_seqs,
                                int total_tokens, int h_qk, int h_v, float scale,
                                const float* s0, float* s_final, void* o, void* workspace,
                                hipStream_t stream) {
  PrefillArgs a;
  a.q = static_cast<const bf16*>(q);
  a.k = static_cast<const bf16*>(k);
  a.v = static_cast<const bf16*>(v);
  a.g = g;
  a.beta = beta;
  a.cu = cu_seqlens;
  a.s0 = s0;
  a.s_final = s_final;
  a.o = static_cast<bf16*>(o);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  const size_t nc = max_chunks(total_tokens, num_seqs);
  a.ws_heads = ws;
  a.ws_kt = ws + nc * (size_t)h_v * kWsHead;
  a.num_seqs = num_seqs;
  a.h_qk = h_qk;
  a.h_v = h_v;
  a.group = h_v / h_qk;
  a.n_chunks_max = (int)nc;
  a.scale = scale;

  if (total_tokens > 0) {
    const size_t pairs = nc * (size_t)h_qk;
    const size_t prep_blocks = (pairs + 7) / 8 * 8 * (size_t)a.group;
    hipLaunchKernelGGL(prep_kernel, dim3((unsigned)prep_blocks), dim3(kThreads), 0, stream, a);
  }
  const size_t pairs = (size_t)num_seqs * h_v;
  const size_t state_blocks = (pairs + 7) / 8 * 16;
  hipLaunchKernelGGL(state_kernel, dim3((unsigned)state_blocks), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace gdn
