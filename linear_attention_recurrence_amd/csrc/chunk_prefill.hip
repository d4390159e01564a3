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
//    cores), then -W on the bf16 matrix cores. Writes -W, P^T with
//    P = scale (Q K^T o Gam o lower-incl), gam, gam_C / gam, and T diag(beta) as a hi + lo
//    bf16 pair in the operand order of the state pass.
//  * state_kernel, walking each sequence's chunks in order with S in fp32 registers, 16 or
//    32 value rows per wave (value rows evolve independently), one to eight workgroups per
//    (sequence, V head) depending on how many heads there are. Per chunk:
//    U~ = T diag(beta) V (by a loading wave when there is one), U = U~ - W S^T,
//    (Q S^T)^T, O^T = scale gam (Q S^T)^T + U^T P^T and the state update on the bf16
//    matrix cores. The next chunk's -W, Q, K, P^T, T diag(beta) and values stream into LDS
//    with direct global-to-LDS loads while the current chunk computes.
//
// Precision: every product keeps one exact bf16 operand (K, Q, V as given); T diag(beta)
// and the decayed U that feeds the state are split into hi + lo bf16 pairs so they keep
// ~16 mantissa bits; S stays in fp32 and is rounded to bf16 only as a product operand.
//
// Matrix-core layout (v_mfma_f32_16x16x32_bf16): lane l holds A[l%16][8*(l/16)+s],
// B[8*(l/16)+s][l%16] for s = 0..7, and C[4*(l/16)+i][l%16] for i = 0..3. A product is
// unchanged when the same permutation is applied to the K index of A and B, so a
// C-layout accumulator pair covering K rows k0..k0+15 and k0+16..k0+31 is a valid
// operand once its partner reads K entries {4g..4g+3, 16+4g..16+4g+3} (g = l/16); the
// products below use that K order. The fp32 16x16x4 instruction has lane l holding
// A[l%16][l/16], B[l/16][l%16] and the same C layout.
//
// Operands whose K index runs down the rows of a row-major LDS image (K and V contracted
// over tokens, P^T) are read with ds_read_b64_tr_b16: within each group of 16 lanes,
// when lane i points at row k0 + i/4, columns n0 + 4(i%4) .. +3, lane j receives rows
// k0 .. k0+3 of column n0 + j.
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {
namespace {

constexpr int kC = 64;          // chunk length
constexpr int kD = 128;         // head dim
constexpr int kThreads = 256;
constexpr size_t kStateCus = 256;   // compute units of the chip
constexpr int kTokPad = kC + 8;     // [token][token] bf16 LDS rows
constexpr int kTokPad4 = kC + 4;    // [token][token] bf16 LDS rows, tight
constexpr int kF32Pad = kC + 4;     // [token][token] fp32 LDS rows

// Workspace: one block per (chunk, V head).
constexpr size_t kWsW = 0;                          // bf16 [64][128]: -W
constexpr size_t kWsP = kWsW + kC * kD * 2;         // bf16 [64][64]: P^T
constexpr size_t kWsGam = kWsP + kC * kC * 2;       // fp32 [64]: gam_r
constexpr size_t kWsLam = kWsGam + kC * 4;          // fp32 [64]: gam_C / gam_r
constexpr size_t kWsG = kWsLam + kC * 4;            // fp32 [64]: G_r (the log-decay prefix sums)
constexpr int kTbFrags = 6;                         // nonzero T diag(beta) operand fragments
constexpr size_t kWsTh = kWsGam + 1024;             // bf16 T diag(beta), hi, operand order (below)
constexpr size_t kWsTl = kWsTh + kTbFrags * 1024;  // bf16 T diag(beta), lo, operand order
constexpr size_t kWsTbg = kWsTl + kTbFrags * 1024; // bf16 -T diag(beta gam), operand order
constexpr size_t kWsHead = kWsTbg + kTbFrags * 1024; // 44032 bytes

// Which parts a block holds depends on how the state pass runs. With few heads (a loading
// wave per workgroup) prep writes -W and P^T; with many heads the state pass forms both on
// chip from Q, K and -T diag(beta gam) (bit for bit the same values), so prep writes
// -T diag(beta gam) instead and reads no Q. The decay factors and T diag(beta) are always
// written.

// T diag(beta) is stored in the order the state pass reads it as the A operand of
// U~ = T diag(beta) V: the fragment of row tile rt and K-step ks holds, for lane
// l = l16 + 16 g4, the eight entries T[16 rt + l16][32 ks + 16 h + 4 g4 + i] (h, i = 0, 1 /
// 0..3, element 4 h + i), so one 16-byte read per lane fetches an operand. T is lower
// triangular, so the fragments with ks > rt / 2 are zero and are not stored: the six others
// are numbered 0, 1 (rt = 0, 1), then 2 + 2 (rt - 2) + ks.
__device__ __forceinline__ constexpr int tb_frag(int rt, int ks) { return rt < 2 ? rt : 2 * rt - 2 + ks; }
// Element offset of entry (r, s) for s a multiple of 4 (r >= s rounded down to the fragment,
// i.e. a stored fragment).
__device__ __forceinline__ int tb_frag_off(int r, int s) {
  return (tb_frag(r >> 4, s >> 5) * 64 + (r & 15) + 16 * ((s >> 2) & 3)) * 8 + 4 * ((s >> 4) & 1);
}

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
  uint8_t* ws;              // per (chunk, V head) blocks
  int num_seqs, h_qk, h_v, group, n_chunks_max;
  float scale;
};

typedef __attribute__((address_space(3))) void* lds_void_ptr;
typedef __bf16 bf16x4_gcc __attribute__((__vector_size__(8)));
typedef __attribute__((address_space(3))) bf16x4_gcc* lds_bf16x4_ptr;

__device__ __forceinline__ bf16x8 lds8(const bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }
__device__ __forceinline__ bf16x4 lds4(const bf16* p) { return *reinterpret_cast<const bf16x4*>(p); }
__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ bf16x4 lds_tr4(const bf16* p) {
  const bf16x4_gcc r = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_ptr)(p));
  return __builtin_bit_cast(bf16x4, r);
}

// ---- LDS images: unpadded rows, 16-byte pieces XOR-swizzled so that the row reads, the
// permuted-K reads and the transpose reads below all hit distinct banks.
// 256-byte rows ([64][128] bf16): piece p of row r at slot p ^ 2(r & 7) ^ ((r >> 3) & 1).
__device__ __forceinline__ int sw256(int r, int col) {
  const int p = col >> 3;
  return r * 128 + ((p ^ ((r & 7) << 1) ^ ((r >> 3) & 1)) << 3) + (col & 7);
}
// 128-byte rows ([R][64] bf16): piece p of row r at slot p ^ 2((r >> 1) & 3).
__device__ __forceinline__ int sw128(int r, int col) {
  const int p = col >> 3;
  return r * 64 + ((p ^ (((r >> 1) & 3) << 1)) << 3) + (col & 7);
}
// Operand in the permuted K order with K along the image row r (the lane's M/N index).
__device__ __forceinline__ bf16x8 perm_row256(const bf16* img, int r, int k0, int g4) {
  return join8(lds4(img + sw256(r, k0 + 4 * g4)), lds4(img + sw256(r, k0 + 16 + 4 * g4)));
}
__device__ __forceinline__ bf16x8 perm_rowpad(const bf16* rowp, int k0, int g4) {
  return join8(lds4(rowp + k0 + 4 * g4), lds4(rowp + k0 + 16 + 4 * g4));
}
// Operand in the permuted K order with K down the image columns (transpose reads):
// lane (l16, g4) gets image rows {k0 + 4 g4 .. +3, k0 + 16 + 4 g4 .. +3} of column n0 + l16.
__device__ __forceinline__ bf16x8 perm_tr256(const bf16* img, int k0, int n0, int g4, int l16) {
  const int r = k0 + 4 * g4 + (l16 >> 2), c = n0 + 4 * (l16 & 3);
  return join8(lds_tr4(img + sw256(r, c)), lds_tr4(img + sw256(r + 16, c)));
}
__device__ __forceinline__ bf16x8 perm_tr128(const bf16* img, int k0, int n0, int g4, int l16) {
  const int r = k0 + 4 * g4 + (l16 >> 2), c = n0 + 4 * (l16 & 3);
  return join8(lds_tr4(img + sw128(r, c)), lds_tr4(img + sw128(r + 16, c)));
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

// Direct global -> LDS copy of rows of a [rows][128] bf16 matrix (256-byte rows) into a
// swizzled image: instruction i of wave w fills image rows 4(4w + i) .. +3. Image row r comes
// from source row min(r, nv - 1) at `src + row * stride`: rows past the chunk end repeat the
// last valid row and only feed results that are discarded or multiplied by zero.
__device__ __forceinline__ void dma_rows256(const bf16* src, size_t stride, int nv, bf16* img,
                                            int i, int w, int lane) {
  const int r = 4 * (4 * w + i) + (lane >> 4);
  const int slot = lane & 15;
  const int piece = slot ^ ((r & 7) << 1) ^ ((r >> 3) & 1);
  const int rs = min(r, nv - 1);
  __builtin_amdgcn_global_load_lds(src + (size_t)rs * stride + piece * 8,
                                   (lds_void_ptr)(img + (16 * w + 4 * i) * kD), 16, 0, 0);
}
// Same for a contiguous [rows][64] bf16 matrix (128-byte rows): instruction i of wave w
// fills image rows 8(nw w + i) .. +7.
__device__ __forceinline__ void dma_rows128(const bf16* src, bf16* img, int i, int w, int nw, int lane) {
  const int r = 8 * (nw * w + i) + (lane >> 3);
  const int slot = lane & 7;
  const int piece = slot ^ (((r >> 1) & 3) << 1);
  __builtin_amdgcn_global_load_lds(src + r * kC + piece * 8, (lds_void_ptr)(img + 8 * (nw * w + i) * kC), 16, 0, 0);
}

// ------------------------------------------------------------------------------------------
// prep_kernel: one workgroup per (chunk, V head)
// ------------------------------------------------------------------------------------------
struct PrepSmem {
  bf16 K[kC * kD];              // swizzled 256-byte rows
  union {
    bf16 Q[kC * kD];            // loads and Q K^T only; then A with T; then -T diag(beta gam)
    float A[kC][kF32Pad];       // A in the strict lower triangle, T transposed in the upper one
    bf16 Tbg[kC][kTokPad];
  } r1;
  alignas(16) float G[kC];
  alignas(16) float beta[kC];
  alignas(16) float gam[kC];
};

// Lower 16 x 16 tile t (0..9, row-major over the lower triangle) of a 64 x 64 product.
__device__ __forceinline__ constexpr int tile_row(int t) { return t < 1 ? 0 : t < 3 ? 1 : t < 6 ? 2 : 3; }
__device__ __forceinline__ constexpr int tile_col(int t) { return t - tile_row(t) * (tile_row(t) + 1) / 2; }

// Tiles FIRST, FIRST + STEP, ... (below 10) of K K^T (ISQ = false) or Q K^T (ISQ = true).
template <bool ISQ, int FIRST, int STEP>
__device__ __forceinline__ void gram_tiles(const PrepSmem& sm, f32x4 (&acc)[5], int g4, int l16) {
  const bf16* Am = ISQ ? sm.r1.Q : sm.K;
#pragma unroll
  for (int jj = 0; jj < 5; ++jj) {
    const int t = FIRST + STEP * jj;
    if (t >= 10) break;
    const int rt = tile_row(t), ct = tile_col(t);
    acc[jj] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      acc[jj] = mfma16x16x32(lds8(Am + sw256(16 * rt + l16, 32 * ks + 8 * g4)),
                             lds8(sm.K + sw256(16 * ct + l16, 32 * ks + 8 * g4)), acc[jj]);
  }
}

// Masked and decayed tiles: A = strictly-lower(beta_r Gam_rs (K K^T)_rs) into LDS, or
// P = scale lower-incl(Gam_rs (Q K^T)_rs), stored transposed to the workspace (8 bytes per
// lane: four adjacent query tokens of one key token).
template <bool ISQ, int FIRST, int STEP>
__device__ __forceinline__ void gram_epilogue(PrepSmem& sm, const f32x4 (&acc)[5], bf16* Pt, float scale,
                                              int g4, int l16) {
  f32x4 Gr[5], Br[5];
  float Gs[5];
#pragma unroll
  for (int jj = 0; jj < 5; ++jj) {   // every LDS read first: the stores into A would order them
    const int t = FIRST + STEP * jj;
    if (t >= 10) break;
    const int rt = tile_row(t), ct = tile_col(t);
    Gr[jj] = *reinterpret_cast<const f32x4*>(&sm.G[16 * rt + 4 * g4]);
    if (!ISQ) Br[jj] = *reinterpret_cast<const f32x4*>(&sm.beta[16 * rt + 4 * g4]);
    Gs[jj] = sm.G[16 * ct + l16];
  }
#pragma unroll
  for (int jj = 0; jj < 5; ++jj) {
    const int t = FIRST + STEP * jj;
    if (t >= 10) break;
    const int rt = tile_row(t), ct = tile_col(t);
    const int s = 16 * ct + l16;
    f32x4 val;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * rt + 4 * g4 + i;
      // G is nonincreasing (every g <= 0 by contract), but the prefix sums above are added
      // in a different order for each token, so G_r - G_s (s <= r) may round to a tiny
      // positive value; the bound keeps every in-chunk ratio at most 1, as it is exactly.
      const float decay = __expf(fminf(Gr[jj][i] - Gs[jj], 0.f));
      if (ISQ) val[i] = s <= r ? scale * decay * acc[jj][i] : 0.f;
      else sm.r1.A[r][s] = s < r ? Br[jj][i] * decay * acc[jj][i] : 0.f;
    }
    if (ISQ) {
      bf16x4 pv;
      pv[0] = to_bf16(val[0]); pv[1] = to_bf16(val[1]); pv[2] = to_bf16(val[2]); pv[3] = to_bf16(val[3]);
      *reinterpret_cast<bf16x4*>(Pt + s * kC + 16 * rt + 4 * g4) = pv;
    }
  }
}

// FULL: write -W and P^T (few heads); otherwise -T diag(beta gam) for the state pass to
// form them (see the workspace layout above).
template <bool FULL>
__global__ __launch_bounds__(kThreads, 4) void prep_kernel(PrefillArgs a) {
  __shared__ PrepSmem sm;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, uniform
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
  uint8_t* wsh = a.ws + ((size_t)c * a.h_v + h) * kWsHead;

  // ---- loads: K, Q rows straight into swizzled LDS images; g, beta ----
  const size_t qk_stride = (size_t)a.h_qk * kD;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    dma_rows256(a.k + (size_t)t0 * qk_stride + (size_t)j * kD, qk_stride, nv, sm.K, i, w, lane);
    if (FULL) dma_rows256(a.q + (size_t)t0 * qk_stride + (size_t)j * kD, qk_stride, nv, sm.r1.Q, i, w, lane);
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
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

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
    reinterpret_cast<float*>(wsh + kWsG)[lane] = x;
  }

  // ---- K K^T and Q K^T: the 10 lower tiles of each, held in registers. With FULL waves
  // 0, 1 take K K^T and waves 2, 3 Q K^T, alternate tiles each; otherwise the four waves
  // share K K^T (tiles w, w + 4, w + 8) ----
  f32x4 acc[5];
  if (FULL) {
    if (w == 0) gram_tiles<false, 0, 2>(sm, acc, g4, l16);
    else if (w == 1) gram_tiles<false, 1, 2>(sm, acc, g4, l16);
    else if (w == 2) gram_tiles<true, 0, 2>(sm, acc, g4, l16);
    else gram_tiles<true, 1, 2>(sm, acc, g4, l16);
  } else {
    if (w == 0) gram_tiles<false, 0, 4>(sm, acc, g4, l16);
    else if (w == 1) gram_tiles<false, 1, 4>(sm, acc, g4, l16);
    else if (w == 2) gram_tiles<false, 2, 4>(sm, acc, g4, l16);
    else gram_tiles<false, 3, 4>(sm, acc, g4, l16);
  }
  __syncthreads();   // Q is consumed (its space becomes A) and G is ready
  bf16* Pt = reinterpret_cast<bf16*>(wsh + kWsP);
  if (FULL) {
    if (w == 0) gram_epilogue<false, 0, 2>(sm, acc, Pt, a.scale, g4, l16);
    else if (w == 1) gram_epilogue<false, 1, 2>(sm, acc, Pt, a.scale, g4, l16);
    else if (w == 2) gram_epilogue<true, 0, 2>(sm, acc, Pt, a.scale, g4, l16);
    else gram_epilogue<true, 1, 2>(sm, acc, Pt, a.scale, g4, l16);
  } else {
    if (w == 0) gram_epilogue<false, 0, 4>(sm, acc, Pt, a.scale, g4, l16);
    else if (w == 1) gram_epilogue<false, 1, 4>(sm, acc, Pt, a.scale, g4, l16);
    else if (w == 2) gram_epilogue<false, 2, 4>(sm, acc, Pt, a.scale, g4, l16);
    else gram_epilogue<false, 3, 4>(sm, acc, Pt, a.scale, g4, l16);
  }
  if (FULL && tid < 128) {   // the strictly upper tiles of P that the read-out's 32-token K-steps see
    const int rt = (tid >> 6) * 2, ln = tid & 63;
    *reinterpret_cast<bf16x4*>(Pt + (16 * (rt + 1) + (ln & 15)) * kC + 16 * rt + 4 * (ln >> 4)) = bf16x4{};
  }
  __syncthreads();

  // ---- T = (I + A)^-1 --------------------------------------------------------------------
  // T is unit lower triangular and A strictly lower triangular, so they share one array: A
  // keeps the strict lower triangle and T[r][c] (r >= c) goes to the mirror position [c][r].
  float (&M)[kC][kF32Pad] = sm.r1.A;
  // diagonal 16 x 16 blocks: wave b inverts block b, lane = column, one column of A at a time
  if (lane < 16) {
    const int b0 = 16 * w, col = lane;
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {   // row r of the block: x_r = e_r - sum_{m < r} A_rm x_m
      f32x4 ar[4];
#pragma unroll
      for (int q = 0; q < (r + 3) / 4; ++q) ar[q] = *reinterpret_cast<const f32x4*>(&M[b0 + r][b0 + 4 * q]);
      float acc = (r == col) ? 1.f : 0.f;
#pragma unroll
      for (int m = 0; m < r; ++m) acc -= ar[m >> 2][m & 3] * x[m];
      x[r] = acc;
      if (r >= col) M[b0 + col][b0 + r] = acc;
    }
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
        for (int ks = 0; ks < 4; ++ks) {
          // T[16 kb + 4 ks + g4][16 b + l16]; within the diagonal block only its lower part
          const float t = M[16 * b + l16][16 * kb + 4 * ks + g4];
          X = mfma_f32(M[16 * i + l16][16 * kb + 4 * ks + g4], (kb > b || 4 * ks + g4 >= l16) ? t : 0.f, X);
        }
      }
      // X in the C layout feeds the next product as B with K order {4g + ks}
      f32x4 Y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const float t = M[16 * i + 4 * g4 + ks][16 * i + l16];   // T[16 i + l16][16 i + 4 g4 + ks]
        Y = mfma_f32(4 * g4 + ks <= l16 ? -t : 0.f, X[ks], Y);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) M[16 * b + l16][16 * i + 4 * g4 + r] = Y[r];
    }
    __syncthreads();
  }

  // ---- operands from T: T diag(beta) as a hi + lo bf16 pair, straight to the workspace
  // in operand order, and -T diag(beta gam) into A's space (A is consumed) or, without
  // FULL, to the workspace in operand order --------------------------------------------------
  // Lane = row r; wave w takes columns s0 = 8 (w + 4 it) .. + 7, so the reads of T's
  // mirrored entries M[s][r] hit distinct banks.
  bf16* Thg = reinterpret_cast<bf16*>(wsh + kWsTh);
  bf16* Tlg = reinterpret_cast<bf16*>(wsh + kWsTl);
  bf16* Tbgg = reinterpret_cast<bf16*>(wsh + kWsTbg);
  bf16x8 hv[2], lv[2], gv[2];
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int r = lane, s0 = 8 * (w + 4 * it);
    float tv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) tv[e] = M[s0 + e][r];
    const f32x4 bv[2] = {*reinterpret_cast<const f32x4*>(&sm.beta[s0]), *reinterpret_cast<const f32x4*>(&sm.beta[s0 + 4])};
    const f32x4 gm[2] = {*reinterpret_cast<const f32x4*>(&sm.gam[s0]), *reinterpret_cast<const f32x4*>(&sm.gam[s0 + 4])};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      // T is lower triangular; the mirror of its strict upper part holds A
      const float tb = (s0 + e <= r) ? tv[e] * bv[e >> 2][e & 3] : 0.f;
      const bf16 hh = to_bf16(tb);
      hv[it][e] = hh;
      lv[it][e] = to_bf16(tb - (float)hh);
      gv[it][e] = to_bf16(-tb * gm[e >> 2][e & 3]);
    }
  }
  __syncthreads();   // T is read; its space takes -T diag(beta gam)
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int r = lane, s0 = 8 * (w + 4 * it);
    if ((s0 >> 5) <= (r >> 4) / 2) {   // a stored (not all-zero) fragment
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int off = tb_frag_off(r, s0 + 4 * hh);
        *reinterpret_cast<bf16x4*>(Thg + off) = bf16x4{hv[it][4 * hh], hv[it][4 * hh + 1], hv[it][4 * hh + 2], hv[it][4 * hh + 3]};
        *reinterpret_cast<bf16x4*>(Tlg + off) = bf16x4{lv[it][4 * hh], lv[it][4 * hh + 1], lv[it][4 * hh + 2], lv[it][4 * hh + 3]};
        if (!FULL)
          *reinterpret_cast<bf16x4*>(Tbgg + off) = bf16x4{gv[it][4 * hh], gv[it][4 * hh + 1], gv[it][4 * hh + 2], gv[it][4 * hh + 3]};
      }
    }
    if (FULL) *reinterpret_cast<bf16x8*>(&sm.r1.Tbg[r][s0]) = gv[it];
  }
  if (!FULL) return;
  __syncthreads();

  // ---- -W = -T diag(beta gam) K; wave w: column tiles 2w, 2w+1. -W is formed transposed
  // (K^T times the transposed operand: the same registers with the roles swapped) so each
  // lane holds four adjacent columns of one -W row, stored as 8-byte pieces.
  bf16* Wg = reinterpret_cast<bf16*>(wsh + kWsW);
#pragma unroll
  for (int cc = 0; cc < 2; ++cc) {
    const int ct = 2 * w + cc;
    bf16x8 bk[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) bk[ks] = perm_tr256(sm.K, 32 * ks, 16 * ct, g4, l16);
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      f32x4 aw = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks <= rt / 2; ++ks)   // T is lower triangular
        aw = mfma16x16x32(bk[ks], perm_rowpad(&sm.r1.Tbg[16 * rt + l16][0], 32 * ks, g4), aw);
      bf16x4 wv;
      wv[0] = to_bf16(aw[0]); wv[1] = to_bf16(aw[1]); wv[2] = to_bf16(aw[2]); wv[3] = to_bf16(aw[3]);
      *reinterpret_cast<bf16x4*>(Wg + (16 * rt + l16) * kD + 16 * ct + 4 * g4) = wv;
    }
  }
}

// ------------------------------------------------------------------------------------------
// state_kernel<NW, NT, DW>: NW waves of NT 16-row value tiles each per workgroup, so
// 8 / (NW NT) workgroups per (sequence, V head), placed on one XCD. Every wave reads the
// chunk's shared operands (-W, Q, K, P^T) from LDS once for all of its tiles: NT = 2 would
// halve the LDS traffic per value row, NT = 1 halves the dependent work per wave. With few
// heads the pass is bound by each wave's chain of dependent steps (small workgroups on many
// CUs); once the heads fill the chip, one workgroup of eight one-tile waves per head keeps
// two waves on each SIMD, which hides the LDS latency that bounds a single wave there.
// (state_ro_kernel, further below, is the fewest-heads shape.)
// ------------------------------------------------------------------------------------------

// LDS of the state pass: the shared per-chunk operands, double buffered as two separate
// objects (so the compiler can tell that reads of one never wait for direct loads into
// the other).
struct StateBuf {
  bf16 W[kC * kD];       // -W, 256-byte rows
  bf16 Pt[kC * kC];      // P^T, 128-byte rows
  bf16 Q[kC * kD];       // 256-byte rows
  bf16 K[kC * kD];       // 256-byte rows
  float gl[4 * kC];      // gam, then gam_C / gam, then G (see dma_piece)
};

// The inputs of U~ = T diag(beta) V, single buffered: T diag(beta) hi and lo in operand
// order, and the workgroup's NTILE value tiles, [tile][token][16] bf16 (32-byte rows).
template <int NTILE>
struct TvBuf {
  bf16 th[kTbFrags * 512];
  bf16 tl[kTbFrags * 512];
  bf16 tbg[kTbFrags * 512];   // -T diag(beta gam), for the shapes that form -W on chip
  bf16 v[NTILE][kC * 16];
};

// Per-lane LDS element offsets, computed once (the swizzles keep K-steps, row tiles and the
// buffer out of the lane-dependent part).
//
// S is held in K order: St[c][2 ks + h][i] = S[row][32 ks + 8 g4 + 4 h + i] for the lane's
// value row of tile c, so the packed operand of K-step ks holds S[row][32 ks + 8 g4 .. + 7]
// and its partners (-W and Q rows) are single 16-byte row reads. The state update produces
// that order by reading K^T columns 32 ks + 8 a + 4 h .. + 3 for output rows 4 a .. 4 a + 3.
struct LaneOffsets {
  int row[4];       // -W and Q row reads: K-step ks (add 2048 per row tile)
  int t128[4];      // P^T transpose reads: column tile
  int k[8];         // K transpose reads: state tile
};

__device__ __forceinline__ void lane_offsets(LaneOffsets& o, int g4, int l16) {
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) o.row[ks] = sw256(l16, 32 * ks + 8 * g4);
  const int rr = 4 * g4 + (l16 >> 2), cc = 4 * (l16 & 3);
#pragma unroll
  for (int x = 0; x < 4; ++x) o.t128[x] = sw128(rr, 16 * x + cc);
#pragma unroll
  for (int x = 0; x < 8; ++x) o.k[x] = sw256(rr, 32 * (x >> 1) + 8 * (l16 & 3) + 4 * (x & 1));
}

// U~ = T diag(beta) V for one 16-row value tile (tokens x value rows, accumulator layout).
// T diag(beta) = hi + lo is lower triangular, so row tile rt needs K-steps 0 .. rt / 2. The
// value operand is read transposed: lane (l16, g4) gets tokens {32 ks + 4 g4 .. +3,
// 32 ks + 16 + 4 g4 .. +3} of value row l16, the K order of the stored T fragments.
__device__ __forceinline__ void utilde_tile(const bf16* th, const bf16* tl, const bf16* vt, f32x4 (&u)[4],
                                            int g4, int l16, int lane) {
  const int vo = (4 * g4 + (l16 >> 2)) * 16 + 4 * (l16 & 3);
  bf16x8 bv[2], ah[kTbFrags], al[kTbFrags];   // every LDS read first, then the products
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) bv[ks] = join8(lds_tr4(vt + vo + 512 * ks), lds_tr4(vt + vo + 512 * ks + 256));
#pragma unroll
  for (int f = 0; f < kTbFrags; ++f) {
    ah[f] = lds8(th + (f * 64 + lane) * 8);
    al[f] = lds8(tl + (f * 64 + lane) * 8);
  }
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks <= rt / 2; ++ks) {
      acc = mfma16x16x32(ah[tb_frag(rt, ks)], bv[ks], acc);
      acc = mfma16x16x32(al[tb_frag(rt, ks)], bv[ks], acc);
    }
    u[rt] = acc;
  }
}

// This wave's share of the direct loads of one chunk's shared operands. The NW waves of a
// workgroup split the sixteen 1 KB instructions of each 16 KB image (-W, Q, K) and the
// eight of P^T. `ni` = 16 / NW instructions per image.
struct DmaPlan {
  int pt[8];        // P^T source offsets (elements)
  int row[16];      // -W / Q / K source rows within the chunk
  int piece[16];    // -W / Q / K source element offsets within the row
  int ni;
};

__device__ __forceinline__ void dma_plan(DmaPlan& d, int ni, int w, int lane) {
  d.ni = ni;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int rq = 4 * (ni * w + i) + (lane >> 4);
    d.row[i] = rq;
    d.piece[i] = ((lane & 15) ^ ((rq & 7) << 1) ^ ((rq >> 3) & 1)) * 8;
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int rp = 8 * ((ni / 2) * w + i) + (lane >> 3);
    d.pt[i] = rp * kC + ((lane & 7) ^ (((rp >> 1) & 3) << 1)) * 8;
  }
}

// Sources and destinations of one chunk's direct loads.
struct DmaChunk {
  const bf16* w;
  const bf16* pt;
  const bf16* qb;       // row 0 of the chunk, this QK head
  const bf16* kb;
  const float* gl;
  const bf16* th;       // T diag(beta) hi, then lo and -T diag(beta gam) (operand order)
  const bf16* vb;       // row 0 of the chunk, this V head, the workgroup's first value row
  bf16* d_w;            // LDS destinations
  bf16* d_pt;
  bf16* d_q;
  bf16* d_k;
  float* d_gl;
  int nv;               // valid rows of the chunk
};

// Number of direct-load instructions per wave per chunk for the shared operands: the three
// 16 KB images, P^T, and the decay factors.
__device__ __forceinline__ constexpr int dma_pieces(int ni) { return 3 * ni + ni / 2 + 1; }

// Issues shared-operand load p (0 <= p < dma_pieces) of a chunk. p is a constant once the
// callers' loops unroll, so each call folds to one instruction.
__device__ __forceinline__ void dma_piece(int p, const DmaChunk& d, const DmaPlan& dp, int qk_stride,
                                          int w, int lane) {
  const int ni = dp.ni;
  if (p < 3 * ni) {
    const int i = p / 3, which = p % 3;
    if (which == 0) {
      __builtin_amdgcn_global_load_lds(d.w + dp.row[i] * kD + dp.piece[i], (lds_void_ptr)(d.d_w + 4 * (ni * w + i) * kD), 16, 0, 0);
    } else {
      // rows past the chunk end repeat the last valid row and only feed discarded results
      const int row = dp.row[i] < d.nv ? dp.row[i] : d.nv - 1;
      const int off = row * qk_stride + dp.piece[i];
      if (which == 1)
        __builtin_amdgcn_global_load_lds(d.qb + off, (lds_void_ptr)(d.d_q + 4 * (ni * w + i) * kD), 16, 0, 0);
      else
        __builtin_amdgcn_global_load_lds(d.kb + off, (lds_void_ptr)(d.d_k + 4 * (ni * w + i) * kD), 16, 0, 0);
    }
    return;
  }
  p -= 3 * ni;
  if (p < ni / 2) {
    __builtin_amdgcn_global_load_lds(d.pt + dp.pt[p], (lds_void_ptr)(d.d_pt + 8 * ((ni / 2) * w + p) * kC), 16, 0, 0);
    return;
  }
  // gam, lam and G: the 1 KB decay-factor area of the block. Every wave issues it
  // (identical data, so the overlapping writes agree): no branch, which would split the
  // scheduling regions around it.
  __builtin_amdgcn_global_load_lds(d.gl + lane * 4, (lds_void_ptr)d.d_gl, 16, 0, 0);
}

// Direct load of stored fragment f: T diag(beta) hi (0..5), lo (6..11), -T diag(beta gam)
// (12..17). A straight 1 KB copy; the three sets are contiguous in the block and in TvBuf.
template <int NTILE>
__device__ __forceinline__ void dma_tb(int f, const DmaChunk& d, TvBuf<NTILE>& tv, int lane) {
  static_assert(kWsTl == kWsTh + kTbFrags * 1024 && kWsTbg == kWsTl + kTbFrags * 1024, "fragment sets");
  const bf16* src = d.th + 512 * f + 8 * lane;
  bf16* dst = tv.th + 512 * f;
  __builtin_amdgcn_global_load_lds(src, (lds_void_ptr)dst, 16, 0, 0);
}

// Direct load of tokens 32 i .. 32 i + 31 of value tile t of the workgroup (two lanes per
// token); rows past the chunk end repeat the last valid row (T diag(beta) is zero there).
template <int NTILE>
__device__ __forceinline__ void dma_v(int t, int i, const DmaChunk& d, TvBuf<NTILE>& tv, int v_stride,
                                      int lane) {
  const int r = 32 * i + (lane >> 1);
  const int row = r < d.nv ? r : d.nv - 1;
  __builtin_amdgcn_global_load_lds(d.vb + row * v_stride + 16 * t + 8 * (lane & 1),
                                   (lds_void_ptr)(tv.v[t] + 512 * i), 16, 0, 0);
}

// Shared-operand loads of chunk slot s of the slots a chunk's compute offers, spread
// evenly: one per state tile of the update (off the chain that leads from U to the next
// state) and, with two value tiles per wave (more compute to hide them behind), one per
// K-step of U.
// When -W and P^T are formed on chip (FORM) the shared operands loaded are Q, K and the decay
// factors: pieces 3 i + 1 and 3 i + 2 of dma_piece, then the decay factors.
__device__ __forceinline__ constexpr int dma_slots(int nt) { return nt == 2 ? 12 : 8; }
__device__ __forceinline__ constexpr int dma_qk_pieces(int ni) { return 2 * ni + 1; }
__device__ __forceinline__ constexpr int dma_qk_piece(int p, int ni) {
  return p < 2 * ni ? 3 * (p / 2) + 1 + (p % 2) : 3 * ni + ni / 2;
}
template <int NI, int NT, bool FORM>
__device__ __forceinline__ void dma_slot(int s, const DmaChunk& d, const DmaPlan& dp, int qk_stride,
                                         int w, int lane) {
  constexpr int P = FORM ? dma_qk_pieces(NI) : dma_pieces(NI);
#pragma unroll
  for (int p = 0; p < P; ++p)
    if (p * dma_slots(NT) / P == s) dma_piece(FORM ? dma_qk_piece(p, NI) : p, d, dp, qk_stride, w, lane);
}

// Sources of chunk c's loads (destinations left unset).
__device__ __forceinline__ DmaChunk dma_src(const PrefillArgs& a, int c, int t0, int t_seq1, int h, int j,
                                           int col_base) {
  DmaChunk d;
  const uint8_t* head = a.ws + ((size_t)c * a.h_v + h) * kWsHead;
  const size_t qk_stride = (size_t)a.h_qk * kD;
  d.w = reinterpret_cast<const bf16*>(head + kWsW);
  d.pt = reinterpret_cast<const bf16*>(head + kWsP);
  d.qb = a.q + (size_t)t0 * qk_stride + (size_t)j * kD;
  d.kb = a.k + (size_t)t0 * qk_stride + (size_t)j * kD;
  d.gl = reinterpret_cast<const float*>(head + kWsGam);
  d.th = reinterpret_cast<const bf16*>(head + kWsTh);

  d.vb = a.v + ((size_t)t0 * a.h_v + h) * kD + col_base;
  d.nv = min(kC, t_seq1 - t0);
  return d;
}

__device__ __forceinline__ DmaChunk dma_chunk(const PrefillArgs& a, StateBuf& dst, int c, int t0, int t_seq1,
                                              int h, int j, int col_base) {
  DmaChunk d = dma_src(a, c, t0, t_seq1, h, j, col_base);
  d.d_w = dst.W;
  d.d_pt = dst.Pt;
  d.d_q = dst.Q;
  d.d_k = dst.K;
  d.d_gl = dst.gl;
  return d;
}

// This wave's loads of the U~ inputs of chunk `d` without a loading wave: a share of the
// T diag(beta) fragments and its own value tiles.
template <int NW, int NT, bool FORM>
__device__ __forceinline__ void dma_tv_share(const DmaChunk& d, TvBuf<NW * NT>& tv, int v_stride, int w,
                                             int lane) {
  constexpr int NF = (FORM ? 3 : 2) * kTbFrags;   // hi, lo (and -T diag(beta gam))
#pragma unroll
  for (int jf = 0; jf < (NF + NW - 1) / NW; ++jf) {
    const int f = w + NW * jf;
    if (f < NF) dma_tb(f, d, tv, lane);
  }
#pragma unroll
  for (int c = 0; c < NT; ++c)
#pragma unroll
    for (int i = 0; i < 2; ++i) dma_v(NT * w + c, i, d, tv, v_stride, lane);
}

// The one-workgroup-per-head shape (no loading wave) forms -W and P^T on chip; the others
// read them from the workspace.
__host__ __device__ constexpr bool forms_w_p(int nw, int nt, bool dw) { return !dw && nw * nt == 8; }

// The many-heads shape forms -W and P^T on chip, into the chunk's LDS buffer, from its Q, K,
// decay factors and -T diag(beta gam), with the products, operand orders and roundings of
// prep_kernel, so the values are bit for bit those prep writes for the other shapes. Wave w
// takes column tiles w, w + NW, ... of -W and tiles w, w + NW, ... of the 10 lower tiles
// of P (P^T is stored by key token, four query tokens per lane).
template <int NW, int NTILE>
__device__ __forceinline__ void form_w_p(StateBuf& cur, const TvBuf<NTILE>& tv, float scale, int w, int g4,
                                         int l16, int lane) {
#pragma unroll
  for (int jc = 0; jc < 8 / NW; ++jc) {
    const int ct = w + NW * jc;
    bf16x8 bk[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) bk[ks] = perm_tr256(cur.K, 32 * ks, 16 * ct, g4, l16);
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      f32x4 aw = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks <= rt / 2; ++ks)
        aw = mfma16x16x32(bk[ks], lds8(tv.tbg + (tb_frag(rt, ks) * 64 + lane) * 8), aw);
      bf16x4 wv;
      wv[0] = to_bf16(aw[0]); wv[1] = to_bf16(aw[1]); wv[2] = to_bf16(aw[2]); wv[3] = to_bf16(aw[3]);
      *reinterpret_cast<bf16x4*>(cur.W + sw256(16 * rt + l16, 16 * ct + 4 * g4)) = wv;
    }
  }
  const float* G = cur.gl + 2 * kC;
#pragma unroll
  for (int jt = 0; jt < (10 + NW - 1) / NW; ++jt) {
    const int t = w + NW * jt;
    if (t >= 10) break;
    const int rt = tile_row(t), ct = tile_col(t);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      acc = mfma16x16x32(lds8(cur.Q + sw256(16 * rt + l16, 32 * ks + 8 * g4)),
                         lds8(cur.K + sw256(16 * ct + l16, 32 * ks + 8 * g4)), acc);
    const f32x4 Gr = *reinterpret_cast<const f32x4*>(&G[16 * rt + 4 * g4]);
    const float Gs = G[16 * ct + l16];
    const int s = 16 * ct + l16;
    bf16x4 pv;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * rt + 4 * g4 + i;
      const float decay = __expf(fminf(Gr[i] - Gs, 0.f));   // bounded as in gram_epilogue
      pv[i] = to_bf16(s <= r ? scale * decay * acc[i] : 0.f);
    }
    *reinterpret_cast<bf16x4*>(cur.Pt + sw128(s, 16 * rt + 4 * g4)) = pv;
  }
}

// One chunk of the state pass for this wave's 16 NT value rows (tiles c at col0 + 16 c),
// reading LDS buffer `cur` while the next chunk (`nx`) streams into the other
// one; its loads are spread over the compute so the vector-memory unit works in the
// background. After a sequence's last chunk `nx` names the following block of the
// workspace and the sequence's last rows: in bounds, and never read. The code has no
// branches, so the scheduler sees each chunk whole. The read-out is formed transposed
// (value rows x tokens) so each lane ends up with four adjacent value rows of one token.
//
// U~ comes either from the loading wave (DW: `my_u`, in the accumulator layout) or, without
// one, from this wave's own products over `tv`, after which a second barrier frees `tv` for
// the next chunk's T diag(beta) and values.
template <int NW, int NT, bool DW>
__device__ __forceinline__ void state_chunk(const PrefillArgs& a, StateBuf& cur, const f32x4* my_u,
                                            TvBuf<NW * NT>& tv, const LaneOffsets& lo, const DmaPlan& dp,
                                            f32x4 (&St)[NT][8], const DmaChunk& nx, int t0, int nv, int h,
                                            int col0, int w, int lane) {
  constexpr int NI = 16 / NW;
  constexpr bool FORM = forms_w_p(NW, NT, DW);
  const int g4 = lane >> 4;
  const int l16 = lane & 15;
  const int qk_stride = a.h_qk * kD;
  // this chunk's direct loads have landed (own share; with a loading wave there are none,
  // and the read-out stores need not complete) ...
  if (!DW) __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();                 // ... everyone's; and the other buffer is free

  // U = U~ - W S^T  (tokens x value rows), starting from U~
  f32x4 U[NT][4], QSt[NT][4];
  if (DW) {
#pragma unroll
    for (int c = 0; c < NT; ++c)
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) U[c][rt] = my_u[(4 * c + rt) * 64 + lane];
  } else {
    if (FORM) form_w_p<NW>(cur, tv, a.scale, w, g4, l16, lane);
#pragma unroll
    for (int c = 0; c < NT; ++c) utilde_tile(tv.th, tv.tl, tv.v[NT * w + c], U[c], g4, l16, lane);
    __syncthreads();               // every wave has read tv (and with FORM, -W and P^T are in)
    dma_tv_share<NW, NT, FORM>(nx, tv, a.h_v * kD, w, lane);
  }
#pragma unroll
  for (int c = 0; c < NT; ++c)
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) QSt[c][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
  // the decay factors this lane uses, read now so their latency hides behind the products:
  // lam4[q] = gam_C / gam of tokens 16 q + 4 g4 .. + 3, gs[nt] = scale gam of token 16 nt + l16
  f32x4 lam4[4];
  float gs[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    lam4[q] = *reinterpret_cast<const f32x4*>(&cur.gl[kC + 16 * q + 4 * g4]);
    gs[q] = cur.gl[16 * q + l16];
  }
  const float gC = cur.gl[kC - 1];

  // S^T as bf16 operands (B of U, A of the transposed read-out)
  bf16x8 Sb[NT][4];
#pragma unroll
  for (int c = 0; c < NT; ++c)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) Sb[c][ks] = pack8(St[c][2 * ks], St[c][2 * ks + 1]);
  const bf16* Wl = cur.W;
  const bf16* Q = cur.Q;
  const bf16* K = cur.K;
  // U -= W S^T first: it is the head of the chain that leads to the next state. Operands
  // of K-step ks + 1 are read while the products of K-step ks run; each operand serves
  // every value tile.
  bf16x8 aw[2][4];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) aw[0][rt] = lds8(Wl + lo.row[0] + 2048 * rt);
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const int cb = ks & 1;
    if (ks + 1 < 4) {
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) aw[cb ^ 1][rt] = lds8(Wl + lo.row[ks + 1] + 2048 * rt);
    }
    if (!DW && NT == 2) dma_slot<NI, NT, FORM>(ks, nx, dp, qk_stride, w, lane);
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int c = 0; c < NT; ++c) U[c][rt] = mfma16x16x32(aw[cb][rt], Sb[c][ks], U[c][rt]);
  }
  // QSt = (Q S^T)^T (value rows x tokens) next: it does not depend on the hi/lo split
  // below, so its products fill the matrix cores while that vector work runs
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    bf16x8 aq[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) aq[rt] = lds8(Q + lo.row[ks] + 2048 * rt);
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int c = 0; c < NT; ++c) QSt[c][rt] = mfma16x16x32(Sb[c][ks], aq[rt], QSt[c][rt]);
  }
  // U as bf16 for the read-out; the decayed U as a hi + lo pair for the state update
  bf16x8 Ub[NT][2], Bh[NT][2], Bl[NT][2];
#pragma unroll
  for (int c = 0; c < NT; ++c)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      Ub[c][ks] = pack8(U[c][2 * ks], U[c][2 * ks + 1]);
      f32x4 hi[2], lw[2];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float u = U[c][2 * ks + hh][i] * lam4[2 * ks + hh][i];
          const float uh = (float)to_bf16(u);
          hi[hh][i] = uh;
          lw[hh][i] = u - uh;
        }
      Bh[c][ks] = pack8(hi[0], hi[1]);
      Bl[c][ks] = pack8(lw[0], lw[1]);
    }
  // S^T <- gam_C S^T + K^T (diag(gam_C / gam) U), with the read-out in between (off the
  // chain to the next state): after state tiles 2 nt and 2 nt + 1, read-out tile nt,
  // O^T = scale gam (Q S^T)^T + U^T P^T, is stored as 8-byte pieces through a buffer
  // resource that ends at the chunk's last valid token (so stores past it are dropped by
  // the hardware range check instead of a branch). Operands of step mt + 1 are read while
  // the products of step mt run.
  const bf16* Pt = cur.Pt;
  const __amdgpu_buffer_rsrc_t orsrc = __builtin_amdgcn_make_buffer_rsrc(
      a.o + ((size_t)t0 * a.h_v + h) * kD, (short)0, nv * a.h_v * kD * 2, 0x00020000);
  bf16x8 ak[2][2];
  ak[0][0] = join8(lds_tr4(K + lo.k[0]), lds_tr4(K + lo.k[0] + 2048));
  ak[0][1] = join8(lds_tr4(K + lo.k[0] + 4096), lds_tr4(K + lo.k[0] + 6144));
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) {
    const int cb = mt & 1;
    if (mt + 1 < 8) {
      const int m1 = mt + 1;
      ak[cb ^ 1][0] = join8(lds_tr4(K + lo.k[m1]), lds_tr4(K + lo.k[m1] + 2048));
      ak[cb ^ 1][1] = join8(lds_tr4(K + lo.k[m1] + 4096), lds_tr4(K + lo.k[m1] + 6144));
    }
    if (!DW) dma_slot<NI, NT, FORM>((NT == 2 ? 4 : 0) + mt, nx, dp, qk_stride, w, lane);
    const int nt = mt >> 1;
    bf16x8 bp[2];
    if (mt & 1) {
#pragma unroll
      for (int ks = 0; ks <= nt / 2; ++ks)
        bp[ks] = join8(lds_tr4(Pt + lo.t128[nt] + 2048 * ks), lds_tr4(Pt + lo.t128[nt] + 2048 * ks + 1024));
    }
#pragma unroll
    for (int c = 0; c < NT; ++c) {
      f32x4 s = St[c][mt] * gC;
      s = mfma16x16x32(ak[cb][0], Bh[c][0], s);
      s = mfma16x16x32(ak[cb][0], Bl[c][0], s);
      s = mfma16x16x32(ak[cb][1], Bh[c][1], s);
      St[c][mt] = mfma16x16x32(ak[cb][1], Bl[c][1], s);
    }
    if (mt & 1) {
      const float gsn = a.scale * gs[nt];
      const int tok = 16 * nt + l16;
#pragma unroll
      for (int c = 0; c < NT; ++c) {
        f32x4 acc = QSt[c][nt] * gsn;
#pragma unroll
        for (int ks = 0; ks <= nt / 2; ++ks) acc = mfma16x16x32(Ub[c][ks], bp[ks], acc);
        bf16x4 ov;
        ov[0] = to_bf16(acc[0]); ov[1] = to_bf16(acc[1]); ov[2] = to_bf16(acc[2]); ov[3] = to_bf16(acc[3]);
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, ov), orsrc,
                                              (tok * a.h_v * kD + col0 + 16 * c + 4 * g4) * 2, 0, 0);
      }
    }
  }
}

// The shared-operand loads of one chunk, issued by one wave (the loading wave of a DW
// workgroup): the three 16 KB images, P^T and the decay factors.
__device__ __forceinline__ void dma_all(const DmaChunk& d, const DmaPlan& dp, int qk_stride, int lane) {
#pragma unroll
  for (int p = 0; p < dma_pieces(16); ++p) dma_piece(p, d, dp, qk_stride, 0, lane);
}

// The U~ inputs of one chunk, issued by one wave (the U~ wave of a DW workgroup): T diag(beta)
// hi and lo and the workgroup's value tiles.
template <int NTILE>
__device__ __forceinline__ void dma_tv_all(const DmaChunk& d, TvBuf<NTILE>& tv, int v_stride, int lane) {
#pragma unroll
  for (int f = 0; f < 2 * kTbFrags; ++f) dma_tb(f, d, tv, lane);
#pragma unroll
  for (int t = 0; t < NTILE; ++t)
#pragma unroll
    for (int i = 0; i < 2; ++i) dma_v(t, i, d, tv, v_stride, lane);
}

// Workgroup barrier for the U~ wave: its LDS reads and writes complete first (lgkmcnt(0)),
// but not its direct loads still in flight, which only it reads, after its own wait. The
// empty asm statements keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void barrier_lds_only() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((15) | (7 << 4) | (0 << 8) | (3 << 14));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// The U~ wave's products for every tile of the workgroup from landed inputs: into the compute
// waves' tile buffers, in the accumulator layout.
template <int NW, int NT>
__device__ __forceinline__ void utilde_all(const TvBuf<NW * NT>& tv, f32x4 (*dst_u)[4 * NT][64], int lane) {
  const int g4 = lane >> 4, l16 = lane & 15;
#pragma unroll
  for (int v = 0; v < NW; ++v)
#pragma unroll
    for (int c = 0; c < NT; ++c) {
      f32x4 u[4];
      utilde_tile(tv.th, tv.tl, tv.v[NT * v + c], u, g4, l16, lane);
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) dst_u[v][4 * c + rt][lane] = u[rt];
    }
}

// DW = true adds two helper waves. The loading wave (wave NW) issues the shared-operand
// loads of the next chunk right after each chunk's barrier and waits for them, so the NW
// compute waves never stall on issuing loads. The U~ wave (wave NW + 1) forms the next
// chunk's U~ for all compute waves into a double buffer of tiles.
template <int NW, int NT, bool DW>
__global__ __launch_bounds__((NW + 2 * DW) * kWave) void state_kernel(PrefillArgs a) {
  __shared__ StateBuf buf0;
  __shared__ StateBuf buf1;
  __shared__ TvBuf<NW * NT> tv;
  __shared__ f32x4 utiles[DW ? 2 : 1][DW ? NW : 1][DW ? 4 * NT : 1][64];
  constexpr int kBlocks = 8 / (NW * NT);      // workgroups per (sequence, V head)
  constexpr int NI = 16 / NW;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, uniform
  const int lane = tid & 63;
  const int g4 = lane >> 4;
  const int l16 = lane & 15;

  // the workgroups of the V heads sharing one QK head (same Q and K) sit on one XCD
  const int per = 8 * a.group * kBlocks;
  const int bid = blockIdx.x;
  const int grp = bid / per, rem = bid % per;
  const int p = grp * 8 + rem % 8;            // (sequence, QK head) pair
  if (p >= a.num_seqs * a.h_qk) return;
  const int sub = rem / 8;                    // V head within the group, value-row block
  const int n = p / a.h_qk, j = p % a.h_qk;
  const int h = j * a.group + sub / kBlocks;
  const int col_base = (sub % kBlocks) * (16 * NT * NW);   // the workgroup's first value row
  const int t_seq0 = a.cu[n], t_seq1 = a.cu[n + 1];
  const int n_chunks = (t_seq1 - t_seq0 + kC - 1) / kC;
  const int c_begin = first_chunk(a.cu, n, lane);
  const int qk_stride = a.h_qk * kD;
  const int v_stride = a.h_v * kD;

  if constexpr (DW) {
    if (w == NW) {   // the loading wave: one barrier per chunk, like the compute waves
      DmaPlan dpl;
      dma_plan(dpl, 16, 0, lane);
      auto issue = [&](int ci, StateBuf& dst) {
        dma_all(dma_chunk(a, dst, c_begin + ci, t_seq0 + ci * kC, t_seq1, h, j, col_base), dpl, qk_stride, lane);
      };
      // even chunks into buf0, odd ones into buf1 (fixed destinations, so the addresses fold)
      if (n_chunks > 0) issue(0, buf0);
      for (int ci = 0; ci < n_chunks; ci += 2) {
        __builtin_amdgcn_s_waitcnt(0);   // chunk ci has landed
        __syncthreads();                 // ... and buf1 is free
        if (ci + 1 < n_chunks) {
          issue(ci + 1, buf1);
          __builtin_amdgcn_s_waitcnt(0);
          __syncthreads();
          if (ci + 2 < n_chunks) issue(ci + 2, buf0);
        }
      }
      return;
    }
    if (w == NW + 1) {   // the U~ wave: chunk ci + 1's U~ during chunk ci
      auto issue = [&](int ci) {   // U~ inputs of chunk ci
        dma_tv_all(dma_src(a, c_begin + ci, t_seq0 + ci * kC, t_seq1, h, j, col_base), tv, v_stride, lane);
      };
      if (n_chunks > 0) {
        issue(0);
        __builtin_amdgcn_s_waitcnt(0);
        utilde_all<NW, NT>(tv, utiles[0], lane);
      }
      for (int ci = 0; ci < n_chunks; ++ci) {
        barrier_lds_only();
        if (ci + 1 < n_chunks) {
          issue(ci + 1);
          __builtin_amdgcn_s_waitcnt(0);
          utilde_all<NW, NT>(tv, utiles[(ci + 1) & 1], lane);
        }
      }
      return;
    }
  }

  const int col0 = col_base + 16 * NT * w;    // this wave's first value row
  LaneOffsets lo;
  lane_offsets(lo, g4, l16);
  DmaPlan dp;
  dma_plan(dp, NI, w, lane);

  // St[c][mt][i] = S[col0 + 16 c + l16][32 (mt / 2) + 8 g4 + 4 (mt % 2) + i]
  f32x4 St[NT][8];
#pragma unroll
  for (int c = 0; c < NT; ++c) {
    const size_t state_off = (((size_t)n * a.h_v + h) * kD + col0 + 16 * c + l16) * kD;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
      St[c][mt] = a.s0 ? *reinterpret_cast<const f32x4*>(a.s0 + state_off + 32 * (mt >> 1) + 8 * g4 + 4 * (mt & 1))
                       : f32x4{0.f, 0.f, 0.f, 0.f};
  }

  if (forms_w_p(NW, NT, DW) && tid < 128) {   // the strictly upper tiles of P that the read-out's 32-token K-steps see
    const int rt = (tid >> 6) * 2, ln = tid & 63;
    const int sr = 16 * (rt + 1) + (ln & 15), col = 16 * rt + 4 * (ln >> 4);
    *reinterpret_cast<bf16x4*>(buf0.Pt + sw128(sr, col)) = bf16x4{};
    *reinterpret_cast<bf16x4*>(buf1.Pt + sw128(sr, col)) = bf16x4{};
  }
  const f32x4* my_u0 = &utiles[0][DW ? w : 0][0][0];
  const f32x4* my_u1 = &utiles[DW ? 1 : 0][DW ? w : 0][0][0];
  if (!DW && n_chunks > 0) {
    const DmaChunk d0 = dma_chunk(a, buf0, c_begin, t_seq0, t_seq1, h, j, col_base);
    dma_tv_share<NW, NT, forms_w_p(NW, NT, DW)>(d0, tv, v_stride, w, lane);
#pragma unroll
    for (int s = 0; s < dma_slots(NT); ++s) dma_slot<NI, NT, forms_w_p(NW, NT, DW)>(s, d0, dp, qk_stride, w, lane);
  }
  // chunks alternate between the two LDS buffers
  for (int ci = 0; ci < n_chunks; ci += 2) {
    const int t0 = t_seq0 + ci * kC;
    const DmaChunk d1 = dma_chunk(a, buf1, c_begin + ci + 1, t0 + kC, t_seq1, h, j, col_base);
    state_chunk<NW, NT, DW>(a, buf0, my_u0, tv, lo, dp, St, d1, t0, min(kC, t_seq1 - t0), h, col0, w, lane);
    if (ci + 1 < n_chunks) {
      const int t1 = t0 + kC;
      const DmaChunk d2 = dma_chunk(a, buf0, c_begin + ci + 2, t1 + kC, t_seq1, h, j, col_base);
      state_chunk<NW, NT, DW>(a, buf1, my_u1, tv, lo, dp, St, d2, t1, min(kC, t_seq1 - t1), h, col0, w, lane);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);   // the last (unused) direct loads land before LDS is released

  if (a.s_final) {
#pragma unroll
    for (int c = 0; c < NT; ++c) {
      const size_t state_off = (((size_t)n * a.h_v + h) * kD + col0 + 16 * c + l16) * kD;
#pragma unroll
      for (int mt = 0; mt < 8; ++mt)
        *reinterpret_cast<f32x4*>(a.s_final + state_off + 32 * (mt >> 1) + 8 * g4 + 4 * (mt & 1)) = St[c][mt];
    }
  }
}

// ------------------------------------------------------------------------------------------
// state_ro_kernel: the fewest-heads state pass (one 16-row value tile per workgroup, eight
// workgroups per head) with the read-out on a wave of its own. The chain wave (wave 0)
// forms U = U~ - W S^T and the state update -- the chain from one chunk's state to the
// next -- and hands S^T and U over as packed bf16 operands. The read-out wave (wave 3)
// forms each chunk's (Q S^T)^T and O^T = scale gam (Q S^T)^T + U^T P^T during the next
// chunk, from its own copies of Q, P^T and the decay factors. The loading wave (wave 1)
// streams -W, K and the decay factors, the U~ wave (wave 2) forms U~ a chunk ahead. One
// barrier per chunk and one at the end; the read-out is the same arithmetic as in
// state_chunk, so results agree bit for bit with the other shapes.
// ------------------------------------------------------------------------------------------

// The chain wave's per-chunk operands, and the read-out wave's.
struct ChainBuf {
  bf16 W[kC * kD];       // -W, 256-byte rows
  bf16 K[kC * kD];       // 256-byte rows
  float gl[4 * kC];      // gam, then gam_C / gam (see dma_piece)
};
struct ReadBuf {
  bf16 Q[kC * kD];       // 256-byte rows
  bf16 Pt[kC * kC];      // P^T, 128-byte rows
  float gl[4 * kC];
};
// What the chain wave hands the read-out wave for one chunk, in lane order: S^T for the
// four K-steps of (Q S^T)^T and U for the two K-steps of U^T P^T.
struct Exchange {
  bf16x8 s[4][64];
  bf16x8 u[2][64];
};

// Loads into a chain buffer (-W, K, decay factors) or a read-out buffer (Q, P^T, decay
// factors), by one wave: the pieces of dma_piece with NI = 16 that each needs.
__device__ __forceinline__ void dma_chain(const PrefillArgs& a, ChainBuf& dst, int c, int t0, int t_seq1, int h,
                                          int j, int col_base, const DmaPlan& dp, int qk_stride, int lane) {
  DmaChunk d = dma_src(a, c, t0, t_seq1, h, j, col_base);
  d.d_w = dst.W;
  d.d_k = dst.K;
  d.d_gl = dst.gl;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    dma_piece(3 * i, d, dp, qk_stride, 0, lane);
    dma_piece(3 * i + 2, d, dp, qk_stride, 0, lane);
  }
  dma_piece(3 * 16 + 8, d, dp, qk_stride, 0, lane);
}
__device__ __forceinline__ void dma_read(const PrefillArgs& a, ReadBuf& dst, int c, int t0, int t_seq1, int h,
                                         int j, int col_base, const DmaPlan& dp, int qk_stride, int lane) {
  DmaChunk d = dma_src(a, c, t0, t_seq1, h, j, col_base);
  d.d_q = dst.Q;
  d.d_pt = dst.Pt;
  d.d_gl = dst.gl;
#pragma unroll
  for (int i = 0; i < 16; ++i) dma_piece(3 * i + 1, d, dp, qk_stride, 0, lane);
#pragma unroll
  for (int i = 0; i < 8; ++i) dma_piece(3 * 16 + i, d, dp, qk_stride, 0, lane);
  dma_piece(3 * 16 + 8, d, dp, qk_stride, 0, lane);
}

// The chain wave's part of one chunk.
__device__ __forceinline__ void chain_chunk(const ChainBuf& cur, const f32x4* my_u, Exchange& xo,
                                            const LaneOffsets& lo, f32x4 (&St)[8], int lane) {
  const int g4 = lane >> 4;
  __syncthreads();                 // the chunk's operands and U~ are in
  f32x4 U[4];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) U[rt] = my_u[rt * 64 + lane];
  f32x4 lam4[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) lam4[q] = *reinterpret_cast<const f32x4*>(&cur.gl[kC + 16 * q + 4 * g4]);
  const float gC = cur.gl[kC - 1];
  // every operand of the chunk is read up front (-W rows for U, then K^T for the update), so
  // the LDS latency overlaps the products instead of stalling each step
  const bf16* Wl = cur.W;
  const bf16* K = cur.K;
  bf16x8 aw[4][4], ak[8][2];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) aw[ks][rt] = lds8(Wl + lo.row[ks] + 2048 * rt);
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) {
    ak[mt][0] = join8(lds_tr4(K + lo.k[mt]), lds_tr4(K + lo.k[mt] + 2048));
    ak[mt][1] = join8(lds_tr4(K + lo.k[mt] + 4096), lds_tr4(K + lo.k[mt] + 6144));
  }
  bf16x8 Sb[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    Sb[ks] = pack8(St[2 * ks], St[2 * ks + 1]);
    xo.s[ks][lane] = Sb[ks];
  }
  // U -= W S^T
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) U[rt] = mfma16x16x32(aw[ks][rt], Sb[ks], U[rt]);
  // U as bf16 for the read-out; the decayed U as a hi + lo pair for the state update
  bf16x8 Bh[2], Bl[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    xo.u[ks][lane] = pack8(U[2 * ks], U[2 * ks + 1]);
    f32x4 hi[2], lw[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float u = U[2 * ks + hh][i] * lam4[2 * ks + hh][i];
        const float uh = (float)to_bf16(u);
        hi[hh][i] = uh;
        lw[hh][i] = u - uh;
      }
    Bh[ks] = pack8(hi[0], hi[1]);
    Bl[ks] = pack8(lw[0], lw[1]);
  }
  // S^T <- gam_C S^T + K^T (diag(gam_C / gam) U)
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) {
    f32x4 s = St[mt] * gC;
    s = mfma16x16x32(ak[mt][0], Bh[0], s);
    s = mfma16x16x32(ak[mt][0], Bl[0], s);
    s = mfma16x16x32(ak[mt][1], Bh[1], s);
    St[mt] = mfma16x16x32(ak[mt][1], Bl[1], s);
  }
}

// The read-out wave's part of one chunk (tokens t0 .. t0 + nv - 1). Every operand is read
// first; once those reads are done `reads_done()` runs (the caller refills `rb` there, so the
// refill's latency overlaps the products).
template <typename F>
__device__ __forceinline__ void readout_chunk(const PrefillArgs& a, const ReadBuf& rb, const Exchange& xo,
                                              const LaneOffsets& lo, int t0, int nv, int h, int col0, int lane,
                                              F reads_done) {
  const int g4 = lane >> 4;
  const int l16 = lane & 15;
  bf16x8 sb[4], aq[4][4], bp[4][2];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    sb[ks] = xo.s[ks][lane];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) aq[ks][rt] = lds8(rb.Q + lo.row[ks] + 2048 * rt);
  }
#pragma unroll
  for (int nt = 0; nt < 4; ++nt)
#pragma unroll
    for (int ks = 0; ks <= nt / 2; ++ks)
      bp[nt][ks] = join8(lds_tr4(rb.Pt + lo.t128[nt] + 2048 * ks), lds_tr4(rb.Pt + lo.t128[nt] + 2048 * ks + 1024));
  float gs[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) gs[q] = rb.gl[16 * q + l16];
  const bf16x8 ub[2] = {xo.u[0][lane], xo.u[1][lane]};
  __builtin_amdgcn_s_waitcnt((15) | (7 << 4) | (0 << 8) | (3 << 14));   // lgkmcnt(0)
  reads_done();
  f32x4 QSt[4];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) QSt[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) QSt[rt] = mfma16x16x32(sb[ks], aq[ks][rt], QSt[rt]);
  const __amdgpu_buffer_rsrc_t orsrc = __builtin_amdgcn_make_buffer_rsrc(
      a.o + ((size_t)t0 * a.h_v + h) * kD, (short)0, nv * a.h_v * kD * 2, 0x00020000);
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    const float gsn = a.scale * gs[nt];
    const int tok = 16 * nt + l16;
    f32x4 acc = QSt[nt] * gsn;
#pragma unroll
    for (int ks = 0; ks <= nt / 2; ++ks) acc = mfma16x16x32(ub[ks], bp[nt][ks], acc);
    bf16x4 ov;
    ov[0] = to_bf16(acc[0]); ov[1] = to_bf16(acc[1]); ov[2] = to_bf16(acc[2]); ov[3] = to_bf16(acc[3]);
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, ov), orsrc,
                                          (tok * a.h_v * kD + col0 + 4 * g4) * 2, 0, 0);
  }
}

__global__ __launch_bounds__(4 * kWave) void state_ro_kernel(PrefillArgs a) {
  __shared__ ChainBuf cb0;
  __shared__ ChainBuf cb1;
  __shared__ TvBuf<1> tv;
  __shared__ f32x4 utiles[2][1][4][64];
  __shared__ Exchange xo0;
  __shared__ Exchange xo1;
  __shared__ ReadBuf rb0;
  __shared__ ReadBuf rb1;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, uniform
  const int lane = tid & 63;
  const int g4 = lane >> 4;
  const int l16 = lane & 15;

  // eight workgroups per head; those of the V heads sharing one QK head sit on one XCD
  const int per = 8 * a.group * 8;
  const int bid = blockIdx.x;
  const int grp = bid / per, rem = bid % per;
  const int p = grp * 8 + rem % 8;            // (sequence, QK head) pair
  if (p >= a.num_seqs * a.h_qk) return;
  const int sub = rem / 8;
  const int n = p / a.h_qk, j = p % a.h_qk;
  const int h = j * a.group + sub / 8;
  const int col0 = (sub % 8) * 16;            // the workgroup's value rows
  const int t_seq0 = a.cu[n], t_seq1 = a.cu[n + 1];
  const int n_chunks = (t_seq1 - t_seq0 + kC - 1) / kC;
  const int c_begin = first_chunk(a.cu, n, lane);
  const int qk_stride = a.h_qk * kD;
  const int v_stride = a.h_v * kD;
  DmaPlan dpl;
  dma_plan(dpl, 16, 0, lane);
  LaneOffsets lo;
  lane_offsets(lo, g4, l16);

  if (w == 1) {   // the loading wave: chunk ci + 1's chain operands during chunk ci
    auto issue = [&](int ci, ChainBuf& dst) {
      dma_chain(a, dst, c_begin + ci, t_seq0 + ci * kC, t_seq1, h, j, col0, dpl, qk_stride, lane);
    };
    if (n_chunks > 0) issue(0, cb0);
    for (int ci = 0; ci < n_chunks; ci += 2) {
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (ci + 1 < n_chunks) {
        issue(ci + 1, cb1);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (ci + 2 < n_chunks) issue(ci + 2, cb0);
      }
    }
    __syncthreads();
    return;
  }
  if (w == 2) {   // the U~ wave: chunk ci + 1's U~ during chunk ci
    auto issue = [&](int ci) {
      dma_tv_all(dma_src(a, c_begin + ci, t_seq0 + ci * kC, t_seq1, h, j, col0), tv, v_stride, lane);
    };
    if (n_chunks > 0) {
      issue(0);
      __builtin_amdgcn_s_waitcnt(0);
      utilde_all<1, 1>(tv, utiles[0], lane);
    }
    for (int ci = 0; ci < n_chunks; ++ci) {
      barrier_lds_only();
      if (ci + 1 < n_chunks) {
        issue(ci + 1);
        __builtin_amdgcn_s_waitcnt(0);
        utilde_all<1, 1>(tv, utiles[(ci + 1) & 1], lane);
      }
    }
    barrier_lds_only();
    return;
  }
  if (w == 3) {   // the read-out wave: chunk ci's read-out after barrier ci + 1
    auto issue = [&](int ci, ReadBuf& dst) {
      dma_read(a, dst, c_begin + ci, t_seq0 + ci * kC, t_seq1, h, j, col0, dpl, qk_stride, lane);
    };
    // chunk ci's read-out from buffer ci % 2, which then takes chunk ci + 2's operands
    auto readout = [&](int ci, ReadBuf& rb, const Exchange& xo) {
      const int t0 = t_seq0 + ci * kC;
      __builtin_amdgcn_s_waitcnt(0);   // its Q, P^T and decay factors have landed
      readout_chunk(a, rb, xo, lo, t0, min(kC, t_seq1 - t0), h, col0, lane, [&] {
        if (ci + 2 < n_chunks) issue(ci + 2, rb);
      });
    };
    if (n_chunks > 0) issue(0, rb0);
    if (n_chunks > 1) issue(1, rb1);
    for (int ci = 0; ci < n_chunks; ci += 2) {
      barrier_lds_only();
      if (ci >= 1) readout(ci - 1, rb1, xo1);
      if (ci + 1 < n_chunks) {
        barrier_lds_only();
        readout(ci, rb0, xo0);
      }
    }
    barrier_lds_only();
    if (n_chunks > 0) {
      if ((n_chunks - 1) & 1) readout(n_chunks - 1, rb1, xo1);
      else readout(n_chunks - 1, rb0, xo0);
    }
    return;
  }

  // the chain wave. St[mt][i] = S[col0 + l16][32 (mt / 2) + 8 g4 + 4 (mt % 2) + i]
  f32x4 St[8];
  const size_t state_off = (((size_t)n * a.h_v + h) * kD + col0 + l16) * kD;
#pragma unroll
  for (int mt = 0; mt < 8; ++mt)
    St[mt] = a.s0 ? *reinterpret_cast<const f32x4*>(a.s0 + state_off + 32 * (mt >> 1) + 8 * g4 + 4 * (mt & 1))
                  : f32x4{0.f, 0.f, 0.f, 0.f};
  for (int ci = 0; ci < n_chunks; ci += 2) {
    chain_chunk(cb0, &utiles[0][0][0][0], xo0, lo, St, lane);
    if (ci + 1 < n_chunks) chain_chunk(cb1, &utiles[1][0][0][0], xo1, lo, St, lane);
  }
  __syncthreads();   // the last chunk's hand-over is visible to the read-out wave
  if (a.s_final) {
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
      *reinterpret_cast<f32x4*>(a.s_final + state_off + 32 * (mt >> 1) + 8 * g4 + 4 * (mt & 1)) = St[mt];
  }
}

}  // namespace

size_t chunk_prefill_workspace_bytes(int total_tokens, int num_seqs, int h_qk, int h_v) {
  (void)h_qk;
  return max_chunks(total_tokens, num_seqs) * (size_t)h_v * kWsHead;
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
  a.ws = static_cast<uint8_t*>(workspace);
  const size_t nc = max_chunks(total_tokens, num_seqs);
  a.num_seqs = num_seqs;
  a.h_qk = h_qk;
  a.h_v = h_v;
  a.group = h_v / h_qk;
  a.n_chunks_max = (int)nc;
  a.scale = scale;

  // the shapes for up to 128 heads read -W and P^T from the workspace; the one-workgroup-
  // per-head shape forms them on chip (forms_w_p)
  const size_t heads = (size_t)num_seqs * h_v;
  const bool full = heads * 2 <= kStateCus;
  if (total_tokens > 0) {
    const size_t pairs = nc * (size_t)h_qk;
    const size_t prep_blocks = (pairs + 7) / 8 * 8 * (size_t)a.group;
    if (full) hipLaunchKernelGGL(prep_kernel<true>, dim3((unsigned)prep_blocks), dim3(kThreads), 0, stream, a);
    else hipLaunchKernelGGL(prep_kernel<false>, dim3((unsigned)prep_blocks), dim3(kThreads), 0, stream, a);
  }
  // With few heads, eight or four workgroups per head of one or two compute waves (one
  // tile each) and helper waves spread the heads over many CUs; once the heads fill the
  // chip, one 8-wave workgroup per head (two waves per SIMD to hide latency) avoids the
  // operand traffic that every workgroup repeats, and forms -W and P^T itself.
  const size_t seq_pairs = (size_t)num_seqs * h_qk;
  const size_t groups = (seq_pairs + 7) / 8 * 8 * (size_t)a.group;
  if (heads * 8 <= kStateCus) {
    hipLaunchKernelGGL(state_ro_kernel, dim3((unsigned)(groups * 8)), dim3(4 * kWave), 0, stream, a);
  } else if (heads * 4 <= kStateCus) {
    hipLaunchKernelGGL((state_kernel<2, 1, true>), dim3((unsigned)(groups * 4)), dim3(4 * kWave), 0, stream, a);
  } else if (heads * 2 <= kStateCus) {
    hipLaunchKernelGGL((state_kernel<4, 1, false>), dim3((unsigned)(groups * 2)), dim3(4 * kWave), 0, stream, a);
  } else {
    hipLaunchKernelGGL((state_kernel<8, 1, false>), dim3((unsigned)groups), dim3(8 * kWave), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace gdn
