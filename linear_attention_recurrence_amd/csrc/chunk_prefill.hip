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
//   U   = T diag(beta) (V - diag(gam) K S^T)          (the chunk's corrections)
//   O   = scale * [ diag(gam) Q S^T + (Q K^T o Gam o lower-incl) U ]
//   S'  = gam_C S + (diag(gam_C / gam) U)^T K
//
// Everything that does not involve S depends on one chunk only, so the work splits in two
// launches that share a workspace:
//
//  * prep_kernel, one workgroup per (chunk, QK head) and one or two of the QK head's V heads,
//    all chunks in parallel: K K^T (and K Q^T, formed once for the V heads that share them)
//    on the bf16 matrix cores, the prefix sums, the unit-lower-triangular inverse T in
//    fp32 (16 x 16 diagonal blocks by substitution, off-diagonal blocks on the fp32 matrix
//    cores). Writes T diag(beta) and P^T, P = scale (Q K^T o Gam o lower-incl), each as a
//    hi + lo bf16 pair in the operand order of the state pass, and gam, gam_C / gam, G.
//  * the state pass, walking each sequence's chunks in order with S in fp32 registers, 16
//    value rows per wave (value rows evolve independently), one to eight workgroups per
//    (sequence, V head) depending on how many heads there are. Per chunk:
//    X = K S^T, R = V - diag(gam) X, U = T diag(beta) R, the state update, and the read-out
//    O^T = scale gam (Q S^T)^T + U^T P^T, all on the bf16 matrix cores. The next chunk's
//    K, Q, T diag(beta), P^T, values and decay factors stream into LDS with direct
//    global-to-LDS loads while the current chunk computes.
//
// Precision: K, Q and V are exact bf16 operands. Every computed operand whose rounding would
// reach the state or cancel in a sum -- S in K S^T, the residual R, T diag(beta), the decayed
// U of the update, and both U and P in the read-out's P U -- is split into a hi + lo bf16
// pair (x = hi + lo to about 16 bits) and multiplied as hi*hi + hi*lo + lo*hi (or both
// halves against an exact operand). With alpha = 1 the state keeps everything it is given
// and K S^T nearly cancels V; with beta near 1 and a repeated key, P U telescopes. Single
// bf16 roundings there cost several times the output and state bounds. Only S in Q S^T stays
// a single bf16 rounding (it feeds no later chunk and nothing cancels against it). S stays
// in fp32.
//
// Matrix-core layout (v_mfma_f32_16x16x32_bf16): lane l holds A[l%16][8*(l/16)+s],
// B[8*(l/16)+s][l%16] for s = 0..7, and C[4*(l/16)+i][l%16] for i = 0..3. A product is
// unchanged when the same permutation is applied to the K index of A and B, so a
// C-layout accumulator pair covering K rows k0..k0+15 and k0+16..k0+31 is a valid
// operand once its partner reads K entries {4g..4g+3, 16+4g..16+4g+3} (g = l/16); the
// products over tokens below use that K order. The fp32 16x16x4 instruction has lane l
// holding A[l%16][l/16], B[l/16][l%16] and the same C layout.
//
// Operands whose K index runs down the rows of a row-major LDS image (K contracted over
// tokens, the value tile) are read with ds_read_b64_tr_b16: within each group of 16 lanes,
// when lane i points at row k0 + i/4, columns n0 + 4(i%4) .. +3, lane j receives rows
// k0 .. k0+3 of column n0 + j.
#include <atomic>
#include <mutex>

#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {

// Device scratch of the prefill variant that allocates nothing (gdn_chunk_prefill_noalloc):
// its workspace lives here, one copy per GPU the library runs on, held until the process
// ends. In host code `scratch` names a host-side stand-in, not the device array: the device
// address comes from hipGetSymbolAddress, once per device (noalloc_scratch below).
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {

constexpr int kC = 64;          // chunk length
constexpr int kD = 128;         // head dim
constexpr size_t kStateCus = 256;   // compute units of the chip
constexpr int kF32Pad = kC + 4;     // [token][token] fp32 LDS rows

// Workspace: one block per (chunk, V head). The two triangular 64 x 64 operands are stored
// as six 1 KB fragments each (below), hi and lo.
constexpr int kFrags = 6;
constexpr size_t kFragBytes = 1024;
constexpr size_t kWsTh = 0;                               // bf16 T diag(beta), hi
constexpr size_t kWsTl = kWsTh + kFrags * kFragBytes;     // bf16 T diag(beta), lo
constexpr size_t kWsPh = kWsTl + kFrags * kFragBytes;     // bf16 P^T, hi
constexpr size_t kWsPl = kWsPh + kFrags * kFragBytes;     // bf16 P^T, lo
constexpr size_t kWsGam = kWsPl + kFrags * kFragBytes;    // fp32 [64]: gam_r
constexpr size_t kWsLam = kWsGam + kC * 4;                // fp32 [64]: gam_C / gam_r
constexpr size_t kWsG = kWsLam + kC * 4;                  // fp32 [64]: G_r
constexpr size_t kWsHead = kWsGam + 1024;                 // 25600 bytes

// With many heads the state pass forms P^T on chip (from Q, K and G, with the products,
// operand order and roundings of prep_kernel, so bit for bit the same values) and prep
// writes no P^T and reads no Q.

// The two lower-triangular operands are stored fragment by fragment in the order the state
// pass reads them, one 16-byte read per lane per fragment:
//  * T diag(beta) is the A operand of U = T diag(beta) R (rows = tokens r, K = tokens s).
//    Fragment (row tile rt, K-step ks) holds, for lane l = l16 + 16 g4, the eight entries
//    T[16 rt + l16][32 ks + 16 h + 4 g4 + i] beta_s (h, i = 0, 1 / 0..3, element 4 h + i).
//  * P^T is the B operand of O^T = U^T P^T (K = key tokens s, columns = query tokens r).
//    Fragment (query tile nt, K-step ks) holds, for lane l16 + 16 g4, the eight entries
//    P[16 nt + l16][32 ks + 16 h + 4 g4 + i].
// Both are lower triangular in (r, s), so fragments with ks > rt / 2 are zero and are not
// stored: the six others are numbered 0, 1 (rt = 0, 1), then 2 + 2 (rt - 2) + ks.
__device__ __forceinline__ constexpr int frag(int rt, int ks) { return rt < 2 ? rt : 2 * rt - 2 + ks; }
// Element offset of T entry (r, s) for s a multiple of 4 (r >= s rounded down to the
// fragment, i.e. a stored fragment).
__device__ __forceinline__ int tb_frag_off(int r, int s) {
  return (frag(r >> 4, s >> 5) * 64 + (r & 15) + 16 * ((s >> 2) & 3)) * 8 + 4 * ((s >> 4) & 1);
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
  // a segmented call (seg_len > 0, fewest-heads shape only): the launches cover chunks
  // seg_lo .. seg_lo + seg_len - 1 of every sequence, chunk seg_lo + i of sequence n in
  // workspace slot n seg_len + i; the state between segments waits in `carry`
  // ([num_seqs][h_v][d_v][d_k] fp32, in the workspace)
  int seg_lo, seg_len;
  float* carry;
};

typedef __attribute__((address_space(3))) void* lds_void_ptr;
typedef __bf16 bf16x4_gcc __attribute__((__vector_size__(8)));
typedef __attribute__((address_space(3))) bf16x4_gcc* lds_bf16x4_ptr;

__device__ __forceinline__ bf16x8 lds8(const bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }
__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
// Transposing LDS read (ds_read_b64_tr_b16). The address-space cast keeps the pointer's
// origin (a __shared__ array) visible to the compiler: from a bare integer address it would
// assume the read may touch bytes that a direct global -> LDS load in flight is writing,
// and make the read wait for every such load.
__device__ __forceinline__ bf16x4 lds_tr4(const bf16* p) {
  const bf16x4_gcc r = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_ptr)p);
  return __builtin_bit_cast(bf16x4, r);
}

// Two fp32 values rounded to bf16 (nearest even) and packed into one word, x in the low half.
__device__ __forceinline__ uint32_t pk_bf16(float x, float y) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t v = {to_bf16(x), to_bf16(y)};
  return __builtin_bit_cast(uint32_t, v);
}

// x = hi + lo for eight fp32 values (two accumulator quads), each half rounded to bf16:
// hi = bf16(x), lo = bf16(x - hi), so hi + lo carries about 16 bits of x. Each pair is
// rounded by one packed conversion and its halves widened back by a shift and a mask (three
// instructions per value). The packed word passes through an empty asm statement: seen
// through, the shift of the pair is rewritten as a second conversion of x alone, one more
// instruction per pair. Contraction stays off: every kernel that calls this must round the
// same way.
__device__ __forceinline__ void split8(f32x4 a, f32x4 b, bf16x8& hi, bf16x8& lo) {
#pragma clang fp contract(off)
  u32x4 h, l;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const float x = p < 2 ? a[2 * p] : b[2 * p - 4];
    const float y = p < 2 ? a[2 * p + 1] : b[2 * p - 3];
    uint32_t w = pk_bf16(x, y);
    asm("" : "+v"(w));
    h[p] = w;
    l[p] = pk_bf16(x - __builtin_bit_cast(float, w << 16), y - __builtin_bit_cast(float, w & 0xffff0000u));
  }
  hi = __builtin_bit_cast(bf16x8, h);
  lo = __builtin_bit_cast(bf16x8, l);
}

// The LDS-space pointer of a generic pointer into __shared__ memory: its low 32 bits are the
// LDS address. (An address-space cast would test the generic pointer for null first.)
__device__ __forceinline__ lds_void_ptr lds_addr(const void* p) {
  return (lds_void_ptr)(uint32_t)(uintptr_t)p;
}

// ---- LDS images: unpadded rows, 16-byte pieces XOR-swizzled against the LDS banks. 256-byte
// rows ([64][128] bf16): piece p of row r at slot p ^ sw_row(r), sw_row(r) = 2 (r mod 8) ^
// bit 1 of r. Measured on gfx950 (bank-conflict counters over access patterns): a 16-byte
// read serves 16 lanes per cycle from 64 four-byte banks, and the bank of a 16-byte slot is
// its position in the 256-byte row with the slot's lowest bit flipped by bits 1 and 3 of
// the row. Against that, the 16 rows of a row read (one piece) land on 16 distinct slots
// (no conflict), and a transposing read (4 rows x 4 pieces, one 8-byte half) on 8, twice
// each, the least a fixed half allows.
__device__ __forceinline__ int sw_row(int r) { return (2 * (r & 7)) ^ ((r >> 1) & 1); }
__device__ __forceinline__ int sw256(int r, int col) {
  const int p = col >> 3;
  return r * 128 + ((p ^ sw_row(r)) << 3) + (col & 7);
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
// swizzled image, 1 KB per instruction: piece i fills image rows 4 i .. 4 i + 3. Image row r
// comes from source row min(r, nv - 1) at byte `r * stride` from `src`: rows past the chunk
// end repeat the last valid row and only feed results that are discarded or multiplied by
// zero. The source address is a uniform base plus a 32-bit lane offset.
__device__ __forceinline__ void dma_rows256(const bf16* src, uint32_t stride, int nv, bf16* img, int i,
                                            int lane) {
  const int r = 4 * i + (lane >> 4);
  const uint32_t piece = (uint32_t)((lane & 15) ^ sw_row(r));
  const uint32_t off = __umul24((uint32_t)min(r, nv - 1), stride) + 16u * piece;
  __builtin_amdgcn_global_load_lds(reinterpret_cast<const uint8_t*>(src) + off, lds_addr(img + 4 * i * kD),
                                   16, 0, 0);
}
// A straight 1 KB copy (16 bytes per lane).
__device__ __forceinline__ void dma_1k(const void* src, void* dst, int lane) {
  __builtin_amdgcn_global_load_lds(reinterpret_cast<const uint8_t*>(src) + 16 * lane, lds_addr(dst), 16, 0, 0);
}
// Tokens 32 i .. 32 i + 31 of a [64][16] bf16 value tile (32-byte rows; two lanes per
// token); rows past the chunk end repeat the last valid row (T diag(beta) is zero there).
// v_stride is in bytes.
__device__ __forceinline__ void dma_vtile(const bf16* vb, uint32_t v_stride, int nv, bf16* tile, int i,
                                          int lane) {
  const uint32_t r = (uint32_t)min(32 * i + (lane >> 1), nv - 1);
  const uint32_t off = __umul24(r, v_stride) + 16u * (lane & 1);
  __builtin_amdgcn_global_load_lds(reinterpret_cast<const uint8_t*>(vb) + off, lds_addr(tile + 512 * i), 16, 0, 0);
}

// Lower 16 x 16 tile t (0..9, row-major over the lower triangle) of a 64 x 64 product.
__device__ __forceinline__ constexpr int tile_row(int t) { return t < 1 ? 0 : t < 3 ? 1 : t < 6 ? 2 : 3; }
__device__ __forceinline__ constexpr int tile_col(int t) { return t - tile_row(t) * (tile_row(t) + 1) / 2; }

// One 16 x 16 tile of X Y^T over the 128 key channels: rows of X from image rows
// 16 xt .. + 15, rows of Y from 16 yt .. + 15 (both swizzled 256-byte-row images).
// C[4 g4 + i][l16] = X[16 xt + 4 g4 + i] . Y[16 yt + l16].
__device__ __forceinline__ f32x4 gram_tile(const bf16* X, const bf16* Y, int xt, int yt, int g4, int l16) {
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
    acc = mfma16x16x32(lds8(X + sw256(16 * xt + l16, 32 * ks + 8 * g4)),
                       lds8(Y + sw256(16 * yt + l16, 32 * ks + 8 * g4)), acc);
  return acc;
}

// P^T tile for key tile ct <= query tile rt, from acc = (K Q^T) tile (ct, rt) (gram_tile with
// X = K, Y = Q): lane (l16, g4) holds P[r][s] for r = 16 rt + l16 and s = 16 ct + 4 g4 + i,
// which are elements 4 (ct % 2) + i of its slot of fragment (rt, ct / 2). Returns hi and lo
// of the four values (zero where s > r). G is the log-decay prefix sum of the chunk.
__device__ __forceinline__ void pt_tile_values(const float* G, f32x4 acc, int rt, int ct, float scale,
                                               int g4, int l16, bf16x4& hi, bf16x4& lo) {
#pragma clang fp contract(off)
  const int r = 16 * rt + l16;
  const float Gr = G[r];
  const f32x4 Gs = *reinterpret_cast<const f32x4*>(&G[16 * ct + 4 * g4]);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int s = 16 * ct + 4 * g4 + i;
    // G is nonincreasing (every g <= 0 by contract), but the prefix sums are added in a
    // different order for each token, so G_r - G_s (s <= r) may round to a tiny positive
    // value; the bound keeps every in-chunk ratio at most 1, as it is exactly.
    const float decay = __expf(fminf(Gr - Gs[i], 0.f));
    const float p = s <= r ? scale * decay * acc[i] : 0.f;
    const bf16 h = to_bf16(p);
    hi[i] = h;
    lo[i] = to_bf16(p - (float)h);
  }
}
// Element offset (bf16) of the 4-element group of tile (ct, rt) in a P^T fragment set.
__device__ __forceinline__ int pt_off(int rt, int ct, int lane) {
  return (frag(rt, ct >> 1) * 64 + lane) * 8 + 4 * (ct & 1);
}

// ------------------------------------------------------------------------------------------
// prep_kernel: one workgroup per (chunk, HP V heads of one QK head)
// ------------------------------------------------------------------------------------------
// The chunk's K (and Q) rows are loaded and their Gram products formed once for the HP V
// heads that share them (two when the heads of a QK head pair up, else one); the decays,
// A, T and the workspace blocks are per V head, four waves each for the triangular solve.
template <bool WITH_P, int HP>
struct PrepSmem {
  union {
    struct {
      bf16 K[kC * kD];          // swizzled 256-byte rows
      bf16 Q[WITH_P ? kC * kD : 8];
    } in;
    // per V head, once the Gram products are in registers: A in the strict lower triangle,
    // T transposed in the upper one
    float M[HP][kC][kF32Pad];
  } r;
  alignas(16) float G[HP][kC];
  alignas(16) float beta[HP][kC];
};

// WITH_P: also K Q^T and P^T (few heads); otherwise the state pass forms P^T itself.
template <bool WITH_P, int HP>
__global__ __launch_bounds__(4 * HP * kWave, HP == 1 ? 4 : 3) void prep_kernel(PrefillArgs a) {
  static_assert(HP == 1 || HP == 2, "one or two V heads per workgroup");
  constexpr int NW = 4 * HP;                      // waves
  __shared__ PrepSmem<WITH_P, HP> sm;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, uniform
  const int lane = tid & 63;
  const int g4 = lane >> 4;
  const int l16 = lane & 15;

  // workgroups of the V heads sharing one QK head sit on the same XCD (blockIdx % 8)
  const int per = a.group / HP;               // workgroups per (chunk, QK head)
  const int bid = blockIdx.x;
  const int grp = bid / (8 * per), rem = bid % (8 * per);
  const int p = grp * 8 + rem % 8;            // (chunk, QK head) pair
  const int gi = (rem / 8) * HP;              // first V head of the workgroup within the QK group
  const int c = p / a.h_qk, j = p % a.h_qk;    // c: the workspace slot
  if (c >= a.n_chunks_max) return;
  int n, local;
  if (a.seg_len) {   // slot n seg_len + i: chunk seg_lo + i of sequence n
    n = c / a.seg_len;
    local = a.seg_lo + c % a.seg_len;
    if (n >= a.num_seqs || local >= seq_chunks(a.cu, n)) return;
  } else {
    locate_chunk(a.cu, a.num_seqs, c, lane, n, local);
    if (n < 0) return;
  }
  const int h0 = j * a.group + gi;            // V heads h0 .. h0 + HP - 1
  const int t0 = a.cu[n] + local * kC;
  const int nv = min(kC, a.cu[n + 1] - t0);
  uint8_t* const ws0 = a.ws + ((size_t)c * a.h_v + h0) * kWsHead;   // head h0 + hh: + hh kWsHead

  // ---- loads: K, Q rows straight into swizzled LDS images; g, beta ----
  constexpr int kPieces = 16 / NW;            // 1 KB pieces (four rows) of each image per wave
  const size_t qk_stride = (size_t)a.h_qk * kD;
#pragma unroll
  for (int i = 0; i < kPieces; ++i) {
    dma_rows256(a.k + (size_t)t0 * qk_stride + (size_t)j * kD, (uint32_t)qk_stride * 2, nv, sm.r.in.K,
                kPieces * w + i, lane);
    if (WITH_P)
      dma_rows256(a.q + (size_t)t0 * qk_stride + (size_t)j * kD, (uint32_t)qk_stride * 2, nv, sm.r.in.Q,
                  kPieces * w + i, lane);
  }
  if (tid < HP * kC) {
    const int hh = tid / kC, r = tid % kC;
    float gg = 0.f, bb = 0.f;
    if (r < nv) {
      gg = a.g[(size_t)(t0 + r) * a.h_v + h0 + hh];
      bb = a.beta[(size_t)(t0 + r) * a.h_v + h0 + hh];
    }
    sm.G[hh][r] = gg;
    sm.beta[hh][r] = bb;
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // ---- K K^T (lower 10 tiles, for A) and, WITH_P, K Q^T (the 10 tiles with key tile <=
  // query tile, for P^T), in registers: WITH_P, the first half of the waves takes K K^T and
  // the second K Q^T, tiles dealt round-robin; otherwise every wave takes K K^T tiles ----
  constexpr int NK = WITH_P ? NW / 2 : NW;    // waves per product
  constexpr int NT = (10 + NK - 1) / NK;      // tiles per wave, at most
  const bool is_p = WITH_P && w >= NK;
  const int first = WITH_P ? w % NK : w;
  f32x4 acc[NT];
#pragma unroll
  for (int jj = 0; jj < NT; ++jj) {
    const int t = first + NK * jj;
    if (t < 10) {
      const int rt = tile_row(t), ct = tile_col(t);
      acc[jj] = is_p ? gram_tile(sm.r.in.K, sm.r.in.Q, ct, rt, g4, l16)
                     : gram_tile(sm.r.in.K, sm.r.in.K, rt, ct, g4, l16);
    }
  }
  // ---- prefix sums of log-decays (wave hh for V head h0 + hh, its Gram tiles issued first) ----
  if (w < HP) {
    float x = sm.G[w][lane];
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float y = __shfl_up(x, off, 64);
      if (lane >= off) x += y;
    }
    const float GC = __shfl(x, 63, 64);
    sm.G[w][lane] = x;
    uint8_t* wsh = ws0 + (size_t)w * kWsHead;
    reinterpret_cast<float*>(wsh + kWsGam)[lane] = __expf(x);
    reinterpret_cast<float*>(wsh + kWsLam)[lane] = __expf(GC - x);
    reinterpret_cast<float*>(wsh + kWsG)[lane] = x;
  }
  __syncthreads();   // K and Q are consumed (their space becomes the M's) and G is ready

  if (is_p) {
    // P^T hi and lo of every V head straight to the workspace (8-byte pieces), and the two
    // all-zero halves of fragments (rt, ks) = (0, 0) and (2, 1) (key tiles 1 and 3 above the
    // diagonal): wave NK + 2 hh + z zeroes half z of V head hh's
#pragma unroll
    for (int hh = 0; hh < HP; ++hh) {
      bf16* Ph = reinterpret_cast<bf16*>(ws0 + (size_t)hh * kWsHead + kWsPh);
      bf16* Pl = reinterpret_cast<bf16*>(ws0 + (size_t)hh * kWsHead + kWsPl);
#pragma unroll
      for (int jj = 0; jj < NT; ++jj) {
        const int t = first + NK * jj;
        if (t < 10) {
          const int rt = tile_row(t), ct = tile_col(t);
          bf16x4 hi, lo;
          pt_tile_values(sm.G[hh], acc[jj], rt, ct, a.scale, g4, l16, hi, lo);
          *reinterpret_cast<bf16x4*>(Ph + pt_off(rt, ct, lane)) = hi;
          *reinterpret_cast<bf16x4*>(Pl + pt_off(rt, ct, lane)) = lo;
        }
      }
    }
    const int q = w - NK, hz = q >> 1, rz = (q & 1) * 2;
    bf16* Ph = reinterpret_cast<bf16*>(ws0 + (size_t)hz * kWsHead + kWsPh);
    bf16* Pl = reinterpret_cast<bf16*>(ws0 + (size_t)hz * kWsHead + kWsPl);
    *reinterpret_cast<bf16x4*>(Ph + pt_off(rz, rz + 1, lane)) = bf16x4{};
    *reinterpret_cast<bf16x4*>(Pl + pt_off(rz, rz + 1, lane)) = bf16x4{};
  } else {
    // A = strictly-lower(beta_r Gam_rs (K K^T)_rs) of every V head into LDS; each head's LDS
    // reads first (the stores into A would order them)
#pragma unroll
    for (int hh = 0; hh < HP; ++hh) {
      f32x4 Gr[NT], Br[NT];
      float Gs[NT];
#pragma unroll
      for (int jj = 0; jj < NT; ++jj) {
        const int t = first + NK * jj;
        if (t < 10) {
          const int rt = tile_row(t), ct = tile_col(t);
          Gr[jj] = *reinterpret_cast<const f32x4*>(&sm.G[hh][16 * rt + 4 * g4]);
          Br[jj] = *reinterpret_cast<const f32x4*>(&sm.beta[hh][16 * rt + 4 * g4]);
          Gs[jj] = sm.G[hh][16 * ct + l16];
        }
      }
#pragma unroll
      for (int jj = 0; jj < NT; ++jj) {
        const int t = first + NK * jj;
        if (t < 10) {
          const int rt = tile_row(t), ct = tile_col(t);
          const int s = 16 * ct + l16;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = 16 * rt + 4 * g4 + i;
            const float decay = __expf(fminf(Gr[jj][i] - Gs[jj], 0.f));   // bounded as in pt_tile_values
            sm.r.M[hh][r][s] = s < r ? Br[jj][i] * decay * acc[jj][i] : 0.f;
          }
        }
      }
    }
  }
  __syncthreads();

  // ---- T = (I + A)^-1 per V head: waves 4 hh .. 4 hh + 3 on V head h0 + hh ----------------
  // T is unit lower triangular and A strictly lower triangular, so they share one array: A
  // keeps the strict lower triangle and T[r][c] (r >= c) goes to the mirror position [c][r].
  const int hh = w >> 2, wl = w & 3;
  float (&M)[kC][kF32Pad] = sm.r.M[hh];
  // diagonal 16 x 16 blocks: the head's first wave inverts all four, 16 lanes per block
  // (block lane / 16, lane = column), one row of A at a time; the other waves wait at the
  // barrier (their lanes would run the same dependent chain, so the SIMDs issue a quarter
  // of the instructions this way)
  if (wl == 0) {
    const int b0 = 16 * (lane >> 4), col = lane & 15;
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {   // row r of the block: x_r = e_r - sum_{m < r} A_rm x_m
      f32x4 ar[4];
#pragma unroll
      for (int q = 0; q < (r + 3) / 4; ++q) ar[q] = *reinterpret_cast<const f32x4*>(&M[b0 + r][b0 + 4 * q]);
      float acc1 = (r == col) ? 1.f : 0.f;
#pragma unroll
      for (int m = 0; m < r; ++m) acc1 -= ar[m >> 2][m & 3] * x[m];
      x[r] = acc1;
      if (r >= col) M[b0 + col][b0 + r] = acc1;
    }
  }
  __syncthreads();
  // off-diagonal block (i, b), i = b + d:  T_ib = -T_ii * sum_{k=b}^{i-1} A_ik T_kb,
  // level by level on the fp32 matrix cores (wave wl handles block (wl + d, wl))
#pragma unroll 1
  for (int d = 1; d < 4; ++d) {
    if (wl < 4 - d) {
      const int b = wl, i = b + d;
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

  // ---- T diag(beta) as a hi + lo bf16 pair, straight to the workspace in operand order.
  // Lane = row r; wave wl takes columns s0 = 8 (wl + 4 it) .. + 7, so the reads of T's
  // mirrored entries M[s][r] hit distinct banks.
  uint8_t* wsh = ws0 + (size_t)hh * kWsHead;
  bf16* Thg = reinterpret_cast<bf16*>(wsh + kWsTh);
  bf16* Tlg = reinterpret_cast<bf16*>(wsh + kWsTl);
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int r = lane, s0 = 8 * (wl + 4 * it);
    if ((s0 >> 5) <= (r >> 4) / 2) {   // a stored (not all-zero) fragment
      f32x4 tv[2];
#pragma unroll
      for (int e = 0; e < 8; ++e) tv[e >> 2][e & 3] = M[s0 + e][r];
      const f32x4 bv[2] = {*reinterpret_cast<const f32x4*>(&sm.beta[hh][s0]),
                           *reinterpret_cast<const f32x4*>(&sm.beta[hh][s0 + 4])};
#pragma unroll
      for (int e = 0; e < 8; ++e)   // T is lower triangular; the mirror of its strict upper part holds A
        tv[e >> 2][e & 3] = (s0 + e <= r) ? tv[e >> 2][e & 3] * bv[e >> 2][e & 3] : 0.f;
      bf16x8 hv, lv;
      split8(tv[0], tv[1], hv, lv);
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const int off = tb_frag_off(r, s0 + 4 * h2);
        *reinterpret_cast<bf16x4*>(Thg + off) = bf16x4{hv[4 * h2], hv[4 * h2 + 1], hv[4 * h2 + 2], hv[4 * h2 + 3]};
        *reinterpret_cast<bf16x4*>(Tlg + off) = bf16x4{lv[4 * h2], lv[4 * h2 + 1], lv[4 * h2 + 2], lv[4 * h2 + 3]};
      }
    }
  }
}

// ------------------------------------------------------------------------------------------
// The state pass: shared per-chunk arithmetic
// ------------------------------------------------------------------------------------------

// Per-lane LDS element offsets, computed once (the swizzles keep K-steps, row tiles and the
// buffer out of the lane-dependent part).
//
// S is held in K order: St[2 ks + h][i] = S[row][32 ks + 8 g4 + 4 h + i] for the lane's
// value row, so the packed operand of K-step ks holds S[row][32 ks + 8 g4 .. + 7] and its
// partners (K and Q rows) are single 16-byte row reads. The state update produces that
// order by reading K^T columns 32 ks + 8 a + 4 h .. + 3 for output rows 4 a .. 4 a + 3.
struct LaneOffsets {
  int row[4];       // K and Q row reads: K-step ks (add 2048 per row tile)
  int k[8];         // K transpose reads: state tile
  int vt;           // value-tile transpose read (add 256 per token tile)
};

__device__ __forceinline__ void lane_offsets(LaneOffsets& o, int g4, int l16) {
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) o.row[ks] = sw256(l16, 32 * ks + 8 * g4);
  const int rr = 4 * g4 + (l16 >> 2);
#pragma unroll
  for (int x = 0; x < 8; ++x) o.k[x] = sw256(rr, 32 * (x >> 1) + 8 * (l16 & 3) + 4 * (x & 1));
  o.vt = rr * 16 + 4 * (l16 & 3);
}

// The operands one chunk of the chain reads from LDS.
struct ChainOps {
  const bf16* K;      // swizzled [64][128]
  const bf16* th;     // T diag(beta) hi, 6 fragments
  const bf16* tl;     // T diag(beta) lo
  const bf16* vt;     // this tile's values, [64][16]
  const float* gl;    // gam[64], then gam_C / gam[64]
};

// One chunk of the chain from one state to the next, for 16 value rows (the lane's row l16
// of the tile), in three parts so that two waves can share it by key halves:
//  chain_x      for key half kh (keys 64 kh .. 64 kh + 63, state tiles 4 kh .. 4 kh + 3):
//               that half of S split into hi + lo and X_kh = K_kh S_kh^T (tokens x rows);
//  chain_u      from X = X_0 + X_1: R = V - diag(gam) X, U = T diag(beta) R, and the decayed
//               U split into hi + lo for the update;
//  chain_update for key half kh: S_kh^T <- gam_C S_kh^T + K_kh^T (diag(gam_C / gam) U).
// The halves of X are always summed as X_0 + X_1, so one wave doing both halves and two
// waves doing one each give the same bits. S's hi half (Sh) is the read-out's operand; U is
// returned in the accumulator layout (token tile rt: rows 16 rt + 4 g4 + i of column l16).
// The parts take their LDS operands in registers (the load_* functions), so a caller can
// issue every read of a chunk at once.

// K rows of key half kh's two K-steps (A operands of X), token tiles 0..3.
__device__ __forceinline__ void load_k_rows(const bf16* K, const LaneOffsets& lo, int kh, bf16x8 (&ak)[2][4]) {
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) ak[j][rt] = lds8(K + lo.row[2 * kh + j] + 2048 * rt);
}
// K^T operands of key half kh's four state tiles (A operands of the update).
__device__ __forceinline__ void load_k_t(const bf16* K, const LaneOffsets& lo, int kh, bf16x8 (&akt)[4][2]) {
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int mt = 4 * kh + m;
    akt[m][0] = join8(lds_tr4(K + lo.k[mt]), lds_tr4(K + lo.k[mt] + 2048));
    akt[m][1] = join8(lds_tr4(K + lo.k[mt] + 4096), lds_tr4(K + lo.k[mt] + 6144));
  }
}
// The operands of chain_u: T diag(beta) hi and lo, the tile's values, gam, gam_C / gam.
struct UOps {
  bf16x8 th[kFrags], tl[kFrags];
  bf16x4 v4[4];
  f32x4 gam4[4], lam4[4];
};
__device__ __forceinline__ void load_u_ops(const ChainOps& c, const LaneOffsets& lo, UOps& u, int lane) {
  const int g4 = lane >> 4;
#pragma unroll
  for (int f = 0; f < kFrags; ++f) {
    u.th[f] = lds8(c.th + (f * 64 + lane) * 8);
    u.tl[f] = lds8(c.tl + (f * 64 + lane) * 8);
  }
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    u.v4[rt] = lds_tr4(c.vt + lo.vt + 256 * rt);
    u.gam4[rt] = *reinterpret_cast<const f32x4*>(&c.gl[16 * rt + 4 * g4]);
    u.lam4[rt] = *reinterpret_cast<const f32x4*>(&c.gl[kC + 16 * rt + 4 * g4]);
  }
}

__device__ __forceinline__ void chain_x(const bf16x8 (&ak)[2][4], const f32x4 (&S)[4], bf16x8 (&Sh)[2],
                                        f32x4 (&X)[4]) {
  bf16x8 Sl[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) split8(S[2 * j], S[2 * j + 1], Sh[j], Sl[j]);
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) X[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < 2; ++j)   // low halves first
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) X[rt] = mfma16x16x32(ak[j][rt], Sl[j], X[rt]);
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) X[rt] = mfma16x16x32(ak[j][rt], Sh[j], X[rt]);
}

__device__ __forceinline__ void chain_u(const UOps& o, const f32x4 (&X0)[4], const f32x4 (&X1)[4],
                                        f32x4 (&U)[4], bf16x8 (&Bh)[2], bf16x8 (&Bl)[2]) {
#pragma clang fp contract(off)
  // R = V - diag(gam) X, then R = Rh + Rl as the B operands of the two 32-token K-steps
  f32x4 R[4];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      R[rt][i] = __builtin_fmaf(-o.gam4[rt][i], X0[rt][i] + X1[rt][i], (float)o.v4[rt][i]);
  bf16x8 Rh[2], Rl[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) split8(R[2 * ks], R[2 * ks + 1], Rh[ks], Rl[ks]);
  // U = T diag(beta) R = Th Rl + Tl Rh + Th Rh (lower triangular: K-steps 0 .. rt / 2). Each
  // token tile accumulates its terms in the order Th Rl, Tl Rh per K-step, then Th Rh per
  // K-step; the four tiles' chains are issued step by step, interleaved, so that no product
  // waits on the one before it in its own chain.
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) U[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int st = 0; st < 6; ++st) {
#pragma unroll
    for (int rt = 3; rt >= 0; --rt) {
      const int nk = rt / 2 + 1;            // K-steps of this tile
      if (st >= 3 * nk) continue;
      const int ks = st < 2 * nk ? st >> 1 : st - 2 * nk;
      if (st >= 2 * nk) U[rt] = mfma16x16x32(o.th[frag(rt, ks)], Rh[ks], U[rt]);
      else if (st & 1) U[rt] = mfma16x16x32(o.tl[frag(rt, ks)], Rh[ks], U[rt]);
      else U[rt] = mfma16x16x32(o.th[frag(rt, ks)], Rl[ks], U[rt]);
    }
  }
  // the decayed U as a hi + lo pair for the update
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
    split8(U[2 * ks] * o.lam4[2 * ks], U[2 * ks + 1] * o.lam4[2 * ks + 1], Bh[ks], Bl[ks]);
}

__device__ __forceinline__ void chain_update(const bf16x8 (&akt)[4][2], f32x4 (&S)[4], const bf16x8 (&Bh)[2],
                                             const bf16x8 (&Bl)[2], float gC) {
#pragma clang fp contract(off)
  // each tile: gam_C S, then the four products in this order; the tiles' chains interleaved
#pragma unroll
  for (int m = 0; m < 4; ++m) S[m] = S[m] * gC;
#pragma unroll
  for (int m = 0; m < 4; ++m) S[m] = mfma16x16x32(akt[m][0], Bh[0], S[m]);
#pragma unroll
  for (int m = 0; m < 4; ++m) S[m] = mfma16x16x32(akt[m][0], Bl[0], S[m]);
#pragma unroll
  for (int m = 0; m < 4; ++m) S[m] = mfma16x16x32(akt[m][1], Bh[1], S[m]);
#pragma unroll
  for (int m = 0; m < 4; ++m) S[m] = mfma16x16x32(akt[m][1], Bl[1], S[m]);
}

// The whole chunk of the chain in one wave: both key halves (S0 = keys 0..63, S1 = 64..127),
// each part's operands read just before it.
__device__ __forceinline__ void chain_chunk(const ChainOps& c, const LaneOffsets& lo, f32x4 (&S0)[4],
                                            f32x4 (&S1)[4], bf16x8 (&Sh)[4], f32x4 (&U)[4], int lane) {
  f32x4 X0[4], X1[4];
  bf16x8 sh0[2], sh1[2], Bh[2], Bl[2];
  {
    bf16x8 ak[2][4];
    load_k_rows(c.K, lo, 0, ak);
    chain_x(ak, S0, sh0, X0);
    load_k_rows(c.K, lo, 1, ak);
    chain_x(ak, S1, sh1, X1);
  }
  Sh[0] = sh0[0]; Sh[1] = sh0[1]; Sh[2] = sh1[0]; Sh[3] = sh1[1];
  {
    UOps uo;
    load_u_ops(c, lo, uo, lane);
    chain_u(uo, X0, X1, U, Bh, Bl);
  }
  const float gC = c.gl[kC - 1];
  bf16x8 akt[4][2];
  load_k_t(c.K, lo, 0, akt);
  chain_update(akt, S0, Bh, Bl, gC);
  load_k_t(c.K, lo, 1, akt);
  chain_update(akt, S1, Bh, Bl, gC);
}

// The operands one chunk of the read-out reads from LDS.
struct ReadOps {
  const bf16* Q;      // swizzled [64][128]
  const bf16* ph;     // P^T hi, 6 fragments
  const bf16* pl;     // P^T lo
  const float* gl;    // gam[64]
};

// The read-out of one chunk for the 16 value rows: O^T = scale gam (Q S^T)^T + U^T P^T with
// S = the state entering the chunk (its hi half Sh) and U from chain_chunk, each O^T tile
// (value rows x 16 tokens) stored as 8-byte pieces of four adjacent value rows through a
// buffer resource that ends at the chunk's last valid token (so stores past it are dropped
// by the hardware range check instead of a branch). `col` is the byte offset of the lane's
// first value row within a token's output row.
__device__ __forceinline__ void readout_chunk(const ReadOps& r, const LaneOffsets& lo, const bf16x8 (&Sh)[4],
                                              const f32x4 (&U)[4], float scale, __amdgpu_buffer_rsrc_t orsrc,
                                              int tok_stride, int col, int lane) {
#pragma clang fp contract(off)
  const int g4 = lane >> 4;
  const int l16 = lane & 15;
  bf16x8 aq[4][4], ph[kFrags], pl[kFrags];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) aq[ks][nt] = lds8(r.Q + lo.row[ks] + 2048 * nt);
#pragma unroll
  for (int f = 0; f < kFrags; ++f) {
    ph[f] = lds8(r.ph + (f * 64 + lane) * 8);
    pl[f] = lds8(r.pl + (f * 64 + lane) * 8);
  }
  float gs[4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) gs[nt] = r.gl[16 * nt + l16];
  // U = Uh + Ul as the A operands (value rows x tokens) of the two 32-token K-steps
  bf16x8 Uh[2], Ul[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) split8(U[2 * ks], U[2 * ks + 1], Uh[ks], Ul[ks]);
  f32x4 QSt[4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) QSt[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) QSt[nt] = mfma16x16x32(Sh[ks], aq[ks][nt], QSt[nt]);
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    f32x4 acc = QSt[nt] * (scale * gs[nt]);
#pragma unroll
    for (int ks = 0; ks <= nt / 2; ++ks) {
      acc = mfma16x16x32(Ul[ks], ph[frag(nt, ks)], acc);
      acc = mfma16x16x32(Uh[ks], pl[frag(nt, ks)], acc);
    }
#pragma unroll
    for (int ks = 0; ks <= nt / 2; ++ks) acc = mfma16x16x32(Uh[ks], ph[frag(nt, ks)], acc);
    bf16x4 ov;
    ov[0] = to_bf16(acc[0]); ov[1] = to_bf16(acc[1]); ov[2] = to_bf16(acc[2]); ov[3] = to_bf16(acc[3]);
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, ov), orsrc,
                                          (16 * nt + l16) * tok_stride + col + 8 * g4, 0, 0);
  }
}

// Sources of chunk c of a sequence for one workgroup (V head h, QK head j, value rows from
// col_base).
struct ChunkSrc {
  const uint8_t* ws;    // the chunk's workspace block
  const bf16* qb;       // row 0 of the chunk, this QK head
  const bf16* kb;
  const bf16* vb;       // row 0 of the chunk, this V head, the workgroup's first value row
  int nv;               // valid rows of the chunk
};

__device__ __forceinline__ ChunkSrc chunk_src(const PrefillArgs& a, int c, int t0, int t_seq1, int h, int j,
                                              int col_base) {
  ChunkSrc s;
  s.ws = a.ws + ((size_t)c * a.h_v + h) * kWsHead;
  const size_t qk_stride = (size_t)a.h_qk * kD;
  s.qb = a.q + (size_t)t0 * qk_stride + (size_t)j * kD;
  s.kb = a.k + (size_t)t0 * qk_stride + (size_t)j * kD;
  s.vb = a.v + ((size_t)t0 * a.h_v + h) * kD + col_base;
  s.nv = min(kC, t_seq1 - t0);
  return s;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t out_rsrc(const PrefillArgs& a, int t0, int nv, int h) {
  return __builtin_amdgcn_make_buffer_rsrc(a.o + ((size_t)t0 * a.h_v + h) * kD, (short)0,
                                           nv * a.h_v * kD * 2, 0x00020000);
}

// Key half kh of the lane's value row: S[mt] = S[row0 + l16][32 (mt' / 2) + 8 g4 + 4 (mt' % 2) + i]
// for state tile mt' = 4 kh + mt.
__device__ __forceinline__ void load_state(const PrefillArgs& a, const float* src, int n, int h, int row0, int kh,
                                           f32x4 (&S)[4], int lane) {
  const int g4 = lane >> 4, l16 = lane & 15;
  const size_t off = (((size_t)n * a.h_v + h) * kD + row0 + l16) * kD + 64 * kh + 8 * g4;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
    S[mt] = src ? *reinterpret_cast<const f32x4*>(src + off + 32 * (mt >> 1) + 4 * (mt & 1))
                : f32x4{0.f, 0.f, 0.f, 0.f};
}
__device__ __forceinline__ void load_state(const PrefillArgs& a, int n, int h, int row0, int kh, f32x4 (&S)[4],
                                           int lane) {
  load_state(a, a.s0, n, h, row0, kh, S, lane);
}
__device__ __forceinline__ void store_state(const PrefillArgs& a, float* dst, int n, int h, int row0, int kh,
                                            const f32x4 (&S)[4], int lane) {
  const int g4 = lane >> 4, l16 = lane & 15;
  const size_t off = (((size_t)n * a.h_v + h) * kD + row0 + l16) * kD + 64 * kh + 8 * g4;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
    *reinterpret_cast<f32x4*>(dst + off + 32 * (mt >> 1) + 4 * (mt & 1)) = S[mt];
}
__device__ __forceinline__ void store_state(const PrefillArgs& a, int n, int h, int row0, int kh,
                                            const f32x4 (&S)[4], int lane) {
  store_state(a, a.s_final, n, h, row0, kh, S, lane);
}

// ------------------------------------------------------------------------------------------
// state_ro_kernel: the fewest-heads state pass (one 16-row value tile per workgroup, eight
// workgroups per head). The chain -- the dependent path from one chunk's state to the next --
// runs on two waves, one per key half (waves 0 and 1: chain_x on their half, an exchange of
// the halves of X through LDS, chain_u each, chain_update on their half). The read-out wave
// (wave 3) forms each chunk's read-out during the next chunk from its own copies of Q, P^T
// and the decay factors, which it loads itself, and S's hi half and U handed over by the
// chain waves. The loading wave (wave 2) streams K, T diag(beta), the value tile and the
// decay factors one chunk ahead. One workgroup barrier per chunk and one at the end; the two
// chain waves also hand the halves of X to each other through LDS mid-chunk. The arithmetic
// is that of the other shapes, so results agree bit for bit.
// ------------------------------------------------------------------------------------------

struct RoChainBuf {
  bf16 K[kC * kD];
  bf16 th[kFrags * 512];
  bf16 tl[kFrags * 512];
  bf16 vt[kC * 16];
  float gl[4 * kC];      // gam, gam_C / gam, G, unused
};
struct RoReadBuf {
  bf16 Q[kC * kD];
  bf16 ph[kFrags * 512];
  bf16 pl[kFrags * 512];
  float gl[4 * kC];
};
// What the chain waves hand the read-out wave for one chunk, in lane order.
struct Exchange {
  bf16x8 sh[4][64];
  f32x4 u[4][64];
};
// The two halves of X, exchanged between the two chain waves, and the handshake: ready[kh]
// counts the chunks whose half kh is in x[kh].
struct XHalves {
  f32x4 x[2][4][64];
  unsigned ready[2];
};

// Wait until the other chain wave has published chunk `count - 1`'s half of X. Both chain
// waves run the same chunks and each publishes its half before it waits for the other's, so
// the wait always ends; the spin is capped all the same (2^22 polls, a fraction of a second),
// so a fault in that reasoning could not hang the GPU. The poll does not sleep: the waiting
// wave has its SIMD to itself, and each poll is one LDS read.
__device__ __forceinline__ void wait_ready(const unsigned* ready, unsigned count) {
  for (int spin = 0; spin < (1 << 22); ++spin) {
    if (__hip_atomic_load(ready, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) >= count) return;
  }
}

// Byte strides of the q/k and v rows.
struct DmaStrides {
  uint32_t qk, v;
};

__device__ __forceinline__ void dma_ro_chain(const ChunkSrc& s, RoChainBuf& d, const DmaStrides& st, int lane) {
#pragma unroll
  for (int i = 0; i < 16; ++i) dma_rows256(s.kb, st.qk, s.nv, d.K, i, lane);
#pragma unroll
  for (int f = 0; f < 2 * kFrags; ++f) dma_1k(s.ws + kWsTh + f * kFragBytes, d.th + 512 * f, lane);
#pragma unroll
  for (int i = 0; i < 2; ++i) dma_vtile(s.vb, st.v, s.nv, d.vt, i, lane);
  dma_1k(s.ws + kWsGam, d.gl, lane);
}
__device__ __forceinline__ void dma_ro_read(const ChunkSrc& s, RoReadBuf& d, const DmaStrides& st, int lane) {
#pragma unroll
  for (int i = 0; i < 16; ++i) dma_rows256(s.qb, st.qk, s.nv, d.Q, i, lane);
#pragma unroll
  for (int f = 0; f < 2 * kFrags; ++f) dma_1k(s.ws + kWsPh + f * kFragBytes, d.ph + 512 * f, lane);
  dma_1k(s.ws + kWsGam, d.gl, lane);
}

// Workgroup barrier for a wave whose direct loads still in flight only it reads, after its
// own wait: its LDS reads and writes complete first (lgkmcnt(0)), the loads do not. The
// empty asm statements keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void barrier_lds_only() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((15) | (7 << 4) | (0 << 8) | (3 << 14));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// A chain wave of state_ro_kernel: key half KH of the state,
// S[mt][i] = S[col0 + l16][64 KH + 32 (mt / 2) + 8 g4 + 4 (mt % 2) + i]. It takes part in the
// workgroup barrier once per chunk, like the other waves; the halves of X pass between the
// two chain waves through xx with its own handshake, which the other waves never wait for.
template <int KH>
__device__ __forceinline__ void ro_chain_wave(const PrefillArgs& a, const RoChainBuf (&cb)[2], Exchange (&xo)[2],
                                              XHalves& xx, const LaneOffsets& lo, int n, int h, int col0,
                                              int n_chunks, const float* s_in, float* s_out, int lane) {
  f32x4 S[4];
  load_state(a, s_in, n, h, col0, KH, S, lane);
  if (lane == 0) xx.ready[KH] = 0;
  for (int ci = 0; ci < n_chunks; ++ci) {
    const RoChainBuf& c = cb[ci & 1];
    Exchange& x = xo[ci & 1];
    __syncthreads();                 // the chunk's operands are in (and the flags are set up)
    // every LDS operand of the chunk at once: the reads overlap each other and the products
    bf16x8 ak[2][4], akt[4][2];
    UOps uo;
    const ChainOps ops{c.K, c.th, c.tl, c.vt, c.gl};
    load_k_rows(c.K, lo, KH, ak);
    load_k_t(c.K, lo, KH, akt);
    load_u_ops(ops, lo, uo, lane);
    const float gC = c.gl[kC - 1];
    bf16x8 sh[2];
    f32x4 X[4];
    chain_x(ak, S, sh, X);
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) xx.x[KH][rt][lane] = X[rt];
    // publish: the half's stores complete before the count moves on
    __builtin_amdgcn_s_waitcnt((15) | (7 << 4) | (0 << 8) | (3 << 14));
    if (lane == 0) __hip_atomic_store(&xx.ready[KH], (unsigned)ci + 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) x.sh[2 * KH + jj][lane] = sh[jj];
    wait_ready(&xx.ready[KH ^ 1], (unsigned)ci + 1);
    f32x4 Xo[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) Xo[rt] = xx.x[KH ^ 1][rt][lane];
    f32x4 U[4];
    bf16x8 Bh[2], Bl[2];
    if (KH == 0) {
      chain_u(uo, X, Xo, U, Bh, Bl);
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) x.u[rt][lane] = U[rt];
    } else {
      chain_u(uo, Xo, X, U, Bh, Bl);
    }
    chain_update(akt, S, Bh, Bl, gC);
  }
  __syncthreads();   // the last chunk's hand-over is visible to the read-out wave
  if (s_out) store_state(a, s_out, n, h, col0, KH, S, lane);
}

__global__ __launch_bounds__(4 * kWave) void state_ro_kernel(PrefillArgs a) {
  __shared__ RoChainBuf cb[2];
  __shared__ Exchange xo[2];
  __shared__ XHalves xx;
  __shared__ RoReadBuf rb[2];
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
  const int seq_chunks_n = (t_seq1 - t_seq0 + kC - 1) / kC;
  // this launch's chunks of the sequence: all of them, or those of the segment
  const int seg_lo = a.seg_len ? a.seg_lo : 0;
  const int n_chunks = a.seg_len ? max(0, min(a.seg_len, seq_chunks_n - seg_lo)) : seq_chunks_n;
  if (seg_lo > 0 && n_chunks == 0) return;   // the sequence ended in an earlier segment
  const int c_begin = a.seg_len ? n * a.seg_len : first_chunk(a.cu, n, lane);
  // state in and out: the caller's, or the carry between segments
  const float* s_in = seg_lo == 0 ? a.s0 : a.carry;
  float* s_out = seg_lo + n_chunks == seq_chunks_n ? a.s_final : a.carry;
  const int t_lo = t_seq0 + seg_lo * kC;
  const int qk_stride = a.h_qk * kD;
  const int v_stride = a.h_v * kD;
  LaneOffsets lo;
  lane_offsets(lo, g4, l16);
  auto src = [&](int ci) { return chunk_src(a, c_begin + ci, t_lo + ci * kC, t_seq1, h, j, col0); };

  DmaStrides dst;
  dst.qk = (uint32_t)qk_stride * 2;
  dst.v = (uint32_t)v_stride * 2;
  if (w == 2) {   // the loading wave: chunk ci + 1's chain operands during chunk ci
    if (n_chunks > 0) dma_ro_chain(src(0), cb[0], dst, lane);
    for (int ci = 0; ci < n_chunks; ++ci) {
      __builtin_amdgcn_s_waitcnt(0);   // chunk ci has landed
      __syncthreads();
      if (ci + 1 < n_chunks) dma_ro_chain(src(ci + 1), cb[(ci + 1) & 1], dst, lane);
    }
    __syncthreads();
    return;
  }
  if (w == 3) {   // the read-out wave: chunk ci's read-out after the barrier of chunk ci + 1
    // chunk ci's read-out from buffer ci % 2, which then takes chunk ci + 2's operands
    auto readout = [&](int ci) {
      const int t0 = t_lo + ci * kC;
      RoReadBuf& r = rb[ci & 1];
      const Exchange& x = xo[ci & 1];
      __builtin_amdgcn_s_waitcnt(0);   // its Q, P^T and decay factors have landed
      bf16x8 sh[4];
      f32x4 u[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) sh[ks] = x.sh[ks][lane];
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) u[rt] = x.u[rt][lane];
      const ReadOps ops{r.Q, r.ph, r.pl, r.gl};
      readout_chunk(ops, lo, sh, u, a.scale, out_rsrc(a, t0, min(kC, t_seq1 - t0), h), v_stride * 2,
                    col0 * 2, lane);
      // every LDS read of the buffer is done before it is refilled
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_waitcnt((15) | (7 << 4) | (0 << 8) | (3 << 14));
      if (ci + 2 < n_chunks) dma_ro_read(src(ci + 2), r, dst, lane);
    };
    if (n_chunks > 0) dma_ro_read(src(0), rb[0], dst, lane);
    if (n_chunks > 1) dma_ro_read(src(1), rb[1], dst, lane);
    for (int ci = 0; ci < n_chunks; ++ci) {
      barrier_lds_only();
      if (ci >= 1) readout(ci - 1);
    }
    barrier_lds_only();
    if (n_chunks > 0) readout(n_chunks - 1);
    return;
  }

  // the chain waves: wave kh holds key half kh of the state (a constant in each branch, so
  // every register array is indexed statically)
  if (w == 0) ro_chain_wave<0>(a, cb, xo, xx, lo, n, h, col0, n_chunks, s_in, s_out, lane);
  else ro_chain_wave<1>(a, cb, xo, xx, lo, n, h, col0, n_chunks, s_in, s_out, lane);
}

// ------------------------------------------------------------------------------------------
// state_kernel<NW, FORM>: NW waves of one 16-row value tile each per workgroup, each wave
// running both the chain and the read-out of its rows, so 8 / NW workgroups per (sequence,
// V head), placed on one XCD. With FORM (one workgroup per head, once the heads outnumber
// the CUs) the workgroup forms P^T itself from the chunk's Q, K and G, with prep's products,
// operand order and roundings, and prep writes none: P^T stays off HBM.
// ------------------------------------------------------------------------------------------

template <int NW>
struct StateBuf {
  bf16 K[kC * kD];
  bf16 Q[kC * kD];
  bf16 th[kFrags * 512];
  bf16 tl[kFrags * 512];
  bf16 ph[kFrags * 512];
  bf16 pl[kFrags * 512];
  float gl[4 * kC];          // gam, gam_C / gam, G, unused
  bf16 vt[NW][kC * 16];
};

// This wave's share of the direct loads of one chunk: 1 KB pieces numbered 0 .. 16 K rows,
// 16 Q rows, 12 T diag(beta) fragments, 12 P^T fragments (not with FORM), the decay factors,
// two per value tile; wave w issues the pieces p = w (mod NW).
template <int NW, bool FORM>
__device__ __forceinline__ void dma_chunk(const ChunkSrc& s, StateBuf<NW>& d, const DmaStrides& st, int w,
                                          int lane) {
  constexpr int kP = FORM ? 0 : 2 * kFrags;
  constexpr int kTotal = 32 + 2 * kFrags + kP + 1 + 2 * NW;
#pragma unroll
  for (int i = 0; i < (kTotal + NW - 1) / NW; ++i) {
    const int p = w + NW * i;
    if (p < 16) dma_rows256(s.kb, st.qk, s.nv, d.K, p, lane);
    else if (p < 32) dma_rows256(s.qb, st.qk, s.nv, d.Q, p - 16, lane);
    else if (p < 32 + 2 * kFrags) dma_1k(s.ws + kWsTh + (p - 32) * kFragBytes, d.th + 512 * (p - 32), lane);
    else if (p < 32 + 2 * kFrags + kP)
      dma_1k(s.ws + kWsPh + (p - 32 - 2 * kFrags) * kFragBytes, d.ph + 512 * (p - 32 - 2 * kFrags), lane);
    else if (p == 32 + 2 * kFrags + kP) dma_1k(s.ws + kWsGam, d.gl, lane);
    else if (p < kTotal) {
      const int q = p - (33 + 2 * kFrags + kP);
      dma_vtile(s.vb + 16 * (q >> 1), st.v, s.nv, d.vt[q >> 1], q & 1, lane);
    }
  }
}

// With FORM, the workgroup's share of P^T for the chunk in `b` (Q, K and G in): wave w takes
// tiles w, w + NW, ... of the 10 (key tile <= query tile), and the two all-zero halves.
template <int NW>
__device__ __forceinline__ void form_pt(StateBuf<NW>& b, float scale, int w, int g4, int l16, int lane) {
#pragma unroll
  for (int jt = 0; jt < (10 + NW - 1) / NW; ++jt) {
    const int t = w + NW * jt;
    if (t < 10) {
      const int rt = tile_row(t), ct = tile_col(t);
      const f32x4 acc = gram_tile(b.K, b.Q, ct, rt, g4, l16);
      bf16x4 hi, lo;
      pt_tile_values(b.gl + 2 * kC, acc, rt, ct, scale, g4, l16, hi, lo);
      *reinterpret_cast<bf16x4*>(b.ph + pt_off(rt, ct, lane)) = hi;
      *reinterpret_cast<bf16x4*>(b.pl + pt_off(rt, ct, lane)) = lo;
    }
  }
  if (w == NW - 1) {
#pragma unroll
    for (int rt = 0; rt < 4; rt += 2) {
      *reinterpret_cast<bf16x4*>(b.ph + pt_off(rt, rt + 1, lane)) = bf16x4{};
      *reinterpret_cast<bf16x4*>(b.pl + pt_off(rt, rt + 1, lane)) = bf16x4{};
    }
  }
}

template <int NW, bool FORM>
__global__ __launch_bounds__(NW * kWave) void state_kernel(PrefillArgs a) {
  __shared__ StateBuf<NW> buf0;
  __shared__ StateBuf<NW> buf1;
  constexpr int kBlocks = 8 / NW;      // workgroups per (sequence, V head)
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
  const int col_base = (sub % kBlocks) * (16 * NW);   // the workgroup's first value row
  const int col0 = col_base + 16 * w;                 // this wave's first value row
  const int t_seq0 = a.cu[n], t_seq1 = a.cu[n + 1];
  const int n_chunks = (t_seq1 - t_seq0 + kC - 1) / kC;
  const int c_begin = first_chunk(a.cu, n, lane);
  const int qk_stride = a.h_qk * kD;
  const int v_stride = a.h_v * kD;
  LaneOffsets lo;
  lane_offsets(lo, g4, l16);
  auto src = [&](int ci) { return chunk_src(a, c_begin + ci, t_seq0 + ci * kC, t_seq1, h, j, col_base); };

  DmaStrides dst;
  dst.qk = (uint32_t)qk_stride * 2;
  dst.v = (uint32_t)v_stride * 2;
  f32x4 S0[4], S1[4];
  load_state(a, n, h, col0, 0, S0, lane);
  load_state(a, n, h, col0, 1, S1, lane);
  auto step = [&](int ci, StateBuf<NW>& cur, StateBuf<NW>& nxt) {
    __builtin_amdgcn_s_waitcnt(0);   // this wave's share of the chunk's loads has landed ...
    __syncthreads();                 // ... and everyone's; the other buffer is free
    if (ci + 1 < n_chunks) dma_chunk<NW, FORM>(src(ci + 1), nxt, dst, w, lane);
    if (FORM) form_pt<NW>(cur, a.scale, w, g4, l16, lane);
    bf16x8 sh[4];
    f32x4 u[4];
    const ChainOps ops{cur.K, cur.th, cur.tl, cur.vt[w], cur.gl};
    chain_chunk(ops, lo, S0, S1, sh, u, lane);
    if (FORM) barrier_lds_only();    // every wave's part of P^T is in (the next chunk's loads may still fly)
    const int t0 = t_seq0 + ci * kC;
    const ReadOps rops{cur.Q, cur.ph, cur.pl, cur.gl};
    readout_chunk(rops, lo, sh, u, a.scale, out_rsrc(a, t0, min(kC, t_seq1 - t0), h), v_stride * 2,
                  col0 * 2, lane);
  };
  if (n_chunks > 0) dma_chunk<NW, FORM>(src(0), buf0, dst, w, lane);
  for (int ci = 0; ci < n_chunks; ci += 2) {
    step(ci, buf0, buf1);
    if (ci + 1 < n_chunks) step(ci + 1, buf1, buf0);
  }
  if (a.s_final) {
    store_state(a, n, h, col0, 0, S0, lane);
    store_state(a, n, h, col0, 1, S1, lane);
  }
}

}  // namespace

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;
}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
      // with device `dev` current: that device's copy of the array
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  return hipSuccess;
}

namespace {

// The fewest-heads shape (up to 64 (sequence, V head) pairs) can run in segments of
// kSegChunks chunks per sequence, a prep launch and a state-pass launch each, so that its
// workspace holds one segment's blocks and the states between segments, whatever the
// sequence lengths. It does when that is smaller than the whole call's blocks.
constexpr int kSegChunks = 64;

size_t segmented_workspace_bytes(int num_seqs, int h_v) {
  return ((size_t)num_seqs * kSegChunks * h_v) * kWsHead + (size_t)num_seqs * h_v * kD * kD * 4;
}

bool prefill_segmented(int total_tokens, int num_seqs, int h_v) {
  const size_t whole = max_chunks(total_tokens, num_seqs) * (size_t)h_v * kWsHead;
  return (size_t)num_seqs * h_v * 8 <= 2 * kStateCus && segmented_workspace_bytes(num_seqs, h_v) < whole;
}

}  // namespace

size_t chunk_prefill_workspace_bytes(int total_tokens, int num_seqs, int h_qk, int h_v) {
  (void)h_qk;
  // with no tokens there are no chunks: no prep launch, and the state pass only copies each
  // initial state to its final state without touching the workspace
  if (total_tokens == 0) return 0;
  if (prefill_segmented(total_tokens, num_seqs, h_v)) return segmented_workspace_bytes(num_seqs, h_v);
  return max_chunks(total_tokens, num_seqs) * (size_t)h_v * kWsHead;
}

namespace {

// The two launches of a chunked prefill.
hipError_t launch_prefill(PrefillArgs a, int total_tokens, hipStream_t stream) {
  // With up to one (sequence, V head) pair per CU the state pass reads P^T from the
  // workspace; beyond, one workgroup per head forms it on chip (no P^T traffic; with every
  // CU busy that costs less than reading it).
  const size_t nc = (size_t)a.n_chunks_max;
  const size_t heads = (size_t)a.num_seqs * a.h_v;
  const bool with_p = heads <= kStateCus;
  if (total_tokens > 0) {
    // V heads of one QK head pair up in the workgroups when their number is even
    const size_t pairs = nc * (size_t)a.h_qk;
    const int hp = a.group % 2 == 0 ? 2 : 1;
    const size_t prep_blocks = (pairs + 7) / 8 * 8 * (size_t)(a.group / hp);
    const dim3 grid((unsigned)prep_blocks), block(4 * hp * kWave);
    if (with_p) {
      if (hp == 2) hipLaunchKernelGGL((prep_kernel<true, 2>), grid, block, 0, stream, a);
      else hipLaunchKernelGGL((prep_kernel<true, 1>), grid, block, 0, stream, a);
    } else {
      if (hp == 2) hipLaunchKernelGGL((prep_kernel<false, 2>), grid, block, 0, stream, a);
      else hipLaunchKernelGGL((prep_kernel<false, 1>), grid, block, 0, stream, a);
    }
  }
  // With few heads, eight or two workgroups per head spread the heads over many CUs: eight,
  // with the chain, the loads and the read-out on waves of their own, up to two rounds of
  // workgroups (64 pairs; its chunk step is so much shorter that two rounds of it beat one
  // round of a shape whose waves run the whole chunk alone); two up to 128 pairs. Beyond,
  // one 8-wave workgroup per head (two waves per SIMD to hide latency) avoids the operand
  // traffic every workgroup repeats, and once the heads outnumber the CUs it forms P^T
  // itself.
  const size_t seq_pairs = (size_t)a.num_seqs * a.h_qk;
  const size_t groups = (seq_pairs + 7) / 8 * 8 * (size_t)a.group;
  if (heads * 8 <= 2 * kStateCus) {
    hipLaunchKernelGGL(state_ro_kernel, dim3((unsigned)(groups * 8)), dim3(4 * kWave), 0, stream, a);
  } else if (heads * 2 <= kStateCus) {
    hipLaunchKernelGGL((state_kernel<4, false>), dim3((unsigned)(groups * 2)), dim3(4 * kWave), 0, stream, a);
  } else if (heads <= kStateCus) {
    hipLaunchKernelGGL((state_kernel<8, false>), dim3((unsigned)groups), dim3(8 * kWave), 0, stream, a);
  } else {
    hipLaunchKernelGGL((state_kernel<8, true>), dim3((unsigned)groups), dim3(8 * kWave), 0, stream, a);
  }
  return hipGetLastError();
}

PrefillArgs prefill_args(const float* g, const float* beta, const int32_t* cu_seqlens, int num_seqs,
                         int total_tokens, int h_qk, int h_v, float scale, const float* s0,
                         float* s_final, void* o, void* workspace) {
  PrefillArgs a{};
  a.g = g;
  a.beta = beta;
  a.cu = cu_seqlens;
  a.s0 = s0;
  a.s_final = s_final;
  a.o = static_cast<bf16*>(o);
  a.ws = static_cast<uint8_t*>(workspace);
  a.num_seqs = num_seqs;
  a.h_qk = h_qk;
  a.h_v = h_v;
  a.group = h_v / h_qk;
  a.n_chunks_max = (int)max_chunks(total_tokens, num_seqs);
  a.scale = scale;
  return a;
}

}  // namespace

hipError_t launch_chunk_prefill(const void* q, const void* k, const void* v, const float* g,
                                const float* beta, const int32_t* cu_seqlens, int num_seqs,
                                int total_tokens, int h_qk, int h_v, float scale,
                                const float* s0, float* s_final, void* o, void* workspace,
                                hipStream_t stream) {
  PrefillArgs a = prefill_args(g, beta, cu_seqlens, num_seqs, total_tokens, h_qk, h_v, scale, s0,
                               s_final, o, workspace);
  a.q = static_cast<const bf16*>(q);
  a.k = static_cast<const bf16*>(k);
  a.v = static_cast<const bf16*>(v);
  if (!prefill_segmented(total_tokens, num_seqs, h_v)) return launch_prefill(a, total_tokens, stream);
  // segments of kSegChunks chunks of every sequence; as many as the longest possible
  // sequence (all the tokens in one) needs (a segment past a sequence's end does nothing)
  a.seg_len = kSegChunks;
  a.n_chunks_max = num_seqs * kSegChunks;
  a.carry = reinterpret_cast<float*>(a.ws + (size_t)num_seqs * kSegChunks * h_v * kWsHead);
  const int n_seg = max(1, ((total_tokens + kC - 1) / kC + kSegChunks - 1) / kSegChunks);
  for (int s = 0; s < n_seg; ++s) {
    a.seg_lo = s * kSegChunks;
    const hipError_t e = launch_prefill(a, total_tokens, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// The front end and the prefill in one call: the front end's q, k and v go to the workspace,
// after the prefill's own blocks, and the prefill reads them there. (Two forms that ran the
// front end inside the prefill's loads instead were measured slower: the conversion then
// lands on the latency-bound prefill kernels at low occupancy, where the standalone pass
// spreads it over the whole chip.)
size_t chunk_prefill_conv_workspace_bytes(int total_tokens, int num_seqs, int h_qk, int h_v) {
  return chunk_prefill_workspace_bytes(total_tokens, num_seqs, h_qk, h_v) +
         (size_t)total_tokens * (2 * h_qk + h_v) * kD * 2;
}

hipError_t launch_chunk_prefill_conv(const void* mixed, const float* conv_weight, int conv_kernel,
                                     float q_scale, const float* g, const float* beta,
                                     const int32_t* cu_seqlens, int num_seqs, int total_tokens,
                                     int h_qk, int h_v, float scale, const float* s0, float* s_final,
                                     void* o, void* workspace, hipStream_t stream) {
  uint8_t* qkv = static_cast<uint8_t*>(workspace) + chunk_prefill_workspace_bytes(total_tokens, num_seqs, h_qk, h_v);
  bf16* q = reinterpret_cast<bf16*>(qkv);
  bf16* k = q + (size_t)total_tokens * h_qk * kD;
  bf16* v = k + (size_t)total_tokens * h_qk * kD;
  if (total_tokens > 0) {
    const hipError_t e = launch_conv_prep(mixed, conv_weight, conv_kernel, cu_seqlens, num_seqs, total_tokens, h_qk,
                                          h_v, q_scale, q, k, v, stream);
    if (e != hipSuccess) return e;
  }
  return launch_chunk_prefill(q, k, v, g, beta, cu_seqlens, num_seqs, total_tokens, h_qk, h_v, scale, s0, s_final,
                              o, workspace, stream);
}

}  // namespace gdn
