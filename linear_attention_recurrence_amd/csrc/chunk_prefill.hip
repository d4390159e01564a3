// chunk_prefill.hip -- chunked gated delta rule prefill on gfx950 bf16 matrix cores.
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
// One workgroup (4 waves) owns one (sequence, V head, block of 64 value rows) and walks the
// sequence's chunks in order, carrying its 64 x 128 slice of S in fp32 registers (value rows
// evolve independently, so slices need no exchange). Per chunk, in LDS:
//   1. load K, Q (and K^T, V^T copies), g, beta; zero-pad the ragged tail (a token with
//      k = q = v = 0, beta = 0, g = 0 leaves S unchanged and emits 0);
//   2. prefix sum of g;
//   3. K K^T and Q K^T lower tiles on the matrix cores -> A (fp32) and P (bf16, with Gam
//      and scale folded in);
//   4. T = (I + A)^-1 in fp32: 16 x 16 diagonal blocks by substitution, then the
//      off-diagonal blocks level by level;
//   5. -W and U~ on the matrix cores (T diag(beta) split into hi + lo bf16 so U~ keeps
//      ~16 mantissa bits; the other operands are exact bf16 inputs);
//   6. per wave (16 value rows): U, O and the state update on the matrix cores. S^T stays
//      in the accumulator layout and is fed back as the B operand with a permuted K order
//      (see below); the decayed U enters the state update as a hi + lo pair.
//
// Matrix-core layout (v_mfma_f32_16x16x32_bf16): lane l holds A[l%16][8*(l/16)+s],
// B[8*(l/16)+s][l%16] for s = 0..7, and C[4*(l/16)+i][l%16] for i = 0..3. A product is
// unchanged when the same permutation is applied to the K index of A and B, so a
// C-layout accumulator pair covering K rows k0..k0+15 and k0+16..k0+31 is a valid B
// operand once its A partner reads K entries {4g..4g+3, 16+4g..16+4g+3} (g = l/16).
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {
namespace {

constexpr int kC = 64;          // chunk length
constexpr int kD = 128;         // head dim
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;
constexpr int kDvBlock = 16 * kWaves;   // value rows per workgroup
constexpr int kRowPad = kD + 8;         // [token][d_k] rows, bf16
constexpr int kTokPad = kC + 8;         // [x][token] rows, bf16
constexpr int kF32Pad = kC + 4;         // [token][token] rows, fp32

struct Smem {
  bf16 K[kC][kRowPad];
  bf16 Q[kC][kRowPad];
  bf16 W[kC][kRowPad];          // -W
  bf16 KT[kD][kTokPad];
  bf16 VT[kDvBlock][kTokPad];
  bf16 P[kC][kTokPad];          // scale * (Q K^T o Gam), lower incl. diagonal
  bf16 Tbg[kC][kTokPad];        // -T diag(beta gam)
  bf16 Tbh[kC][kTokPad];        // T diag(beta), high part
  bf16 Tbl[kC][kTokPad];        // T diag(beta), low part
  float A[kC][kF32Pad];
  float T[kC][kF32Pad];
  float X[3][16][17];
  float G[kC];
  float gam[kC];
  float beta[kC];
};

struct ChunkArgs {
  const bf16* q;
  const bf16* k;
  const bf16* v;
  const float* g;
  const float* beta;
  const int32_t* cu;
  const float* s0;
  float* s_final;
  bf16* o;
  int num_seqs, h_qk, h_v;
  float scale;
};

// (row tile, col tile) of the 10 lower tiles and the 6 strictly upper tiles of a 4x4 grid
__device__ __forceinline__ void lower_tile(int t, int& rt, int& ct) {
  rt = t < 1 ? 0 : t < 3 ? 1 : t < 6 ? 2 : 3;
  ct = t - rt * (rt + 1) / 2;
}
__device__ __forceinline__ void upper_tile(int t, int& rt, int& ct) {
  rt = t < 3 ? 0 : t < 5 ? 1 : 2;
  ct = t < 3 ? t + 1 : t < 5 ? t - 1 : 3;
}

__device__ __forceinline__ bf16x8 lds8(const bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }
__device__ __forceinline__ bf16x4 lds4(const bf16* p) { return *reinterpret_cast<const bf16x4*>(p); }
// A operand whose K order matches a C-layout accumulator pair (see the header comment)
__device__ __forceinline__ bf16x8 lds_perm(const bf16* row, int k0, int g4) {
  return join8(lds4(row + k0 + 4 * g4), lds4(row + k0 + 16 + 4 * g4));
}

__global__ __launch_bounds__(kThreads) void chunk_prefill_kernel(ChunkArgs a) {
  __shared__ Smem sm;
  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int g4 = lane >> 4;
  const int l16 = lane & 15;

  constexpr int kBlocks = kD / kDvBlock;
  int bid = blockIdx.x;
  const int dvb = bid % kBlocks;
  bid /= kBlocks;
  const int h = bid % a.h_v;
  const int n = bid / a.h_v;
  const int j = h / (a.h_v / a.h_qk);
  const int t_seq0 = a.cu[n];
  const int t_seq1 = a.cu[n + 1];
  const int col_blk = dvb * kDvBlock;          // first value row of this workgroup
  const int my_col = col_blk + 16 * w + l16;   // value row owned by this lane
  const size_t state_off = (((size_t)n * a.h_v + h) * kD + my_col) * kD;

  // St[mt][i] = S[my_col][16*mt + 4*g4 + i]
  f32x4 St[8];
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) {
    if (a.s0) St[mt] = *reinterpret_cast<const f32x4*>(a.s0 + state_off + 16 * mt + 4 * g4);
    else St[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  for (int c0 = t_seq0; c0 < t_seq1; c0 += kC) {
    const int nv = min(kC, t_seq1 - c0);
    __syncthreads();   // every wave is done with the previous chunk's LDS

    // ---- 1. load ---------------------------------------------------------------------
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int p = tid + kThreads * i;          // 1024 pieces of 8 bf16
      const int row = p >> 4, cb = p & 15;
      bf16x8 kv = {}, qv = {};
      if (row < nv) {
        const size_t off = ((size_t)(c0 + row) * a.h_qk + j) * kD + cb * 8;
        kv = *reinterpret_cast<const bf16x8*>(a.k + off);
        qv = *reinterpret_cast<const bf16x8*>(a.q + off);
      }
      *reinterpret_cast<bf16x8*>(&sm.K[row][cb * 8]) = kv;
      *reinterpret_cast<bf16x8*>(&sm.Q[row][cb * 8]) = qv;
#pragma unroll
      for (int e = 0; e < 8; ++e) sm.KT[cb * 8 + e][row] = kv[e];
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int p = tid + kThreads * i;          // 512 pieces of 8 bf16
      const int row = p >> 3, cb = p & 7;
      bf16x8 vv = {};
      if (row < nv)
        vv = *reinterpret_cast<const bf16x8*>(a.v + ((size_t)(c0 + row) * a.h_v + h) * kD +
                                              col_blk + cb * 8);
#pragma unroll
      for (int e = 0; e < 8; ++e) sm.VT[cb * 8 + e][row] = vv[e];
    }
    if (tid < kC) {
      float gg = 0.f, bb = 0.f;
      if (tid < nv) {
        gg = a.g[(size_t)(c0 + tid) * a.h_v + h];
        bb = a.beta[(size_t)(c0 + tid) * a.h_v + h];
      }
      sm.G[tid] = gg;
      sm.beta[tid] = bb;
    }
    __syncthreads();

    // ---- 2. inclusive prefix sum of log-decays -----------------------------------------
    if (w == 0) {
      float x = sm.G[lane];
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
      }
      sm.G[lane] = x;
      sm.gam[lane] = __expf(x);
    }
    __syncthreads();

    // ---- 3. K K^T -> A, Q K^T -> P (lower tiles), zero upper tiles ----------------------
    for (int job = w; job < 20; job += kWaves) {
      const bool isq = job >= 10;
      int rt, ct;
      lower_tile(isq ? job - 10 : job, rt, ct);
      const bf16* arow = isq ? &sm.Q[16 * rt + l16][0] : &sm.K[16 * rt + l16][0];
      const bf16* brow = &sm.K[16 * ct + l16][0];
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        acc = mfma16x16x32(lds8(arow + 32 * ks + 8 * g4), lds8(brow + 32 * ks + 8 * g4), acc);
      const int s = 16 * ct + l16;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * rt + 4 * g4 + i;
        const float decay = __expf(fminf(sm.G[r] - sm.G[s], 0.f));
        if (isq) sm.P[r][s] = to_bf16(s <= r ? a.scale * decay * acc[i] : 0.f);
        else sm.A[r][s] = s < r ? sm.beta[r] * decay * acc[i] : 0.f;
      }
    }
    for (int e = tid; e < 6 * 256; e += kThreads) {
      int rt, ct;
      upper_tile(e >> 8, rt, ct);
      const int r = 16 * rt + ((e & 255) >> 4), s = 16 * ct + (e & 15);
      sm.P[r][s] = to_bf16(0.f);
      sm.A[r][s] = 0.f;
      sm.T[r][s] = 0.f;
    }
    __syncthreads();

    // ---- 4. T = (I + A)^-1 ----------------------------------------------------------------
    // 4a. diagonal 16x16 blocks: wave b inverts block b, one lane per column
    if (lane < 16) {
      const int b0 = 16 * w, c = lane;
      float x[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) x[r] = (r == c) ? 1.f : 0.f;
#pragma unroll
      for (int r = 1; r < 16; ++r) {
        float s = 0.f;
#pragma unroll
        for (int m = 0; m < r; ++m) s += sm.A[b0 + r][b0 + m] * x[m];
        if (r > c) x[r] = -s;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) sm.T[b0 + r][b0 + c] = x[r];
    }
    __syncthreads();
    // 4b. block (i, b), i = b + d: T_ib = -T_ii * sum_{k=b}^{i-1} A_ik T_kb
#pragma unroll 1
    for (int d = 1; d < 4; ++d) {
      const int jobs = 4 - d;
      for (int e = tid; e < jobs * 256; e += kThreads) {
        const int b = e >> 8, r = (e & 255) >> 4, c = e & 15, i = b + d;
        float s = 0.f;
        for (int m = 16 * b; m < 16 * i; ++m) s += sm.A[16 * i + r][m] * sm.T[m][16 * b + c];
        sm.X[b][r][c] = s;
      }
      __syncthreads();
      for (int e = tid; e < jobs * 256; e += kThreads) {
        const int b = e >> 8, r = (e & 255) >> 4, c = e & 15, i = b + d;
        float s = 0.f;
#pragma unroll
        for (int m = 0; m < 16; ++m) s += sm.T[16 * i + r][16 * i + m] * sm.X[b][m][c];
        sm.T[16 * i + r][16 * b + c] = -s;
      }
      __syncthreads();
    }

    // ---- 5a. operands from T ----------------------------------------------------------------
    for (int e = tid; e < kC * kC; e += kThreads) {
      const int r = e >> 6, s = e & 63;
      const float tb = sm.T[r][s] * sm.beta[s];
      sm.Tbg[r][s] = to_bf16(-tb * sm.gam[s]);
      const bf16 hi = to_bf16(tb);
      sm.Tbh[r][s] = hi;
      sm.Tbl[r][s] = to_bf16(tb - (float)hi);
    }
    __syncthreads();

    // ---- 5b. -W = (-T diag(beta gam)) K; wave w: columns tiles 2w, 2w+1 ---------------------
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      const int ct = 2 * w + cc;
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks <= rt / 2; ++ks)
          acc = mfma16x16x32(lds8(&sm.Tbg[16 * rt + l16][32 * ks + 8 * g4]),
                             lds8(&sm.KT[16 * ct + l16][32 * ks + 8 * g4]), acc);
#pragma unroll
        for (int i = 0; i < 4; ++i) sm.W[16 * rt + 4 * g4 + i][16 * ct + l16] = to_bf16(acc[i]);
      }
    }
    // ---- 5c. U~ = T diag(beta) V for this wave's 16 value rows (hi + lo) --------------------
    f32x4 U[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      U[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks <= rt / 2; ++ks) {
        const bf16x8 bv = lds8(&sm.VT[16 * w + l16][32 * ks + 8 * g4]);
        U[rt] = mfma16x16x32(lds8(&sm.Tbh[16 * rt + l16][32 * ks + 8 * g4]), bv, U[rt]);
        U[rt] = mfma16x16x32(lds8(&sm.Tbl[16 * rt + l16][32 * ks + 8 * g4]), bv, U[rt]);
      }
    }
    __syncthreads();   // -W complete

    // ---- 6. the state pass for this wave's 16 value rows ------------------------------------
    bf16x8 Sb[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) Sb[ks] = pack8(St[2 * ks], St[2 * ks + 1]);
    // U = U~ - W S^T
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      const bf16* wrow = &sm.W[16 * rt + l16][0];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) U[rt] = mfma16x16x32(lds_perm(wrow, 32 * ks, g4), Sb[ks], U[rt]);
    }
    // O = scale gam (Q S^T) + P U
    bf16x8 Ub[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) Ub[ks] = pack8(U[2 * ks], U[2 * ks + 1]);
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      const bf16* qrow = &sm.Q[16 * rt + l16][0];
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) acc = mfma16x16x32(lds_perm(qrow, 32 * ks, g4), Sb[ks], acc);
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] *= a.scale * sm.gam[16 * rt + 4 * g4 + i];
      const bf16* prow = &sm.P[16 * rt + l16][0];
#pragma unroll
      for (int ks = 0; ks <= rt / 2; ++ks) acc = mfma16x16x32(lds_perm(prow, 32 * ks, g4), Ub[ks], acc);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * rt + 4 * g4 + i;
        if (r < nv) a.o[((size_t)(c0 + r) * a.h_v + h) * kD + my_col] = to_bf16(acc[i]);
      }
    }
    // S^T <- gam_C S^T + K^T (diag(gam_C / gam) U), the decayed U as hi + lo
    const float GC = sm.G[kC - 1];
    const float gC = sm.gam[kC - 1];
    f32x4 Uh[4], Ul[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float u = U[rt][i] * __expf(GC - sm.G[16 * rt + 4 * g4 + i]);
        const float hi = (float)to_bf16(u);
        Uh[rt][i] = hi;
        Ul[rt][i] = u - hi;
      }
    }
    bf16x8 Bh[2], Bl[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      Bh[ks] = pack8(Uh[2 * ks], Uh[2 * ks + 1]);
      Bl[ks] = pack8(Ul[2 * ks], Ul[2 * ks + 1]);
    }
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
      St[mt] *= gC;
      const bf16* krow = &sm.KT[16 * mt + l16][0];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const bf16x8 ak = lds_perm(krow, 32 * ks, g4);
        St[mt] = mfma16x16x32(ak, Bh[ks], St[mt]);
        St[mt] = mfma16x16x32(ak, Bl[ks], St[mt]);
      }
    }
  }

  if (a.s_final) {
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
      *reinterpret_cast<f32x4*>(a.s_final + state_off + 16 * mt + 4 * g4) = St[mt];
  }
}

}  // namespace

hipError_t launch_chunk_prefill(const void* q, const void* k, const void* v, const float* g,
                                const float* beta, const int32_t* cu_seqlens, int num_seqs,
                                int h_qk, int h_v, float scale, const float* s0,
                                float* s_final, void* o, hipStream_t stream) {
  ChunkArgs a;
  a.q = static_cast<const bf16*>(q);
  a.k = static_cast<const bf16*>(k);
  a.v = static_cast<const bf16*>(v);
  a.g = g;
  a.beta = beta;
  a.cu = cu_seqlens;
  a.s0 = s0;
  a.s_final = s_final;
  a.o = static_cast<bf16*>(o);
  a.num_seqs = num_seqs;
  a.h_qk = h_qk;
  a.h_v = h_v;
  a.scale = scale;
  const dim3 grid((unsigned)num_seqs * (unsigned)h_v * (kD / kDvBlock));
  hipLaunchKernelGGL(chunk_prefill_kernel, grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace gdn
