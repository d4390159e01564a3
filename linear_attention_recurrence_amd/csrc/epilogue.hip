// epilogue.hip -- the output epilogue after the token mixer (gfx950).
//
// For each (token, V head) vector x of d_v = 128 read-out channels and the gate input z at
// the same place:
//     out = x / sqrt(mean(x^2) + eps) * (1 + w) * gate(z),   gate = sigmoid or SiLU
// The norm is the zero-centred RMS norm that the architecture knowledge-base page
// "Qwen3-Next 80B-A3B" names in its "Architecture" table (row "Norm type"), taken over one
// head at a time; the gate is the output gate of section "01 . GatedDeltaNet(config)" of
// page "Qwen3-Next 80B-A3B -- The Evolving Transformer", which decides how much of the
// recurrent read-out reaches the output. The pages give no formula for either; the norm
// comes first and the gate multiplies its result.
//
// Layout: 16 lanes per vector, 8 consecutive channels per lane (one 16-byte load of bf16),
// so a wave holds 4 vectors and the mean square is finished by four exchanges inside a
// 16-lane DPP row. Memory bound: 768 bytes per vector in bf16 (o and z read, out written);
// the 512-byte weight vector stays in cache.
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {
namespace {

constexpr int kVecPerBlock = 16;   // 256 threads

// The loads return the words as stored; widen() turns them into fp32. o and z are read once,
// so their loads are non-temporal (100 MB with the inputs rotated so no cache holds them:
// 19.7 against 21.9 us); the weight vector is read cached.
template <typename IO> struct Raw8 { u32x4 w[sizeof(IO) / 2]; };

template <typename IO>
__device__ __forceinline__ Raw8<IO> load_nt(const IO* p) {
  Raw8<IO> r;
#pragma unroll
  for (int i = 0; i < (int)(sizeof(IO) / 2); ++i)
    r.w[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p) + i);
  return r;
}
__device__ __forceinline__ void widen(const Raw8<bf16>& r, float (&x)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __builtin_bit_cast(float, r.w[0][i] << 16);
    x[2 * i + 1] = __builtin_bit_cast(float, r.w[0][i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void widen(const Raw8<float>& r, float (&x)[8]) {
#pragma unroll
  // the element is copied out first: a bit cast applied to a vector element itself reads
  // element 0 of the vector with this compiler
  for (int i = 0; i < 8; ++i) x[i] = __builtin_bit_cast(float, (uint32_t)r.w[i / 4][i % 4]);
}
__device__ __forceinline__ void store8(bf16* p, const float (&y)[8]) {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = to_bf16(y[i]);
  *reinterpret_cast<bf16x8*>(p) = r;
}
__device__ __forceinline__ void store8(float* p, const float (&y)[8]) {
  reinterpret_cast<f32x4*>(p)[0] = f32x4{y[0], y[1], y[2], y[3]};
  reinterpret_cast<f32x4*>(p)[1] = f32x4{y[4], y[5], y[6], y[7]};
}

// SILU selects the gate z * sigmoid(z); otherwise sigmoid(z). A 16-lane group past the
// last vector reads the last vector (its lanes run the same code, so the row exchanges
// stay within live data) and stores nothing.
template <typename IO, bool SILU>
__global__ __launch_bounds__(256) void gated_rmsnorm_kernel(const IO* o, const IO* z, const float* w,
                                                            IO* out, long long n_vec, float eps) {
  const int lane16 = threadIdx.x & 15;
  const long long vec = (long long)blockIdx.x * kVecPerBlock + (threadIdx.x >> 4);
  const bool live = vec < n_vec;
  const size_t base = (size_t)(live ? vec : n_vec - 1) * kHeadDim + 8 * lane16;
  Raw8<IO> ro = load_nt(o + base), rz = load_nt(z + base);
  f32x4 w0 = reinterpret_cast<const f32x4*>(w + 8 * lane16)[0];
  f32x4 w1 = reinterpret_cast<const f32x4*>(w + 8 * lane16)[1];
  // z and w feed only the stored result; left free, the compiler issues their loads inside
  // the store's branch, after the mean square has waited for o: two memory round trips
  // instead of one. Passing them through an empty asm here keeps all the loads together.
#pragma unroll
  for (int i = 0; i < (int)(sizeof(IO) / 2); ++i) asm volatile("" : "+v"(rz.w[i]));
  asm volatile("" : "+v"(w0), "+v"(w1));
  float x[8], zg[8], wt[8];
  widen(ro, x);
  widen(rz, zg);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    wt[i] = w0[i];
    wt[4 + i] = w1[i];
  }
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) ss += x[i] * x[i];
  ss += xor_lane(ss, 1);
  ss += xor_lane(ss, 2);
  ss += xor_lane(ss, 4);
  ss += xor_lane(ss, 8);
  const float inv_rms = rsqrtf(ss * (1.f / kHeadDim) + eps);
  float y[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float sig = 1.f / (1.f + __expf(-zg[i]));
    y[i] = x[i] * inv_rms * (1.f + wt[i]) * (SILU ? zg[i] * sig : sig);
  }
  if (live) store8(out + base, y);
}

template <typename IO>
hipError_t launch_typed(const void* o, const void* z, const float* w, void* out, long long n_vec,
                        float eps, bool silu, hipStream_t stream) {
  const dim3 grid((unsigned)((n_vec + kVecPerBlock - 1) / kVecPerBlock)), block(256);
  const IO* po = static_cast<const IO*>(o);
  const IO* pz = static_cast<const IO*>(z);
  IO* pout = static_cast<IO*>(out);
  if (silu)
    hipLaunchKernelGGL((gated_rmsnorm_kernel<IO, true>), grid, block, 0, stream, po, pz, w, pout, n_vec, eps);
  else
    hipLaunchKernelGGL((gated_rmsnorm_kernel<IO, false>), grid, block, 0, stream, po, pz, w, pout, n_vec, eps);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gated_rmsnorm(const void* o, const void* z, bool io_bf16, const float* weight,
                                long long n_vec, float eps, bool silu, void* out,
                                hipStream_t stream) {
  if (n_vec == 0) return hipSuccess;
  return io_bf16 ? launch_typed<bf16>(o, z, weight, out, n_vec, eps, silu, stream)
                 : launch_typed<float>(o, z, weight, out, n_vec, eps, silu, stream);
}

}  // namespace gdn
