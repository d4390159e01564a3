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

__device__ __forceinline__ void load8(const bf16* p, float (&x)[8]) {
  const u32x4 w = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __builtin_bit_cast(float, w[i] << 16);
    x[2 * i + 1] = __builtin_bit_cast(float, w[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void load8(const float* p, float (&x)[8]) {
  const f32x4 a = reinterpret_cast<const f32x4*>(p)[0];
  const f32x4 b = reinterpret_cast<const f32x4*>(p)[1];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[i] = a[i];
    x[4 + i] = b[i];
  }
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
  float x[8], zg[8], wt[8];
  load8(o + base, x);
  load8(z + base, zg);
  load8(w + 8 * lane16, wt);
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
