// gdn_device.h -- device-side helpers shared by the gfx950 kernels of libgdn.
//
// bf16 <-> fp32 conversion (round to nearest even), packed operand types for the CDNA4
// matrix-core builtins, and wave-level exchanges.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef __bf16 bf16;
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kHeadDim = 128;
constexpr int kWave = 64;

// fp32 -> bf16, round to nearest even (the compiler's conversion does RNE on gfx950).
__device__ __forceinline__ bf16 to_bf16(float x) { return (bf16)x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }

__device__ __forceinline__ f32x4 load4(const bf16* p) {
  bf16x4 v = *reinterpret_cast<const bf16x4*>(p);
  return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
}
__device__ __forceinline__ f32x4 load4(const float* p) {
  return *reinterpret_cast<const f32x4*>(p);
}
__device__ __forceinline__ float load1(const bf16* p) { return (float)*p; }
__device__ __forceinline__ float load1(const float* p) { return *p; }
__device__ __forceinline__ void store1(bf16* p, float x) { *p = to_bf16(x); }
__device__ __forceinline__ void store1(float* p, float x) { *p = x; }

// Eight bf16 from two groups of four fp32 (the A/B operand of a 16x16x32 bf16 MFMA).
__device__ __forceinline__ bf16x8 pack8(f32x4 a, f32x4 b) {
  bf16x8 r;
  r[0] = to_bf16(a[0]); r[1] = to_bf16(a[1]); r[2] = to_bf16(a[2]); r[3] = to_bf16(a[3]);
  r[4] = to_bf16(b[0]); r[5] = to_bf16(b[1]); r[6] = to_bf16(b[2]); r[7] = to_bf16(b[3]);
  return r;
}

// Two 4-element bf16 halves read from separate places, joined into one operand.
__device__ __forceinline__ bf16x8 join8(bf16x4 a, bf16x4 b) {
  return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// D = A(16x32) * B(32x16) + C on the bf16 matrix cores, fp32 accumulation.
// Lane l holds A[l%16][8*(l/16) .. +7], B[8*(l/16) .. +7][l%16], C[4*(l/16) .. +3][l%16].
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Lane exchanges within a half-wave without the LDS crossbar where the pattern stays inside
// a 16-lane row: the value of lane l ^ m, by DPP for m = 1 and 2 (quad permutes), 4 (half-row
// mirror, then quad reversal: l ^ 7 ^ 3), 8 (row rotation by 8), and by ds_swizzle (xor mask
// within 32 lanes) for m = 16. Pure data movement: sums built from it are unchanged. Every
// DPP pattern here reads a lane of the same row and all rows and banks are written, so the
// move needs no old value (none is materialised) and the bound control never applies.
__device__ __forceinline__ float xor_lane(float x, int m) {
  const int v = __builtin_bit_cast(int, x);
  int r;
  switch (m) {
    case 1: r = __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, true); break;
    case 2: r = __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, true); break;
    case 4: r = __builtin_amdgcn_mov_dpp(__builtin_amdgcn_mov_dpp(v, 0x141, 0xF, 0xF, true),
                                         0x1B, 0xF, 0xF, true); break;
    case 8: r = __builtin_amdgcn_mov_dpp(v, 0x128, 0xF, 0xF, true); break;
    default: r = __builtin_amdgcn_ds_swizzle(v, 0x401F); break;   // m = 16
  }
  return __builtin_bit_cast(float, r);
}

// Sum over the 32 lanes of each half-wave; every lane receives its half's total.
__device__ __forceinline__ float half_wave_sum(float x) {
  x += __shfl_xor(x, 16, 32);
  x += __shfl_xor(x, 8, 32);
  x += __shfl_xor(x, 4, 32);
  x += __shfl_xor(x, 2, 32);
  x += __shfl_xor(x, 1, 32);
  return x;
}

}  // namespace gdn
