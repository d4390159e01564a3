// conv_device.h -- device code of the front end shared by the kernels that produce its
// outputs (the packed front end, its decode-time form, and the decode step that runs the
// front end itself), so that every one of them computes each output with the same code.
//
// The front end is the short causal depthwise convolution that section "01 .
// GatedDeltaNet(config)" of page "Qwen3-Next 80B-A3B -- The Evolving Transformer" places
// before the recurrence, followed by SiLU, the L2 normalisation of each q and k head and a
// scale on q.
#pragma once

#include "gdn_device.h"

namespace gdn {

// The taps of this thread's 8 channels: wt[0][e] multiplies the current token, wt[d][e] the
// token d positions earlier (zero past the kernel size K).
__device__ __forceinline__ void load_taps(const float* w, int K, int c0, float (&wt)[4][8]) {
  if (K == 4) {   // the model's kernel: each channel's taps are one 16-byte load
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const f32x4 t = *reinterpret_cast<const f32x4*>(w + (size_t)(c0 + e) * 4);
#pragma unroll
      for (int d = 0; d < 4; ++d) wt[d][e] = t[3 - d];
    }
    return;
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
#pragma unroll
    for (int d = 0; d < 4; ++d) wt[d][e] = (d < K) ? w[(size_t)(c0 + e) * K + (K - 1 - d)] : 0.f;
  }
}

// One token of this thread's 8 channels from its input x0 and the inputs h1, h2, h3 one,
// two and three tokens earlier: the convolution, SiLU and, for q and k heads, the head's L2
// normalisation over the 16 lanes that share the head (and the q scale). The prefill and
// decode kernels both produce every output through this function.
__device__ __forceinline__ bf16x8 conv_token(const float (&wt)[4][8], const float (&x0)[8], const float (&h1)[8],
                                             const float (&h2)[8], const float (&h3)[8], bool is_q, bool is_k,
                                             float q_scale) {
  // Every operation is spelled out (explicit fused multiply-adds, no contraction left to the
  // compiler), so each kernel that includes this computes the same bits whatever the code
  // around it: the compiler's own contraction choices differed between instantiations.
#pragma clang fp contract(off)
  float z[8];
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float y = __builtin_fmaf(wt[3][e], h3[e], __builtin_fmaf(wt[2][e], h2[e],
                    __builtin_fmaf(wt[1][e], h1[e], wt[0][e] * x0[e])));
    z[e] = y * __builtin_amdgcn_rcpf(1.f + __expf(-y));   // hardware 1-ulp reciprocal
    ss = __builtin_fmaf(z[e], z[e], ss);
  }
  bf16x8 out;
  if (is_q || is_k) {
    ss += __shfl_xor(ss, 8, 16);
    ss += __shfl_xor(ss, 4, 16);
    ss += __shfl_xor(ss, 2, 16);
    ss += __shfl_xor(ss, 1, 16);
    // 1 / max(||z||, 1e-12) = rsqrt(max(||z||^2, 1e-24)), hardware 1-ulp rsqrt
    const float f = (is_q ? q_scale : 1.f) * __builtin_amdgcn_rsqf(fmaxf(ss, 1e-24f));
#pragma unroll
    for (int e = 0; e < 8; ++e) out[e] = to_bf16(z[e] * f);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) out[e] = to_bf16(z[e]);
  }
  return out;
}

}  // namespace gdn
