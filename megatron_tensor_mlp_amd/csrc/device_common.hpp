// Device-side types and element-wise functions shared by the gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tpmlp {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Activation codes, equal to tp_act in tpmlp.h.
enum : int { ACT_NONE = 0, ACT_RELU = 1, ACT_GELU_TANH = 2, ACT_GELU_ERF = 3, ACT_SWIGLU = 4 };

// Element-wise activations in fp32.  The pages name GeLU and Swish without a
// formula; the published definitions are used, evaluated with the device math
// library (tanhf, erff, expf).
//   GeLU tanh form: 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3)))
//   GeLU erf form:  0.5 x (1 + erf(x / sqrt 2))
//   SiLU (Swish, slope 1): x / (1 + exp(-x))
template <int ACT>
__device__ __forceinline__ float activate(float x) {
  if constexpr (ACT == ACT_RELU) {
    return x > 0.0f ? x : 0.0f;
  } else if constexpr (ACT == ACT_GELU_TANH) {
    const float c = 0.7978845608028654f;  // sqrt(2/pi)
    return 0.5f * x * (1.0f + tanhf(c * (x + 0.044715f * x * x * x)));
  } else if constexpr (ACT == ACT_GELU_ERF) {
    return 0.5f * x * (1.0f + erff(x * 0.7071067811865476f));
  } else if constexpr (ACT == ACT_SWIGLU) {  // the SiLU half of SwiGLU
    return x / (1.0f + expf(-x));
  } else {
    return x;
  }
}

__device__ __forceinline__ float silu(float x) { return activate<ACT_SWIGLU>(x); }

// Epilogue forms of the activations whose result is rounded to bf16 next:
// the exponential and the reciprocal are single instructions (v_exp_f32,
// v_rcp_f32, each within about an fp32 ulp), far below bf16's 2^-8.
//   SiLU:  x / (1 + 2^(-x log2 e))
//   tanh:  1 - 2 / (1 + 2^(2 z log2 e))   (for the GeLU tanh form)
__device__ __forceinline__ float silu_fast(float x) {
  return x * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * x));
}
__device__ __forceinline__ float tanh_fast(float z) {
  return 1.0f - 2.0f * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(2.8853900817779268f * z));
}
template <int ACT>
__device__ __forceinline__ float activate_fast(float x) {
  if constexpr (ACT == ACT_GELU_TANH) {
    const float c = 0.7978845608028654f;  // sqrt(2/pi)
    return 0.5f * x * (1.0f + tanh_fast(c * (x + 0.044715f * x * x * x)));
  } else if constexpr (ACT == ACT_SWIGLU) {
    return silu_fast(x);
  } else {
    return activate<ACT>(x);
  }
}

// Lanes 2j and 2j+1 exchange a 32-bit value (DPP quad permutation 1,0,3,2).
__device__ __forceinline__ uint32_t swap_adjacent_lanes(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);
}

// Derivatives of the activations (for the backward pass), from the
// definitions above by the chain rule:
//   GeLU tanh form: with t = tanh(sqrt(2/pi) (x + 0.044715 x^3)),
//                   0.5 (1 + t) + 0.5 x (1 - t^2) sqrt(2/pi) (1 + 3 * 0.044715 x^2)
//   GeLU erf form:  0.5 (1 + erf(x / sqrt 2)) + x exp(-x^2 / 2) / sqrt(2 pi)
//   SiLU:           s (1 + x (1 - s)), s = 1 / (1 + exp(-x))
//   ReLU:           1 for x > 0, else 0
template <int ACT>
__device__ __forceinline__ float dactivate(float x) {
  if constexpr (ACT == ACT_RELU) {
    return x > 0.0f ? 1.0f : 0.0f;
  } else if constexpr (ACT == ACT_GELU_TANH) {
    const float c = 0.7978845608028654f;  // sqrt(2/pi)
    const float t = tanhf(c * (x + 0.044715f * x * x * x));
    return 0.5f * (1.0f + t) + 0.5f * x * (1.0f - t * t) * c * (1.0f + 0.134145f * x * x);
  } else if constexpr (ACT == ACT_GELU_ERF) {
    return 0.5f * (1.0f + erff(x * 0.7071067811865476f)) +
           x * expf(-0.5f * x * x) * 0.3989422804014327f;  // 1/sqrt(2 pi)
  } else if constexpr (ACT == ACT_SWIGLU) {  // SiLU'
    const float s = 1.0f / (1.0f + expf(-x));
    return s * (1.0f + x * (1.0f - s));
  } else {
    return 1.0f;
  }
}

// fp32 -> bf16, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ bf16 to_bf16(float x) { return (bf16)x; }

__device__ __forceinline__ float bf16_bits_to_float(uint32_t lo16) {
  return __uint_as_float(lo16 << 16);
}

// Combine the low (or high) 16-bit halves of two dwords into one dword:
// result = lo_half(a) | lo_half(b) << 16   (or the high halves).
__device__ __forceinline__ uint32_t pack_lo(uint32_t a, uint32_t b) {
  return (a & 0xffffu) | (b << 16);
}
__device__ __forceinline__ uint32_t pack_hi(uint32_t a, uint32_t b) {
  return (a >> 16) | (b & 0xffff0000u);
}

}  // namespace tpmlp
