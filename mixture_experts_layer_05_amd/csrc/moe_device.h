// Device-side helpers shared by the MoE kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

constexpr int kWave = 64;

// bf16 <-> fp32 ---------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// round-to-nearest-even fp32 -> bf16 (finite inputs; NaN kept quiet)
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return static_cast<uint32_t>(f32_to_bf16(lo)) | (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
}

// wave64 reductions ------------------------------------------------------
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// wave64 reductions without LDS: DPP within each 16-lane row (xor 1 and 2
// by quad permutation, then the half-row and row mirrors), then the four
// row results read as scalars.  The result is wave-uniform.
template <int kCtrl>
__device__ __forceinline__ int dpp_(int v) {
  return __builtin_amdgcn_update_dpp(v, v, kCtrl, 0xf, 0xf, false);
}
constexpr int kDppXor1 = 0xb1, kDppXor2 = 0x4e, kDppHalfMirror = 0x141, kDppMirror = 0x140;

__device__ __forceinline__ float wave_max_dpp(float v) {
  v = fmaxf(v, __int_as_float(dpp_<kDppXor1>(__float_as_int(v))));
  v = fmaxf(v, __int_as_float(dpp_<kDppXor2>(__float_as_int(v))));
  v = fmaxf(v, __int_as_float(dpp_<kDppHalfMirror>(__float_as_int(v))));
  v = fmaxf(v, __int_as_float(dpp_<kDppMirror>(__float_as_int(v))));
  const int b = __float_as_int(v);
  return fmaxf(fmaxf(__int_as_float(__builtin_amdgcn_readlane(b, 0)),
                     __int_as_float(__builtin_amdgcn_readlane(b, 16))),
               fmaxf(__int_as_float(__builtin_amdgcn_readlane(b, 32)),
                     __int_as_float(__builtin_amdgcn_readlane(b, 48))));
}
__device__ __forceinline__ int wave_min_dpp(int v) {
  v = min(v, dpp_<kDppXor1>(v));
  v = min(v, dpp_<kDppXor2>(v));
  v = min(v, dpp_<kDppHalfMirror>(v));
  v = min(v, dpp_<kDppMirror>(v));
  return min(min(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
             min(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
}
// sum in a fixed order: pairs, quads, half rows, rows, then rows 0..3
__device__ __forceinline__ float wave_sum_dpp(float v) {
  v += __int_as_float(dpp_<kDppXor1>(__float_as_int(v)));
  v += __int_as_float(dpp_<kDppXor2>(__float_as_int(v)));
  v += __int_as_float(dpp_<kDppHalfMirror>(__float_as_int(v)));
  v += __int_as_float(dpp_<kDppMirror>(__float_as_int(v)));
  const int b = __float_as_int(v);
  return (__int_as_float(__builtin_amdgcn_readlane(b, 0)) +
          __int_as_float(__builtin_amdgcn_readlane(b, 16))) +
         (__int_as_float(__builtin_amdgcn_readlane(b, 32)) +
          __int_as_float(__builtin_amdgcn_readlane(b, 48)));
}

__device__ __forceinline__ float sigmoidf_(float z) { return 1.0f / (1.0f + expf(-z)); }

// Epilogue forms: e^-z as 2^(-z log2 e) and the hardware reciprocal (about
// one ulp each); z -> -inf gives 2^+inf = inf and a sigmoid of 0.
__device__ __forceinline__ float sigmoid_fast(float z) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(z * -1.4426950408889634f));
}

typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2v;
// four fp32 -> four bf16 in 8 bytes, hardware round-to-nearest-even
__device__ __forceinline__ u32x2 pack4_bf16(float a, float b, float c, float d) {
  const f32x2 lo = {a, b}, hi = {c, d};
  return u32x2{__builtin_bit_cast(uint32_t, __builtin_convertvector(lo, bf16x2v)),
               __builtin_bit_cast(uint32_t, __builtin_convertvector(hi, bf16x2v))};
}
// silu(z) = z * sigmoid(z); written as a quotient so that very negative z
// (expf(-z) = +inf) gives -0 instead of NaN.
__device__ __forceinline__ float siluf_(float z) { return z / (1.0f + expf(-z)); }

__device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }

}  // namespace moe
