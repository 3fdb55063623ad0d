// Device-side helpers shared by the gfx950 kernels: element types, MFMA fragment traits,
// wave64 reductions. Lane layouts of the MFMA instructions used here (checked on gfx950):
//   v_mfma_f32_16x16x32_bf16: A lane l holds row l%16, k = 8*(l/16) .. +7;
//                             B lane l holds col l%16, k = 8*(l/16) .. +7;
//                             C lane l holds col l%16, rows 4*(l/16) .. +3.
//   v_mfma_f32_16x16x4f32:    A row l%16, k = l/16; B col l%16, k = l/16; C as above.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mor {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int WAVE = 64;
#define MOR_MAX_REC_DEV 8

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
// Round to nearest even (the gfx950 conversion instruction).
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }

// Four consecutive elements of T, stored with one vector store.
template <typename T> struct Vec4;
template <> struct Vec4<float> {
  typedef float4 type;
  static __device__ __forceinline__ void store(float* p, float a, float b, float c, float d) {
    *reinterpret_cast<float4*>(p) = make_float4(a, b, c, d);
  }
};
template <> struct Vec4<bf16> {
  static __device__ __forceinline__ void store(bf16* p, float a, float b, float c, float d) {
    bf16x4 v = {(bf16)a, (bf16)b, (bf16)c, (bf16)d};
    *reinterpret_cast<bf16x4*>(p) = v;
  }
};

// One MFMA step: KSTEP k-elements per instruction, KW of them per lane.
template <typename T> struct Mma;
template <> struct Mma<bf16> {
  static constexpr int KSTEP = 32, KW = 8;
  typedef bf16x8 frag;
  static __device__ __forceinline__ frag load(const bf16* p) {
    return *reinterpret_cast<const bf16x8*>(p);
  }
  static __device__ __forceinline__ f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};
template <> struct Mma<float> {
  static constexpr int KSTEP = 4, KW = 1;
  typedef float frag;
  static __device__ __forceinline__ frag load(const float* p) { return *p; }
  static __device__ __forceinline__ f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
};

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Fixed-order fp32 dot product of one row with w (the router logit order): lane l sums
// x[i]*w[i] for i = l, l+64, ... ascending, product and sum each rounded (no contraction),
// then the partials fold as p_l + p_{l+o}, o = 32..1. Every lane returns the result.
// Product and sum rounded separately: these operations carry no contraction flag, so they
// are never fused into an FMA.
__device__ __forceinline__ float mul_rn(float a, float b) {
#pragma clang fp contract(off)
  return a * b;
}
__device__ __forceinline__ float add_rn(float a, float b) {
#pragma clang fp contract(off)
  return a + b;
}

__device__ __forceinline__ float fold_fixed(float p) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) p = add_rn(p, __shfl_xor(p, o));
  return p;
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (WAVE - 1); }

}  // namespace mor
