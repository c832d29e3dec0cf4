// Device-side helpers shared by the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace mla {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }

template <typename T>
__device__ __forceinline__ T from_f32(float x);
template <>
__device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }  // RNE

// Wave-wide (64 lanes) reductions.
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Reductions over lane pairs (i, i ^ 16) and (i, i ^ 32) with the gfx950 row-swap
// instructions (one VALU op each, no LDS round trip).  With both operands holding v, the two
// results of v_permlane16_swap are v[i & ~16] and v[i | 16] in every lane i (for
// v_permlane32_swap, v[i & ~32] and v[i | 32]): the lane's own value and its partner's.
// (The results are copied to scalars before the bit casts: a bit cast applied directly to an
// element of the returned vector reads element 0 whatever the index.)
__device__ __forceinline__ void pair16(float v, float* a, float* b) {
  const unsigned u = __builtin_bit_cast(unsigned, v);
  const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const unsigned r0 = r[0], r1 = r[1];
  *a = __builtin_bit_cast(float, r0);
  *b = __builtin_bit_cast(float, r1);
}
__device__ __forceinline__ void pair32(float v, float* a, float* b) {
  const unsigned u = __builtin_bit_cast(unsigned, v);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  const unsigned r0 = r[0], r1 = r[1];
  *a = __builtin_bit_cast(float, r0);
  *b = __builtin_bit_cast(float, r1);
}
__device__ __forceinline__ float max_xor16(float v) { float a, b; pair16(v, &a, &b); return fmaxf(a, b); }
__device__ __forceinline__ float max_xor32(float v) { float a, b; pair32(v, &a, &b); return fmaxf(a, b); }
__device__ __forceinline__ float sum_xor16(float v) { float a, b; pair16(v, &a, &b); return a + b; }
__device__ __forceinline__ float sum_xor32(float v) { float a, b; pair32(v, &a, &b); return a + b; }

// RoPE frequencies theta^(-2k/d_rope) for k < d_rope/2, computed on the host in fp64 and
// passed by value as a kernel argument (d_rope <= 256).
struct RopeFreq {
  double f[128];
};

// cos/sin of the rotation angle pos * f: the product and its reduction to [-pi, pi] are done
// in fp64 (positions reach 2^26), the trigonometric functions in fp32 on the reduced angle.
// Tokens query token qi of s_q sees in sequence b: the causal limit L - s_q + 1 + qi, with L =
// seqlens[b] clamped to [0, max_seqlen] as the split plan clamps it (s_q = 1: L).
__device__ __forceinline__ int causal_limit(const int32_t* seqlens, int b, int max_seqlen, int sq,
                                            int qi) {
  return min(max(seqlens[b], 0), max_seqlen) - sq + 1 + qi;
}

__device__ __forceinline__ void rope_cos_sin(int pos, double f, float* c, float* s) {
  constexpr double kTwoPi = 6.283185307179586476925286766559;
  double a = (double)pos * f;
  a -= kTwoPi * rint(a * (1.0 / kTwoPi));
  sincosf((float)a, s, c);
}

}  // namespace mla
