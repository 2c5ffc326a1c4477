// Device helpers shared by the gfx950 kernels: element types, conversions,
// MFMA fragments and RoPE angles.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ga {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kWave = 64;

// ---- element conversions ---------------------------------------------------
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return static_cast<float>(x); }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) {
  return static_cast<bf16>(x);  // round to nearest even (v_cvt_pk_bf16_f32)
}

// ---- 8-element operand fragment -------------------------------------------
// One lane's share of an MFMA operand with 8 values along the reduction
// index: a bf16 fragment feeds one K=32/K=16 bf16 MFMA; an fp32 fragment feeds
// eight K=4/K=2 fp32 MFMAs, element j of every lane forming MFMA j.  The
// reduction index is a sum, so any fixed map of (lane group, j) to k works as
// long as both operands use the same one.
template <typename T> struct Frag8;
template <> struct Frag8<bf16> { bf16x8 v; };
template <> struct Frag8<float> { float v[8]; };

template <typename T> struct Frag4;
template <> struct Frag4<bf16> { bf16x4 v; };
template <> struct Frag4<float> { float v[4]; };

// 16 bytes (bf16) or 32 bytes (fp32) from memory into a fragment.
__device__ __forceinline__ void load_frag(Frag8<bf16>& f, const bf16* p) {
  f.v = *reinterpret_cast<const bf16x8*>(p);
}
__device__ __forceinline__ void load_frag(Frag8<float>& f, const float* p) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p);
  const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
  f.v[0] = a[0]; f.v[1] = a[1]; f.v[2] = a[2]; f.v[3] = a[3];
  f.v[4] = b[0]; f.v[5] = b[1]; f.v[6] = b[2]; f.v[7] = b[3];
}

// C[32x32] += A[32x16] * B[16x32]; lane l holds row (A) / column (B) l%32.
__device__ __forceinline__ void mma32(f32x16& c, const Frag8<bf16>& a, const Frag8<bf16>& b) {
  c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.v, b.v, c, 0, 0, 0);
}
__device__ __forceinline__ void mma32(f32x16& c, const Frag8<float>& a, const Frag8<float>& b) {
#pragma unroll
  for (int j = 0; j < 8; ++j) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.v[j], b.v[j], c, 0, 0, 0);
}

// C[16x16] += A[16x32] * B[32x16]; lane l holds row (A) / column (B) l%16.
__device__ __forceinline__ void mma16(f32x4& c, const Frag8<bf16>& a, const Frag8<bf16>& b) {
  c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, c, 0, 0, 0);
}
__device__ __forceinline__ void mma16(f32x4& c, const Frag8<float>& a, const Frag8<float>& b) {
#pragma unroll
  for (int j = 0; j < 8; ++j) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[j], b.v[j], c, 0, 0, 0);
}

// C[16x16] += A[16x16] * B[16x16], 4 values per lane along the reduction index.
__device__ __forceinline__ void mma16k16(f32x4& c, const Frag4<bf16>& a, const Frag4<bf16>& b) {
  c = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a.v),
                                                __builtin_bit_cast(s16x4, b.v), c, 0, 0, 0);
}
__device__ __forceinline__ void mma16k16(f32x4& c, const Frag4<float>& a, const Frag4<float>& b) {
#pragma unroll
  for (int j = 0; j < 4; ++j) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[j], b.v[j], c, 0, 0, 0);
}

template <typename T> __device__ __forceinline__ void frag_set(Frag8<T>& f, int j, float x);
template <> __device__ __forceinline__ void frag_set(Frag8<bf16>& f, int j, float x) { f.v[j] = from_f32<bf16>(x); }
template <> __device__ __forceinline__ void frag_set(Frag8<float>& f, int j, float x) { f.v[j] = x; }
template <typename T> __device__ __forceinline__ void frag_set(Frag4<T>& f, int j, float x);
template <> __device__ __forceinline__ void frag_set(Frag4<bf16>& f, int j, float x) { f.v[j] = from_f32<bf16>(x); }
template <> __device__ __forceinline__ void frag_set(Frag4<float>& f, int j, float x) { f.v[j] = x; }

// ---- RoPE angles -----------------------------------------------------------
// Pair i of a head of dim d turns by pos * theta^(-2i/d).  The product and the
// sine/cosine are taken in fp64 (fp32 loses the angle at long positions) and
// rounded to fp32 once.
__device__ __forceinline__ double rope_omega(int pair, int head_dim, double log2_theta) {
  return exp2(-(2.0 * pair / head_dim) * log2_theta);
}
__device__ __forceinline__ f32x2 rope_cos_sin(double angle) {
  double s, c;
  sincos(angle, &s, &c);
  f32x2 r;
  r[0] = static_cast<float>(c);
  r[1] = static_cast<float>(s);
  return r;
}

// Rotate the pair (x0, x1) counter-clockwise by the angle with (cos, sin) = cs.
__device__ __forceinline__ void rotate_pair(float& x0, float& x1, f32x2 cs) {
  const float a = x0 * cs[0] - x1 * cs[1];
  const float b = x0 * cs[1] + x1 * cs[0];
  x0 = a;
  x1 = b;
}

// ---- wave helpers ----------------------------------------------------------
__device__ __forceinline__ float wave_xor(float x, int mask) { return __shfl_xor(x, mask, kWave); }

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

}  // namespace ga
