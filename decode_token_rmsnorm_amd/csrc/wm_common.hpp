// wm_common.hpp — element types, 16-byte fragments and the MFMA step shared
// by the GEMM and attention kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wm {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Elements per 16-byte fragment.
template <typename T> struct Elt;
template <> struct Elt<float> { static constexpr int E16 = 4; };
template <> struct Elt<bf16> { static constexpr int E16 = 8; };

__device__ __forceinline__ float to_f(float x) { return x; }
__device__ __forceinline__ float to_f(bf16 x) { return (float)x; }
template <typename T> __device__ __forceinline__ T from_f(float x);
template <> __device__ __forceinline__ float from_f<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f<bf16>(float x) { return (bf16)x; }

// One 16x16 output tile step of D += A * B^T where every lane supplies one
// 16-byte fragment of A (row lane%16) and of B (column lane%16), both covering
// the same k-slice for lane group lane/16.  bf16: one 16x16x32 MFMA over 32 k.
// float: four 16x16x4 MFMAs, element e of every lane forming the e-th one,
// together covering 16 k.  The accumulator layout is the same for both: lane
// holds rows 4*(lane/16)+i (i<4) of column lane%16.
template <typename T> __device__ __forceinline__ void mma16(f32x4 &acc, const u32x4 &a, const u32x4 &b);

template <> __device__ __forceinline__ void mma16<bf16>(f32x4 &acc, const u32x4 &a, const u32x4 &b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), acc,
                                                0, 0, 0);
}

// (Vector elements are passed by value: a bit cast applied directly to an
// ext-vector element lvalue was seen to read element 0 for every e.)
template <> __device__ __forceinline__ void mma16<float>(f32x4 &acc, const u32x4 &a, const u32x4 &b) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t ae = a[e], be = b[e];
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(ae), __uint_as_float(be), acc, 0, 0, 0);
  }
}

// Unpack / pack a 16-byte fragment to / from floats.
template <typename T> __device__ __forceinline__ void unpack16(const u32x4 &v, float *f);
template <> __device__ __forceinline__ void unpack16<float>(const u32x4 &v, float *f) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t x = v[e];
    f[e] = __uint_as_float(x);
  }
}
template <> __device__ __forceinline__ void unpack16<bf16>(const u32x4 &v, float *f) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t x = v[e];
    f[2 * e] = __uint_as_float(x << 16);
    f[2 * e + 1] = __uint_as_float(x & 0xffff0000u);
  }
}
template <typename T> __device__ __forceinline__ u32x4 pack16(const float *f);
template <> __device__ __forceinline__ u32x4 pack16<float>(const float *f) {
  u32x4 v;
#pragma unroll
  for (int e = 0; e < 4; ++e) v[e] = __float_as_uint(f[e]);
  return v;
}
// (a pair converted as one 2-vector becomes a single v_cvt_pk_bf16_f32, RNE)
template <> __device__ __forceinline__ u32x4 pack16<bf16>(const float *f) {
  u32x4 v;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const bf16x2 p = {(bf16)f[2 * e], (bf16)f[2 * e + 1]};
    v[e] = __builtin_bit_cast(uint32_t, p);
  }
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Sum over aligned groups of `width` lanes (width a power of two <= 64).
__device__ __forceinline__ float group_sum(float v, int width) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1)
    if (o < width) v += __shfl_xor(v, o);
  return v;
}

// x * sigmoid(x) with the hardware reciprocal (1 ulp) instead of a full
// IEEE division.
__device__ __forceinline__ float silu(float x) { return x * __builtin_amdgcn_rcpf(1.0f + __expf(-x)); }

}  // namespace wm
