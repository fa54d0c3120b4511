/*
 * kda_common.h -- device-side building blocks shared by the KDA kernels
 * (gfx950, wave64): element types, bf16 rounding, the gate of eq. (5), and
 * the 32x32 MFMA tile used for every dense contraction.
 */
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

constexpr int kD = 128;     // d_k = d_v
constexpr int kChunk = 16;  // tokens per chunk
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kGateFloor = -5.0f;  // g_min of eq. (5)

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }

template <typename T>
__device__ __forceinline__ T from_f32(float x);
template <>
__device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }  // round to nearest even

/* Eq. (5) in base 2: g * log2(e) = -5 log2(e) sigmoid(a), using the hardware
 * exp2 and reciprocal (both within about one ulp). */
__device__ __forceinline__ float gate_log2(float a) {
  float e = __builtin_amdgcn_exp2f(-a * kLog2e);
  return (kGateFloor * kLog2e) * __builtin_amdgcn_rcpf(1.0f + e);
}

/*
 * MFMA operands.  One K16 fragment is 8 values per lane covering a K = 16
 * slice of a contraction: lane l supplies row (A) or column (B) l % 32, and
 * its half l / 32 together with the slot s in 0..7 names the k index.  The
 * hardware pairs slot s of half h in A with slot s of half h in B, so any
 * fixed assignment of the 16 k indices to (h, s) gives the same product as
 * long as both operands use it.
 *
 * The kernels use the assignment induced by the 32x32 accumulator layout
 * (lane l, register 4i + j holds row 8i + 4(l/32) + j of column l % 32): for a
 * block of 16 rows, slot s of half h is row kappa(h, s) = 8(s/4) + 4h + s%4.
 * With that assignment the first or last 8 accumulator registers of a tile
 * are directly a K16 fragment of the tile's rows, so a result can feed the
 * next contraction without moving data between lanes.
 */
__host__ __device__ constexpr int kappa(int h, int s) { return 8 * (s / 4) + 4 * h + (s % 4); }
__host__ __device__ constexpr int kappa_half(int r) { return (r / 4) % 2; }            // h with kappa(h, s) = r
__host__ __device__ constexpr int kappa_slot(int r) { return 4 * (r / 8) + (r % 4); }  // s with kappa(h, s) = r

template <typename T>
struct Frag;
template <>
struct Frag<bf16> {
  bf16x8 v;
};
template <>
struct Frag<float> {
  float v[8];
};

/* acc += A(32 x 16) * B(16 x 32) for one K16 fragment pair. */
__device__ __forceinline__ void mfma_k16(f32x16& acc, const Frag<bf16>& a, const Frag<bf16>& b) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.v, b.v, acc, 0, 0, 0);
}
__device__ __forceinline__ void mfma_k16(f32x16& acc, const Frag<float>& a, const Frag<float>& b) {
#pragma unroll
  for (int s = 0; s < 8; ++s) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.v[s], b.v[s], acc, 0, 0, 0);
}

/* Fragment from 8 consecutive accumulator registers acc[base .. base+7]. */
template <typename T>
__device__ __forceinline__ Frag<T> frag_from_acc(const f32x16& acc, int base);
template <>
__device__ __forceinline__ Frag<bf16> frag_from_acc<bf16>(const f32x16& acc, int base) {
  Frag<bf16> f;
#pragma unroll
  for (int s = 0; s < 8; ++s) f.v[s] = (bf16)acc[base + s];
  return f;
}
template <>
__device__ __forceinline__ Frag<float> frag_from_acc<float>(const f32x16& acc, int base) {
  Frag<float> f;
#pragma unroll
  for (int s = 0; s < 8; ++s) f.v[s] = acc[base + s];
  return f;
}

template <typename T>
__device__ __forceinline__ Frag<T> frag_from_f32(const float* x);
template <>
__device__ __forceinline__ Frag<bf16> frag_from_f32<bf16>(const float* x) {
  Frag<bf16> f;
#pragma unroll
  for (int s = 0; s < 8; ++s) f.v[s] = (bf16)x[s];
  return f;
}
template <>
__device__ __forceinline__ Frag<float> frag_from_f32<float>(const float* x) {
  Frag<float> f;
#pragma unroll
  for (int s = 0; s < 8; ++s) f.v[s] = x[s];
  return f;
}

template <typename T>
__device__ __forceinline__ Frag<T> frag_zero() {
  float z[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  return frag_from_f32<T>(z);
}

/* Load one K16 fragment (8 contiguous elements) from LDS. */
template <typename T>
__device__ __forceinline__ Frag<T> frag_load(const T* p) {
  Frag<T> f;
  if constexpr (sizeof(T) == 2) {
    f.v = *reinterpret_cast<const bf16x8*>(p);
  } else {
    const f32x4* q = reinterpret_cast<const f32x4*>(p);
    f32x4 lo = q[0], hi = q[1];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      f.v[s] = lo[s];
      f.v[4 + s] = hi[s];
    }
  }
  return f;
}

}  // namespace kda
