/*
 * kda_common.h -- device-side building blocks shared by the KDA kernels
 * (gfx950, wave64): element types, bf16 rounding, the gate of eq. (5), and
 * the 16x16 MFMA tiles used for every dense contraction.
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
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

/* Four floats to bf16 (round to nearest even) as two packed conversions.
 * Converting the halves as 2-vectors, joined as 32-bit words, keeps the
 * compiler on the packed instruction; a 4-vector taken straight from an MFMA
 * result is otherwise converted one element at a time and re-packed with
 * permutes. */
__device__ __forceinline__ bf16x4 pack_bf16x4(const f32x4& x) {
  const bf16x2 lo = __builtin_convertvector(__builtin_shufflevector(x, x, 0, 1), bf16x2);
  const bf16x2 hi = __builtin_convertvector(__builtin_shufflevector(x, x, 2, 3), bf16x2);
  typedef uint32_t pair_t __attribute__((ext_vector_type(2)));
  const pair_t u = {__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
  return __builtin_bit_cast(bf16x4, u);
}

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }

template <typename T>
__device__ __forceinline__ T from_f32(float x);
template <>
__device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }  // round to nearest even

/*
 * Buffer resources: a base address and a size in bytes, held in scalar
 * registers.  Loads through them take a 32-bit per-lane byte offset and return
 * zero beyond the size (stores there are dropped), so a chunk's loads need no
 * 64-bit address arithmetic and no branch for a ragged tail.
 */
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRsrcWord3 = 0x00020000;  // raw, untyped 32-bit access (gfx9 family)
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int n = bytes <= 0 ? 0 : (int)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, n, kRsrcWord3);
}

/* A loaded input element held in its own 32-bit register until it is used
 * (bf16: the raw bits, zero-extended; fp32: the bits of the value). */
template <typename IO>
struct Raw;
template <>
struct Raw<bf16> {
  __device__ __forceinline__ static uint32_t load(rsrc_t r, int off) {
    return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
  }
  __device__ __forceinline__ static float f32(uint32_t x) { return __uint_as_float(x << 16); }
  __device__ __forceinline__ static void store(rsrc_t r, int off, float x) {
    __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, (bf16)x), r, off, 0, 0);
  }
};
template <>
struct Raw<float> {
  __device__ __forceinline__ static uint32_t load(rsrc_t r, int off) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
  }
  __device__ __forceinline__ static float f32(uint32_t x) { return __uint_as_float(x); }
  __device__ __forceinline__ static void store(rsrc_t r, int off, float x) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), r, off, 0, 0);
  }
};
__device__ __forceinline__ float load_f32(rsrc_t r, int off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}

/* Eq. (5) in base 2 without the floor factor: sigmoid(a) via the hardware
 * exp2 and reciprocal (each within about one ulp); g * log2(e) is
 * (-5 log2 e) times this. */
__device__ __forceinline__ float sigmoid_fast(float a) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-a * kLog2e));
}

/*
 * MFMA operands (16x16 tiles, wave64).  Lane l supplies row (A) or column
 * (B) l % 16 of its operand; its group h = l / 16 and a slot index name the
 * k index.  The hardware pairs slot s of group h in A with slot s of group h
 * in B, so any fixed assignment of k indices to (h, s) gives the same
 * product as long as both operands use it.
 *
 *   K = 16 fragments (4 slots):  k = 4h + s  -- the natural order, which is
 *     also where the 16x16 accumulator keeps its rows (lane l, register j
 *     holds row 4(l/16) + j of column l % 16), so a result feeds the next
 *     contraction as its B operand without moving data between lanes.
 *   K = 32 fragments (8 slots):  k = kappa(h, s) = 16 (s / 4) + 4 h + s % 4,
 *     the rows that the accumulators of two stacked 16-row tiles put in lane
 *     group h, again so that accumulators convert in place.
 */
__host__ __device__ constexpr int kappa(int h, int s) { return 16 * (s / 4) + 4 * h + (s % 4); }
__host__ __device__ constexpr int kappa_group(int r) { return (r % 16) / 4; }          // h with kappa(h, s) = r
__host__ __device__ constexpr int kappa_slot(int r) { return 4 * (r / 16) + (r % 4); }  // s with kappa(h, s) = r

template <typename T>
struct Frag8;  // K = 32 fragment
template <>
struct Frag8<bf16> {
  bf16x8 v;
};
template <>
struct Frag8<float> {
  float v[8];
};
template <typename T>
struct Frag4;  // K = 16 fragment
template <>
struct Frag4<bf16> {
  bf16x4 v;
};
template <>
struct Frag4<float> {
  float v[4];
};

/* acc(16x16) += A(16 x 32) B(32 x 16) */
__device__ __forceinline__ void mfma_k32(f32x4& acc, const Frag8<bf16>& a, const Frag8<bf16>& b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, acc, 0, 0, 0);
}
__device__ __forceinline__ void mfma_k32(f32x4& acc, const Frag8<float>& a, const Frag8<float>& b) {
#pragma unroll
  for (int s = 0; s < 8; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[s], b.v[s], acc, 0, 0, 0);
}
/* acc(16x16) += A(16 x 16) B(16 x 16) */
__device__ __forceinline__ void mfma_k16(f32x4& acc, const Frag4<bf16>& a, const Frag4<bf16>& b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a.v, b.v, acc, 0, 0, 0);
}
__device__ __forceinline__ void mfma_k16(f32x4& acc, const Frag4<float>& a, const Frag4<float>& b) {
#pragma unroll
  for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[s], b.v[s], acc, 0, 0, 0);
}

template <typename T>
__device__ __forceinline__ Frag4<T> frag4(float x0, float x1, float x2, float x3) {
  Frag4<T> f;
  f.v[0] = from_f32<T>(x0);
  f.v[1] = from_f32<T>(x1);
  f.v[2] = from_f32<T>(x2);
  f.v[3] = from_f32<T>(x3);
  return f;
}
template <typename T>
__device__ __forceinline__ Frag4<T> frag4(const f32x4& x) {
  if constexpr (sizeof(T) == 2) {
    Frag4<T> f;
    f.v = pack_bf16x4(x);
    return f;
  } else {
    return frag4<T>(x[0], x[1], x[2], x[3]);
  }
}
/* K = 32 fragment from two stacked accumulator tiles (rows 0..15, 16..31). */
template <typename T>
__device__ __forceinline__ Frag8<T> frag8(const f32x4& lo, const f32x4& hi) {
  Frag8<T> f;
  if constexpr (sizeof(T) == 2) {
    f.v = __builtin_shufflevector(pack_bf16x4(lo), pack_bf16x4(hi), 0, 1, 2,
                                  3, 4, 5, 6, 7);
  } else {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      f.v[s] = lo[s];
      f.v[4 + s] = hi[s];
    }
  }
  return f;
}

template <typename T>
__device__ __forceinline__ Frag8<T> load_frag8(const T* p) {
  Frag8<T> f;
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
template <typename T>
__device__ __forceinline__ Frag4<T> load_frag4(const T* p) {
  Frag4<T> f;
  if constexpr (sizeof(T) == 2) {
    f.v = *reinterpret_cast<const bf16x4*>(p);
  } else {
    f32x4 x = *reinterpret_cast<const f32x4*>(p);
#pragma unroll
    for (int s = 0; s < 4; ++s) f.v[s] = x[s];
  }
  return f;
}
template <typename T>
__device__ __forceinline__ void store_frag4(T* p, const Frag4<T>& f) {
  if constexpr (sizeof(T) == 2) {
    *reinterpret_cast<bf16x4*>(p) = f.v;
  } else {
    f32x4 x = {f.v[0], f.v[1], f.v[2], f.v[3]};
    *reinterpret_cast<f32x4*>(p) = x;
  }
}

}  // namespace kda
