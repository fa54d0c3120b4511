/*
 * kda_bf16_tiles.h -- LDS and register helpers of the bf16 prefill kernels
 * (gfx950): transposing LDS reads, bf16 packing, DPP broadcasts and the
 * wave / workgroup synchronisation they rely on.
 *
 * ds_read_b64_tr_b16 transposes 16-bit elements across the lanes of each
 * 16-lane group while it reads: lane i, element j of the result is element
 * i % 4 of the 8 bytes that lane 4j + i/4 addressed.
 */
#pragma once

#include "kda_common.h"

namespace kda {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ __forceinline__ bf16x4 lds_tr(const bf16* p) {
  return __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p)));
}
__device__ __forceinline__ bf16x4 lds_b64(const bf16* p) { return *reinterpret_cast<const bf16x4*>(p); }
__device__ __forceinline__ void lds_put(bf16* p, const f32x4& x) {
  *reinterpret_cast<bf16x4*>(p) = pack_bf16x4(x);
}
__device__ __forceinline__ f32x4 bf16x4_to_f32(bf16x4 b) {
  const u32x2 u = __builtin_bit_cast(u32x2, b);
  f32x4 r = {__uint_as_float(u[0] << 16), __uint_as_float(u[0] & 0xffff0000u), __uint_as_float(u[1] << 16),
             __uint_as_float(u[1] & 0xffff0000u)};
  return r;
}
__device__ __forceinline__ Frag8<bf16> cat8(bf16x4 lo, bf16x4 hi) {
  Frag8<bf16> f;
  f.v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return f;
}
__device__ __forceinline__ Frag4<bf16> f4(bf16x4 x) {
  Frag4<bf16> f;
  f.v = x;
  return f;
}
/* The value of lane J of this lane's quad (DPP quad permutation). */
template <int J>
__device__ __forceinline__ float quad_bcast(float x) {
  constexpr int ctrl = J | (J << 2) | (J << 4) | (J << 6);
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), ctrl, 0xf, 0xf, true));  // folds into the user
}
/* The value of the lane N places further round this lane's 16-lane row
 * (DPP row_ror:N, 1 <= N <= 15). */
template <int N>
__device__ __forceinline__ float row_ror(float x) {
  static_assert(N >= 1 && N <= 15, "row_ror takes 1 .. 15");
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x120 + N, 0xf, 0xf, false));
}
/* s_waitcnt vmcnt(0), the other counters untouched (gfx9 encoding). */
__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0 | (0x7 << 4) | (0xf << 8)); }
/* Workgroup barrier (the same fences as __syncthreads).  Kernels whose waves
 * run separate loops call it the same number of times on every path. */
__device__ __forceinline__ void block_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

}  // namespace kda
