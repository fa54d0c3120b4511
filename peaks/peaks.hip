/*
 * peaks.hip -- micro-benchmarks that measure what the MI355X reaches on the
 * two roofs the KDA kernels are held against, on the same box and in the same
 * run: a streaming device copy (HBM bandwidth) and back-to-back bf16 / fp32
 * MFMA loops (matrix throughput).  Measurement infrastructure only: the
 * kernels of the KDA path neither use nor link this library.
 *
 *   peaks_copy        dst = src, 16 bytes a lane per access with the
 *                     non-temporal hint, grid-stride over the buffer
 *   peaks_read        the same reads alone (decode and prefill read far
 *                     more than they write)
 *   peaks_mfma_bf16   every wave issues iters x 8 independent
 *                     v_mfma_f32_16x16x32_bf16 (16 x 16 x 32 x 2 flops each)
 *   peaks_mfma_f32    the same with v_mfma_f32_16x16x4_f32 (16 x 16 x 4 x 2)
 *                     (and 4 independent v_mfma_f32_32x32x16_bf16 per iteration)
 *   peaks_valu        8 independent chains a lane of v_exp_f32, v_rcp_f32 or
 *                     v_mul_f32: how long a transcendental instruction holds
 *                     the VALU against a plain one
 * The MFMA results are summed and stored, so nothing is optimised away.
 */
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kThreads = 256;
constexpr int kUnroll = 4;

__global__ __launch_bounds__(kThreads) void copy_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                        uint64_t n) {
  const uint64_t stride = (uint64_t)gridDim.x * kThreads;
  uint64_t i = (uint64_t)blockIdx.x * kThreads + threadIdx.x;
  // whole groups of kUnroll accesses: every index < n
  for (; i + (kUnroll - 1) * stride < n; i += kUnroll * stride) {
    u32x4 x[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) x[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) __builtin_nontemporal_store(x[u], dst + i + u * stride);
  }
  for (; i < n; i += stride) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

/* A read-only pass (a sum, stored per thread so nothing is optimised away). */
__global__ __launch_bounds__(kThreads) void read_kernel(const u32x4* __restrict__ src, uint32_t* __restrict__ out,
                                                        uint64_t n) {
  const uint64_t stride = (uint64_t)gridDim.x * kThreads;
  uint64_t i = (uint64_t)blockIdx.x * kThreads + threadIdx.x;
  u32x4 acc = {0, 0, 0, 0};
  for (; i + (kUnroll - 1) * stride < n; i += kUnroll * stride) {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc += __builtin_nontemporal_load(src + i + u * stride);
  }
  for (; i < n; i += stride) acc += __builtin_nontemporal_load(src + i);
  out[(size_t)blockIdx.x * kThreads + threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

typedef float f32x16 __attribute__((ext_vector_type(16)));

/* v_mfma_f32_32x32x16_bf16 (32 x 32 x 16 x 2 flops), four independent accumulators. */
__global__ __launch_bounds__(kThreads) void mfma32_kernel(float* __restrict__ out, int iters) {
  const int t = threadIdx.x;
  f32x16 acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[j][e] = 0.0f;
  bf16x8 a, b;
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    a[s] = (__bf16)(0.001f * (float)((t + s) & 7));
    b[s] = (__bf16)(0.002f * (float)((t * 3 + s) & 7));
  }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[j][e];
  out[(size_t)blockIdx.x * kThreads + t] = s;
}

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

/* v_mfma_f32_16x16x16_bf16 (16 x 16 x 16 x 2 flops), 16 independent accumulators. */
__global__ __launch_bounds__(kThreads) void mfma16k16_kernel(float* __restrict__ out, int iters) {
  const int t = threadIdx.x;
  f32x4 acc[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) acc[j] = f32x4{0, 0, 0, 0};
  bf16x4 a, b;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    a[s] = (__bf16)(0.001f * (float)((t + s) & 7));
    b[s] = (__bf16)(0.002f * (float)((t * 3 + s) & 7));
  }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, acc[j], 0, 0, 0);
  }
  f32x4 s = acc[0];
#pragma unroll
  for (int j = 1; j < 16; ++j) s += acc[j];
  out[(size_t)blockIdx.x * kThreads + t] = s[0] + s[1] + s[2] + s[3];
}

template <bool kBf16>
__global__ __launch_bounds__(kThreads) void mfma_kernel(float* __restrict__ out, int iters) {
  const int t = threadIdx.x;
  f32x4 acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = f32x4{0, 0, 0, 0};
  if constexpr (kBf16) {
    bf16x8 a, b;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      a[s] = (__bf16)(0.001f * (float)((t + s) & 7));
      b[s] = (__bf16)(0.002f * (float)((t * 3 + s) & 7));
    }
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[j], 0, 0, 0);
    }
  } else {
    const float a = 0.001f * (float)(t & 7), b = 0.002f * (float)((t * 3) & 7);
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc[j], 0, 0, 0);
    }
  }
  f32x4 s = acc[0];
#pragma unroll
  for (int j = 1; j < 8; ++j) s += acc[j];
  out[(size_t)blockIdx.x * kThreads + t] = s[0] + s[1] + s[2] + s[3];
}

/* op 0: v_exp_f32, 1: v_rcp_f32, 2: v_mul_f32; iters x 8 instructions a wave. */
template <int kOp>
__global__ __launch_bounds__(kThreads) void valu_kernel(float* __restrict__ out, int iters) {
  float x[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) x[j] = 0.5f + 0.001f * (float)(threadIdx.x + j);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if constexpr (kOp == 0)
        x[j] = __builtin_amdgcn_exp2f(x[j]);
      else if constexpr (kOp == 1)
        x[j] = __builtin_amdgcn_rcpf(x[j]);
      else
        x[j] = x[j] * 1.0001f;
    }
    // each chain stays a chain of single instructions (no reassociation)
    asm volatile("" : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), "+v"(x[4]), "+v"(x[5]), "+v"(x[6]), "+v"(x[7]));
  }
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) s += x[j];
  out[(size_t)blockIdx.x * kThreads + threadIdx.x] = s;
}

}  // namespace

extern "C" {

/* Copies bytes (a multiple of 16; both pointers 16-byte aligned) on the
 * stream with `blocks` workgroups of 256 threads.  Returns a hipError_t. */
int peaks_copy(const void* src, void* dst, uint64_t bytes, int blocks, void* stream) {
  if ((bytes & 15) != 0 || ((uintptr_t)src & 15) != 0 || ((uintptr_t)dst & 15) != 0 || blocks <= 0)
    return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(copy_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, (hipStream_t)stream,
                     (const u32x4*)src, (u32x4*)dst, bytes / 16);
  return (int)hipGetLastError();
}

/* Reads bytes (a multiple of 16, 16-byte aligned) with `blocks` workgroups
 * of 256 threads; out holds blocks x 256 words.  Returns a hipError_t. */
int peaks_read(const void* src, uint32_t* out, uint64_t bytes, int blocks, void* stream) {
  if ((bytes & 15) != 0 || ((uintptr_t)src & 15) != 0 || blocks <= 0) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(read_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, (hipStream_t)stream, (const u32x4*)src,
                     out, bytes / 16);
  return (int)hipGetLastError();
}

/* `blocks` workgroups of 256 threads, each wave issuing iters x 8 MFMAs;
 * out holds blocks x 256 floats.  bf16 = 1: the 16x16x32 bf16 instruction,
 * 2: iters x 4 of the 32x32x16 bf16 one, 3: iters x 16 of the 16x16x16 bf16
 * one (the same flops in each), 0: the fp32 one.
 * Returns a hipError_t. */
int peaks_mfma(float* out, int blocks, int iters, int bf16, void* stream) {
  if (blocks <= 0 || iters <= 0) return (int)hipErrorInvalidValue;
  if (bf16 == 2)  // 32x32x16 bf16: iters x 4 instructions of twice the work
    hipLaunchKernelGGL(mfma32_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, (hipStream_t)stream, out, iters);
  else if (bf16 == 3)  // 16x16x16 bf16: iters x 16 instructions of half the work
    hipLaunchKernelGGL(mfma16k16_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, (hipStream_t)stream, out, iters);
  else if (bf16)
    hipLaunchKernelGGL(mfma_kernel<true>, dim3((unsigned)blocks), dim3(kThreads), 0, (hipStream_t)stream, out, iters);
  else
    hipLaunchKernelGGL(mfma_kernel<false>, dim3((unsigned)blocks), dim3(kThreads), 0, (hipStream_t)stream, out, iters);
  return (int)hipGetLastError();
}

/* `blocks` workgroups of 256 threads, each wave issuing iters x 8 VALU
 * instructions of kind op (0 v_exp_f32, 1 v_rcp_f32, 2 v_mul_f32); out
 * holds blocks x 256 floats.  Returns a hipError_t. */
int peaks_valu(float* out, int blocks, int iters, int op, void* stream) {
  if (blocks <= 0 || iters <= 0 || op < 0 || op > 2) return (int)hipErrorInvalidValue;
  if (op == 0)
    hipLaunchKernelGGL(valu_kernel<0>, dim3((unsigned)blocks), dim3(kThreads), 0, (hipStream_t)stream, out, iters);
  else if (op == 1)
    hipLaunchKernelGGL(valu_kernel<1>, dim3((unsigned)blocks), dim3(kThreads), 0, (hipStream_t)stream, out, iters);
  else
    hipLaunchKernelGGL(valu_kernel<2>, dim3((unsigned)blocks), dim3(kThreads), 0, (hipStream_t)stream, out, iters);
  return (int)hipGetLastError();
}

}  // extern "C"
