/*
 * kda_epilogue.hip -- the weight-free output side of eq. (6) on the page
 * "Kimi K3：从三条信息流到完整系统": y = sigmoid(z) * RMSNorm(o), where o is
 * the recurrent output of one (token, head) row of 128 value channels, the
 * RMSNorm is head-wise with no learned scale, o / sqrt(mean(o^2) + eps), and
 * z = W_g x is the gate's pre-activation (W_g and the output projection W_o
 * stay with the caller).
 *
 * Bound by HBM: a row reads o and z once and writes y once.  A lane takes 16
 * bytes of a row per operand (8 bf16 or 4 fp32 channels), so a wave moves
 * 1 KiB per access; the row's sum of squares is reduced over its lanes.
 * y may be o itself: every lane reads its elements before it writes them.
 */
#include "kda_common.h"
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int kNormThreads = 256;

// A lane takes 16 bytes of a row: 8 bf16 or 4 fp32 channels; a row spans
// kD / kPerLane lanes and a wave 64 kPerLane / kD rows.
template <typename IO>
struct Lanes {
  static constexpr int kPerLane = 16 / (int)sizeof(IO);
  static constexpr int kRowLanes = kD / kPerLane;
  static constexpr int kRowsPerWave = 64 / kRowLanes;
  static constexpr int kRowsPerBlock = kRowsPerWave * kNormThreads / 64;
};

__device__ __forceinline__ void unpack(const u32x4 w, float (&f)[4], float) {
#pragma unroll
  for (int j = 0; j < 4; ++j) f[j] = __uint_as_float(w[j]);
}
__device__ __forceinline__ void unpack(const u32x4 w, float (&f)[8], bf16) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    f[2 * j] = __uint_as_float(w[j] << 16);
    f[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
  }
}
__device__ __forceinline__ u32x4 pack(const float (&f)[4]) {
  return u32x4{__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]), __float_as_uint(f[3])};
}
__device__ __forceinline__ u32x4 pack(const float (&f)[8]) {
  auto bits = [](float x) { return (uint32_t)__builtin_bit_cast(uint16_t, (bf16)x); };  // round to nearest even
  u32x4 w;
#pragma unroll
  for (int j = 0; j < 4; ++j) w[j] = bits(f[2 * j]) | (bits(f[2 * j + 1]) << 16);
  return w;
}

template <typename IO>
__global__ __launch_bounds__(kNormThreads) void gate_norm_kernel(const IO* o, const IO* z, IO* y, int64_t rows,
                                                                float eps) {
  using L = Lanes<IO>;
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * L::kRowsPerBlock + L::kRowsPerWave * (threadIdx.x >> 6) + lane / L::kRowLanes;
  const bool live = row < rows;
  const int64_t at = row * kD + L::kPerLane * (lane % L::kRowLanes);
  float ov[L::kPerLane], zv[L::kPerLane];
  u32x4 ow = {0, 0, 0, 0}, zw = {0, 0, 0, 0};
  if (live) {
    ow = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(o + at));
    zw = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(z + at));
  }
  unpack(ow, ov, IO());
  unpack(zw, zv, IO());
  float ss = 0.0f;
#pragma unroll
  for (int j = 0; j < L::kPerLane; ++j) ss += ov[j] * ov[j];
#pragma unroll
  for (int off = L::kRowLanes / 2; off >= 1; off >>= 1) ss += __shfl_xor(ss, off, 64);  // within the row's lanes
  const float inv = 1.0f / sqrtf(ss * (1.0f / kD) + eps);
  float out[L::kPerLane];
#pragma unroll
  for (int j = 0; j < L::kPerLane; ++j) out[j] = ov[j] * inv / (1.0f + expf(-zv[j]));
  if (live) __builtin_nontemporal_store(pack(out), reinterpret_cast<u32x4*>(y + at));  // streamed through once
}

}  // namespace

hipError_t launch_output_gate_norm(const void* o, const void* z, void* y, int64_t rows, float eps, bool bf16_io,
                                   hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  const int per_block = bf16_io ? Lanes<bf16>::kRowsPerBlock : Lanes<float>::kRowsPerBlock;
  const unsigned grid = (unsigned)((rows + per_block - 1) / per_block);
  if (bf16_io) {
    hipLaunchKernelGGL(gate_norm_kernel<bf16>, dim3(grid), dim3(kNormThreads), 0, stream, (const bf16*)o,
                       (const bf16*)z, (bf16*)y, rows, eps);
  } else {
    hipLaunchKernelGGL(gate_norm_kernel<float>, dim3(grid), dim3(kNormThreads), 0, stream, (const float*)o,
                       (const float*)z, (float*)y, rows, eps);
  }
  return hipGetLastError();
}

}  // namespace kda
