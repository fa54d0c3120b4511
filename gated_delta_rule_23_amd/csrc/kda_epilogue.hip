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
 * 1 KiB per access, and covers four rows whose loads all go out first; the
 * row's sum of squares is reduced over its lanes by DPP rotations, and the
 * sigmoid and the reciprocal square root are single instructions
 * (v_exp_f32, v_rcp_f32, v_rsq_f32).  y may be o itself: every lane reads
 * its elements before it writes them.
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

// Rows a thread covers: the loads of all of them go out before any is used.
constexpr int kNormUnroll = 4;

// The sum over the lanes of one row: a row of bf16 channels spans one 16-lane
// DPP row (four rotations), a row of fp32 channels two (then a row swap).
template <typename IO>
__device__ __forceinline__ float row_sum(float x) {
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x128, 0xf, 0xf, false));  // row_ror:8
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x124, 0xf, 0xf, false));  // row_ror:4
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x122, 0xf, 0xf, false));  // row_ror:2
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x121, 0xf, 0xf, false));  // row_ror:1
  if constexpr (Lanes<IO>::kRowLanes == 32) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  return x;
}

template <typename IO>
__global__ __launch_bounds__(kNormThreads) void gate_norm_kernel(const IO* o, const IO* z, IO* y, int64_t rows,
                                                                float eps) {
  using L = Lanes<IO>;
  static_assert(L::kRowLanes == 16 || L::kRowLanes == 32, "a row spans one or two DPP rows");
  const int lane = threadIdx.x & 63;
  // rows of block b: kNormUnroll slabs of kRowsPerBlock, thread row i of slab u
  const int64_t row0 = (int64_t)blockIdx.x * (kNormUnroll * L::kRowsPerBlock) +
                       L::kRowsPerWave * (threadIdx.x >> 6) + lane / L::kRowLanes;
  const int col = L::kPerLane * (lane % L::kRowLanes);
  u32x4 ow[kNormUnroll], zw[kNormUnroll];
#pragma unroll
  for (int u = 0; u < kNormUnroll; ++u) {
    const int64_t row = row0 + (int64_t)u * L::kRowsPerBlock;
    ow[u] = zw[u] = u32x4{0, 0, 0, 0};
    if (row < rows) {
      ow[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(o + row * kD + col));
      zw[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(z + row * kD + col));
    }
  }
#pragma unroll
  for (int u = 0; u < kNormUnroll; ++u) {
    const int64_t row = row0 + (int64_t)u * L::kRowsPerBlock;
    float ov[L::kPerLane], zv[L::kPerLane];
    unpack(ow[u], ov, IO());
    unpack(zw[u], zv, IO());
    float ss = 0.0f;
#pragma unroll
    for (int j = 0; j < L::kPerLane; ++j) ss = fmaf(ov[j], ov[j], ss);
    const float inv = __builtin_amdgcn_rsqf(fmaf(row_sum<IO>(ss), 1.0f / kD, eps));
    float out[L::kPerLane];
#pragma unroll
    for (int j = 0; j < L::kPerLane; ++j) out[j] = ov[j] * inv * sigmoid_fast(zv[j]);
    if (row < rows) __builtin_nontemporal_store(pack(out), reinterpret_cast<u32x4*>(y + row * kD + col));  // streamed through once
  }
}

}  // namespace

hipError_t launch_output_gate_norm(const void* o, const void* z, void* y, int64_t rows, float eps, bool bf16_io,
                                   hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  const int per_block = kNormUnroll * (bf16_io ? Lanes<bf16>::kRowsPerBlock : Lanes<float>::kRowsPerBlock);
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
