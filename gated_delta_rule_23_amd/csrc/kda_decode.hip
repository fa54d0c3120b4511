/*
 * kda_decode.hip -- one recurrent KDA step per (batch, head), state updated
 * in place (page "Kimi K3：从三条信息流到完整系统", eq. (1) in its expanded
 * form, section "KDA 是带逐通道遗忘的 delta rule"):
 *
 *   alpha = exp(-5 sigmoid(a))
 *   x = S^T (alpha * k),  y = S^T (alpha * q)        one pass over S
 *   e = v - x                                          residual vs the decayed prediction
 *   o = y + beta (q . k) e                             = S_new^T q
 *   S_new = Diag(alpha) S + beta k e^T                 written back over S
 *
 * The step is bound by HBM traffic: each state entry is read once and
 * written once (2 x 64 KiB per head), against 4 x 128 input values.  A
 * 1024-thread workgroup holds one (b, h) state in registers between its read
 * and its write: thread t holds the float4 columns 4 (t % 32) .. +3 of rows
 * t / 32 + 32 m, m = 0..3, so every wave reads and writes two whole 512-byte
 * rows per instruction.  The grid strides over the states (four workgroups
 * per compute unit), and each workgroup issues the loads of its next state
 * before the three barriers of the current one: the read stream continues
 * while a state is reduced and written back, where one workgroup per state
 * left the memory system idle during its barriers (measured on 256 x 96
 * states: 0.578 ms with one state per workgroup, 0.518 ms with the prefetch
 * and four workgroups per compute unit, 0.521-0.530 ms with two to twelve).  State
 * loads and stores carry the non-temporal hint (the state streams through
 * once per step).
 */
#include "kda_common.h"
#include "kda_internal.h"

namespace kda {

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

constexpr int kDecodeThreads = 1024;
constexpr int kRowGroups = kDecodeThreads / 32;  // thread t: rows t / 32 + kRowGroups m
constexpr int kRowsPerThread = kD / kRowGroups;
constexpr int kWorkgroupsPerCU = 4;

template <typename IO>
__global__ __launch_bounds__(kDecodeThreads) void decode_kernel(const IO* __restrict__ q, const IO* __restrict__ k,
                                                     const IO* __restrict__ v, const IO* __restrict__ a,
                                                     const float* __restrict__ beta, float* __restrict__ state,
                                                     IO* __restrict__ o, int units) {
  // Per-channel values of the state in hand, in two sets used by alternate
  // states: a set is rewritten two states later, after every thread has
  // passed the first barrier of the state in between.
  __shared__ float s_alpha[2][kD], s_ak[2][kD], s_aq[2][kD], s_k[2][kD];
  __shared__ float s_be[kD];
  __shared__ f32x4 s_part[kRowGroups / 2][2][32];  // per wave: partial x and y, float4 per column group
  __shared__ float s_dot[2][2];

  const int t = threadIdx.x;
  const int cg = t & 31, rg = t >> 5;
  auto load_state = [&](int u, f32x4 (&dst)[kRowsPerThread]) {
    const float* S = state + (size_t)u * kD * kD;
#pragma unroll
    for (int m = 0; m < kRowsPerThread; ++m)
      dst[m] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(S + (size_t)(rg + kRowGroups * m) * kD + 4 * cg));
  };

  int unit = blockIdx.x;  // b * H + h
  f32x4 s[kRowsPerThread];
  if (unit < units) load_state(unit, s);
  for (int set = 0; unit < units; set ^= 1) {
    const size_t row = (size_t)unit * kD;
    if (t < kD) {
      const float qi = to_f32(q[row + t]), ki = to_f32(k[row + t]), ai = to_f32(a[row + t]);
      const float al = expf(kGateFloor / (1.0f + expf(-ai)));
      s_alpha[set][t] = al;
      s_ak[set][t] = al * ki;
      s_aq[set][t] = al * qi;
      s_k[set][t] = ki;
      const float d = wave_sum(qi * ki);
      if ((t & 63) == 0) s_dot[set][t >> 6] = d;
    }
    const int next = unit + (int)gridDim.x;
    f32x4 sn[kRowsPerThread];
    if (next < units) load_state(next, sn);  // in flight until the next pass
    __syncthreads();

    f32x4 x = {0, 0, 0, 0}, y = {0, 0, 0, 0};
#pragma unroll
    for (int m = 0; m < kRowsPerThread; ++m) {
      const int i = rg + kRowGroups * m;
      x += s_ak[set][i] * s[m];
      y += s_aq[set][i] * s[m];
    }
    // the two row groups of a wave (lanes 0..31 and 32..63, same columns) combined by a half swap
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const auto sx = __builtin_amdgcn_permlane32_swap(__float_as_uint(x[j]), __float_as_uint(x[j]), false, false);
      const auto sy = __builtin_amdgcn_permlane32_swap(__float_as_uint(y[j]), __float_as_uint(y[j]), false, false);
      x[j] = __uint_as_float(sx[0]) + __uint_as_float(sx[1]);
      y[j] = __uint_as_float(sy[0]) + __uint_as_float(sy[1]);
    }
    if ((t & 63) < 32) {
      s_part[t >> 6][0][cg] = x;
      s_part[t >> 6][1][cg] = y;
    }
    __syncthreads();

    if (t < kD) {
      const float* px = reinterpret_cast<const float*>(&s_part[0][0][0]);
      float xs = 0.0f, ys = 0.0f;
#pragma unroll
      for (int r = 0; r < kRowGroups / 2; ++r) {
        xs += px[(r * 2 + 0) * kD + t];
        ys += px[(r * 2 + 1) * kD + t];
      }
      const float bt = beta[unit];
      const float e = to_f32(v[row + t]) - xs;
      o[row + t] = from_f32<IO>(ys + bt * (s_dot[set][0] + s_dot[set][1]) * e);
      s_be[t] = bt * e;
    }
    __syncthreads();

    float* S = state + (size_t)unit * kD * kD;
    const f32x4 be = *reinterpret_cast<const f32x4*>(&s_be[4 * cg]);
#pragma unroll
    for (int m = 0; m < kRowsPerThread; ++m) {
      const int i = rg + kRowGroups * m;
      __builtin_nontemporal_store(s_alpha[set][i] * s[m] + s_k[set][i] * be,
                                  reinterpret_cast<f32x4*>(S + (size_t)i * kD + 4 * cg));
    }
#pragma unroll
    for (int m = 0; m < kRowsPerThread; ++m) s[m] = sn[m];
    unit = next;
  }
}

hipError_t launch_decode(const void* q, const void* k, const void* v, const void* a, const float* beta, float* state,
                         void* o, int units, bool bf16_io, hipStream_t stream) {
  if (units == 0) return hipSuccess;
  int cus = 0;
  const hipError_t err = device_cu_count(stream, &cus);
  if (err != hipSuccess) return err;
  const int64_t slots = (int64_t)kWorkgroupsPerCU * (cus > 0 ? cus : 1);
  const unsigned grid = (unsigned)(units < slots ? units : slots);
  if (bf16_io) {
    hipLaunchKernelGGL(decode_kernel<bf16>, dim3(grid), dim3(kDecodeThreads), 0, stream, (const bf16*)q, (const bf16*)k,
                       (const bf16*)v, (const bf16*)a, beta, state, (bf16*)o, units);
  } else {
    hipLaunchKernelGGL(decode_kernel<float>, dim3(grid), dim3(kDecodeThreads), 0, stream, (const float*)q,
                       (const float*)k, (const float*)v, (const float*)a, beta, state, (float*)o, units);
  }
  return hipGetLastError();
}

}  // namespace kda
