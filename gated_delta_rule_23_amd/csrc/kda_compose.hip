/*
 * kda_compose.hip -- the prefix composition of segment fragments of the page
 * "Kimi K3：从三条信息流到完整系统", section "FlashKDA 与 KCP" (eq. (17)):
 * a segment j of a sequence acts on its entering state as S -> M_j S + E_j
 * (the recurrence is affine in S), so the entering states follow as
 *   S_in[0] = S0,  S_in[j + 1] = M_j S_in[j] + E_j.
 * M_j is the segment's transition (its state run from S = I with v = 0) and
 * E_j its state run from zero; both come from the packed prefill.
 *
 * One 256-thread workgroup per (sequence b, head h), serial over the P
 * segments: the state in LDS (fp32, 64 KiB) and M_j staged transposed in LDS
 * (64 KiB); thread t computes row t / 2, columns 64 (t % 2) .. +63 of
 * M_j S + E_j in registers.  fp32 throughout.
 */
#include "kda_common.h"
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int kComposeThreads = 256;

__global__ __launch_bounds__(kComposeThreads) void compose_kernel(const float* __restrict__ M,
                                                                  const float* __restrict__ E,
                                                                  const float* __restrict__ S0, float* __restrict__ S_in,
                                                                  int P, int H) {
  __shared__ float s_state[kD][kD];  // S, row-major
  __shared__ float s_mt[kD][kD];     // M_j transposed: s_mt[i][r] = M_j[r][i]
  const int b = blockIdx.x / H, h = blockIdx.x % H;
  const int t = threadIdx.x, r = t >> 1, c0 = 64 * (t & 1);
  auto state_at = [&](const float* base, int j) { return base + (((size_t)b * P + j) * H + h) * kD * kD; };
  // S_in[0] = S0 (or zeros)
  for (int e = t; e < kD * kD; e += kComposeThreads)
    s_state[e / kD][e % kD] = S0 ? S0[((size_t)b * H + h) * kD * kD + e] : 0.0f;
  __syncthreads();
  for (int j = 0; j < P; ++j) {
    float* out = S_in + (((size_t)b * P + j) * H + h) * kD * kD;
    for (int e = t; e < kD * kD; e += kComposeThreads) out[e] = s_state[e / kD][e % kD];
    if (j + 1 == P) break;
    const float* Mj = state_at(M, j);
    for (int e = t; e < kD * kD; e += kComposeThreads) s_mt[e % kD][e / kD] = Mj[e];
    __syncthreads();
    const float* Ej = state_at(E, j) + (size_t)r * kD + c0;
    float acc[64];
#pragma unroll
    for (int c = 0; c < 64; ++c) acc[c] = Ej[c];
    for (int i = 0; i < kD; ++i) {
      const float m = s_mt[i][r];
#pragma unroll
      for (int c = 0; c < 64; ++c) acc[c] = fmaf(m, s_state[i][c0 + c], acc[c]);
    }
    __syncthreads();  // every thread has read S and M_j
#pragma unroll
    for (int c = 0; c < 64; ++c) s_state[r][c0 + c] = acc[c];
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_compose(const float* M, const float* E, const float* S0, float* S_in, int B, int P, int H,
                          hipStream_t stream) {
  if (B == 0 || H == 0 || P == 0) return hipSuccess;
  hipLaunchKernelGGL(compose_kernel, dim3((unsigned)(B * H)), dim3(kComposeThreads), 0, stream, M, E, S0, S_in, P, H);
  return hipGetLastError();
}

}  // namespace kda
