/*
 * kda_compose.hip -- the prefix composition of segment fragments of the page
 * "Kimi K3：从三条信息流到完整系统", section "FlashKDA 与 KCP" (eq. (17)):
 * a segment j of a sequence acts on its entering state as S -> M_j S + E_j
 * (the recurrence is affine in S), so the entering states follow as
 *   S_in[0] = S0,  S_in[j + 1] = M_j S_in[j] + E_j.
 * M_j is the segment's transition (its state run from S = I with v = 0) and
 * E_j its state run from zero; both come from the packed prefill.
 *
 * Each column of S evolves on its own (S -> M S + E acts on the rows), so a
 * (sequence b, head h) takes kColGroups 256-thread workgroups of 16 columns
 * each, serial over the P segments: its columns of S in LDS, M_j staged
 * transposed in LDS (64 KiB, read by all of them, rows padded to 129 floats:
 * the staging writes of consecutive threads go down a column, which unpadded
 * would put all of them in one bank); thread t computes row t / 2, columns
 * 8 (t % 2) .. +7 of its group in registers.  fp32 throughout.
 */
#include "kda_common.h"
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int kComposeThreads = 256;
constexpr int kColGroups = 8;
constexpr int kGroupCols = kD / kColGroups;  // 16

__global__ __launch_bounds__(kComposeThreads) void compose_kernel(const float* __restrict__ M,
                                                                  const float* __restrict__ E,
                                                                  const float* __restrict__ S0, float* __restrict__ S_in,
                                                                  int P, int H, int frag_segs) {
  __shared__ float s_state[kD][kGroupCols];  // this group's columns of S
  __shared__ float s_mt[kD][kD + 1];         // M_j transposed: s_mt[i][r] = M_j[r][i]; rows padded by one
                                             // float, so the transposing writes spread over the banks
  const int unit = blockIdx.x / kColGroups, g = blockIdx.x % kColGroups;
  const int b = unit / H, h = unit % H;
  const int t = threadIdx.x, r = t >> 1, cl = 8 * (t & 1), col = kGroupCols * g + cl;
  auto at = [&](int j) { return (((size_t)b * P + j) * H + h) * kD * kD; };             // S_in
  auto frag = [&](int j) { return (((size_t)b * frag_segs + j) * H + h) * kD * kD; };  // M, E
  for (int e = t; e < kD * kGroupCols; e += kComposeThreads) {
    const int rr = e / kGroupCols, cc = e % kGroupCols;
    s_state[rr][cc] = S0 ? S0[((size_t)b * H + h) * kD * kD + (size_t)rr * kD + kGroupCols * g + cc] : 0.0f;
  }
  __syncthreads();
  for (int j = 0; j < P; ++j) {
    float* out = S_in + at(j);
#pragma unroll
    for (int c = 0; c < 8; ++c) out[(size_t)r * kD + col + c] = s_state[r][cl + c];
    if (j + 1 == P) break;
    const float* Mj = M + frag(j);
    for (int e = t; e < kD * kD; e += kComposeThreads) s_mt[e % kD][e / kD] = Mj[e];
    __syncthreads();
    const float* Ej = E + frag(j) + (size_t)r * kD + col;
    float acc[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] = Ej[c];
    for (int i = 0; i < kD; ++i) {
      const float m = s_mt[i][r];
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[c] = fmaf(m, s_state[i][cl + c], acc[c]);
    }
    __syncthreads();  // every thread has read S and M_j
#pragma unroll
    for (int c = 0; c < 8; ++c) s_state[r][cl + c] = acc[c];
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_compose(const float* M, const float* E, const float* S0, float* S_in, int B, int P, int H,
                          int frag_segs, hipStream_t stream) {
  if (B == 0 || H == 0 || P == 0) return hipSuccess;
  hipLaunchKernelGGL(compose_kernel, dim3((unsigned)(B * H * kColGroups)), dim3(kComposeThreads), 0, stream, M, E, S0,
                     S_in, P, H, frag_segs);
  return hipGetLastError();
}

}  // namespace kda
