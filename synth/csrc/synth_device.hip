/*
 * synth_device.hip -- device generator for the seeded synthetic KDA inputs.
 * Same arithmetic as the host generator (synth_core.h, built with
 * floating-point contraction off), so both produce identical bits; used to
 * fill large inputs directly in device memory.
 */
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "synth_core.h"

__global__ void synth_rows_kernel(synth_row_recipe r, int dtype, int b0, int t0, int h0, int nt, int nh,
                                  uint64_t n_rows, void* dst) {
  uint64_t n = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (n >= n_rows) return;
  uint64_t hh = n % (uint64_t)nh, tt = (n / (uint64_t)nh) % (uint64_t)nt, bb = n / ((uint64_t)nh * (uint64_t)nt);
  uint32_t b = (uint32_t)(b0 + bb), t = (uint32_t)(t0 + tt), h = (uint32_t)(h0 + hh);
  double div = synth_row_divisor(&r, b, t, h);
  for (uint32_t g = 0; g < SYNTH_D / 4; ++g) {
    double z[4];
    synth_row_group(&r, b, t, h, g, z);
    for (int c = 0; c < 4; ++c) synth_store(dst, n * SYNTH_D + 4 * g + c, dtype, z[c] / div);
  }
}

__global__ void synth_beta_kernel(uint32_t seed, int dtype, int b0, int t0, int h0, int nt, int nh, uint64_t n_total,
                                  void* dst) {
  uint64_t n = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (n >= n_total) return;
  uint64_t hh = n % (uint64_t)nh, tt = (n / (uint64_t)nh) % (uint64_t)nt, bb = n / ((uint64_t)nh * (uint64_t)nt);
  synth_store(dst, n, dtype, synth_beta(seed, (uint32_t)(b0 + bb), (uint32_t)(t0 + tt), (uint32_t)(h0 + hh)));
}

__global__ void synth_state_kernel(uint32_t seed, double scale, int dtype, int b0, int h0, int nh, uint64_t n_rows,
                                   void* dst) {
  uint64_t n = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (n >= n_rows) return;
  uint64_t i = n % SYNTH_D, hh = (n / SYNTH_D) % (uint64_t)nh, bb = n / ((uint64_t)SYNTH_D * (uint64_t)nh);
  for (uint32_t g = 0; g < SYNTH_D / 4; ++g) {
    double z[4];
    synth_state4(seed, scale, (uint32_t)(b0 + bb), (uint32_t)(h0 + hh), (uint32_t)i, g, z);
    for (int c = 0; c < 4; ++c) synth_store(dst, n * SYNTH_D + 4 * g + c, dtype, z[c]);
  }
}

static int synth_grid(uint64_t n, dim3* grid) {
  uint64_t blocks = (n + 255) / 256;
  if (blocks > 0x7FFFFFFFull) return -1;
  *grid = dim3((unsigned)(blocks ? blocks : 1));
  return 0;
}

extern "C" {

/* Device twins of synth_rows_host / synth_beta_host / synth_state_host: dst is
 * a device pointer, work is enqueued on `stream`. Returns 0, -1 on bad
 * arguments, -2 if the launch failed. */
int synth_rows_device(const synth_row_recipe* recipe, int dtype, int b0, int nb, int t0, int nt, int h0, int nh,
                      void* dst, void* stream) {
  if (!recipe || nb < 0 || nt < 0 || nh < 0 || b0 < 0 || t0 < 0 || h0 < 0 || dtype < 0 || dtype > 2) return -1;
  uint64_t n = (uint64_t)nb * (uint64_t)nt * (uint64_t)nh;
  if (n == 0) return 0;
  if (!dst) return -1;
  dim3 grid;
  if (synth_grid(n, &grid)) return -1;
  hipLaunchKernelGGL(synth_rows_kernel, grid, dim3(256), 0, (hipStream_t)stream, *recipe, dtype, b0, t0, h0, nt, nh, n,
                     dst);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}

int synth_beta_device(uint32_t seed, int dtype, int b0, int nb, int t0, int nt, int h0, int nh, void* dst,
                      void* stream) {
  if (nb < 0 || nt < 0 || nh < 0 || b0 < 0 || t0 < 0 || h0 < 0 || dtype < 0 || dtype > 2) return -1;
  uint64_t n = (uint64_t)nb * (uint64_t)nt * (uint64_t)nh;
  if (n == 0) return 0;
  if (!dst) return -1;
  dim3 grid;
  if (synth_grid(n, &grid)) return -1;
  hipLaunchKernelGGL(synth_beta_kernel, grid, dim3(256), 0, (hipStream_t)stream, seed, dtype, b0, t0, h0, nt, nh, n,
                     dst);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}

int synth_state_device(uint32_t seed, double scale, int dtype, int b0, int nb, int h0, int nh, void* dst,
                       void* stream) {
  if (nb < 0 || nh < 0 || b0 < 0 || h0 < 0 || dtype < 0 || dtype > 2) return -1;
  uint64_t n = (uint64_t)nb * (uint64_t)nh * SYNTH_D;
  if (n == 0) return 0;
  if (!dst) return -1;
  dim3 grid;
  if (synth_grid(n, &grid)) return -1;
  hipLaunchKernelGGL(synth_state_kernel, grid, dim3(256), 0, (hipStream_t)stream, seed, scale, dtype, b0, h0, nh, n,
                     dst);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}

}  // extern "C"
