/*
 * kda_chunk.hip -- chunkwise KDA prefill on gfx950.
 *
 * Per (batch, head) the sequence is cut into chunks of C = 16 tokens.  With S
 * the state entering a chunk, b_r = sum_{s<=r} g_s the in-chunk cumulative
 * log-decay (eq. (3): Gamma_r = e^{b_r} = gamma^{1->r}) and
 *   Qh = Q * Gamma,  Kh = K * Gamma,  Kt = K / Gamma,  Kb = K * Gamma_C / Gamma,
 * eq. (4) of the page "Kimi K3：从三条信息流到完整系统" (section
 * "从投影到 Chunkwise 的完整接口") gives
 *   A  = Tril(Qh Kt^T)                       (diagonal kept: a token reads its own write)
 *   O  = Qh S + A Vt                         (inter-chunk + intra-chunk)
 * with the pseudo-value Vt = U - W S.  The pages leave U, W and the state
 * carry to Kimi Linear; substituting S_r = Diag(Gamma_r) R_r into eq. (1)
 * gives
 *   L  = StrictTril(Kh Kt^T),  M = (I + Diag(beta) L)^{-1} Diag(beta)
 *   Vt = M (V - Kh S)                        (U = M V, W = M Kh)
 *   S' = Diag(Gamma_C) S + Kb^T Vt.
 * The bounded gate (eq. (5), section "下界 log-decay 是一个 kernel 设计")
 * keeps b in [-80, 0] over a 16-token chunk, so Kt = K e^{-b} stays below
 * e^80 and every factor is representable in fp32 and bf16: the dense form is
 * used for every tile, with no per-pair path.
 *
 * Mapping (one workgroup per (b, h), 4 waves):
 *   - state: wave w keeps columns 32w .. 32w+31 of S (128 x 32 fp32) in four
 *     32x32 MFMA accumulator tiles for the whole sequence;
 *   - per chunk, all 256 threads compute the gate, the cumulative decay and
 *     the scaled operands (thread = key channel x half of the tokens) and
 *     write them to LDS already in MFMA fragment order;
 *   - wave 0 forms the two 16x16 Gram matrices on MFMA and inverts the unit
 *     lower-triangular (I + Diag(beta) L) by forward substitution in fp32;
 *   - every wave then runs the serial part on its columns: P = [Kh; Qh] S,
 *     [Vt; A Vt] = [M; A M] (V - Kh S), O = Qh S + A Vt,
 *     S <- Diag(Gamma_C) S + Kb^T Vt -- 13 32x32x16 MFMAs per chunk.
 * Contractions take bf16 operands with fp32 accumulation for bf16 I/O, and
 * fp32 operands (32x32x2 fp32 MFMA) for fp32 I/O.  The state stays fp32.
 */
#include "kda_common.h"
#include "kda_internal.h"

namespace kda {

template <typename OT>
struct ChunkSmem {
  OT xf[8][2][32][8];   // [Kh; Qh] as A fragments of P = X S: [k-block][half][row][slot]
  OT kf[8][2][16][8];   // Kt as B fragments of the Gram products: [k-block][half][token][slot]
  OT kbf[4][2][32][8];  // Kb^T as A fragments of the state update: [row tile][half][channel][slot]
  OT maf[2][32][8];     // [M; A M] as the A fragment over the chunk's tokens
  float v[kChunk][kD];  // V in fp32
  float lmat[kChunk][kChunk + 1];
  float amat[kChunk][kChunk + 1];
  float beta[kChunk];
  float gamma_c[kD];    // Gamma_C per key channel
  float half_sum[kD];   // log2-decay summed over tokens 0..7, per key channel
};

template <typename IO, typename OT>
__global__ __launch_bounds__(256) void chunk_fwd_kernel(const IO* __restrict__ q, const IO* __restrict__ k,
                                                        const IO* __restrict__ v, const IO* __restrict__ a,
                                                        const float* __restrict__ beta,
                                                        const float* initial_state, IO* __restrict__ o,
                                                        float* final_state, int T, int H) {
  __shared__ ChunkSmem<OT> sm;
  const int unit = blockIdx.x;  // b * H + h
  const int bb = unit / H, hh = unit % H;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int n = lane & 31, half = lane >> 5;
  const int col = 32 * wave + n;  // state column owned by this lane in the serial part

  // elementwise role: key channel c, tokens 8 th .. 8 th + 7
  const int c = tid & (kD - 1), th = tid >> 7;

  const size_t rs = (size_t)H * kD;  // token stride of a row tensor
  const size_t base = ((size_t)bb * T * H + hh) * kD;

  // ---------------------------------------------------------------- state in
  f32x16 sacc[4];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      int row = 32 * rt + 8 * (r / 4) + 4 * half + (r % 4);
      sacc[rt][r] = initial_state ? initial_state[((size_t)unit * kD + row) * kD + col] : 0.0f;
    }
  }

  for (int t0 = 0; t0 < T; t0 += kChunk) {
    const int nvalid = min(kChunk, T - t0);

    // ------------------------------------------------ gate and decay cumsum
    float qv[8], kv[8], cs[8];
    float run = 0.0f;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      int tok = 8 * th + r;
      float g = 0.0f;
      qv[r] = 0.0f;
      kv[r] = 0.0f;
      if (tok < nvalid) {
        size_t idx = base + (size_t)(t0 + tok) * rs + c;
        g = gate_log2(to_f32(a[idx]));
        qv[r] = to_f32(q[idx]);
        kv[r] = to_f32(k[idx]);
      }
      run += g;
      cs[r] = run;
    }
    if (th == 0) sm.half_sum[c] = run;
    {
      int tok = tid >> 4, c8 = 8 * (tid & 15);
#pragma unroll
      for (int e = 0; e < 8; ++e)
        sm.v[tok][c8 + e] = tok < nvalid ? to_f32(v[base + (size_t)(t0 + tok) * rs + c8 + e]) : 0.0f;
      if (tid < kChunk) sm.beta[tid] = tid < nvalid ? beta[((size_t)bb * T + t0 + tid) * H + hh] : 0.0f;
    }
    __syncthreads();

    // ------------------------------------------------ scaled operands -> LDS
    {
      const float prefix = th ? sm.half_sum[c] : 0.0f;
      const int kb = c >> 4, fh = kappa_half(c & 15), fs = kappa_slot(c & 15);
      if (th == 1) sm.gamma_c[c] = __builtin_amdgcn_exp2f(prefix + run);  // Gamma_C = e^{b_C}
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        int tok = 8 * th + r;
        float b2 = prefix + cs[r];
        float gam = __builtin_amdgcn_exp2f(b2);
        float inv = __builtin_amdgcn_exp2f(-b2);
        sm.xf[kb][fh][tok][fs] = from_f32<OT>(kv[r] * gam);
        sm.xf[kb][fh][kChunk + tok][fs] = from_f32<OT>(qv[r] * gam);
        kv[r] *= inv;  // Kt, kept for Kb below
        sm.kf[kb][fh][tok][fs] = from_f32<OT>(kv[r]);
      }
    }
    __syncthreads();
    {
      // Kb = Kt * Gamma_C: Gamma_C of this channel was written by the second token half.
      const int rt = c >> 5, m = c & 31;
      const float gc = sm.gamma_c[c];
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        int tok = 8 * th + r;
        sm.kbf[rt][kappa_half(tok)][m][kappa_slot(tok)] = from_f32<OT>(kv[r] * gc);
      }
    }

    // ------------------------------------------------ Gram matrices (wave 0)
    if (wave == 0) {
      f32x16 g = {};
#pragma unroll
      for (int kb = 0; kb < 8; ++kb) {
        Frag<OT> fa = frag_load<OT>(&sm.xf[kb][half][n][0]);
        Frag<OT> fb = n < kChunk ? frag_load<OT>(&sm.kf[kb][half][n][0]) : frag_zero<OT>();
        mfma_k16(g, fa, fb);
      }
      if (n < kChunk) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          int row = 8 * (r / 4) + 4 * half + (r % 4);
          if (row < kChunk)
            sm.lmat[row][n] = g[r];
          else
            sm.amat[row - kChunk][n] = g[r];
        }
      }
    }
    __syncthreads();

    // ------------------------------------------------ (I + Diag(beta) L)^{-1} Diag(beta) and A times it
    if (wave == 0 && lane < kChunk) {
      const int j = lane;
      float tcol[kChunk];
#pragma unroll
      for (int r = 0; r < kChunk; ++r) {
        float acc = 0.0f;
#pragma unroll
        for (int s = 0; s < r; ++s) acc += sm.lmat[r][s] * tcol[s];
        tcol[r] = (r == j ? 1.0f : 0.0f) - sm.beta[r] * acc;
      }
      const float bj = sm.beta[j];
      const int fh = kappa_half(j), fs = kappa_slot(j);
#pragma unroll
      for (int r = 0; r < kChunk; ++r) tcol[r] *= bj;  // column j of M
#pragma unroll
      for (int r = 0; r < kChunk; ++r) {
        float am = 0.0f;
#pragma unroll
        for (int s = 0; s <= r; ++s) am += sm.amat[r][s] * tcol[s];
        sm.maf[fh][r][fs] = from_f32<OT>(tcol[r]);
        sm.maf[fh][16 + r][fs] = from_f32<OT>(am);
      }
    }
    __syncthreads();

    // ------------------------------------------------ serial part on this wave's columns
    {
      Frag<OT> sf[8];
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        sf[2 * rt] = frag_from_acc<OT>(sacc[rt], 0);
        sf[2 * rt + 1] = frag_from_acc<OT>(sacc[rt], 8);
      }
      f32x16 p = {};
#pragma unroll
      for (int kb = 0; kb < 8; ++kb) mfma_k16(p, frag_load<OT>(&sm.xf[kb][half][n][0]), sf[kb]);

      float rres[8];
#pragma unroll
      for (int s = 0; s < 8; ++s) rres[s] = sm.v[kappa(half, s)][col] - p[s];
      f32x16 d = {};
      mfma_k16(d, frag_load<OT>(&sm.maf[half][n][0]), frag_from_f32<OT>(rres));

#pragma unroll
      for (int s = 0; s < 8; ++s) {
        int tok = kappa(half, s);
        if (tok < nvalid) o[base + (size_t)(t0 + tok) * rs + col] = from_f32<IO>(p[8 + s] + d[8 + s]);
      }

      Frag<OT> vt = frag_from_acc<OT>(d, 0);
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[rt][r] *= sm.gamma_c[32 * rt + 8 * (r / 4) + 4 * half + (r % 4)];
        mfma_k16(sacc[rt], frag_load<OT>(&sm.kbf[rt][half][n][0]), vt);
      }
    }
    __syncthreads();
  }

  // ---------------------------------------------------------------- state out
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      int row = 32 * rt + 8 * (r / 4) + 4 * half + (r % 4);
      final_state[((size_t)unit * kD + row) * kD + col] = sacc[rt][r];
    }
  }
}

hipError_t launch_chunk_fwd(const void* q, const void* k, const void* v, const void* a, const float* beta,
                            const float* initial_state, void* o, float* final_state, int B, int T, int H,
                            bool bf16_io, hipStream_t stream) {
  const int units = B * H;
  if (units == 0) return hipSuccess;
  if (bf16_io) {
    hipLaunchKernelGGL((chunk_fwd_kernel<bf16, bf16>), dim3(units), dim3(256), 0, stream, (const bf16*)q,
                       (const bf16*)k, (const bf16*)v, (const bf16*)a, beta, initial_state, (bf16*)o, final_state, T,
                       H);
  } else {
    hipLaunchKernelGGL((chunk_fwd_kernel<float, float>), dim3(units), dim3(256), 0, stream, (const float*)q,
                       (const float*)k, (const float*)v, (const float*)a, beta, initial_state, (float*)o, final_state,
                       T, H);
  }
  return hipGetLastError();
}

}  // namespace kda
