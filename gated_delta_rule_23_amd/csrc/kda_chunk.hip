/*
 * kda_chunk.hip -- chunkwise KDA prefill on gfx950.
 *
 * The method (page "Kimi K3：从三条信息流到完整系统", wineandchord.com).
 * Per (batch, head) the sequence is cut into chunks of C = 16 tokens.  With S
 * the state entering a chunk, b_r = sum_{s<=r} g_s the in-chunk cumulative
 * log-decay (eq. (3) of section "从投影到 Chunkwise 的完整接口":
 * Gamma_r = e^{b_r} = gamma^{1->r}) and
 *   Qh = Q * Gamma,  Kh = K * Gamma,  Kt = K / Gamma,  Kb = K * Gamma_C / Gamma,
 * eq. (4) gives
 *   A  = Tril(Qh Kt^T)        (diagonal kept: a token reads its own write)
 *   O  = Qh S + A Vt          (inter-chunk + intra-chunk)
 * with the pseudo-value Vt = U - W S.  The pages leave U, W and the state
 * carry to Kimi Linear; substituting S_r = Diag(Gamma_r) R_r into eq. (1)
 * (section "KDA 是带逐通道遗忘的 delta rule") gives
 *   L  = StrictTril(Kh Kt^T),   M = (I + Diag(beta) L)^{-1} Diag(beta),
 *   Vt = M (V - Kh S)           (U = M V, W = M Kh),
 *   S' = Diag(Gamma_C) S + Kb^T Vt.
 * The bounded gate (eq. (5), section "下界 log-decay 是一个 kernel 设计")
 * keeps b in [-80, 0] over 16 tokens, so Kt = K e^{-b} <= e^80 |K| and every
 * factor is representable in fp32 and bf16: all tiles take the dense path.
 *
 * Mapping: one 512-thread workgroup (8 waves, two per SIMD) per (b, h).
 * Lane l of wave w owns state column 16w + l%16 and key channel 16w + l%16;
 * its group h = l/16 covers tokens 4h .. 4h+3 of a chunk.
 *   - The 128 x 128 fp32 state stays in MFMA accumulators for the whole
 *     sequence: each wave keeps 128 x 16 of it in eight 16x16 tiles.
 *   - Three chunks are in flight.  In iteration i:
 *       chain(i-2):  P = [Kh; Qh] S, [Vt; A Vt] = [M; A M] (V - Kh S),
 *                    O = Qh S + A Vt, S <- Diag(Gamma_C) S + Kb^T Vt
 *                    (18 MFMAs per wave, all waves, their own columns);
 *       inverse(i-1): one wave forms the 16x16 Gram products on MFMA and
 *                    (I + N)^{-1} = (I - N)(I + N^2)(I + N^4)(I + N^8) for the
 *                    nilpotent N = Diag(beta) L, also on MFMA;
 *       gate(i):     every lane: g = -5 sigmoid(a), cumulative sums, the four
 *                    scaled operands, written to LDS in MFMA fragment order;
 *       loads(i+1):  the next chunk's q, k, a, beta and V go to registers;
 *       store(i-3):  the output tile staged in LDS goes out in 16-byte rows.
 *     One workgroup barrier per iteration separates producers and consumers
 *     of the three LDS stages.
 * Contractions take bf16 operands with fp32 accumulation for bf16 I/O, and
 * fp32 operands (16x16x4 fp32 MFMA) for fp32 I/O.  The state stays fp32.
 */
#include "kda_common.h"
#include "kda_internal.h"

namespace kda {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kStages = 3;
constexpr float kGateLog2 = kGateFloor * kLog2e;  // g * log2(e) = kGateLog2 * sigmoid(a)

/* One chunk's operands, in the order the MFMA lanes read them. */
template <typename OT>
struct Stage {
  OT xf[2][4][64][8];  // [Kh | Qh][block of 32 key channels][lane][slot]: A of P = X S, and of the Gram products
  OT kf[4][64][8];     // Kt: [block of 32 key channels][lane][slot]
  OT kbf[8][64][4];    // Kb^T: [tile of 16 key channels][lane][token slot]: A of the state update
  OT maf[2][64][4];    // [M | A M]: A of [Vt; A Vt] = [M; A M] R
  float gamma_c[kD];   // Gamma_C per key channel
  float beta[kChunk];
};

template <typename IO, typename OT>
struct Smem {
  Stage<OT> st[kStages];
  IO ostage[2][kChunk][kD];         // output tiles waiting for their coalesced store
  float tscratch[kChunk][kChunk + 1];  // transpose scratch of the inverse
};

template <typename IO, typename OT>
__global__ __launch_bounds__(kThreads) void chunk_fwd_kernel(const IO* __restrict__ q, const IO* __restrict__ k,
                                                             const IO* __restrict__ v, const IO* __restrict__ a,
                                                             const float* __restrict__ beta,
                                                             const float* initial_state, IO* __restrict__ o,
                                                             float* final_state, int T, int H) {
  __shared__ Smem<IO, OT> sm;
  const int unit = blockIdx.x;  // b * H + h
  const int bb = unit / H, hh = unit % H;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int n = lane & 15, h = lane >> 4;
  const int col = 16 * wave + n;  // state column and key channel of this lane
  const size_t rs = (size_t)H * kD;  // token stride of a row tensor
  const size_t base = ((size_t)bb * T * H + hh) * kD;
  const int nchunks = (T + kChunk - 1) / kChunk;

  // fragment coordinates of this lane's key channel inside the K = 32 blocks
  const int kb_c = col >> 5;
  const int grp_c = kappa_group(col & 31), slot_c = kappa_slot(col & 31);

  // ---------------------------------------------------------------- state in
  f32x4 sacc[8];
#pragma unroll
  for (int rt = 0; rt < 8; ++rt)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int row = 16 * rt + 4 * h + j;
      sacc[rt][j] = initial_state ? initial_state[((size_t)unit * kD + row) * kD + col] : 0.0f;
    }

  // Registers carried between iterations: raw q, k, a, beta of the next gate
  // pass and V of the next serial step.  Every iteration loads a chunk index
  // clamped into range and a token clamped to T - 1, so the loads issue back
  // to back with no branch; tokens past the end are masked where used.  Each
  // element keeps its own 32-bit register until used, so no wait follows the
  // loads: they complete under the next iteration's work.
  typedef typename Raw<IO>::type RT;
  RT rq[4], rk[4], ra[4], rv[4];
  float rb[4];
  auto load_raw = [&](int x, RT* lq, RT* lk, RT* la, float* lb) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int t = min(x * kChunk + 4 * h + j, T - 1);
      const size_t idx = base + (size_t)t * rs + col;
      lq[j] = Raw<IO>::load(q, idx);
      lk[j] = Raw<IO>::load(k, idx);
      la[j] = Raw<IO>::load(a, idx);
      lb[j] = beta[((size_t)bb * T + t) * H + hh];
    }
  };
  auto load_v = [&](int x, RT* lv) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int t = min(x * kChunk + 4 * h + j, T - 1);
      lv[j] = Raw<IO>::load(v, base + (size_t)t * rs + col);
    }
  };
  const int last = max(nchunks - 1, 0);
  if (nchunks > 0) {
    load_raw(0, rq, rk, ra, rb);
    load_v(0, rv);
  }

  for (int i = 0; i < nchunks + 3; ++i) {
    // ------------------------------------------------ loads for the next iteration
    RT nq[4], nk[4], na[4], nv[4];
    float nb[4];
    if (nchunks > 0) {
      load_raw(min(i + 1, last), nq, nk, na, nb);
      load_v(min(max(i - 1, 0), last), nv);
    }

    // ------------------------------------------------ chain(i - 2): the serial part
    if (i - 2 >= 0 && i - 2 < nchunks) {
      const int x = i - 2;
      Stage<OT>& st = sm.st[x % kStages];
      f32x4 pk = {0, 0, 0, 0}, pq = {0, 0, 0, 0};
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        Frag8<OT> sf = frag8<OT>(sacc[2 * kb], sacc[2 * kb + 1]);
        mfma_k32(pk, load_frag8<OT>(&st.xf[0][kb][lane][0]), sf);
        mfma_k32(pq, load_frag8<OT>(&st.xf[1][kb][lane][0]), sf);
      }
      const int nvalid = min(kChunk, T - x * kChunk);
      float rr[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) rr[j] = (4 * h + j < nvalid ? Raw<IO>::f32(rv[j]) : 0.0f) - pk[j];
      Frag4<OT> fr = frag4<OT>(rr[0], rr[1], rr[2], rr[3]);
      f32x4 dm = {0, 0, 0, 0}, da = {0, 0, 0, 0};
      mfma_k16(dm, load_frag4<OT>(&st.maf[0][lane][0]), fr);
      mfma_k16(da, load_frag4<OT>(&st.maf[1][lane][0]), fr);
#pragma unroll
      for (int j = 0; j < 4; ++j) sm.ostage[x & 1][4 * h + j][col] = from_f32<IO>(pq[j] + da[j]);
      Frag4<OT> fv = frag4<OT>(dm);
#pragma unroll
      for (int rt = 0; rt < 8; ++rt) {
        f32x4 gc = *reinterpret_cast<const f32x4*>(&st.gamma_c[16 * rt + 4 * h]);
        sacc[rt] *= gc;
        mfma_k16(sacc[rt], load_frag4<OT>(&st.kbf[rt][lane][0]), fv);
      }
    }

    // ------------------------------------------------ inverse(i - 1): one wave
    if (i - 1 >= 0 && i - 1 < nchunks && wave == (i - 1) % kWaves) {
      const int x = i - 1;
      Stage<OT>& st = sm.st[x % kStages];
      // C layouts (lane (n, h), register j <-> row r = 4h + j, column n):
      //   gkt = Kt Kh^T = (Kh Kt^T)^T,  gqt = Kt Qh^T = (Qh Kt^T)^T
      f32x4 gkt = {0, 0, 0, 0}, gqt = {0, 0, 0, 0};
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        Frag8<OT> fa = load_frag8<OT>(&st.kf[kb][lane][0]);
        mfma_k32(gkt, fa, load_frag8<OT>(&st.xf[0][kb][lane][0]));
        mfma_k32(gqt, fa, load_frag8<OT>(&st.xf[1][kb][lane][0]));
      }
      const float bn = st.beta[n];
      f32x4 nt, at;  // N^T and A^T; N[r][c] = beta_r L[r][c] for r > c, A = Tril(Qh Kt^T)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        int r = 4 * h + j;
        nt[j] = n > r ? bn * gkt[j] : 0.0f;
        at[j] = n >= r ? gqt[j] : 0.0f;
        sm.tscratch[r][n] = nt[j];
      }
      // lanes read each other's writes: order them explicitly within the wave
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      f32x4 nc, y;  // N, and Y0 = I - N
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        nc[j] = sm.tscratch[n][4 * h + j];
        y[j] = (4 * h + j == n ? 1.0f : 0.0f) - nc[j];
      }
      // A operand of X = C layout of X^T, so (N^p, (N^p)^T) pairs feed each other.
      f32x4 n2c = {0, 0, 0, 0}, n2t = {0, 0, 0, 0}, n4c = {0, 0, 0, 0}, n4t = {0, 0, 0, 0}, n8t = {0, 0, 0, 0};
      mfma_k16(n2c, frag4<OT>(nt), frag4<OT>(nc));
      mfma_k16(n2t, frag4<OT>(nc), frag4<OT>(nt));
      mfma_k16(y, frag4<OT>(n2t), frag4<OT>(y));  // Y1 = (I + N^2) Y0
      mfma_k16(n4c, frag4<OT>(n2t), frag4<OT>(n2c));
      mfma_k16(n4t, frag4<OT>(n2c), frag4<OT>(n2t));
      mfma_k16(y, frag4<OT>(n4t), frag4<OT>(y));  // Y2 = (I + N^4) Y1
      mfma_k16(n8t, frag4<OT>(n4c), frag4<OT>(n4t));
      mfma_k16(y, frag4<OT>(n8t), frag4<OT>(y));  // (I + N)^{-1} = (I + N^8) Y2
      f32x4 m = y * bn;                           // M = (I + N)^{-1} Diag(beta)
      f32x4 am = {0, 0, 0, 0};
      mfma_k16(am, frag4<OT>(at), frag4<OT>(m));  // A M
      // A fragments of [M; A M]: lane (row r, group n/4), slot n % 4
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        int r = 4 * h + j;
        st.maf[0][(n >> 2) * 16 + r][n & 3] = from_f32<OT>(m[j]);
        st.maf[1][(n >> 2) * 16 + r][n & 3] = from_f32<OT>(am[j]);
      }
    }

    // ------------------------------------------------ gate(i): this lane's channel, tokens 4h .. 4h+3
    if (i < nchunks) {
      const int x = i;
      Stage<OT>& st = sm.st[x % kStages];
      const int nvalid = min(kChunk, T - x * kChunk);
      float b[4], qm[4], km[4], bm[4];
      float run = 0.0f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bool ok = 4 * h + j < nvalid;  // padded tokens: g = 0, q = k = 0, beta = 0
        float g2 = ok ? kGateLog2 * sigmoid_fast(Raw<IO>::f32(ra[j])) : 0.0f;
        qm[j] = ok ? Raw<IO>::f32(rq[j]) : 0.0f;
        km[j] = ok ? Raw<IO>::f32(rk[j]) : 0.0f;
        bm[j] = ok ? rb[j] : 0.0f;
        run += g2;
        b[j] = run;
      }
      // prefix over the four token groups of this channel (lanes n, n+16, n+32, n+48)
      float u = run;
      float t1 = __shfl_up(u, 16, 64);
      u += h >= 1 ? t1 : 0.0f;
      float t2 = __shfl_up(u, 32, 64);
      u += h >= 2 ? t2 : 0.0f;
      const float prefix = u - run;
      const float bc = __shfl(u, n + 48, 64);  // log2 of Gamma_C
      const float gam_c = __builtin_amdgcn_exp2f(bc);
      float kbar[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = 4 * h + j;
        float b2 = b[j] + prefix;
        float gam = __builtin_amdgcn_exp2f(b2);
        float inv = __builtin_amdgcn_exp2f(-b2);
        float kt = km[j] * inv;
        const int fl = grp_c * 16 + r;
        st.xf[0][kb_c][fl][slot_c] = from_f32<OT>(km[j] * gam);
        st.xf[1][kb_c][fl][slot_c] = from_f32<OT>(qm[j] * gam);
        st.kf[kb_c][fl][slot_c] = from_f32<OT>(kt);
        kbar[j] = kt * gam_c;
      }
      store_frag4<OT>(&st.kbf[wave][lane][0], frag4<OT>(kbar[0], kbar[1], kbar[2], kbar[3]));
      if (h == 0) st.gamma_c[col] = gam_c;
      if (n == 0) {
#pragma unroll
        for (int j = 0; j < 4; ++j) st.beta[4 * h + j] = bm[j];
      }
    }

    // ------------------------------------------------ store(i - 3): staged output tile
    if (i - 3 >= 0 && i - 3 < nchunks && tid < 256) {
      const int x = i - 3;
      const int tok = tid >> 4, c8 = 8 * (tid & 15);
      const int t = x * kChunk + tok;
      if (t < T) {
        const IO* src = &sm.ostage[x & 1][tok][c8];
        IO* dst = o + base + (size_t)t * rs + c8;
        if constexpr (sizeof(IO) == 2) {
          *reinterpret_cast<bf16x8*>(dst) = *reinterpret_cast<const bf16x8*>(src);
        } else {
          reinterpret_cast<f32x4*>(dst)[0] = reinterpret_cast<const f32x4*>(src)[0];
          reinterpret_cast<f32x4*>(dst)[1] = reinterpret_cast<const f32x4*>(src)[1];
        }
      }
    }

    __syncthreads();
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      rq[j] = nq[j];
      rk[j] = nk[j];
      ra[j] = na[j];
      rb[j] = nb[j];
      rv[j] = nv[j];
    }
  }

  // ---------------------------------------------------------------- state out
#pragma unroll
  for (int rt = 0; rt < 8; ++rt)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int row = 16 * rt + 4 * h + j;
      final_state[((size_t)unit * kD + row) * kD + col] = sacc[rt][j];
    }
}

hipError_t launch_chunk_fwd(const void* q, const void* k, const void* v, const void* a, const float* beta,
                            const float* initial_state, void* o, float* final_state, int B, int T, int H,
                            bool bf16_io, hipStream_t stream) {
  const int units = B * H;
  if (units == 0) return hipSuccess;
  if (bf16_io) {
    hipLaunchKernelGGL((chunk_fwd_kernel<bf16, bf16>), dim3(units), dim3(kThreads), 0, stream, (const bf16*)q,
                       (const bf16*)k, (const bf16*)v, (const bf16*)a, beta, initial_state, (bf16*)o, final_state, T,
                       H);
  } else {
    hipLaunchKernelGGL((chunk_fwd_kernel<float, float>), dim3(units), dim3(kThreads), 0, stream, (const float*)q,
                       (const float*)k, (const float*)v, (const float*)a, beta, initial_state, (float*)o, final_state,
                       T, H);
  }
  return hipGetLastError();
}

}  // namespace kda
