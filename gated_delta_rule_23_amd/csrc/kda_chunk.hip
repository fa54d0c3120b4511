/*
 * kda_chunk.hip -- chunkwise KDA prefill on gfx950: the general kernel, used
 * for fp32 I/O (bf16 I/O has its own kernel in kda_prefill_bf16.hip).
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
 * Mapping: kParts 512-thread workgroups (8 waves, two per SIMD) per (b, h):
 * one, or, while more per (b, h) still fit on the device at once, two or
 * four, each owning 128 / kParts state columns.  Lane l of wave w gates key
 * channel 16w + l%16 and owns state column 16w + l%16 (one workgroup) or
 * (128 / kParts) part + 16w + l%16 (waves w < 8 / kParts only; the other
 * waves then take the Gram products and the solve); its group h = l/16
 * covers tokens 4h .. 4h+3 of a chunk.
 *   - The 128 x 128 fp32 state stays in MFMA accumulators for the whole
 *     sequence: each chain wave keeps 128 x 16 of it in eight 16x16 tiles.
 *     The chain's fp32 MFMAs bound the iteration; with two workgroups a
 *     SIMD runs one chain wave instead of two.
 *   - Four chunks are in flight.  In iteration i:
 *       chain(i-3):  P = [Kh; Qh] S, [Vt; A Vt] = [M; A M] (V - Kh S),
 *                    O = Qh S + A Vt (stored straight from registers),
 *                    S <- Diag(Gamma_C) S + Kb^T Vt
 *                    (18 MFMAs per chain wave, their own columns);
 *       solve(i-2):  one wave forms (I + N)^{-1} = (I - N)(I + N^2)(I + N^4)(I + N^8)
 *                    for the nilpotent N = Diag(beta) L on MFMA, then M and A M;
 *       gram(i-1):   another wave (on another SIMD) forms the 16x16 Gram
 *                    products on MFMA and masks them into N and A;
 *       gate(i):     every lane: g = -5 sigmoid(a), cumulative sums, the four
 *                    scaled operands, written to LDS in MFMA fragment order;
 *       loads:       the next gate's q, k, a, beta and the next chain's V go to
 *                    registers through buffer loads sized to the chunk, which
 *                    return zero past T.
 *     One workgroup barrier per iteration separates producers and consumers
 *     of the four LDS stages.
 * The kernel is written for an operand type OT and runs with OT = fp32 (fp32
 * operands on the 16x16x4 fp32 MFMA, fp32 accumulation); the state stays
 * fp32.
 */
#include <type_traits>

#include "kda_common.h"
#include "kda_internal.h"

namespace kda {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kStages = 4;
constexpr float kGateLog2 = kGateFloor * kLog2e;  // g * log2(e) = kGateLog2 * sigmoid(a)

/* One chunk's operands, in the order the MFMA lanes read them. */
template <typename OT>
struct Stage {
  alignas(16) OT xf[2][4][64][8];  // [Kh | Qh][block of 32 key channels][lane][slot]: A of P = X S and of the Gram products
  alignas(16) OT kf[4][64][8];     // Kt: [block of 32 key channels][lane][slot]
  alignas(16) OT kbf[8][64][4];    // Kb^T: [tile of 16 key channels][lane][token slot]: A of the state update
  alignas(16) OT maf[2][64][4];    // [M | A M]: A of [Vt; A Vt] = [M; A M] R
  alignas(16) OT nf[3][64][4];     // N^T, N, A^T in C layout: operands of the solve
  alignas(16) float gamma_c[kD];   // Gamma_C per key channel
  alignas(16) float beta[kChunk];
};

template <typename OT>
struct Smem {
  Stage<OT> st[kStages];
  alignas(16) float prefix[kWaves][kChunk][4];  // per wave: [key channel][token group] partial sums of the gate
};

/* Run-time options of the general kernel (PrefillOptions of kda_internal.h,
 * the checkpoint interval in chunks). */
struct ChunkArgs {
  float* states;
  int state_every, n_states;
  const int* cu_seqlens;
  int seg_len, seg_count, last_only;
  int mode, gate;
  int units, trans_units;  // units of the launch; kModeTransFrag: the transition runs among them
};

template <typename IO, typename OT, int kParts>
__global__ __launch_bounds__(kThreads) void chunk_fwd_kernel(const IO* __restrict__ q, const IO* __restrict__ k,
                                                             const IO* __restrict__ v, const IO* __restrict__ a,
                                                             const float* __restrict__ beta,
                                                             const float* initial_state, IO* __restrict__ o,
                                                             float* final_state, int T_all, int H, ChunkArgs args) {
  __shared__ Smem<OT> sm;
  float* const states = args.states;
  const int state_every = args.state_every, n_states = args.n_states;
  const bool state_only = args.mode >= kModeFragment;      // no o
  // With kModeTransFrag, unit b H + h below args.trans_units is a
  // transition run and b H + h + trans_units the fragment run of the same
  // segment; the final states land at the unit index.  With several
  // workgroups per unit they come in groups of 8 kParts: slot s takes column
  // part s / 8 of unit 8 grp + s % 8 (dispatch deals workgroups to the XCDs
  // round robin, so all parts of a unit share an XCD and its L2).
  static_assert(kParts == 1 || kParts == 2 || kParts == 4, "one, two or four workgroups per unit");
  constexpr int kChainW = kWaves / kParts;  // waves holding state columns
  // Four workgroups per unit: the solve and the Gram products rotate over the
  // waves of SIMDs 2 and 3, the two chain waves having SIMDs 0 and 1 (111
  // against 116 us on 2 heads x 512 tokens, rotating over all six).
  constexpr int kOffChain[4] = {2, 3, 6, 7};
  const int unit = kParts > 1 ? 8 * (int)(blockIdx.x / (8 * kParts)) + (int)(blockIdx.x & 7) : (int)blockIdx.x;
  const int part = kParts > 1 ? (int)((blockIdx.x >> 3) % kParts) : 0;
  if (unit >= args.units) return;  // whole workgroup, before any barrier
  const int half_units = args.mode == kModeTransFrag ? args.trans_units : 0;
  const bool transition = args.mode == kModeTransition || unit < half_units;  // S0 = I, v = 0
  const int gate_mode = args.gate;
  const int seq_unit = unit >= half_units ? unit - half_units : unit;
  const int bb = seq_unit / H, hh = seq_unit % H;
  // The sequence's first token and length: b T_all and T_all; for packed
  // sequences, cu_seqlens[b] .. cu_seqlens[b + 1] clamped to [0, T_all] (so
  // any contents of cu_seqlens keep every access inside the tensors); for
  // segments, segment j = b % seg_count of sequence b / seg_count.
  int64_t tok0 = (int64_t)bb * T_all;
  int T = T_all;
  int out_unit = unit;
  bool write_final = true;
  if (args.seg_len > 0) {
    const int sb = bb / args.seg_count, j = bb % args.seg_count, s0 = j * args.seg_len;
    tok0 = (int64_t)sb * T_all + s0;
    T = max(0, min(args.seg_len, T_all - s0));
    if (args.last_only) {
      write_final = j == args.seg_count - 1;
      out_unit = sb * H + hh;
    }
  } else if (args.cu_seqlens) {
    const int c0 = min(max(args.cu_seqlens[bb], 0), T_all);
    const int c1 = min(max(args.cu_seqlens[bb + 1], c0), T_all);
    tok0 = c0;
    T = c1 - c0;
  }
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int n = lane & 15, h = lane >> 4;
  // The gate: wave w gates key channels 16w .. 16w+15 (group w).  With four
  // workgroups per unit the two chain waves gate none: waves 6 and 7 (SIMDs
  // 2 and 3) also gate their groups 0 and 1.
  constexpr bool kGatePairs = kParts == 4;
  constexpr int kGS = kGatePairs ? 2 : 1;  // gate groups per wave, at most
  const bool gate_wave = !kGatePairs || wave >= 2;
  const int n_groups = kGatePairs && wave >= 6 ? 2 : 1;
  const int g0 = wave;  // the first group; the second (waves 6 and 7) is wave - 6
  // the state column of this lane: chain waves only (the first 8 / kParts)
  const bool chain_wave = wave < kChainW;
  const int col = (kD / kParts) * part + 16 * (wave % kChainW) + n;
  const int nchunks = (T + kChunk - 1) / kChunk;

  // This (b, h) sequence: rows of token t start at seq + t * H * 128.
  const int64_t tok_elems = (int64_t)H * kD;
  const int64_t seq_off = (tok0 * H + hh) * kD;
  const float* beta_seq = beta + tok0 * H + hh;
  // Byte offsets of this lane's four tokens (4h .. 4h+3) inside a chunk:
  // its gate channel (q, k, a), its state column (v, o) and beta.
  int off_row[kGS][4], off_col[4], off_beta[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
#pragma unroll
    for (int gs = 0; gs < kGS; ++gs)
      off_row[gs][j] = (int)(((4 * h + j) * tok_elems + 16 * (gs == 0 ? g0 : max(wave - 6, 0)) + n) * (int64_t)sizeof(IO));
    off_col[j] = (int)(((4 * h + j) * tok_elems + col) * (int64_t)sizeof(IO));
    off_beta[j] = (4 * h + j) * H * (int)sizeof(float);
  }
  // Chunk x of a row tensor / of beta as a buffer resource sized to the
  // chunk's valid tokens: loads past T (or of chunks outside [0, nchunks))
  // return 0 and stores there are dropped.  The sizes take three values and
  // the bases advance by one chunk stride per iteration, so a descriptor costs
  // a few scalar instructions.
  const int64_t rows_step = (int64_t)kChunk * tok_elems * (int64_t)sizeof(IO);
  const int64_t beta_step = (int64_t)kChunk * H * (int64_t)sizeof(float);
  const int tail = T - (nchunks - 1) * kChunk;  // tokens in the last chunk (nchunks > 0)
  const int rows_full = (int)(((kChunk - 1) * tok_elems + kD) * (int64_t)sizeof(IO));
  const int rows_tail = (int)(((int64_t)(tail - 1) * tok_elems + kD) * (int64_t)sizeof(IO));
  const int beta_full = ((kChunk - 1) * H + 1) * (int)sizeof(float);
  const int beta_tail = ((tail - 1) * H + 1) * (int)sizeof(float);
  auto rows_bytes = [&](int x) { return (unsigned)x < (unsigned)nchunks ? (x == nchunks - 1 ? rows_tail : rows_full) : 0; };
  auto beta_bytes = [&](int x) { return (unsigned)x < (unsigned)nchunks ? (x == nchunks - 1 ? beta_tail : beta_full) : 0; };
  const char* q_seq = reinterpret_cast<const char*>(q + seq_off);
  const char* k_seq = reinterpret_cast<const char*>(k + seq_off);
  const char* a_seq = reinterpret_cast<const char*>(a + seq_off);
  const char* v_seq = reinterpret_cast<const char*>(v + seq_off);
  const char* o_seq = reinterpret_cast<const char*>(o + seq_off);
  const char* b_seq = reinterpret_cast<const char*>(beta_seq);

  // ---------------------------------------------------------------- state in
  f32x4 sacc[8];
#pragma unroll
  for (int rt = 0; rt < 8; ++rt)  // zeros, or the identity for a transition run
#pragma unroll
    for (int j = 0; j < 4; ++j) sacc[rt][j] = transition && 16 * rt + 4 * h + j == col ? 1.0f : 0.0f;
  if (initial_state && !transition && chain_wave) {  // one test, so the loads issue back to back
#pragma unroll
    for (int rt = 0; rt < 8; ++rt)
#pragma unroll
      for (int j = 0; j < 4; ++j) sacc[rt][j] = initial_state[((size_t)unit * kD + 16 * rt + 4 * h + j) * kD + col];
  }

  // Prefetch registers: q, k, a, beta of the next gate pass and V of the next
  // serial step.  Two sets alternate between consecutive iterations, and every
  // element keeps its own 32-bit register, so no wait follows the loads: they
  // complete under the next iteration's work.
  struct Regs {
    uint32_t q[kGS][4], k[kGS][4], a[kGS][4], v[4];
    float b[4];
  };
  // x: chunk index; rows_off / beta_off: x chunk strides in bytes
  // (a scalar gate's fp32 logits are [.., H] like beta; with no gate a is not read)
  const char* ga_seq = reinterpret_cast<const char*>(reinterpret_cast<const float*>(a) + tok0 * H + hh);
  auto load_gate_inputs = [&](int x, int64_t rows_off, int64_t beta_off, Regs& r) {
    const int nb = rows_bytes(x);
    const rsrc_t rq = make_rsrc(q_seq + rows_off, nb), rk = make_rsrc(k_seq + rows_off, nb),
                 ra = make_rsrc(a_seq + rows_off, gate_mode == kGateChannel ? nb : 0),
                 rg = make_rsrc(ga_seq + beta_off, gate_mode == kGateScalar ? beta_bytes(x) : 0),
                 rb = make_rsrc(b_seq + beta_off, beta_bytes(x));
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int gs = 0; gs < kGS; ++gs) {
        if (gs >= n_groups) break;
        r.q[gs][j] = Raw<IO>::load(rq, off_row[gs][j]);
        r.k[gs][j] = Raw<IO>::load(rk, off_row[gs][j]);
        // the gate logit as fp32 bits (zero-sized resources return 0 without reading)
        r.a[gs][j] = gate_mode == kGateScalar
                         ? __builtin_amdgcn_raw_buffer_load_b32(rg, off_beta[j], 0, 0)
                         : __float_as_uint(Raw<IO>::f32(Raw<IO>::load(ra, off_row[gs][j])));
      }
      r.b[j] = load_f32(rb, off_beta[j]);
    }
  };
  auto load_chain_inputs = [&](int x, int64_t rows_off, Regs& r) {
    const rsrc_t rv = make_rsrc(v_seq + rows_off, transition ? 0 : rows_bytes(x));  // v = 0 in a transition run
#pragma unroll
    for (int j = 0; j < 4; ++j) r.v[j] = Raw<IO>::load(rv, off_col[j]);
  };

  // The 16x16 identity as a B operand.  A x I hands A back in accumulator
  // layout, i.e. transposed across lanes: rows that sit one per lane (a key
  // channel's four tokens) come back as four consecutive rows per lane, which
  // is the order the MFMA fragments want.  The product is exact.
  const Frag4<OT> ident = frag4<OT>(4 * h == n ? 1.0f : 0.0f, 4 * h + 1 == n ? 1.0f : 0.0f,
                                    4 * h + 2 == n ? 1.0f : 0.0f, 4 * h + 3 == n ? 1.0f : 0.0f);
  auto transpose16 = [&](const f32x4& x) {
    f32x4 d = {0, 0, 0, 0};
    mfma_k16(d, frag4<OT>(x), ident);
    return frag4<OT>(d);
  };

  // ------------------------------------------------ gate: group g (g0, or wave - 6 for gs = 1), lane channel 16 g + l%16, tokens 4h .. 4h+3
  auto gate = [&](const Regs& cur, int gs, Stage<OT>& st, int nvalid, auto ragged) {
    const int g = gs == 0 ? g0 : wave - 6, gch = 16 * g + n;
    float b[4];
    float run = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      // no gate: g = 0 (alpha = 1)
      float g2 = gate_mode == kGateNone ? 0.0f : kGateLog2 * sigmoid_fast(__uint_as_float(cur.a[gs][j]));
      if constexpr (decltype(ragged)::value) g2 = 4 * h + j < nvalid ? g2 : 0.0f;  // padded tokens: g = 0
      run += g2;
      b[j] = run;
    }
    // prefix over the four token groups of this channel, through LDS
    float* pre = &sm.prefix[g][n][0];
    pre[h] = run;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");  // lanes read each other's writes
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const f32x4 part = *reinterpret_cast<const f32x4*>(pre);
    const float prefix = (h > 0 ? part[0] : 0.0f) + (h > 1 ? part[1] : 0.0f) + (h > 2 ? part[2] : 0.0f);
    const float gam_c = __builtin_amdgcn_exp2f((part[0] + part[1]) + (part[2] + part[3]));  // Gamma_C
    f32x4 kh, qh, kt, kbar;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float b2 = b[j] + prefix;
      const float gam = __builtin_amdgcn_exp2f(b2);
      const float inv = __builtin_amdgcn_exp2f(-b2);
      const float kk = Raw<IO>::f32(cur.k[gs][j]), qq = Raw<IO>::f32(cur.q[gs][j]);  // zero past T
      kh[j] = kk * gam;
      qh[j] = qq * gam;
      kt[j] = kk * inv;
      kbar[j] = kt[j] * gam_c;
    }
    // Transposes: afterwards lane (token l%16, group h) holds key channels
    // 16w + 4h .. 16w + 4h + 3, i.e. slots 0..3 (even w) or 4..7 (odd w) of
    // its K = 32 fragment row in block w / 2.  The three are independent.
    f32x4 tkh = {0, 0, 0, 0}, tqh = {0, 0, 0, 0}, tkt = {0, 0, 0, 0};
    mfma_k16(tkh, frag4<OT>(kh), ident);
    mfma_k16(tqh, frag4<OT>(qh), ident);
    mfma_k16(tkt, frag4<OT>(kt), ident);
    store_frag4<OT>(&st.kbf[g][lane][0], frag4<OT>(kbar));  // already channel-major
    if (h == 0) st.gamma_c[gch] = gam_c;
    if (n == 0) {
#pragma unroll
      for (int j = 0; j < 4; ++j) st.beta[4 * h + j] = cur.b[j];  // zero past T
    }
    const int kb_w = g >> 1, so = 4 * (g & 1);
    store_frag4<OT>(&st.xf[0][kb_w][lane][so], frag4<OT>(tkh));
    store_frag4<OT>(&st.xf[1][kb_w][lane][so], frag4<OT>(tqh));
    store_frag4<OT>(&st.kf[kb_w][lane][so], frag4<OT>(tkt));
  };

  // Byte offset of chunk i + 1 (rows and beta); chunk i + 1 - d is d strides lower.
  int64_t rows_next = rows_step, beta_next = beta_step;
  auto step = [&](int i, const Regs& cur, Regs& nxt) {
    // ------------------------------------------------ loads for the next iteration
    if (gate_wave) load_gate_inputs(i + 1, rows_next, beta_next, nxt);
    if (chain_wave) load_chain_inputs(i - 2, rows_next - 3 * rows_step, nxt);

    // ------------------------------------------------ chain(i - 3): the serial part
    if (chain_wave && i - 3 >= 0 && i - 3 < nchunks) {
      const int x = i - 3;
      const Stage<OT>& st = sm.st[x % kStages];
      // operands from LDS first, so their latency hides behind the conversions
      Frag8<OT> fk[4], fq[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        fk[kb] = load_frag8<OT>(&st.xf[0][kb][lane][0]);
        fq[kb] = load_frag8<OT>(&st.xf[1][kb][lane][0]);
      }
      const Frag4<OT> fm = load_frag4<OT>(&st.maf[0][lane][0]);
      const Frag4<OT> fam = load_frag4<OT>(&st.maf[1][lane][0]);
      Frag4<OT> fkb[8];
      f32x4 gc[8];
#pragma unroll
      for (int rt = 0; rt < 8; ++rt) {
        fkb[rt] = load_frag4<OT>(&st.kbf[rt][lane][0]);
        gc[rt] = *reinterpret_cast<const f32x4*>(&st.gamma_c[16 * rt + 4 * h]);
      }
      Frag8<OT> sf[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) sf[kb] = frag8<OT>(sacc[2 * kb], sacc[2 * kb + 1]);
      // Kh S first, so the residual is formed while Qh S runs
      f32x4 pk = {0, 0, 0, 0}, pq = {0, 0, 0, 0};
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) mfma_k32(pk, fk[kb], sf[kb]);
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) mfma_k32(pq, fq[kb], sf[kb]);
      // V is zero past T (and M has zero columns there), so padded tokens add nothing.
      Frag4<OT> fr = frag4<OT>(Raw<IO>::f32(cur.v[0]) - pk[0], Raw<IO>::f32(cur.v[1]) - pk[1],
                               Raw<IO>::f32(cur.v[2]) - pk[2], Raw<IO>::f32(cur.v[3]) - pk[3]);
      f32x4 dm = {0, 0, 0, 0}, da = {0, 0, 0, 0};
      mfma_k16(dm, fm, fr);
      mfma_k16(da, fam, fr);
#pragma unroll
      for (int rt = 0; rt < 8; ++rt) sacc[rt] *= gc[rt];  // Diag(Gamma_C) S, under the two MFMAs
      const Frag4<OT> fv = frag4<OT>(dm);
#pragma unroll
      for (int rt = 0; rt < 8; ++rt) mfma_k16(sacc[rt], fkb[rt], fv);
      // O rows 4h .. 4h+3 of this column; stores past T are dropped
      const rsrc_t ro = make_rsrc(o_seq + rows_next - 4 * rows_step, state_only ? 0 : rows_bytes(x));
#pragma unroll
      for (int j = 0; j < 4; ++j) Raw<IO>::store(ro, off_col[j], pq[j] + da[j]);
      // checkpoint: the state after token 16 (x + 1), when that is a multiple of the interval
      if (states && (x + 1) % state_every == 0 && (x + 1) / state_every <= n_states) {
        float* dst = states + ((size_t)unit * n_states + (x + 1) / state_every - 1) * kD * kD;
#pragma unroll
        for (int rt = 0; rt < 8; ++rt)
#pragma unroll
          for (int j = 0; j < 4; ++j) dst[(size_t)(16 * rt + 4 * h + j) * kD + col] = sacc[rt][j];
      }
    }

    // ------------------------------------------------ solve(i - 2): one wave
    // (several workgroups per unit: on the waves that hold no state)
    if (i - 2 >= 0 && i - 2 < nchunks &&
        wave == (kParts == 4   ? kOffChain[(i - 2) & 3]
                 : kParts > 1 ? kChainW + (i - 2) % (kWaves - kChainW)
                              : (i - 2) % kWaves)) {
      Stage<OT>& st = sm.st[(i - 2) % kStages];
      const Frag4<OT> fnt = load_frag4<OT>(&st.nf[0][lane][0]);
      const Frag4<OT> fnc = load_frag4<OT>(&st.nf[1][lane][0]);
      const Frag4<OT> fat = load_frag4<OT>(&st.nf[2][lane][0]);
      f32x4 y;  // Y0 = I - N
#pragma unroll
      for (int j = 0; j < 4; ++j) y[j] = (4 * h + j == n ? 1.0f : 0.0f) - to_f32(fnc.v[j]);
      // A operand of X = C layout of X^T, so (N^p, (N^p)^T) pairs feed each other.
      f32x4 n2c = {0, 0, 0, 0}, n2t = {0, 0, 0, 0}, n4c = {0, 0, 0, 0}, n4t = {0, 0, 0, 0}, n8t = {0, 0, 0, 0};
      mfma_k16(n2c, fnt, fnc);
      mfma_k16(n2t, fnc, fnt);
      mfma_k16(y, frag4<OT>(n2t), frag4<OT>(y));  // Y1 = (I + N^2) Y0
      mfma_k16(n4c, frag4<OT>(n2t), frag4<OT>(n2c));
      mfma_k16(n4t, frag4<OT>(n2c), frag4<OT>(n2t));
      mfma_k16(y, frag4<OT>(n4t), frag4<OT>(y));  // Y2 = (I + N^4) Y1
      mfma_k16(n8t, frag4<OT>(n4c), frag4<OT>(n4t));
      mfma_k16(y, frag4<OT>(n8t), frag4<OT>(y));  // (I + N)^{-1} = (I + N^8) Y2
      const f32x4 m = y * st.beta[n];             // M = (I + N)^{-1} Diag(beta)
      f32x4 am = {0, 0, 0, 0};
      mfma_k16(am, fat, frag4<OT>(m));  // A M
      // A fragments of [M; A M] = their accumulator layouts transposed
      store_frag4<OT>(&st.maf[0][lane][0], transpose16(m));
      store_frag4<OT>(&st.maf[1][lane][0], transpose16(am));
    }

    // ------------------------------------------------ gram(i - 1): another wave, another SIMD
    if (i - 1 >= 0 && i - 1 < nchunks &&
        wave == (kParts == 4   ? kOffChain[(i + 1) & 3]
                 : kParts > 1 ? kChainW + (i + 1) % (kWaves - kChainW)
                              : (i + 3) % kWaves)) {
      Stage<OT>& st = sm.st[(i - 1) % kStages];
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
      }
      store_frag4<OT>(&st.nf[0][lane][0], frag4<OT>(nt));
      store_frag4<OT>(&st.nf[1][lane][0], transpose16(nt));  // C layout of N
      store_frag4<OT>(&st.nf[2][lane][0], frag4<OT>(at));
    }

    // ------------------------------------------------ gate(i)
    if (i < nchunks && gate_wave) {
      const int nvalid = min(kChunk, T - i * kChunk);
      Stage<OT>& st = sm.st[i % kStages];
#pragma unroll
      for (int gs = 0; gs < kGS; ++gs) {
        if (gs >= n_groups) break;
        if (nvalid == kChunk)
          gate(cur, gs, st, nvalid, std::false_type());
        else
          gate(cur, gs, st, nvalid, std::true_type());
      }
    }

    __syncthreads();
    rows_next += rows_step;
    beta_next += beta_step;
  };

  Regs A, B;
  if (gate_wave) load_gate_inputs(0, 0, 0, A);
  for (int i = 0; i < nchunks + 3; i += 2) {
    step(i, A, B);
    step(i + 1, B, A);
  }

  // ---------------------------------------------------------------- state out
  if (write_final && chain_wave) {
#pragma unroll
    for (int rt = 0; rt < 8; ++rt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        int row = 16 * rt + 4 * h + j;
        final_state[((size_t)out_unit * kD + row) * kD + col] = sacc[rt][j];
      }
  }
}

hipError_t launch_chunk_fwd(const void* q, const void* k, const void* v, const void* a, const float* beta,
                            const float* initial_state, void* o, float* final_state, int B, int T, int H,
                            bool bf16_io, hipStream_t stream, const PrefillOptions& opt_in) {
  PrefillOptions opt = opt_in;
  const int seqs = opt.seg_len > 0 ? B * opt.seg_count : B;
  const int trans_units = opt.mode == kModeTransFrag ? seqs * H : 0;
  const int units = seqs * H + trans_units;
  if (units == 0) return hipSuccess;
  // the interval in chunks and the number of checkpoints (none: no checkpoint output)
  const int every_tokens = opt.states ? opt.state_every : 0;
  opt.n_states = opt.states ? T / every_tokens : 0;
  opt.state_every = opt.states ? every_tokens / kChunk : 0;
  if (opt.n_states == 0) opt.states = nullptr;
  if (bf16_io) {
    if (opt.states) opt.mode = kModeEmit;
    else if ((opt.cu_seqlens || opt.seg_len > 0) && opt.mode == kModePlain) opt.mode = kModePacked;
    return launch_chunk_fwd_bf16(q, k, v, a, beta, initial_state, o, final_state, B, T, H, stream, opt);
  }
  const ChunkArgs args = {opt.states, opt.state_every, opt.n_states, opt.cu_seqlens, opt.seg_len, opt.seg_count,
                          opt.last_only ? 1 : 0, opt.mode, opt.gate, units, trans_units};
  // Two or four workgroups per unit while they all fit on the device at once
  // (one per compute unit, whole groups of 8 units).
  int cus = 0;
  hipError_t e = device_cu_count(stream, &cus);
  if (e != hipSuccess) return e;
  const int64_t groups = ((int64_t)units + 7) / 8;
  const int parts = 32 * groups <= cus ? 4 : 16 * groups <= cus ? 2 : 1;
  auto launch = [&](auto kernel, int64_t grid) {
    hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(kThreads), 0, stream, (const float*)q, (const float*)k,
                       (const float*)v, (const float*)a, beta, initial_state, (float*)o, final_state, T, H, args);
  };
  if (parts == 4)
    launch(chunk_fwd_kernel<float, float, 4>, 32 * groups);
  else if (parts == 2)
    launch(chunk_fwd_kernel<float, float, 2>, 16 * groups);
  else
    launch(chunk_fwd_kernel<float, float, 1>, units);
  e = hipGetLastError();
  // fp32 I/O: the output gate and norm as a second pass over o
  if (e == hipSuccess && opt.z != nullptr)
    e = launch_output_gate_norm(o, opt.z, o, (int64_t)seqs * T * H, opt.eps, false, stream);
  return e;
}

}  // namespace kda
