/*
 * kda_prefill_bf16.hip -- chunkwise KDA prefill for bf16 q, k, v, a, o on gfx950.
 *
 * Same chunk algebra as the general kernel in kda_chunk.hip (page "Kimi
 * K3：从三条信息流到完整系统", eq. (1), (3), (4), (5)); per chunk of C = 16
 * tokens, with b the in-chunk cumulative log-decay and Gamma = e^b:
 *   Kh = K Gamma, Qh = Q Gamma, Kt = K / Gamma, Kb = K Gamma_C / Gamma,
 *   N  = Diag(beta) StrictTril(Kh Kt^T),  A = Tril(Qh Kt^T),
 *   M  = (I + N)^{-1} Diag(beta),  W = M Kh,  U = M V,
 *   Vt = U - W S,   O = Qh S + A Vt,   S' = Diag(Gamma_C) S + Kb^T Vt.
 * Folding M into W and U before the state arrives leaves three MFMA rounds
 * on the serial path (W S and Qh S, then A Vt and the state update).
 *
 * Mapping: 512-thread workgroups, 8 waves, two per SIMD (768 threads, three
 * per SIMD, with two workgroups per sequence).  The columns of S
 * (value channels) evolve independently given the per-chunk operands, so a
 * (b, h) sequence is served by one workgroup owning all 128 state columns or,
 * while more workgroups per sequence still fit on the device at once, by two
 * owning 64 each or four owning 32 (kCT, the 16-column tiles per chain wave
 * holding state, is 2 or 1; with four, chain waves 2 and 3 hold none and
 * take the Gram products, the solve and the O stores); they then repeat the
 * column-independent per-chunk work, which costs nothing on CUs that would
 * be idle and shortens the serial step each one runs.  Wave
 * c < 4 (the chain wave of SIMD c) owns kCT 16-column tiles of the state
 * (8 kCT 16x16 fp32 accumulator tiles) and wave 4 + g (the gate wave of SIMD
 * g) owns key channels 32g .. 32g+31 of the gate, so every SIMD pairs the
 * MFMA-heavy serial step with the VALU-heavy gate.  With two workgroups per
 * sequence, wave 8 + b (the helper wave of SIMD b) takes from the chain
 * waves all they do besides U and the serial step: the input loads, W, the
 * O stores, the Gram products and the solve.  Iteration i of the main loop
 * does, separated by one workgroup barrier:
 *   inputs:      beta, q, k, a of chunk i+2 and v of chunk i-1 loaded
 *                straight into LDS token-major (buffer_load ... lds, 16 bytes
 *                a lane, whole 256-byte rows), loader wave w (the helper
 *                waves with two workgroups per sequence, the chain waves with
 *                four, the gate waves with one) taking tensor w % 4 of q, k,
 *                a, v;
 *   gate waves:  gate(i): lane (channel 32g + l%32, tokens 8(l/32) .. +7)
 *                with the per-channel gate (the scalar and no-gate modes:
 *                two channels, tokens 4(l/16) .. +3): g, the cumulative sums
 *                and the four scaled operands, stored channel-major;
 *   chain waves: store_o(i-5) (helper wave 0 with two workgroups, chain
 *                wave 3 with four); prep(i-3):
 *                their tiles of W = M Kh (the helper waves' with two) and
 *                U = M V;
 *                chain(i-4): P = [W; Qh] S, Vt = U - P_W, O = P_Q + A Vt,
 *                S <- Diag(Gamma_C) S + Kb^T Vt; then, on chain waves 1, 2
 *                and 3 (helper waves 1, 2, 3 with two workgroups, chain
 *                waves 2 and 3 with four), gram(i-1) as two products (Kt
 *                Kh^T masked into N, Kt Qh^T into A) and solve(i-2):
 *                (I + N)^{-1} = (I - N)(I + N^2)(I + N^4)(I + N^8) (N is
 *                nilpotent, the product is exact) and M.
 * Operands change between token-major and channel-major through
 * ds_read_b64_tr_b16, which transposes 16-bit elements across the lanes of
 * each 16-lane group while it reads: lane i, element j of the result is
 * element i % 4 of what lane 4j + i/4 addressed.  A 16-row tile with rows of
 * 16 elements read at byte 8 * lane thus arrives with lane i holding column
 * i, rows 4(l/16) .. +3 -- the accumulator (and B operand) layout -- while a
 * plain 8-byte read of row i, elements 4(l/16) .. +3 gives the A layout.
 * Channel-major tiles keep a row's four 8-byte token groups in the order
 * group ^ ((row / 4) % 4): with it the plain accesses of a wave (16 rows x 4
 * groups) and the transposing reads (4 whole rows per 16 lanes) both spread
 * over all LDS banks, where the unpermuted plain pattern costs 8x as long.
 */
#include <type_traits>

#include "kda_bf16_tiles.h"
#include "kda_common.h"
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int kChainWaves = 4;  // waves 0..3: the serial part, 16 kCT state columns each
/* Threads of a workgroup: a chain and a gate wave per SIMD, and with two
 * workgroups per sequence (kLay 1) a helper wave per SIMD as well. */
constexpr int threads_of(int lay) { return 64 * (lay == 1 ? 3 : 2) * kChainWaves; }
constexpr int kORow = 136;     // O staging row: 128 columns + 8 pad (the four rows one 2-byte write covers hit distinct banks)
constexpr float kGateLog2 = kGateFloor * kLog2e;
constexpr float kInvGateLog2 = 1.0f / kGateLog2;

/* g log2(e) = kGateLog2 sigmoid(a) = 1 / ((1 + 2^(-a log2 e)) / kGateLog2): the gate's log-decay in log2 units. */
__device__ __forceinline__ float gate_log2(float a) {
  return __builtin_amdgcn_rcpf(fmaf(__builtin_amdgcn_exp2f(-a * kLog2e), kInvGateLog2, kInvGateLog2));
}


/* LDS rings.  A chunk x lives in slot x % (ring size); the ring a buffer
 * belongs to follows from the iteration that writes it and the last one that
 * reads it.  Buffers of one ring share a slot, so one base address per ring
 * and iteration serves all of them (the rest are immediate offsets). */
struct Ring5 {
  alignas(16) bf16 qh[kD][kChunk];          // channel-major [channel][token]: gate (x) -> gram (x+1), chain (x+4)
  alignas(16) bf16 kb[kD][kChunk];          // gate (x) -> chain (x+4)
  alignas(16) bf16 am[kChunk][kChunk];      // A: gram (x+1) -> chain (x+4)
  alignas(16) float gamma_c[4][4][8];       // Gamma_C[16 rt + 4 g + q] at [g][q][rt]: gate (x) -> chain (x+4)
};
struct Ring4 {
  alignas(16) bf16 kh[kD][kChunk];          // gate (x) -> gram (x+1), prep (x+3)
};
struct Ring2 {
  alignas(16) bf16 kt[kD][kChunk];           // gate (x) -> gram (x+1)
  alignas(16) bf16 w[kD][kChunk];            // prep (x+3) -> chain (x+4)
  alignas(16) bf16 n[kChunk][kChunk];        // N: gram (x+1) -> solve (x+2)
  alignas(16) bf16 mt[kChunk][kChunk];       // M^T: solve (x+2) -> prep (x+3)
  alignas(16) bf16 ost[kChunk][kORow];       // O, token-major: chain (x) at x+4 -> stored at x+5
};
struct Smem {
  Ring5 r5[5];
  Ring4 r4[4];
  Ring2 r2[2];
};
/* Inputs, written by the loads themselves (buffer_load ... lds: lane l's
 * bytes land at the instruction's LDS base + 16 l, or + 4 l for beta).  A
 * token-major row of 128 channels is therefore 256 bytes with no padding; its
 * 16-byte slots sit XOR-permuted (in_swz_ch for q, k and a under the
 * per-channel gate, in_swz otherwise) to keep the transposing reads of the
 * gate and of prep free of bank conflicts. */
struct InQKA {
  alignas(16) bf16 t[3][kChunk][kD];  // q, k, a of chunk x (slot x % 3): loaded at x-2 -> gate (x)
};
struct InV {
  alignas(16) bf16 t[kChunk][kD];  // v of chunk x (slot x % 3): loaded at x+1 -> prep (x+3)
};
struct InBeta {
  alignas(16) float t[kChunk];  // beta of chunk x (slot x % 5): loaded at x-2 -> gram (x+1), solve (x+2)
};

/* 16-byte slot s of staged input row r is stored at slot s ^ in_swz(r): a
 * 16-lane group of a transposing read touches rows 4h .. 4h+3 and two slots
 * of each, which then cover 8 distinct slots; the two groups of a half wave
 * (h even, h odd) fall 8 slots apart. */
__device__ __forceinline__ int in_swz(int r) { return (2 * (r & 3)) ^ (8 * ((r >> 2) & 1)); }
__device__ __forceinline__ int in_off(int r, int col) { return r * kD + 8 * ((col >> 3) ^ in_swz(r)) + (col & 7); }
/* q, k and a for the per-channel gate, whose lanes hold eight tokens of one
 * channel: a half wave's transposing read touches four rows and four slots
 * (two 16-channel tiles), which in_swz_ch spreads over 16 distinct slots. */
__device__ __forceinline__ int in_swz_ch(int r) { return 4 * (r & 3); }
__device__ __forceinline__ int in_off_ch(int r, int col) { return r * kD + 8 * ((col >> 3) ^ in_swz_ch(r)) + (col & 7); }

typedef __attribute__((address_space(3))) void lds_void;

/* Loads straight into LDS (buffer_load ... lds): M0 holds the LDS base, and
 * an instruction reading M0 needs one wait state after the scalar write.
 * Written as inline assembly so that the compiler does not order every later
 * LDS access of the wave behind them: the caller waits for these loads itself
 * (vmcnt) before the workgroup barrier that publishes the data.
 *
 * Four rows of 16 bytes a lane (lane l at lds_base + 16 l + 1024 j for row
 * j): the instruction offset 1024 j is added to both the LDS and the global
 * address, so one M0 serves all four and the global offsets v1 .. v3 take
 * it back. */
__device__ __forceinline__ void load_4rows_to_lds(rsrc_t r, uint32_t lds_base, int v0, int v1, int v2, int v3) {
  asm volatile(
      "s_mov_b32 m0, %0\n\ts_nop 0\n\t"
      "buffer_load_dwordx4 %1, %5, 0 offen lds\n\t"
      "buffer_load_dwordx4 %2, %5, 0 offen offset:1024 lds\n\t"
      "buffer_load_dwordx4 %3, %5, 0 offen offset:2048 lds\n\t"
      "buffer_load_dwordx4 %4, %5, 0 offen offset:3072 lds" ::"s"(lds_base),
      "v"(v0), "v"(v1), "v"(v2), "v"(v3), "s"(r)
      : "memory", "m0");
}
/* 4 bytes per lane (lane l at lds_base + 4 l). */
__device__ __forceinline__ void load_b32_to_lds(rsrc_t r, uint32_t lds_base, int voff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, 0 offen lds" ::"s"(lds_base), "v"(voff),
               "s"(r)
               : "memory", "m0");
}

// kMode (PrefillMode): kModeEmit also writes the state checkpoints (every
// state_every chunks, n_states of them per sequence); from kModePacked on the
// sequences are delimited by cu_seqlens or cut into segments of seg_len
// tokens (seg_count per sequence); kModeFragment writes only the final
// states; kModeTransition also starts every sequence from the identity and
// reads no v (the segment's transition matrix); kModeTransFrag runs both,
// the transitions as units below trans_units and the fragments above.
// kGate (kda_gate): the gate per key channel, one fp32 logit per token and
// head, or none (alpha = 1).
// kNorm (one workgroup per sequence only): y = sigmoid(z) * RMSNorm(O) is
// stored in place of O (eq. (6) without its projections).
template <int kLay, int kMode, int kGate, bool kNorm>
__global__ __launch_bounds__(threads_of(kLay)) void chunk_fwd_bf16_kernel(const bf16* __restrict__ q,
                                                                  const bf16* __restrict__ k,
                                                                  const bf16* __restrict__ v,
                                                                  const bf16* __restrict__ a,
                                                                  const float* __restrict__ beta,
                                                                  const float* initial_state, bf16* __restrict__ o,
                                                                  float* final_state, int T_all, int H, int unit0,
                                                                  int unit_end, float* states, int state_every,
                                                                  int n_states, const int* cu_seqlens, int seg_len,
                                                                  int seg_count, int last_only,
                                                                  const bf16* __restrict__ z, float eps,
                                                                  int trans_units) {
  // kLay: 2 one workgroup per sequence (two 16-column state tiles a chain
  // wave), 1 two workgroups (one tile a chain wave), 4 four workgroups (one
  // tile on chain waves 0 and 1; waves 2 and 3 hold no state).
  static_assert(kLay == 1 || kLay == 2 || kLay == 4, "one, two or four workgroups per sequence");
  constexpr int kCT = kLay == 2 ? 2 : 1;          // 16-column state tiles per state-holding chain wave
  constexpr int kParts = kLay == 2 ? 1 : kLay == 1 ? 2 : 4;  // workgroups per sequence
  static_assert(!kNorm || kCT == 2, "the fused norm needs every value channel of a row in one workgroup");
  constexpr bool kEmit = kMode == kModeEmit;
  constexpr bool kVarlen = kMode >= kModePacked;
  constexpr bool kStateOnly = kMode >= kModeFragment;     // no O: neither Qh S nor A is formed
  constexpr bool kTransition = kMode == kModeTransition;  // S0 = I, v = 0
  constexpr bool kTransFrag = kMode == kModeTransFrag;    // units below trans_units: transition runs
  __shared__ Smem sm;
  __shared__ InQKA s_qka[3];
  __shared__ InV s_v[3];
  __shared__ InBeta s_beta[5];
  __shared__ InBeta s_ga[kGate == kGateScalar ? 5 : 1];  // scalar gate logits of chunk x (slot x % 5)
  // This launch serves units (b * H + h) unit0 .. unit_end - 1.  One
  // workgroup per sequence: workgroup i takes unit unit0 + i.  Several:
  // workgroups come in groups of 8 kParts, slot s taking column part s / 8 of
  // unit 8 grp + s % 8 (from unit0); dispatch deals workgroups to the XCDs
  // round robin, so all parts of a unit share an XCD and its L2 (they load
  // the same input rows).
  const int unit = unit0 + (kParts == 1 ? (int)blockIdx.x
                                        : 8 * (int)(blockIdx.x / (8 * kParts)) + (int)(blockIdx.x & 7));
  const int part = kParts == 1 ? 0 : (int)((blockIdx.x >> 3) % kParts);
  if (unit >= unit_end) return;  // whole workgroup, before any barrier
  // A transition run (S0 = I, v = 0); with kTransFrag unit u < trans_units
  // is the transition run and u + trans_units the fragment run of the same
  // segment, whose final states land at index u.
  const bool trans = kTransition || (kTransFrag && unit < trans_units);
  const int seq_unit = kTransFrag && unit >= trans_units ? unit - trans_units : unit;
  const int bb = seq_unit / H, hh = seq_unit % H;
  // The sequence's first token and length: b T_all and T_all, or, for packed
  // sequences, cu_seqlens[b] .. cu_seqlens[b + 1] clamped to [0, T_all] (so
  // any contents of cu_seqlens keep every access inside the tensors).
  int64_t tok0 = (int64_t)bb * T_all;
  int T = T_all;
  // Where the final state goes: this unit's slot, or, for the last segment
  // of a sequence cut into segments (last_only), the sequence's own slot.
  int out_unit = unit;
  bool write_final = true;
  if constexpr (kVarlen) {
    if (seg_len > 0) {
      // segment j of sequence sb: tokens j seg_len .. of the sequence's T_all
      const int sb = bb / seg_count, j = bb % seg_count;
      const int s0 = j * seg_len;
      tok0 = (int64_t)sb * T_all + s0;
      T = max(0, min(seg_len, T_all - s0));
      if (last_only) {
        write_final = j == seg_count - 1;
        out_unit = sb * H + hh;
      }
    } else {
      const int c0 = min(max(cu_seqlens[bb], 0), T_all);
      const int c1 = min(max(cu_seqlens[bb + 1], c0), T_all);
      tok0 = c0;
      T = c1 - c0;
    }
  }
  // The wave index is uniform; saying so keeps everything derived from it
  // (buffer resources, branch conditions) in scalar registers.
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int n = lane & 15, h = lane >> 4;
  const int nchunks = (T + kChunk - 1) / kChunk;
  // Iterations of the main loop (both wave kinds, an even count): chunk x
  // passes gate at x, gram at x+1, solve at x+2, prep at x+3, chain at x+4.
  const int nsteps = (nchunks + 5) & ~1;

  // ---------------------------------------------------------------- addressing
  // Token t of this sequence starts tok_bytes * t bytes into its tensor.  A
  // chunk is a buffer resource sized to its valid tokens (loads past T return
  // 0, stores there are dropped; chunks outside [0, nchunks) have size 0).
  const int64_t seq_off = (tok0 * H + hh) * kD;
  const int tok_bytes = H * kD * (int)sizeof(bf16);
  const int64_t rows_step = (int64_t)kChunk * tok_bytes;
  const int64_t beta_step = (int64_t)kChunk * H * (int64_t)sizeof(float);
  const int tail = T - (nchunks - 1) * kChunk;
  const int rows_full = (kChunk - 1) * tok_bytes + kD * (int)sizeof(bf16);
  const int rows_tail = (tail - 1) * tok_bytes + kD * (int)sizeof(bf16);
  const int beta_full = ((kChunk - 1) * H + 1) * (int)sizeof(float);
  const int beta_tail = ((tail - 1) * H + 1) * (int)sizeof(float);
  auto rows_bytes = [&](int x) { return (unsigned)x < (unsigned)nchunks ? (x == nchunks - 1 ? rows_tail : rows_full) : 0; };
  auto beta_bytes = [&](int x) { return (unsigned)x < (unsigned)nchunks ? (x == nchunks - 1 ? beta_tail : beta_full) : 0; };

  // LDS element offsets inside a channel-major block of 16 rows x 16 tokens:
  // the plain access of lane (l%16, h) (row l%16, tokens 4h ..) and the
  // transposing read (rows 4h + (l%16)/4, tokens 4(l%4) ..), group-permuted.
  const int pl_sw = n * kChunk + 4 * (h ^ (n >> 2));
  const int tr_sw = (4 * h + (n >> 2)) * kChunk + 4 * ((n & 3) ^ h);

  // ---------------------------------------------------------------- inputs
  // Loader wave w (the helper waves with two workgroups per sequence, the
  // chain waves with four, whose serial step leaves room, the gate waves
  // with one) loads tensor w % 4 (q, k, a, v) straight into LDS: in
  // iteration i, q, k or a of chunk i+2 and v of chunk i-1 (needed only by
  // prep, three iterations later), four instructions of four rows each;
  // loader 0 also beta of chunk i+2.
  constexpr bool kHelp = kLay == 1;  // waves 8..11: one helper wave per SIMD
  constexpr bool kLoadsOnChain = kLay == 4;
  constexpr bool kLoadsOnGate = kLay == 2;
  const int ldw = wave & 3;
  const char* ld_seq = reinterpret_cast<const char*>((ldw == 0 ? q : ldw == 1 ? k : ldw == 2 ? a : v) + seq_off);
  const char* beta_seq = reinterpret_cast<const char*>(beta + tok0 * H + hh);
  const int beta_off = n * H * (int)sizeof(float);
  int voff_row[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = 4 * j + h;
    const int sw = kGate == kGateChannel && ldw < 3 ? in_swz_ch(row) : in_swz(row);
    voff_row[j] = row * tok_bytes + 16 * (n ^ sw) - 1024 * j;
  }
  // full: the chunks are known to be whole, their resources need no range tests
  auto dma_rows = [&](int x, bf16* dst, auto full) {
    constexpr bool kFull = decltype(full)::value;
    const rsrc_t r = make_rsrc(ld_seq + x * rows_step, kFull ? rows_full : rows_bytes(x));
    // instruction j: rows 4j .. 4j+3, lane (n, h) row 4j + h, stored slot n
    // the instruction offset 1024 j adds to both addresses: the global one takes it back in voff
    load_4rows_to_lds(r, (uint32_t)(uintptr_t)(lds_void*)dst, voff_row[0], voff_row[1], voff_row[2], voff_row[3]);
  };
  // beta (loader 0, lanes 0..15: token l) and q, k or a (loaders 0..2) of chunk i+2
  // (the scalar gate's fp32 logits, [.., H] like beta, come with beta from
  // loader 0 and a's rows are not loaded; with no gate, neither)
  const char* ga_seq = reinterpret_cast<const char*>(reinterpret_cast<const float*>(a) + tok0 * H + hh);
  auto load_qka = [&](int i, auto full) {
    constexpr bool kFull = decltype(full)::value;
    if (ldw == 0 && lane < kChunk) {
      const int nb = kFull ? beta_full : beta_bytes(i + 2);
      load_b32_to_lds(make_rsrc(beta_seq + (i + 2) * beta_step, nb),
                      (uint32_t)(uintptr_t)(lds_void*)&s_beta[(i + 2) % 5].t[0], beta_off);
      if constexpr (kGate == kGateScalar)
        load_b32_to_lds(make_rsrc(ga_seq + (i + 2) * beta_step, nb),
                        (uint32_t)(uintptr_t)(lds_void*)&s_ga[(i + 2) % 5].t[0], beta_off);
    }
    if (ldw < (kGate == kGateChannel ? 3 : 2)) dma_rows(i + 2, &s_qka[(i + 2) % 3].t[ldw][0][0], full);
  };
  // v of chunk i-1 (loader 3), into the slot prep reads last at iteration i-1
  auto load_v = [&](int i, auto full) {
    if (!trans && ldw == 3) dma_rows(i - 1, &s_v[(i + 2) % 3].t[0][0], full);
  };
  auto load_inputs = [&](int i, auto full) {
    load_qka(i, full);
    load_v(i, full);
  };
  // Before the barrier that hands chunk operands on: every load but the
  // last four issued (at least this iteration's rows) has landed.
  auto wait_inputs = [&]() { __builtin_amdgcn_s_waitcnt(4 | (0x7 << 4) | (0xf << 8)); };

  // ---------------------------------------------------------------- gram(x): N and A, on two chain waves
  auto gram = [&](int x, auto want_n, auto want_a) {
    constexpr bool kN = decltype(want_n)::value, kA = decltype(want_a)::value;
    const bf16* tkt = &sm.r2[x & 1].kt[0][0];
    const bf16* tkh = &sm.r4[x & 3].kh[0][0];
    const bf16* tqh = &sm.r5[x % 5].qh[0][0];
    // C layouts: gkt = Kt Kh^T, lane (token c, h), register j <-> token r = 4h + j:
    // (Kh Kt^T)[c][r]; likewise gqt holds (Qh Kt^T)[c][r].
    f32x4 gkt = {0, 0, 0, 0}, gqt = {0, 0, 0, 0};
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const int lo = 32 * kb * kChunk + tr_sw, hi = lo + 16 * kChunk;
      const Frag8<bf16> fkt = cat8(lds_tr(tkt + lo), lds_tr(tkt + hi));
      if constexpr (kN) mfma_k32(gkt, fkt, cat8(lds_tr(tkh + lo), lds_tr(tkh + hi)));
      if constexpr (kA) mfma_k32(gqt, fkt, cat8(lds_tr(tqh + lo), lds_tr(tqh + hi)));
    }
    // N[c][r] = beta_c L[c][r] (c > r), A[c][r] (c >= r)
    if constexpr (kN) {
      const float bn = s_beta[x % 5].t[n];
      f32x4 nn;
#pragma unroll
      for (int j = 0; j < 4; ++j) nn[j] = n > 4 * h + j ? bn * gkt[j] : 0.0f;
      lds_put(&sm.r2[x & 1].n[0][0] + pl_sw, nn);  // N, rows c
    }
    if constexpr (kA) {
      f32x4 aq;
#pragma unroll
      for (int j = 0; j < 4; ++j) aq[j] = n >= 4 * h + j ? gqt[j] : 0.0f;
      lds_put(&sm.r5[x % 5].am[0][0] + pl_sw, aq);  // A, rows c
    }
  };

  // ---------------------------------------------------------------- solve(x): on another
  auto solve = [&](int x) {
    const bf16* tn = &sm.r2[x & 1].n[0][0];
    const Frag4<bf16> fnt = f4(lds_b64(tn + pl_sw));  // A layout of N
    const Frag4<bf16> fnc = f4(lds_tr(tn + tr_sw));   // C layout of N
    f32x4 y;  // Y0 = I - N (C layout)
    const f32x4 nc = bf16x4_to_f32(fnc.v);
#pragma unroll
    for (int j = 0; j < 4; ++j) y[j] = (4 * h + j == n ? 1.0f : 0.0f) - nc[j];
    // The A layout of X is the C layout of X^T, so the pairs (N^p, (N^p)^T) feed each other.
    f32x4 n2c = {0, 0, 0, 0}, n2t = {0, 0, 0, 0}, n4c = {0, 0, 0, 0}, n4t = {0, 0, 0, 0}, n8t = {0, 0, 0, 0};
    mfma_k16(n2c, fnt, fnc);
    mfma_k16(n2t, fnc, fnt);
    mfma_k16(y, frag4<bf16>(n2t), frag4<bf16>(y));  // (I + N^2) Y0
    mfma_k16(n4c, frag4<bf16>(n2t), frag4<bf16>(n2c));
    mfma_k16(n4t, frag4<bf16>(n2c), frag4<bf16>(n2t));
    mfma_k16(y, frag4<bf16>(n4t), frag4<bf16>(y));  // (I + N^4) Y1
    mfma_k16(n8t, frag4<bf16>(n4c), frag4<bf16>(n4t));
    mfma_k16(y, frag4<bf16>(n8t), frag4<bf16>(y));  // (I + N)^{-1} = (I + N^8) Y2
    const f32x4 m = y * s_beta[x % 5].t[n];            // M = (I + N)^{-1} Diag(beta), C layout
    lds_put(&sm.r2[x & 1].mt[0][0] + pl_sw, m);        // M^T, rows c
  };

  // ---------------------------------------------------------------- prep_w(x): W tiles
  // W = M Kh for key channels 32b .. 32b+31 (all 128 across b = 0..3: every
  // workgroup needs all of W), from fm, the A layout of M.
  auto m_frag = [&](int x) { return f4(lds_tr(&sm.r2[x & 1].mt[0][0] + tr_sw)); };
  auto prep_w = [&](int x, int b, const Frag4<bf16>& fm) {
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      const int blk = (32 * b + 16 * ct) * kChunk;  // rows 32b + 16ct ..
      const Frag4<bf16> fkh = f4(lds_b64(&sm.r4[x & 3].kh[0][0] + blk + pl_sw));  // B layout of Kh
      f32x4 wc = {0, 0, 0, 0};
      mfma_k16(wc, fm, fkh);
      lds_put(&sm.r2[x & 1].w[0][0] + blk + pl_sw, wc);  // channel-major W
    }
  };

  // ---------------------------------------------------------------- store_o(x): O to HBM
  // O of chunk x from the LDS tile to o, 16 bytes a lane, every store
  // instruction writing whole rows, by wave c of the chain waves (or of the
  // helper waves).  Two workgroups per sequence: helper wave 0 stores this
  // workgroup's 128-byte half of all 16 rows, lane (n, h) rows 2h + n/8 and
  // 8 + 2h + n/8.  Four: chain wave 3 stores the 64-byte quarter.  One:
  // chain wave c stores rows 4c .. 4c+3.
  const char* o_seq = reinterpret_cast<const char*>(o + seq_off);
  u32x4 zbuf = {0, 0, 0, 0};  // z rows of the O tile stored next (kNorm)
  auto store_o = [&](int x, auto all, int c) {
    const rsrc_t ro = make_rsrc(o_seq + x * rows_step, decltype(all)::value ? rows_full : rows_bytes(x));
    auto store_row = [&](int tok, int cb) {
      const u32x4 val = *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(&sm.r2[x & 1].ost[tok][0]) + cb);
      __builtin_amdgcn_raw_buffer_store_b128(val, ro, tok * tok_bytes + cb, 0, 0);
    };
    if constexpr (kParts == 2) {
      store_row(2 * h + (n >> 3), 128 * part + 16 * (n & 7));
      store_row(8 + 2 * h + (n >> 3), 128 * part + 16 * (n & 7));
    } else if constexpr (kParts == 4) {
      // chain wave 3 (no state): this workgroup's 64-byte quarter of all 16 rows, lane l row l / 4
      store_row(lane >> 2, 64 * part + 16 * (lane & 3));
    } else if constexpr (kNorm) {
      // y = sigmoid(z) o / sqrt(mean(o^2) + eps) over the row's 128 value
      // channels: lane (n, h) holds channels 8n .. 8n+7 of token 4c + h,
      // and the 16 lanes of a DPP row hold the whole row.
      const int tok = 4 * c + h;
      const u32x4 ov = *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(&sm.r2[x & 1].ost[tok][0]) + 16 * n);
      float f[8], ss = 0.0f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        f[2 * e] = __uint_as_float(ov[e] << 16);
        f[2 * e + 1] = __uint_as_float(ov[e] & 0xffff0000u);
        ss = fmaf(f[2 * e], f[2 * e], ss);
        ss = fmaf(f[2 * e + 1], f[2 * e + 1], ss);
      }
      ss += row_ror<8>(ss);
      ss += row_ror<4>(ss);
      ss += row_ror<2>(ss);
      ss += row_ror<1>(ss);
      const float r = __builtin_amdgcn_rsqf(fmaf(ss, 1.0f / kD, eps));
      u32x4 yv;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float y0 = f[2 * e] * r * sigmoid_fast(__uint_as_float(zbuf[e] << 16));
        const float y1 = f[2 * e + 1] * r * sigmoid_fast(__uint_as_float(zbuf[e] & 0xffff0000u));
        const bf16x2 yb = __builtin_convertvector(f32x2{y0, y1}, bf16x2);  // round to nearest even
        yv[e] = __builtin_bit_cast(uint32_t, yb);
      }
      __builtin_amdgcn_raw_buffer_store_b128(yv, ro, tok * tok_bytes + 16 * n, 0, 0);
    } else {
      store_row(4 * c + h, 16 * n);
    }
  };
  // the wave that stores O: chain wave 3 with four workgroups, helper wave 0 with two, every chain wave with one
  auto stores_o = [&](int c) { return kParts == 4 ? c == 3 : kParts == 2 ? c == 0 : true; };

  if (wave < kChainWaves) {
    // ================================================================ chain wave c: columns col0 .. col0 + 16 kCT - 1
    const int c = wave;
    // With three waves a SIMD, the serial step goes first when the chain wave
    // and another are both ready to issue (399 against 403 us on 8K tokens x
    // 96 heads; a higher priority for the helper waves instead: 412 us).
    if constexpr (kHelp) __builtin_amdgcn_s_setprio(1);
    const int col0 = kCT == 2 ? 32 * c : (kD / kParts) * part + 16 * c;
    // four workgroups per sequence: chain waves 2 and 3 hold no state
    const bool holds_state = kParts < 4 || c < 2;
    f32x4 sacc[kCT][8];  // [column tile][row tile]: lane holds S[16 rt + 4h + j][col0 + 16 ct + l%16]
    const bool has_s0 = !trans && initial_state != nullptr;  // one test, so the loads below issue back to back
#pragma unroll
    for (int ct = 0; ct < kCT; ++ct)
#pragma unroll
      for (int rt = 0; rt < 8; ++rt)
#pragma unroll
        for (int j = 0; j < 4; ++j)  // zeros, or the identity for a transition run
          sacc[ct][rt][j] = trans && 16 * rt + 4 * h + j == col0 + 16 * ct + n ? 1.0f : 0.0f;
    if (has_s0 && holds_state) {
#pragma unroll
      for (int ct = 0; ct < kCT; ++ct)
#pragma unroll
        for (int rt = 0; rt < 8; ++rt)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            sacc[ct][rt][j] = initial_state[((size_t)unit * kD + 16 * rt + 4 * h + j) * kD + col0 + 16 * ct + n];
      // waited for here: left to their first use, inside the loop, the
      // waits would be repeated every iteration
      wait_vmem_all();
    }
    // U tiles travel from prep (x) to chain (x) one iteration later in
    // registers; two sets alternate between consecutive iterations.
    f32x4 ua[kCT], ub[kCT];
#pragma unroll
    for (int ct = 0; ct < kCT; ++ct) ua[ct] = ub[ct] = f32x4{0, 0, 0, 0};
    // With the helper waves, Gamma_C of the chunk the next iteration's chain
    // step takes is read one iteration early (two sets alternate like the U
    // tiles), so that the decay of S runs under that step's first MFMAs
    // instead of waiting on an LDS read issued after the barrier (398.8 ->
    // 383.4 us on 8K tokens x 96 heads; no change in the other layouts, which
    // read it in the step).
    constexpr bool kGcAhead = kHelp;
    f32x4 gca[2], gcb[2];
    gca[0] = gca[1] = gcb[0] = gcb[1] = f32x4{0, 0, 0, 0};

    // ------------------------------------------------------------ prep(x): W and U tiles
    // W for key channels 32c .. 32c+31 (on the helper waves when there are
    // any); U = M V for this wave's state columns.
    auto prep = [&](int x, f32x4 (&u_out)[kCT]) {
      const Frag4<bf16> fm = m_frag(x);  // A layout of M
      if constexpr (!kHelp) prep_w(x, c, fm);
#pragma unroll
      for (int ct = 0; ct < kCT; ++ct) {
        f32x4 uc = {0, 0, 0, 0};  // v = 0 in a transition run: U = 0 (and none without state)
        if (!trans && holds_state) {
          const Frag4<bf16> fv =  // B layout of V, columns col0 + 16ct ..
              f4(lds_tr(&s_v[x % 3].t[0][0] + in_off(4 * h + (n >> 2), col0 + 16 * ct + 4 * (n & 3))));
          mfma_k16(uc, fm, fv);
        }
        u_out[ct] = uc;
      }
    };

    // ------------------------------------------------------------ chain(x): the serial part
    auto chain = [&](int x, const f32x4 (&u)[kCT], const f32x4 (&gcv)[2]) {
      const bf16* tw = &sm.r2[x & 1].w[0][0];
      const bf16* tq = &sm.r5[x % 5].qh[0][0];
      const bf16* tb = &sm.r5[x % 5].kb[0][0];
      Frag8<bf16> fw[4], fq[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const int lo = 32 * kb * kChunk + tr_sw, hi = lo + 16 * kChunk;
        fw[kb] = cat8(lds_tr(tw + lo), lds_tr(tw + hi));
        if constexpr (!kStateOnly) fq[kb] = cat8(lds_tr(tq + lo), lds_tr(tq + hi));
      }
      Frag4<bf16> fa;
      if constexpr (!kStateOnly) fa = f4(lds_b64(&sm.r5[x % 5].am[0][0] + pl_sw));  // A layout of A
      Frag4<bf16> fkb[8];
#pragma unroll
      for (int rt = 0; rt < 8; ++rt) fkb[rt] = f4(lds_b64(tb + 16 * rt * kChunk + pl_sw));  // A layout of Kb^T
      // Gamma_C[16 rt + 4h + l%4] for all rt; row 16 rt + 4h + j comes from lane j of the quad
      f32x4 g_lo, g_hi;
      if constexpr (kGcAhead) {
        g_lo = gcv[0];
        g_hi = gcv[1];
      } else {
        const f32x4* gp = reinterpret_cast<const f32x4*>(&sm.r5[x % 5].gamma_c[h][n & 3][0]);
        g_lo = gp[0];
        g_hi = gp[1];
      }
      f32x4 pw[kCT], pq[kCT];
#pragma unroll
      for (int ct = 0; ct < kCT; ++ct) {
        Frag8<bf16> sf[4];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) sf[kb] = frag8<bf16>(sacc[ct][2 * kb], sacc[ct][2 * kb + 1]);
        pw[ct] = f32x4{0, 0, 0, 0};
        pq[ct] = f32x4{0, 0, 0, 0};
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) mfma_k32(pw[ct], fw[kb], sf[kb]);
        if constexpr (!kStateOnly) {
#pragma unroll
          for (int kb = 0; kb < 4; ++kb) mfma_k32(pq[ct], fq[kb], sf[kb]);
        }
      }
#pragma unroll
      for (int ct = 0; ct < kCT; ++ct) {
        // Diag(Gamma_C) S, under the MFMAs above (alpha = 1 without a gate)
        if constexpr (kGate != kGateNone) {
#pragma unroll
          for (int rt = 0; rt < 8; ++rt) {
            float g = rt < 4 ? g_lo[rt] : g_hi[rt - 4];
            if (ct == 1) asm volatile("" : "+v"(g));  // a separate copy, so each broadcast folds into its multiply
            sacc[ct][rt][0] *= quad_bcast<0>(g);
            sacc[ct][rt][1] *= quad_bcast<1>(g);
            sacc[ct][rt][2] *= quad_bcast<2>(g);
            sacc[ct][rt][3] *= quad_bcast<3>(g);
          }
        }
        // Vt = U - W S (zero for padded tokens: U and W have zero rows there)
        const Frag4<bf16> fv = frag4<bf16>(u[ct] - pw[ct]);
        f32x4 da = {0, 0, 0, 0};
        if constexpr (!kStateOnly) mfma_k16(da, fa, fv);
#pragma unroll
        for (int rt = 0; rt < 8; ++rt) mfma_k16(sacc[ct][rt], fkb[rt], fv);
        if constexpr (!kStateOnly) {
          // O = Qh S + A Vt into the token-major tile; stored from there next iteration
          const bf16x4 ob = pack_bf16x4(pq[ct] + da);
          bf16* ot = &sm.r2[x & 1].ost[4 * h][col0 + 16 * ct + n];
#pragma unroll
          for (int j = 0; j < 4; ++j) ot[j * kORow] = ob[j];
        }
      }
    };
    // The state after chunk x (token 16 (x + 1)) into checkpoint (x + 1) / state_every - 1.  The
    // chunk count of the next checkpoint is carried from one to the next (no division per chunk).
    int next_emit = state_every;
    const int last_emit = state_every * n_states;
    auto emit_state = [&](int x) {
      float* dst = states + ((size_t)unit * n_states + (x + 1) / state_every - 1) * kD * kD;
#pragma unroll
      for (int ct = 0; ct < kCT; ++ct)
#pragma unroll
        for (int rt = 0; rt < 8; ++rt)
#pragma unroll
          for (int j = 0; j < 4; ++j) dst[(size_t)(16 * rt + 4 * h + j) * kD + col0 + 16 * ct + n] = sacc[ct][rt][j];
    };
    // z of chunk x for the fused norm, one iteration before its rows are stored
    const char* z_seq = reinterpret_cast<const char*>(z + seq_off);
    auto load_z = [&](int x, auto all) {
      const rsrc_t rz = make_rsrc(z_seq + x * rows_step, decltype(all)::value ? rows_full : rows_bytes(x));
      zbuf = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rz, (4 * c + h) * tok_bytes + 16 * n, 0, 0));
    };

    // With the loads here (four workgroups per sequence), beta, q, k and a
    // of chunk x land during iteration x-2.
    if constexpr (kLoadsOnChain) {
      load_inputs(-2, std::false_type());
      load_inputs(-1, std::false_type());
      wait_inputs();
    }
    block_sync();  // inputs of chunk 0 in LDS
    // With one workgroup per sequence the two Gram products and the solve
    // ride on chain waves 1, 2 and 3 (three different SIMDs), whose serial
    // step leaves room before the barrier; wave 0 takes none.  Role: 0 Gram
    // N, 1 Gram A, 2 solve, 3 none; with four workgroups per sequence the
    // two waves without state take them: 4 both Gram products, 5 the solve;
    // with two, the helper waves do, and the chain waves take none.  kRole <
    // 0 looks it up at run time.
    auto citer = [&](int i, const f32x4 (&u_use)[kCT], f32x4 (&u_make)[kCT], const f32x4 (&g_use)[2],
                     f32x4 (&g_make)[2], auto all, auto role)
                     __attribute__((always_inline)) {
      constexpr bool kAll = decltype(all)::value;
      constexpr int kRole = decltype(role)::value;
      constexpr int kRoleOf[kChainWaves] = {3, kParts == 4 ? 3 : 0, kParts == 4 ? 4 : 1, kParts == 4 ? 5 : 2};
      const int r = kHelp ? 3 : kRole >= 0 ? kRole : kRoleOf[c];
      // Gamma_C of chunk i - 3 for the next iteration's chain step (gate(i - 3)
      // wrote it; its ring slot is next written by gate(i + 2))
      if constexpr (kGcAhead && kGate != kGateNone)
        if (holds_state && (kAll || (i >= 3 && i - 3 < nchunks))) {
          const f32x4* gp = reinterpret_cast<const f32x4*>(&sm.r5[(i - 3) % 5].gamma_c[h][n & 3][0]);
          g_make[0] = gp[0];
          g_make[1] = gp[1];
        }
      // the stores go out before the input loads, which wait_inputs then leaves in flight
      if (!kHelp && !kStateOnly && stores_o(c) && (kAll || (i >= 5 && i - 5 < nchunks))) store_o(i - 5, all, c);
      if (kNorm && (kAll || (i >= 4 && i - 4 < nchunks))) load_z(i - 4, all);
      if constexpr (kLoadsOnChain) load_qka(i, all);
      if (kAll || (i >= 3 && i - 3 < nchunks)) prep(i - 3, u_make);
      if constexpr (kLoadsOnChain) load_v(i, all);
      if (holds_state && (kAll || (i >= 4 && i - 4 < nchunks))) chain(i - 4, u_use, g_use);
      if constexpr (kEmit)
        if (holds_state && i - 3 == next_emit && next_emit <= last_emit) {  // chunk i - 4 ends a checkpoint interval
          emit_state(i - 4);
          next_emit += state_every;
        }
      if ((kAll || (i >= 1 && i - 1 < nchunks)) && r == 0) gram(i - 1, std::true_type(), std::false_type());
      if ((kAll || (i >= 1 && i - 1 < nchunks)) && r == 1 && !kStateOnly)
        gram(i - 1, std::false_type(), std::true_type());
      if constexpr (kParts == 4) {
        if ((kAll || (i >= 1 && i - 1 < nchunks)) && r == 4) {
          if constexpr (kStateOnly)
            gram(i - 1, std::true_type(), std::false_type());
          else
            gram(i - 1, std::true_type(), std::true_type());
        }
      }
      if ((kAll || (i >= 2 && i - 2 < nchunks)) && (r == 2 || (kParts == 4 && r == 5))) solve(i - 2);
      if constexpr (kLoadsOnChain) {
        wait_inputs();
      }
      block_sync();
    };
    auto step2 = [&](int i, auto all, auto role) __attribute__((always_inline)) {
      citer(i, ua, ub, gca, gcb, all, role);
      citer(i + 1, ub, ua, gcb, gca, all, role);
    };
    using RunTimeRole = std::integral_constant<int, -1>;
    // Iterations 5 <= i <= nchunks - 4 have every section active and load a
    // whole chunk (i + 2 < nchunks - 1): those run without range tests (pairs
    // start at even i).  With four workgroups per sequence they run in one
    // copy of the loop per role, so that a wave's Gram or solve products share
    // a basic block with its chain step and the compiler interleaves the two
    // dependency chains; with two tiles the copies would spill registers.
    int i = 0;
    for (; i < 6 && i < nsteps; i += 2) step2(i, std::false_type(), RunTimeRole());
    auto steady = [&](auto role) __attribute__((always_inline)) {
      for (; i + 1 <= nchunks - 4; i += 2) step2(i, std::true_type(), role);
    };
    if constexpr (kCT == 2)
      steady(RunTimeRole());
    else if constexpr (kHelp)
      steady(std::integral_constant<int, 3>());
    else if (kParts == 4 && c < 2)
      steady(std::integral_constant<int, 3>());
    else if (kParts == 4 && c == 2)
      steady(std::integral_constant<int, 4>());
    else if (kParts == 4)
      steady(std::integral_constant<int, 5>());
    else if (c == 1)
      steady(std::integral_constant<int, 0>());
    else if (c == 2)
      steady(std::integral_constant<int, 1>());
    else if (c == 3)
      steady(std::integral_constant<int, 2>());
    else
      steady(std::integral_constant<int, 3>());
    for (; i < nsteps; i += 2) step2(i, std::false_type(), RunTimeRole());
    if (!kHelp && !kStateOnly && stores_o(c) && nchunks > 0 && nsteps < nchunks + 5)
      store_o(nchunks - 1, std::false_type(), c);  // not reached inside the loop

    if (write_final && holds_state) {
#pragma unroll
      for (int ct = 0; ct < kCT; ++ct)
#pragma unroll
        for (int rt = 0; rt < 8; ++rt)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const size_t idx = ((size_t)out_unit * kD + 16 * rt + 4 * h + j) * kD + col0 + 16 * ct + n;
            final_state[idx] = sacc[ct][rt][j];
          }
    }
  } else if (!kHelp || wave < 2 * kChainWaves) {
    // ================================================================ gate wave g: key channels 32g .. 32g+31
    const int g = wave - kChainWaves;
    // -------------------------------------------------------------- gate(x)
    // Lane (l%16, h) handles channels 32g + l%16 and 32g + 16 + l%16 (tiles
    // cs = 0, 1), tokens 4h .. 4h+3.
    struct GateIn {
      bf16x4 q[2], k[2], a[2];
    };
    // Per-channel gate: lane (l%16, h) holds channel 32g + 16(h%2) + l%16, tokens
    // 8(h/2) .. 8(h/2)+7 (in[0]: the first four, in[1]: the next four).
    const int gt = h >> 1, gcol = 32 * g + 16 * (h & 1);
    auto gate_read = [&](int x, GateIn& in) {
      if constexpr (kGate == kGateChannel) {
        // the slot's byte offset, uniform and opaque to loop strength reduction,
        // so each read address is one add and the tensor offsets immediates
        int slot = (x % 3) * (int)sizeof(InQKA);
        asm volatile("" : "+s"(slot));
        const char* tile = reinterpret_cast<const char*>(&s_qka[0].t[0][0][0]) + slot;
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          const char* p = tile + 2 * in_off_ch(8 * gt + 4 * r + (n >> 2), gcol + 4 * (n & 3));
          in.q[r] = lds_tr(reinterpret_cast<const bf16*>(p));
          in.k[r] = lds_tr(reinterpret_cast<const bf16*>(p + kChunk * kD * 2));
          in.a[r] = lds_tr(reinterpret_cast<const bf16*>(p + 2 * kChunk * kD * 2));
        }
        return;
      }
      // Lane (l%16, h) addresses row 4h + (l%16)/4, elements 32g + 16cs + 4(l%4) ..;
      // the transposing read returns channel 32g + 16cs + l%16, tokens 4h .. 4h+3.
      const bf16* tile = &s_qka[x % 3].t[0][0][0];
#pragma unroll
      for (int cs = 0; cs < 2; ++cs) {
        const int off = in_off(4 * h + (n >> 2), 32 * g + 16 * cs + 4 * (n & 3));
        in.q[cs] = lds_tr(tile + off);
        in.k[cs] = lds_tr(tile + kChunk * kD + off);
        if constexpr (kGate == kGateChannel) in.a[cs] = lds_tr(tile + 2 * kChunk * kD + off);
      }
    };
    // 0/1 weights of the two exchanged partial sums in this lane's exclusive prefix
    const float w_odd = (h & 1) ? 1.0f : 0.0f, w_hi = h >= 2 ? 1.0f : 0.0f;
    const float w_half = gt ? 1.0f : 0.0f;  // the per-channel gate's prefix weight
    auto gate = [&](int x, const GateIn& in, auto ragged) {
      if constexpr (kGate == kGateNone) {
        // alpha = 1: Gamma = Gamma_C = 1, so Kh = Kt = Kb = K and Qh = Q (the
        // chain skips the decay multiply); the bf16 inputs go out unchanged.
#pragma unroll
        for (int cs = 0; cs < 2; ++cs) {
          const int cm = (32 * g + 16 * cs) * kChunk + pl_sw;
          *reinterpret_cast<bf16x4*>(&sm.r4[x & 3].kh[0][0] + cm) = in.k[cs];
          if constexpr (!kStateOnly) *reinterpret_cast<bf16x4*>(&sm.r5[x % 5].qh[0][0] + cm) = in.q[cs];
          *reinterpret_cast<bf16x4*>(&sm.r2[x & 1].kt[0][0] + cm) = in.k[cs];
          *reinterpret_cast<bf16x4*>(&sm.r5[x % 5].kb[0][0] + cm) = in.k[cs];
        }
        return;
      }
      if constexpr (kGate == kGateScalar) {
        // One logit per token: sigmoid, the cumulative sums and the four
        // decay factors are per token, shared by both channel tiles.
        const f32x4 la = *reinterpret_cast<const f32x4*>(&s_ga[x % 5].t[4 * h]);
        float b[4], run = 0.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float sg = gate_log2(la[j]);
          if constexpr (decltype(ragged)::value) sg = x * kChunk + 4 * h + j < T ? sg : 0.0f;  // padded tokens: g = 0
          run = j == 0 ? sg : run + sg;
          b[j] = run;
        }
        const auto eo = __builtin_amdgcn_permlane16_swap(__float_as_uint(run), __float_as_uint(run), false, false);
        const float e = __uint_as_float(eo[0]), pair = e + __uint_as_float(eo[1]);
        const auto zz = __builtin_amdgcn_permlane32_swap(__float_as_uint(pair), __float_as_uint(pair), false, false);
        const float z_lo = __uint_as_float(zz[0]);
        const float prefix = fmaf(w_hi, z_lo, w_odd * e);
        const float gam_c = __builtin_amdgcn_exp2f(z_lo + __uint_as_float(zz[1]));
        f32x4 gam, inv;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float b2 = b[j] + prefix;
          gam[j] = __builtin_amdgcn_exp2f(b2);
          inv[j] = __builtin_amdgcn_exp2f(-b2);
        }
#pragma unroll
        for (int cs = 0; cs < 2; ++cs) {
          const f32x4 kk = bf16x4_to_f32(in.k[cs]), qq = bf16x4_to_f32(in.q[cs]);
          const f32x4 kt = kk * inv;
          const int cm = (32 * g + 16 * cs) * kChunk + pl_sw;
          lds_put(&sm.r4[x & 3].kh[0][0] + cm, kk * gam);
          if constexpr (!kStateOnly) lds_put(&sm.r5[x % 5].qh[0][0] + cm, qq * gam);
          lds_put(&sm.r2[x & 1].kt[0][0] + cm, kt);
          lds_put(&sm.r5[x % 5].kb[0][0] + cm, kt * gam_c);
          if (h == 0) sm.r5[x % 5].gamma_c[n >> 2][n & 3][2 * g + cs] = gam_c;
        }
        return;
      }
      // Sums are kept in log2 units: c = g log2(e) summed over the lane's
      // eight tokens, then the other half's total from the lanes 32 away.
      float c[8];
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const f32x4 aa = bf16x4_to_f32(in.a[r]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float sg = gate_log2(aa[j]);
          if constexpr (decltype(ragged)::value)
            sg = x * kChunk + 8 * gt + 4 * r + j < T ? sg : 0.0f;  // padded tokens: g = 0
          c[4 * r + j] = r == 0 && j == 0 ? sg : c[4 * r + j - 1] + sg;
        }
      }
      // z[0] = tokens 0..7's total, z[1] = tokens 8..15's, in every lane
      const auto zz = __builtin_amdgcn_permlane32_swap(__float_as_uint(c[7]), __float_as_uint(c[7]), false, false);
      const float z0 = __uint_as_float(zz[0]);
      const float prefix = w_half * z0;
      const float gam_c = __builtin_amdgcn_exp2f(z0 + __uint_as_float(zz[1]));
      const int row = gcol + n;  // channel-major row of this lane's channel
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const f32x4 kk = bf16x4_to_f32(in.k[r]), qq = bf16x4_to_f32(in.q[r]);
        f32x4 kh, qh, kt, kb;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float b2 = c[4 * r + j] + prefix;
          const float gam = __builtin_amdgcn_exp2f(b2);
          const float inv = __builtin_amdgcn_exp2f(-b2);
          kh[j] = kk[j] * gam;
          qh[j] = qq[j] * gam;
          kt[j] = kk[j] * inv;
          kb[j] = kt[j] * gam_c;
        }
        const int cm = row * kChunk + 4 * ((2 * gt + r) ^ (n >> 2));  // tokens 8gt + 4r .., group-permuted
        lds_put(&sm.r4[x & 3].kh[0][0] + cm, kh);
        if constexpr (!kStateOnly) lds_put(&sm.r5[x % 5].qh[0][0] + cm, qh);
        lds_put(&sm.r2[x & 1].kt[0][0] + cm, kt);
        lds_put(&sm.r5[x % 5].kb[0][0] + cm, kb);
      }
      if (gt == 0) sm.r5[x % 5].gamma_c[n >> 2][n & 3][2 * g + (h & 1)] = gam_c;
    };

    // With the loads here (one workgroup per sequence), as wherever they are
    // issued: beta, q, k and a of chunk x land during iteration x-2.
    auto step = [&](int i) {
      GateIn gin;
      if (i < nchunks) gate_read(i, gin);
      if constexpr (kLoadsOnGate) load_inputs(i, std::false_type());
      if (i < nchunks) {
        if (i < nchunks - 1 || tail == kChunk)
          gate(i, gin, std::false_type());
        else
          gate(i, gin, std::true_type());
      }
      if constexpr (kLoadsOnGate) {
        wait_inputs();
      }
      block_sync();
    };

    if constexpr (kLoadsOnGate) {
      load_inputs(-2, std::false_type());
      load_inputs(-1, std::false_type());
      wait_inputs();
    }
    block_sync();
    for (int i = 0; i < nsteps; ++i) step(i);
  } else if constexpr (kHelp) {
    // ================================================================ helper wave b (two workgroups per sequence)
    // Everything around the chain waves' serial step that is not the gate:
    // helper b loads tensor b (and beta), forms W for key channels 32b ..
    // 32b+31 and takes one more part: 0 the O stores, 1 Gram N, 2 Gram A, 3
    // the solve.  The chain waves are then left with U and the serial step.
    const int b = wave - 2 * kChainWaves;
    auto hiter = [&](int i, auto all, auto role) __attribute__((always_inline)) {
      constexpr bool kAll = decltype(all)::value;
      constexpr int kRole = decltype(role)::value;
      const int r = kRole >= 0 ? kRole : b;
      // the stores go out before the input loads, which wait_inputs then leaves in flight
      if (!kStateOnly && r == 0 && (kAll || (i >= 5 && i - 5 < nchunks))) store_o(i - 5, all, 0);
      load_qka(i, all);
      if (kAll || (i >= 3 && i - 3 < nchunks)) prep_w(i - 3, r, m_frag(i - 3));
      load_v(i, all);
      if ((kAll || (i >= 1 && i - 1 < nchunks)) && r == 1) gram(i - 1, std::true_type(), std::false_type());
      if ((kAll || (i >= 1 && i - 1 < nchunks)) && r == 2 && !kStateOnly)
        gram(i - 1, std::false_type(), std::true_type());
      if ((kAll || (i >= 2 && i - 2 < nchunks)) && r == 3) solve(i - 2);
      wait_inputs();
      block_sync();
    };
    load_inputs(-2, std::false_type());
    load_inputs(-1, std::false_type());
    wait_inputs();
    block_sync();  // inputs of chunk 0 in LDS
    using RunTimeRole = std::integral_constant<int, -1>;
    // the same iterations as the chain waves' loop, in one copy per helper
    int i = 0;
    for (; i < 6 && i < nsteps; ++i) hiter(i, std::false_type(), RunTimeRole());
    auto steady = [&](auto role) __attribute__((always_inline)) {
      for (; i + 1 <= nchunks - 4; i += 2) {
        hiter(i, std::true_type(), role);
        hiter(i + 1, std::true_type(), role);
      }
    };
    if (b == 0)
      steady(std::integral_constant<int, 0>());
    else if (b == 1)
      steady(std::integral_constant<int, 1>());
    else if (b == 2)
      steady(std::integral_constant<int, 2>());
    else
      steady(std::integral_constant<int, 3>());
    for (; i < nsteps; ++i) hiter(i, std::false_type(), RunTimeRole());
    if (!kStateOnly && b == 0 && nchunks > 0 && nsteps < nchunks + 5)
      store_o(nchunks - 1, std::false_type(), 0);  // not reached inside the loop
  }
}

}  // namespace

namespace {

typedef void (*PrefillKernel)(const bf16*, const bf16*, const bf16*, const bf16*, const float*, const float*, bf16*,
                              float*, int, int, int, int, float*, int, int, const int*, int, int, int, const bf16*,
                              float, int);

/* The kernel for a layout, mode, gate and norm; the gate variants and the
 * fused norm exist for the plain mode only (the norm with one workgroup per
 * sequence), others return NULL. */
template <int kLay>
PrefillKernel pick_kernel(int mode, int gate, bool norm) {
  constexpr int kCT = kLay;  // the layout (kLay of the kernel)
  if (norm) {
    if constexpr (kCT == 2) {
      if (mode == kModePlain && gate == kGateChannel) return chunk_fwd_bf16_kernel<2, kModePlain, kGateChannel, true>;
    }
    return nullptr;
  }
  if (gate == kGateScalar) return mode == kModePlain ? chunk_fwd_bf16_kernel<kCT, kModePlain, kGateScalar, false> : nullptr;
  if (gate == kGateNone) return mode == kModePlain ? chunk_fwd_bf16_kernel<kCT, kModePlain, kGateNone, false> : nullptr;
  switch (mode) {
    case kModePlain: return chunk_fwd_bf16_kernel<kCT, kModePlain, kGateChannel, false>;
    case kModeEmit: return chunk_fwd_bf16_kernel<kCT, kModeEmit, kGateChannel, false>;
    case kModePacked: return chunk_fwd_bf16_kernel<kCT, kModePacked, kGateChannel, false>;
    case kModeFragment: return chunk_fwd_bf16_kernel<kCT, kModeFragment, kGateChannel, false>;
    case kModeTransition: return chunk_fwd_bf16_kernel<kCT, kModeTransition, kGateChannel, false>;
    case kModeTransFrag: return chunk_fwd_bf16_kernel<kCT, kModeTransFrag, kGateChannel, false>;
  }
  return nullptr;
}

}  // namespace

hipError_t launch_chunk_fwd_bf16(const void* q, const void* k, const void* v, const void* a, const float* beta,
                                 const float* initial_state, void* o, float* final_state, int B, int T, int H,
                                 hipStream_t stream, const PrefillOptions& opt) {
  // B counts the kernel's sequences: with segments, B sequences of T tokens
  // each make B * seg_count of them
  const int seqs = opt.seg_len > 0 ? B * opt.seg_count : B;
  const int trans_units = opt.mode == kModeTransFrag ? seqs * H : 0;
  const int units = seqs * H + trans_units;
  if (units == 0) return hipSuccess;
  int cus = 0;
  const hipError_t err = device_cu_count(stream, &cus);
  if (err != hipSuccess) return err;
  bool norm = opt.z != nullptr;
  // The fused norm needs one workgroup per sequence.  Where the plain prefill
  // would run every sequence as a workgroup pair at once, the pairs' halved
  // serial step outweighs the saved pass over o (8K tokens x 96 heads: 0.651
  // ms fused against 0.577 ms in two passes; 4 x 96 sequences of 32K tokens:
  // 5.82 ms fused against 6.65 ms): there the prefill writes o into y and the
  // norm runs in place over it.
  const bool norm_in_place = norm && opt.mode == kModePlain && units <= 8 * (cus / 16);
  if (norm_in_place) norm = false;
  PrefillKernel k_quarters = pick_kernel<4>(opt.mode, opt.gate, norm);
  PrefillKernel k_pairs = pick_kernel<1>(opt.mode, opt.gate, norm);
  PrefillKernel k_single = pick_kernel<2>(opt.mode, opt.gate, norm);
  if (!k_single) return hipErrorInvalidValue;  // not instantiated: the API checks never ask for one
  // parts: workgroups per sequence (1, 2 or 4), in groups of 8 sequences when more than one
  auto launch = [&](int parts, int u0, int u1) {
    const unsigned grid =
        parts == 1 ? (unsigned)(u1 - u0) : (unsigned)(8 * parts * (((int64_t)(u1 - u0) + 7) / 8));
    hipLaunchKernelGGL(parts == 4 ? k_quarters : parts == 2 ? k_pairs : k_single, dim3(grid),
                       dim3(threads_of(parts == 4 ? 4 : parts == 2 ? 1 : 2)), 0,
                       stream, (const bf16*)q, (const bf16*)k, (const bf16*)v, (const bf16*)a, beta, initial_state,
                       (bf16*)o, final_state, T, H, u0, u1, opt.states, opt.state_every, opt.n_states, opt.cu_seqlens,
                       opt.seg_len, opt.seg_count, opt.last_only ? 1 : 0, norm ? (const bf16*)opt.z : nullptr,
                       opt.eps, trans_units);
  };
  // Sequences that fit on the device at once as four or two workgroups each
  // (one per compute unit, whole groups of 8); the fused norm needs a whole
  // row of O in one workgroup, so it always runs one workgroup per sequence.
  const int quarter_units = k_quarters ? 8 * (cus / 32) : 0;
  const int pair_units = k_pairs ? 8 * (cus / 16) : 0;
  auto fit = [&](int n) { return n <= quarter_units ? 4 : n <= pair_units ? 2 : 1; };
  if (units <= cus) {
    launch(fit(units), 0, units);  // one round
  } else {
    // Several rounds of one workgroup per sequence; a partial last round
    // that fits as pairs or quarters runs so, in a launch of its own.
    const int rest = units % cus;
    if (rest != 0 && fit(rest) > 1) {
      launch(1, 0, units - rest);
      launch(fit(rest), units - rest, units);
    } else {
      launch(1, 0, units);
    }
  }
  hipError_t e = hipGetLastError();
  if (e == hipSuccess && norm_in_place)
    e = launch_output_gate_norm(o, opt.z, o, (int64_t)units * T, opt.eps, true, stream);
  return e;
}

}  // namespace kda
