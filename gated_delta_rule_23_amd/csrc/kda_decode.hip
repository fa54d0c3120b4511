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

// kGate (GateMode): a per key channel, one fp32 logit per (b, h) (a read as
// [units] fp32), or no gate (alpha = 1, a not read).
template <typename IO, int kGate>
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
      const float qi = to_f32(q[row + t]), ki = to_f32(k[row + t]);
      float al = 1.0f;
      if constexpr (kGate == kGateChannel) al = expf(kGateFloor / (1.0f + expf(-to_f32(a[row + t]))));
      if constexpr (kGate == kGateScalar)
        al = expf(kGateFloor / (1.0f + expf(-reinterpret_cast<const float*>(a)[unit])));
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

// ------------------------------------------------------------------ several tokens per state
// K tokens of each (b, h) in one pass: the state is read once, stepped through
// the K tokens in registers, and written once, after the first n_commit[b]
// tokens (or not at all for n_commit[b] = 0); every token's output is
// written.  This is the replay of an accepted draft prefix that the page
// "Kimi K3：从三条信息流到完整系统" (section "recurrent speculative decoding
// 不能复制整个状态") and the page "Kimi K3: Two point eight trillion
// parameters, open weights, and forty-seven pages of how" (section "The
// machine underneath") describe: the state after any accepted prefix follows
// from the cached per-token inputs, and tokens past the prefix are never
// committed.
//
// Layout: a 256-thread workgroup per state, wave w owning columns 32w ..
// 32w+31 of all 128 rows; lane l holds columns 32w + 4(l%8) .. +3 of rows
// l/8 + 8m, m = 0..15, so each load or store instruction moves eight whole
// 128-byte row segments.  A column's sums over the rows (x and y of the step)
// then stay inside its wave (a DPP rotate and two half swaps), so a token
// needs no barrier: the waves only share the per-channel values of the
// tokens, which the workgroup stages in LDS eight tokens at a time behind one
// barrier (thread t: channel t / 2, tokens 4 (t % 2) .. +3 of the group), and
// it loads the next group's inputs (or the next state's first group and the
// state itself) into registers right after staging.  The gate's transcendentals
// are single instructions (v_exp_f32, v_rcp_f32) with the log-decay summed in
// log2 units, and the staging's q . k partial sums stay in registers (DPP and
// lane swaps).  A state moves from its prefetch registers into the working
// ones only after its first group is staged: the copy waits for every memory
// access issued before it, the previous state's committing stores included,
// and the staging gives those time to drain.
//
// Within a group the registers hold T = Diag(1/D_j) S_j, where D_j is the
// product of the decays alpha of the group's tokens up to j (per key channel;
// each token's log-decay is at least -5, so D_j >= e^-40 over eight tokens).
// Since Diag(alpha_j) S_{j-1} = Diag(D_j) T_{j-1}, the step reads
//   x = T^T (D_j k_j),  y = T^T (D_j q_j),  T += (k_j / D_j) (beta e)^T,
// one multiply-add per state entry instead of a multiply and a multiply-add;
// S = Diag(D_j) T is formed only where it is needed: at the group's end
// before the next group, and for the committed state.
constexpr int kMultiThreads = 256;
constexpr float kInvGateLog2 = 1.0f / (kGateFloor * kLog2e);
constexpr int kMultiRows = kD / 8;  // rows per lane
constexpr int kGroupTokens = 8;     // tokens staged per LDS set
constexpr int kStagePerThread = kGroupTokens * kD / kMultiThreads;  // 4

__device__ __forceinline__ float sum_row_pairs(float x) {
  // x + (the lane 8 away within its 16-lane row), then across rows 0-1 / 2-3,
  // then across the two halves: the sum over lane bits 3, 4 and 5
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x128, 0xf, 0xf, false));  // row_ror:8
  const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(r16[0]) + __uint_as_float(r16[1]);
  const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r32[0]) + __uint_as_float(r32[1]);
}

// The sum over the 32 lanes of a wave with the same lane parity: rotations
// by 8, 4 and 2 within each 16-lane row keep the parity, then the rows are
// combined by two swaps, all in registers.
__device__ __forceinline__ float sum_same_parity(float x) {
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x128, 0xf, 0xf, false));  // row_ror:8
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x124, 0xf, 0xf, false));  // row_ror:4
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x122, 0xf, 0xf, false));  // row_ror:2
  const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(r16[0]) + __uint_as_float(r16[1]);
  const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r32[0]) + __uint_as_float(r32[1]);
}

// Four consecutive output values through a buffer resource: one 8-byte
// (bf16) or 16-byte (fp32) store.
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
constexpr int kNonTemporal = 2;  // buffer access cache policy: the nt bit (the state streams through once)
template <typename IO>
__device__ __forceinline__ void store4(rsrc_t r, int off, f32x4 x);
template <>
__device__ __forceinline__ void store4<float>(rsrc_t r, int off, f32x4 x) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, x), r, off, 0, 0);
}
template <>
__device__ __forceinline__ void store4<bf16>(rsrc_t r, int off, f32x4 x) {
  auto bits = [](float f) { return (uint32_t)__builtin_bit_cast(uint16_t, (bf16)f); };  // round to nearest even
  __builtin_amdgcn_raw_buffer_store_b64(u32x2{bits(x[0]) | (bits(x[1]) << 16), bits(x[2]) | (bits(x[3]) << 16)}, r,
                                        off, 0, 0);
}

template <typename IO, int kGate>
__global__ __launch_bounds__(kMultiThreads, 2) void decode_multi_kernel(
    const IO* __restrict__ q, const IO* __restrict__ k, const IO* __restrict__ v, const IO* __restrict__ a,
    const float* __restrict__ beta, float* __restrict__ state, IO* __restrict__ o, const int* __restrict__ n_commit,
    int units, int H, int K) {
  // per token and key channel: (D k, D q) for the sums, (k / D, D) for the update and the rescale
  __shared__ f32x2 s_kq[2][kGroupTokens][kD], s_kd[2][kGroupTokens][kD];
  __shared__ float s_v[2][kGroupTokens][kD];
  __shared__ float s_beta[2][kGroupTokens];
  __shared__ f32x4 s_qk[2][kGroupTokens];  // q . k, one partial sum per wave

  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int c0 = 32 * w + 4 * (lane & 7);  // this lane's four columns
  const int r0 = lane >> 3;                // and rows r0 + 8m
  const int sc = t >> 1, sh = t & 1;       // staging: channel sc, tokens 4 sh + i
  // a state through a buffer resource: one 32-bit lane offset, row block m at 4 KiB m
  const int st_off = (r0 * kD + c0) * (int)sizeof(float);
  auto state_rsrc = [&](int u) { return make_rsrc(state + (size_t)u * kD * kD, kD * kD * (int64_t)sizeof(float)); };
  auto load_state = [&](int u, f32x4 (&dst)[kMultiRows]) {
    const rsrc_t r = state_rsrc(u);
#pragma unroll
    for (int m = 0; m < kMultiRows; ++m)
      dst[m] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, st_off, 8 * m * kD * (int)sizeof(float),
                                                                               kNonTemporal));
  };
  // Token j of unit u = b H + h is row (b K + j) H + h of the [B, K, H, .]
  // inputs: a unit's K rows of a tensor are one buffer resource (loads past
  // its last row return 0), addressed by 32-bit offsets j H 128 + channel.
  const int tok_elems = H * kD;
  auto first_row = [&](int u) { return ((size_t)(u / H) * K) * H + (u % H); };
  auto rows_rsrc = [&](const IO* base, int u) {
    return make_rsrc(base + first_row(u) * kD, ((int64_t)(K - 1) * tok_elems + kD) * (int64_t)sizeof(IO));
  };
  struct Staged {
    uint32_t q[kStagePerThread], k[kStagePerThread], a[kStagePerThread], v[kStagePerThread];
    float b[kStagePerThread];
  };
  auto load_group = [&](int u, int g, Staged& in) {
    const rsrc_t rq = rows_rsrc(q, u), rk = rows_rsrc(k, u), ra = rows_rsrc(a, u), rv = rows_rsrc(v, u);
    const int64_t scalar_bytes = ((int64_t)(K - 1) * H + 1) * (int64_t)sizeof(float);
    const rsrc_t rb = make_rsrc(beta + first_row(u), scalar_bytes);
#pragma unroll
    for (int i = 0; i < kStagePerThread; ++i) {
      const int j = kGroupTokens * g + kStagePerThread * sh + i;
      const int off = (j * tok_elems + sc) * (int)sizeof(IO);
      in.q[i] = Raw<IO>::load(rq, off);
      in.k[i] = Raw<IO>::load(rk, off);
      if constexpr (kGate == kGateChannel) in.a[i] = Raw<IO>::load(ra, off);
      if constexpr (kGate == kGateScalar)  // [B, K, H] fp32, like beta
        in.a[i] = __builtin_amdgcn_raw_buffer_load_b32(
            make_rsrc(reinterpret_cast<const float*>(a) + first_row(u), scalar_bytes), j * H * (int)sizeof(float), 0, 0);
      if constexpr (kGate == kGateNone) in.a[i] = 0;
      in.v[i] = Raw<IO>::load(rv, off);
      in.b[i] = load_f32(rb, j * H * (int)sizeof(float));
    }
  };
  auto commit_count = [&](int u) {
    const int c = n_commit ? n_commit[u / H] : K;
    return c < 0 ? 0 : (c > K ? K : c);
  };

  const int ngroups = (K + kGroupTokens - 1) / kGroupTokens;
  int unit = blockIdx.x;
  f32x4 s[kMultiRows], sn[kMultiRows];
  Staged in = {};
  int nc = 0, nc_next = 0;
  if (unit < units) {
    load_state(unit, sn);
    load_group(unit, 0, in);
    nc = commit_count(unit);
  }
  int set = 0;
  while (unit < units) {
    const int next = unit + (int)gridDim.x;
    const rsrc_t o_rsrc = rows_rsrc(o, unit);
    for (int g = 0; g < ngroups; ++g, set ^= 1) {
      // Stage the group's per-channel values.  Tokens past K load as zeros
      // and are never read back.  log2 D is the running sum of
      // g log2(e) = -5 log2(e) sigmoid(a) over the group's tokens; the lane
      // with the later four tokens adds its partner's (lane - 1) total.
      float lg[kStagePerThread], run = 0.0f;
#pragma unroll
      for (int i = 0; i < kStagePerThread; ++i) {
        if constexpr (kGate != kGateNone) {
          const float ai = kGate == kGateChannel ? Raw<IO>::f32(in.a[i]) : __uint_as_float(in.a[i]);
          // g log2(e) = -5 log2(e) sigmoid(a) = 1 / ((1 + 2^(-a log2 e)) / (-5 log2 e))
          run += __builtin_amdgcn_rcpf(fmaf(__builtin_amdgcn_exp2f(-ai * kLog2e), kInvGateLog2, kInvGateLog2));
        }
        lg[i] = run;
      }
      const float before = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(run), 0xB1, 0xf, 0xf, false));
      const float carry = sh ? before : 0.0f;  // quad_perm [1, 0, 3, 2]: the partner lane's total
#pragma unroll
      for (int i = 0; i < kStagePerThread; ++i) {
        const int jj = kStagePerThread * sh + i;
        const float qi = Raw<IO>::f32(in.q[i]), ki = Raw<IO>::f32(in.k[i]);
        const float l2d = lg[i] + carry;
        const float dd = __builtin_amdgcn_exp2f(l2d), di = __builtin_amdgcn_exp2f(-l2d);
        s_kq[set][jj][sc] = f32x2{dd * ki, dd * qi};
        s_kd[set][jj][sc] = f32x2{ki * di, dd};
        s_v[set][jj][sc] = Raw<IO>::f32(in.v[i]);
        if (sc == 0) s_beta[set][jj] = in.b[i];
        const float part = sum_same_parity(qi * ki);
        if (lane < 2) s_qk[set][jj][w] = part;
      }
      // The state enters its registers after its first group is staged, so
      // the previous state's committing stores, which the copy waits for
      // with everything issued before it, have the staging's time to drain.
      if (g == 0) {
#pragma unroll
        for (int m = 0; m < kMultiRows; ++m) s[m] = sn[m];
      }
      // inputs of the next group, or of the next state's first group with the state itself
      if (g + 1 < ngroups) {
        load_group(unit, g + 1, in);
      } else if (next < units) {
        load_group(next, 0, in);
        load_state(next, sn);
        nc_next = commit_count(next);
      }
      __syncthreads();

      const int jn = K - kGroupTokens * g < kGroupTokens ? K - kGroupTokens * g : kGroupTokens;
#pragma unroll 1
      for (int jj = 0; jj < jn; ++jj) {
        const int j = kGroupTokens * g + jj;
        // x = T^T (D k), y = T^T (D q) over this lane's rows, then over the wave's rows
        f32x4 x = {0, 0, 0, 0}, y = {0, 0, 0, 0};
#pragma unroll
        for (int m = 0; m < kMultiRows; ++m) {
          const f32x2 kq = s_kq[set][jj][r0 + 8 * m];
          x += kq[0] * s[m];
          y += kq[1] * s[m];
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          x[c] = sum_row_pairs(x[c]);
          y[c] = sum_row_pairs(y[c]);
        }
        const f32x4 qk4 = s_qk[set][jj];
        const float bt = s_beta[set][jj], qk = (qk4[0] + qk4[1]) + (qk4[2] + qk4[3]);
        const f32x4 e = *reinterpret_cast<const f32x4*>(&s_v[set][jj][c0]) - x;
        const f32x4 be = bt * e;
        if (r0 == 0) store4<IO>(o_rsrc, (j * tok_elems + c0) * (int)sizeof(IO), y + (bt * qk) * e);
        // T += (k / D) (beta e)^T
#pragma unroll
        for (int m = 0; m < kMultiRows; ++m) s[m] += s_kd[set][jj][r0 + 8 * m][0] * be;
        if (j + 1 == nc) {  // commit S = Diag(D) T
          // The whole offset goes in the lane offset and soffset stays 0: a
          // 16-byte buffer store with a register soffset was seen to store
          // its last dword after the next instruction had overwritten it
          // (the compiler inserts no wait for that form), and with soffset 0
          // the compiler keeps the store's data registers intact.
          const rsrc_t r = state_rsrc(unit);
#pragma unroll
          for (int m = 0; m < kMultiRows; ++m)
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, s_kd[set][jj][r0 + 8 * m][1] * s[m]), r,
                                                   st_off + 8 * m * kD * (int)sizeof(float), 0, kNonTemporal);
        }
      }
      if (g + 1 < ngroups) {  // S = Diag(D) T enters the next group
#pragma unroll
        for (int m = 0; m < kMultiRows; ++m) s[m] *= s_kd[set][kGroupTokens - 1][r0 + 8 * m][1];
      }
    }
    nc = nc_next;
    unit = next;
  }
}

namespace {

template <int kGate>
void launch_multi_gate(unsigned grid, hipStream_t stream, const void* q, const void* k, const void* v, const void* a,
                       const float* beta, float* state, void* o, const int* n_commit, int units, int H, int K,
                       bool bf16_io) {
  if (bf16_io)
    hipLaunchKernelGGL((decode_multi_kernel<bf16, kGate>), dim3(grid), dim3(kMultiThreads), 0, stream, (const bf16*)q,
                       (const bf16*)k, (const bf16*)v, (const bf16*)a, beta, state, (bf16*)o, n_commit, units, H, K);
  else
    hipLaunchKernelGGL((decode_multi_kernel<float, kGate>), dim3(grid), dim3(kMultiThreads), 0, stream,
                       (const float*)q, (const float*)k, (const float*)v, (const float*)a, beta, state, (float*)o,
                       n_commit, units, H, K);
}

template <int kGate>
void launch_decode_gate(unsigned grid, hipStream_t stream, const void* q, const void* k, const void* v, const void* a,
                        const float* beta, float* state, void* o, int units, bool bf16_io) {
  if (bf16_io)
    hipLaunchKernelGGL((decode_kernel<bf16, kGate>), dim3(grid), dim3(kDecodeThreads), 0, stream, (const bf16*)q,
                       (const bf16*)k, (const bf16*)v, (const bf16*)a, beta, state, (bf16*)o, units);
  else
    hipLaunchKernelGGL((decode_kernel<float, kGate>), dim3(grid), dim3(kDecodeThreads), 0, stream, (const float*)q,
                       (const float*)k, (const float*)v, (const float*)a, beta, state, (float*)o, units);
}

}  // namespace

hipError_t launch_decode_multi(const void* q, const void* k, const void* v, const void* a, const float* beta,
                               float* state, void* o, const int* n_commit, int units, int H, int K, bool bf16_io,
                               int gate, hipStream_t stream) {
  if (units == 0 || K == 0) return hipSuccess;
  // One token, every state committed: the [B, 1, H, .] rows are the single
  // step's [B, H, .] rows, and its kernel streams the state faster.
  if (K == 1 && !n_commit) return launch_decode(q, k, v, a, beta, state, o, units, bf16_io, gate, stream);
  // More than one staging group, every token committed: that is a prefill of
  // K tokens from the state into the state (also one read and one write of
  // it, the initial state read before the final one is written), whose
  // chunkwise MFMA form costs nearly the same for any K up to 32 while this
  // kernel's token loop grows with K (256 x 96 states: K = 9 0.79 against
  // 0.83 ms, K = 16 0.82 against 1.16 ms, K = 32 0.94 against 2.08 ms).
  if (K > kGroupTokens && !n_commit) {
    PrefillOptions opt;
    opt.gate = gate;
    return launch_chunk_fwd(q, k, v, a, beta, state, o, state, units / H, K, H, bf16_io, stream, opt);
  }
  int cus = 0;
  const hipError_t err = device_cu_count(stream, &cus);
  if (err != hipSuccess) return err;
  // two resident workgroups per compute unit (a wave holds 128 state registers
  // and as many for the next state's)
  const int64_t slots = 2 * (int64_t)(cus > 0 ? cus : 1);
  const unsigned grid = (unsigned)(units < slots ? units : slots);
  if (gate == kGateScalar)
    launch_multi_gate<kGateScalar>(grid, stream, q, k, v, a, beta, state, o, n_commit, units, H, K, bf16_io);
  else if (gate == kGateNone)
    launch_multi_gate<kGateNone>(grid, stream, q, k, v, a, beta, state, o, n_commit, units, H, K, bf16_io);
  else
    launch_multi_gate<kGateChannel>(grid, stream, q, k, v, a, beta, state, o, n_commit, units, H, K, bf16_io);
  return hipGetLastError();
}

hipError_t launch_decode(const void* q, const void* k, const void* v, const void* a, const float* beta, float* state,
                         void* o, int units, bool bf16_io, int gate, hipStream_t stream) {
  if (units == 0) return hipSuccess;
  int cus = 0;
  const hipError_t err = device_cu_count(stream, &cus);
  if (err != hipSuccess) return err;
  const int64_t slots = (int64_t)kWorkgroupsPerCU * (cus > 0 ? cus : 1);
  const unsigned grid = (unsigned)(units < slots ? units : slots);
  if (gate == kGateScalar)
    launch_decode_gate<kGateScalar>(grid, stream, q, k, v, a, beta, state, o, units, bf16_io);
  else if (gate == kGateNone)
    launch_decode_gate<kGateNone>(grid, stream, q, k, v, a, beta, state, o, units, bf16_io);
  else
    launch_decode_gate<kGateChannel>(grid, stream, q, k, v, a, beta, state, o, units, bf16_io);
  return hipGetLastError();
}

}  // namespace kda
