/*
 * kda_internal.h -- launchers behind the C ABI (include/kda.h).  Arguments
 * are validated by the caller (kda_api.cpp) before these run.
 */
#pragma once

#include <hip/hip_runtime.h>

namespace kda {

/* What a prefill launch reads and writes beyond plain eq. (1) over [B, T, H]. */
enum PrefillMode : int {
  kModePlain = 0,      // o and the final state
  kModeEmit = 1,       // also the state checkpoints
  kModePacked = 2,     // sequences delimited by cu_seqlens, or cut into segments
  kModeFragment = 3,   // segments: final states only (no o)
  kModeTransition = 4, // segments: final states only, from S0 = I with v = 0 (the transition matrix)
  kModeTransFrag = 5   // both in one launch: units [0, U) the transitions, [U, 2U) the fragments of
                       //      the same segments, the final states of both into one [2U, 128, 128] array
};
/* The gate (kda_gate of include/kda.h). */
enum GateMode : int {
  kGateChannel = 0,  // a [.., Dk] in the I/O type: one logit per key channel
  kGateScalar = 1,   // a [..] fp32: one logit per token and head
  kGateNone = 2      // alpha = 1; a is not read
};

struct PrefillOptions {
  float* states = nullptr;        // kModeEmit: [units, n_states, 128, 128]
  int state_every = 0;            // checkpoint interval (tokens for launch_chunk_fwd, chunks below it)
  int n_states = 0;
  const int* cu_seqlens = nullptr;  // kModePacked: [B + 1] offsets into T packed tokens
  int seg_len = 0;                // > 0: each of the B sequences of T tokens is cut into seg_count
  int seg_count = 0;              //      segments of seg_len tokens (the kernel's sequence b P + j)
  bool last_only = false;         // segments: the final state only from each sequence's last
                                  //      segment, into slot b H + h
  int mode = kModePlain;
  int gate = kGateChannel;
  const void* z = nullptr;        // non-NULL: o receives sigmoid(z) * RMSNorm(O) (eq. (6) without projections)
  float eps = 0.0f;
};

/* Compute units of the device the stream runs on (the current device for the
 * null stream), looked up once per device (kda_api.cpp). */
hipError_t device_cu_count(hipStream_t stream, int* cus);

/* units = B * H states; q, k, v, a, o are [units, 128] (a [units] fp32 for a
 * scalar gate); beta [units]; state [units, 128, 128]. */
hipError_t launch_decode(const void* q, const void* k, const void* v, const void* a, const float* beta, float* state,
                         void* o, int units, bool bf16_io, int gate, hipStream_t stream);

/* K tokens per state: q, k, v, a, o are [B, K, H, 128] with units = B * H
 * (a [B, K, H] fp32 for a scalar gate); beta [B, K, H]; n_commit [B] (NULL =
 * K) tokens committed to the state. */
hipError_t launch_decode_multi(const void* q, const void* k, const void* v, const void* a, const float* beta,
                               float* state, void* o, const int* n_commit, int units, int H, int K, bool bf16_io,
                               int gate, hipStream_t stream);

/* Chunkwise prefill over [B, T, H, 128] rows: fp32 or bf16 I/O (kda_chunk.hip).
 * opt.states: NULL, or [B, H, T / state_every, 128, 128] checkpoints, the
 * state after every state_every tokens (a multiple of 16).  opt.cu_seqlens:
 * NULL, or [B + 1] token offsets of B sequences packed along the T tokens of
 * one row (then no checkpoints). */
hipError_t launch_chunk_fwd(const void* q, const void* k, const void* v, const void* a, const float* beta,
                            const float* initial_state, void* o, float* final_state, int B, int T, int H,
                            bool bf16_io, hipStream_t stream, const PrefillOptions& opt = PrefillOptions());

/* y = sigmoid(z) * o / sqrt(mean(o^2) + eps) over rows of 128 channels (kda_epilogue.hip). */
hipError_t launch_output_gate_norm(const void* o, const void* z, void* y, int64_t rows, float eps, bool bf16_io,
                                   hipStream_t stream);

/* Entering states of P segments per (b, h) from their fragments (kda_compose.hip):
 * M, E [B * frag_segs, H, 128, 128] (sequence b's segment j at b * frag_segs + j, j < P - 1 read),
 * S_in [B * P, H, 128, 128], S0 [B, H, 128, 128] or NULL. */
hipError_t launch_compose(const float* M, const float* E, const float* S0, float* S_in, int B, int P, int H,
                          int frag_segs, hipStream_t stream);

/* The bf16 I/O prefill (kda_prefill_bf16.hip); launch_chunk_fwd dispatches to
 * it with the checkpoint interval in chunks. */
hipError_t launch_chunk_fwd_bf16(const void* q, const void* k, const void* v, const void* a, const float* beta,
                                 const float* initial_state, void* o, float* final_state, int B, int T, int H,
                                 hipStream_t stream, const PrefillOptions& opt);

/* The sequence split (kda_split.hip): each of the B sequences cut into P
 * segments of seg_len tokens; workspace holds split_workspace_bytes(B, P, H). */
size_t split_workspace_bytes(int B, int P, int H);
hipError_t launch_split(const void* q, const void* k, const void* v, const void* a, const float* beta,
                        const float* initial_state, void* o, float* final_state, int B, int T, int H, int P,
                        int seg_len, bool bf16_io, void* workspace, hipStream_t stream);
/* The file-scope scratch of kda_chunk_fwd_split_noalloc on the stream's
 * device (its device address, looked up once per device) and its size. */
hipError_t split_noalloc_scratch(hipStream_t stream, void** ptr);
extern const size_t kSplitScratchBytes;
}  // namespace kda
