/*
 * kda_internal.h -- launchers behind the C ABI (include/kda.h).  Arguments
 * are validated by the caller (kda_api.cpp) before these run.
 */
#pragma once

#include <hip/hip_runtime.h>

namespace kda {

/* Compute units of the device the stream runs on (the current device for the
 * null stream), looked up once per device (kda_api.cpp). */
hipError_t device_cu_count(hipStream_t stream, int* cus);

/* units = B * H states; q, k, v, a, o are [units, 128]; beta [units];
 * state [units, 128, 128]. */
hipError_t launch_decode(const void* q, const void* k, const void* v, const void* a, const float* beta, float* state,
                         void* o, int units, bool bf16_io, hipStream_t stream);

/* K tokens per state: q, k, v, a, o are [B, K, H, 128] with units = B * H;
 * beta [B, K, H]; n_commit [B] (NULL = K) tokens committed to the state. */
hipError_t launch_decode_multi(const void* q, const void* k, const void* v, const void* a, const float* beta,
                               float* state, void* o, const int* n_commit, int units, int H, int K, bool bf16_io,
                               hipStream_t stream);

/* Chunkwise prefill over [B, T, H, 128] rows: fp32 or bf16 I/O (kda_chunk.hip).
 * states: NULL, or [B, H, T / state_every, 128, 128] checkpoints, the state
 * after every state_every tokens (a multiple of 16).  cu_seqlens: NULL, or
 * [B + 1] token offsets of B sequences packed along the T tokens of one row
 * (then no checkpoints). */
hipError_t launch_chunk_fwd(const void* q, const void* k, const void* v, const void* a, const float* beta,
                            const float* initial_state, void* o, float* final_state, int B, int T, int H,
                            bool bf16_io, hipStream_t stream, float* states = nullptr, int state_every = 0,
                            const int* cu_seqlens = nullptr);

/* y = sigmoid(z) * o / sqrt(mean(o^2) + eps) over rows of 128 channels (kda_epilogue.hip). */
hipError_t launch_output_gate_norm(const void* o, const void* z, void* y, int64_t rows, float eps, bool bf16_io,
                                   hipStream_t stream);

/* Entering states of P segments per (b, h) from their fragments (kda_compose.hip):
 * M, E, S_in [B * P, H, 128, 128] (sequence b's segment j at b * P + j), S0 [B, H, 128, 128] or NULL. */
hipError_t launch_compose(const float* M, const float* E, const float* S0, float* S_in, int B, int P, int H,
                          hipStream_t stream);

/* The bf16 I/O prefill (kda_prefill_bf16.hip); launch_chunk_fwd dispatches to it. */
hipError_t launch_chunk_fwd_bf16(const void* q, const void* k, const void* v, const void* a, const float* beta,
                                 const float* initial_state, void* o, float* final_state, int B, int T, int H,
                                 hipStream_t stream, float* states, int state_every, int n_states,
                                 const int* cu_seqlens);

}  // namespace kda
