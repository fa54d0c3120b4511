/*
 * kda.h -- C ABI of libkda: the Kimi Delta Attention (KDA) forward pass on
 * AMD Instinct MI355X (gfx950).
 *
 * The operation (page "Kimi K3：从三条信息流到完整系统", wineandchord.com):
 *   per (batch b, head h), for t = 1..T, with key channels i and value channels j,
 *     g_t     = -5 * sigmoid(a_t)                       eq. (5), section "下界 log-decay 是一个 kernel 设计"
 *     alpha_t = exp(g_t)                                 (per key channel, in (e^-5, 1])
 *     S_t     = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
 *     o_t     = S_t^T q_t                                eq. (1), section "KDA 是带逐通道遗忘的 delta rule"
 *   The output reads the state after token t's own write, and the decay acts
 *   before the delta correction, as the reference step in that section fixes.
 *   S has Dk rows (key channels) and Dv columns (value channels).
 *   The learned scale e^A of eq. (5) is folded into a by the caller.
 *   The family's other rules (the delta rule, alpha = 1, and the
 *   scalar-gated delta rule) have entry points of their own (kda_gate).
 *
 * Conventions for every entry point:
 *   - Every pointer is a device pointer (hipMalloc'd or equivalent), row-major,
 *     contiguous and 16-byte aligned.  The library allocates nothing and keeps
 *     no pointer after returning.  Between calls it keeps only a per-device
 *     cache of the compute-unit count and each thread's last error text, so
 *     it is re-entrant and thread-safe.
 *   - Work is enqueued on `hip_stream` (NULL = the default stream) and runs
 *     asynchronously; the caller keeps every buffer alive until the stream has
 *     completed.  No entry point synchronises the host.
 *   - Arguments are checked before anything is launched.  A non-OK status
 *     means nothing was enqueued (KDA_ERR_INVALID_ARGUMENT, KDA_ERR_UNSUPPORTED)
 *     or the launch itself failed (KDA_ERR_HIP); kda_last_error() then holds a
 *     description for the calling thread.  Faults during execution surface at
 *     the caller's next synchronisation.  NaN and out-of-range values are not
 *     checked; beta is expected in [0, 1].
 *   - Only Dk = Dv = 128 is implemented (K3's head dimension); other positive
 *     sizes return KDA_ERR_UNSUPPORTED.
 *   - B * H is at most 2^31 - 2^20; larger counts return
 *     KDA_ERR_INVALID_ARGUMENT.
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KDA_OK = 0,
  KDA_ERR_INVALID_ARGUMENT = 1, /* NULL or misaligned pointer, negative size, overflow, bad enum */
  KDA_ERR_UNSUPPORTED = 2,      /* a valid request this library does not implement (Dk, Dv != 128; H > 65536 in prefill) */
  KDA_ERR_HIP = 3               /* the HIP runtime reported an error at launch */
} kda_status;

typedef enum {
  KDA_F32 = 0,  /* q, k, v, a, o are fp32 */
  KDA_BF16 = 1  /* q, k, v, a, o are bf16; beta and states stay fp32 */
} kda_dtype;

/*
 * The gate of the *_gated entry points: the members of the family of update
 * rules the notebook "Kimi K3: Two point eight trillion parameters, open
 * weights, and forty-seven pages of how" compares (section "The sequence
 * axis"), all through the bounded gate g = -5 sigmoid(a) of eq. (5):
 *   KDA_GATE_CHANNEL  a has one logit per key channel ([.., Dk] in the I/O
 *                     dtype, 16-byte aligned): KDA, as in the plain entries;
 *   KDA_GATE_SCALAR   a has one fp32 logit per token and head ([..] shaped
 *                     like beta, 4-byte aligned): the scalar-gated delta rule;
 *   KDA_GATE_NONE     alpha = 1, a is not read (may be NULL): the delta rule.
 */
typedef enum {
  KDA_GATE_CHANNEL = 0,
  KDA_GATE_SCALAR = 1,
  KDA_GATE_NONE = 2
} kda_gate;

/*
 * Chunkwise prefill: T tokens of B independent sequences, H heads each.
 * Computed in chunks of 16 tokens (the pages' 16-token tile, whose cumulative
 * log-decay stays in [-80, 0]: section "下界 log-decay 是一个 kernel 设计"),
 * inside each chunk by eq. (3)-(4) of section "从投影到 Chunkwise 的完整接口"
 * and carrying an fp32 state between chunks.
 *
 *   q, k, a        [B, T, H, Dk]  dtype                      (read)
 *   v              [B, T, H, Dv]  dtype                      (read)
 *   beta           [B, T, H]      fp32                       (read)
 *   initial_state  [B, H, Dk, Dv] fp32, or NULL for zeros    (read)
 *   o              [B, T, H, Dv]  dtype                      (written)
 *   final_state    [B, H, Dk, Dv] fp32                       (written; may be the
 *                  same buffer as initial_state, any other overlap is undefined)
 *
 * H is at most 65536 (one chunk of one tensor must span less than 2^31
 * bytes); larger H fails with KDA_ERR_UNSUPPORTED.
 * T need not be a multiple of 16: the last chunk is partial, with the same
 * result as padding it with tokens of beta = 0, g = 0 and q = 0.  T = 0 copies
 * initial_state (or zeros) into final_state; q, k, v, a, beta and o may then
 * be NULL.  Feeding final_state back as initial_state for the next T' tokens
 * gives the result of one call over T + T' tokens (up to rounding).
 */
kda_status kda_chunk_fwd(const void* q, const void* k, const void* v, const void* a, const float* beta,
                         const float* initial_state, void* o, float* final_state, int B, int T, int H, int Dk,
                         int Dv, kda_dtype dtype, void* hip_stream);

/*
 * kda_chunk_fwd with a choice of gate (kda_gate above): the gate logits a are
 * [B, T, H, Dk] in dtype (KDA_GATE_CHANNEL), [B, T, H] fp32 (KDA_GATE_SCALAR),
 * or not read (KDA_GATE_NONE).  Every other argument and result is as in
 * kda_chunk_fwd, which is this call with KDA_GATE_CHANNEL.  A bad gate
 * value returns KDA_ERR_INVALID_ARGUMENT.
 */
kda_status kda_chunk_fwd_gated(const void* q, const void* k, const void* v, const void* a, const float* beta,
                               const float* initial_state, void* o, float* final_state, int B, int T, int H, int Dk,
                               int Dv, kda_dtype dtype, kda_gate gate, void* hip_stream);

/*
 * kda_chunk_fwd followed by the output side of eq. (6) of the page "Kimi
 * K3：从三条信息流到完整系统" without its projections: instead of o the call
 * writes
 *
 *   y = sigmoid(z) * o / sqrt(mean(o^2) + eps)     per (token, head) row of Dv channels,
 *
 * the head-wise RMSNorm (no learned scale) of the recurrent output, gated by
 * z = W_g x from the caller.
 *
 *   z   [B, T, H, Dv]  dtype  (read)
 *   y   [B, T, H, Dv]  dtype  (written)
 *
 * With bf16 I/O and more (sequence, head) pairs than run as workgroup pairs
 * at once, the norm is fused into the prefill's output store and o never
 * reaches memory; otherwise (and with fp32 I/O) o is written into y and the
 * norm runs in place over it, which is faster there.  Either way the norm is
 * taken of o rounded to dtype.  Every other argument is as in kda_chunk_fwd;
 * eps must be finite and >= 0.
 */
kda_status kda_chunk_fwd_norm(const void* q, const void* k, const void* v, const void* a, const float* beta,
                              const float* initial_state, const void* z, float eps, void* y, float* final_state, int B,
                              int T, int H, int Dk, int Dv, kda_dtype dtype, void* hip_stream);

/*
 * kda_chunk_fwd that also writes state checkpoints: the state after tokens
 * E, 2E, ..., n E of every sequence, n = floor(T / E), for E = state_every, a
 * positive multiple of 16 (the chunk).  These are the sparse KDA state
 * checkpoints of the page "Kimi K3：从三条信息流到完整系统", section
 * "hybrid prefix cache" (saved at hash-block or turn boundaries so that a
 * cached prefix can resume from them); the notebook "Kimi K3: Two point eight
 * trillion parameters, open weights, and forty-seven pages of how" describes
 * the same in its section "The machine underneath".
 *
 *   states   [B, H, n, Dk, Dv] fp32 (written; may be NULL when n = 0)
 *
 * Every other argument, and o and final_state, are as in kda_chunk_fwd, with
 * the same results.  Resuming from checkpoint i (as initial_state) over
 * tokens E (i + 1) .. T - 1 gives the rest of the outputs and the same final
 * state (up to rounding).  state_every <= 0 or not a multiple of 16 returns
 * KDA_ERR_INVALID_ARGUMENT.
 */
kda_status kda_chunk_fwd_states(const void* q, const void* k, const void* v, const void* a, const float* beta,
                                const float* initial_state, void* o, float* final_state, float* states,
                                int state_every, int B, int T, int H, int Dk, int Dv, kda_dtype dtype,
                                void* hip_stream);

/*
 * kda_chunk_fwd over N sequences of different lengths packed one after
 * another along the token axis (the usual layout of a serving batch):
 * sequence n is tokens cu_seqlens[n] .. cu_seqlens[n + 1] - 1 of the packed
 * rows, and each (sequence, head) is an independent KDA recurrence exactly
 * as in kda_chunk_fwd.
 *
 *   q, k, a        [T, H, Dk]     dtype   (read; T = cu_seqlens[N], the packed length)
 *   v              [T, H, Dv]     dtype   (read)
 *   beta           [T, H]         fp32    (read)
 *   cu_seqlens     [N + 1]        int32 on the device, 4-byte aligned: 0 = cu_seqlens[0]
 *                                 <= cu_seqlens[1] <= ... <= cu_seqlens[N] = T
 *   initial_state  [N, H, Dk, Dv] fp32, or NULL for zeros   (read)
 *   o              [T, H, Dv]     dtype   (written)
 *   final_state    [N, H, Dk, Dv] fp32    (written; may be initial_state)
 *
 * The library cannot read cu_seqlens on the host; offsets outside [0, T] are
 * clamped to it and a decreasing pair gives an empty sequence, so no access
 * leaves the buffers whatever its contents (sequences that overlap leave the
 * shared rows of o undefined).  A sequence of length 0 copies its initial
 * state.  The same limits as kda_chunk_fwd apply (H <= 65536).
 */
kda_status kda_chunk_fwd_varlen(const void* q, const void* k, const void* v, const void* a, const float* beta,
                                const int* cu_seqlens, const float* initial_state, void* o, float* final_state, int N,
                                int T, int H, int Dk, int Dv, kda_dtype dtype, void* hip_stream);

/*
 * kda_chunk_fwd with each sequence cut into segments that run side by side:
 * the page "Kimi K3：从三条信息流到完整系统", section "FlashKDA 与 KCP",
 * eq. (17), on one device.  A segment acts on the state it enters with as
 * S -> M S + E (eq. (1) is affine in S): the library runs every segment but
 * the last of each sequence from S = I with v = 0 (its transition M) and
 * from zero (its fragment E), composes the entering states
 * S_in[j + 1] = M_j S_in[j] + E_j from S_in[0] = initial_state, and runs all
 * segments again from those, writing o and the final states.  Three passes
 * of the state path for `segments` times the (sequence, head) parallelism:
 * worth it when B * H leaves most compute units idle.
 *
 * Segments are whole 16-token chunks: L = ceil(ceil(T / segments) / 16) * 16
 * tokens each, ceil(T / L) of them (the last takes the rest).  Arguments and
 * results are those of kda_chunk_fwd (up to rounding: the composition adds
 * fp32 products of the segments' states), plus
 *
 *   segments         >= 1; 1 (or T <= 16) runs kda_chunk_fwd itself
 *   workspace        device memory of at least kda_chunk_fwd_split_workspace
 *                    (B, T, H, segments) bytes, 16-byte aligned, owned by the
 *                    caller; its contents on entry do not matter and it must
 *                    not overlap any other argument; may be NULL when that
 *                    size is 0
 *   workspace_bytes  its size; a smaller one returns KDA_ERR_INVALID_ARGUMENT
 *
 * initial_state may be final_state (it is read before final_state is
 * written).  Only the per-channel gate (kda_chunk_fwd's a) is taken.
 */
size_t kda_chunk_fwd_split_workspace(int B, int T, int H, int segments);
kda_status kda_chunk_fwd_split(const void* q, const void* k, const void* v, const void* a, const float* beta,
                               const float* initial_state, void* o, float* final_state, int segments,
                               void* workspace, size_t workspace_bytes, int B, int T, int H, int Dk, int Dv,
                               kda_dtype dtype, void* hip_stream);

/*
 * kda_chunk_fwd_split for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same computation and results, with the workspace taken
 * from a scratch array the library holds on every GPU it runs on (64 MiB
 * each, kept until the process ends).  Nothing is allocated and nothing
 * needs to start at zero.  A split needing more than 64 MiB
 * (kda_chunk_fwd_split_workspace above: 192 KiB per (sequence, head,
 * segment), e.g. 8 heads x 16 segments = 23 MiB) returns
 * KDA_ERR_INVALID_ARGUMENT.  Every call on one GPU shares that GPU's array:
 * calls that overlap in time on one GPU (other streams, other host threads)
 * race on it and must be ordered by the caller.
 */
kda_status kda_chunk_fwd_split_noalloc(const void* q, const void* k, const void* v, const void* a, const float* beta,
                                       const float* initial_state, void* o, float* final_state, int segments, int B,
                                       int T, int H, int Dk, int Dv, kda_dtype dtype, void* hip_stream);

/*
 * One recurrent decode step: eq. (1) applied to a single token of each of B
 * sequences and H heads, updating the state in place (read once, written
 * once).
 *
 *   q, k, a   [B, H, Dk]      dtype   (read)
 *   v         [B, H, Dv]      dtype   (read)
 *   beta      [B, H]          fp32    (read)
 *   state     [B, H, Dk, Dv]  fp32    (read, then overwritten with S_t)
 *   o         [B, H, Dv]      dtype   (written)
 */
kda_status kda_decode_step(const void* q, const void* k, const void* v, const void* a, const float* beta,
                           float* state, void* o, int B, int H, int Dk, int Dv, kda_dtype dtype,
                           void* hip_stream);

/* kda_decode_step with a choice of gate: a is [B, H, Dk] in dtype
 * (KDA_GATE_CHANNEL), [B, H] fp32 (KDA_GATE_SCALAR) or not read
 * (KDA_GATE_NONE). */
kda_status kda_decode_step_gated(const void* q, const void* k, const void* v, const void* a, const float* beta,
                                 float* state, void* o, int B, int H, int Dk, int Dv, kda_dtype dtype, kda_gate gate,
                                 void* hip_stream);

/*
 * K tokens of each sequence in one pass, for speculative decoding: the state
 * is read once, stepped through the tokens in order (each step as in
 * kda_decode_step), and written once, holding the state after the first
 * n_commit[b] tokens of batch row b; the tokens after them are never
 * committed.  Every token's output is written, read from the running state
 * after that token (so outputs past n_commit[b] are those of the uncommitted
 * continuation).  The page "Kimi K3：从三条信息流到完整系统" (section
 * "recurrent speculative decoding 不能复制整个状态") and the page "Kimi K3:
 * Two point eight trillion parameters, open weights, and forty-seven pages of
 * how" (section "The machine underneath") describe this replay: cache the
 * drafted tokens' inputs, verify, then replay only the accepted prefix from
 * the committed state, with no per-position state snapshots.  Verifying a
 * draft takes n_commit = 0 (outputs only, state untouched); committing m
 * accepted tokens takes them again with n_commit = m.
 *
 *   q, k, a   [B, K, H, Dk]   dtype   (read)
 *   v         [B, K, H, Dv]   dtype   (read)
 *   beta      [B, K, H]       fp32    (read)
 *   state     [B, H, Dk, Dv]  fp32    (read; overwritten with the state after
 *                                      n_commit[b] tokens, left untouched where
 *                                      n_commit[b] = 0)
 *   o         [B, K, H, Dv]   dtype   (written, all K tokens)
 *   n_commit  [B] int32 on the device, 4-byte aligned, or NULL for K; values
 *             outside [0, K] are clamped to it (the library does not read
 *             device memory on the host, so it cannot reject them)
 *
 * K = 0 (or B * H = 0) enqueues nothing.  With K = 1 and n_commit NULL the
 * result is that of kda_decode_step; with K > 8 and n_commit NULL, that of
 * kda_chunk_fwd over the K tokens with state as both initial and final state
 * (the chunkwise form, cheaper there than the token loop).  K * H is at
 * most 4194303 (a sequence's K rows of one tensor must span less than 2^31
 * bytes); larger products fail with KDA_ERR_UNSUPPORTED.
 */
kda_status kda_decode_multi(const void* q, const void* k, const void* v, const void* a, const float* beta,
                            float* state, void* o, const int* n_commit, int B, int K, int H, int Dk, int Dv,
                            kda_dtype dtype, void* hip_stream);

/* kda_decode_multi with a choice of gate: a is [B, K, H, Dk] in dtype
 * (KDA_GATE_CHANNEL), [B, K, H] fp32 (KDA_GATE_SCALAR) or not read
 * (KDA_GATE_NONE). */
kda_status kda_decode_multi_gated(const void* q, const void* k, const void* v, const void* a, const float* beta,
                                  float* state, void* o, const int* n_commit, int B, int K, int H, int Dk, int Dv,
                                  kda_dtype dtype, kda_gate gate, void* hip_stream);

/*
 * The output side of eq. (6) of the page "Kimi K3：从三条信息流到完整系统"
 * without its two projections: y = sigmoid(z) * o / sqrt(mean(o^2) + eps),
 * the head-wise RMSNorm (no learned scale) of each row of Dv value channels
 * of the recurrent output o, gated by z = W_g x computed by the caller.
 *
 *   o, z   [rows, Dv]  dtype  (read; rows = B * T * H for a prefill's o)
 *   y      [rows, Dv]  dtype  (written; may be o itself)
 *
 * Dv = 128 only.  eps must be finite and non-negative (a zero row gives zeros
 * for eps > 0).
 */
kda_status kda_output_gate_norm(const void* o, const void* z, void* y, int64_t rows, int Dv, float eps,
                                kda_dtype dtype, void* hip_stream);

/*
 * Entering states of P consecutive segments of each sequence, from their
 * fragments: the page "Kimi K3：从三条信息流到完整系统", section "FlashKDA 与
 * KCP", eq. (17).  A segment acts on its entering state as S -> M S + E
 * (eq. (1) is affine in S): M is the segment's state run from S = I with
 * v = 0, E its state run from zero, both from kda_chunk_fwd_varlen over the
 * segments.  Then S_in[0] = S0 and S_in[j + 1] = M_j S_in[j] + E_j, in fp32.
 * With S_in as the segments' initial states, kda_chunk_fwd_varlen gives the
 * whole sequences' outputs and final states: the split of a long sequence
 * over more compute units (gated_delta_rule_23_amd.kda_chunk_fwd_split).
 *
 *   M, E   [B * P, H, Dk, Dk] / [B * P, H, Dk, Dv] fp32 (read; segment j of
 *          sequence b at b * P + j; the last segment's are not read)
 *   S0     [B, H, Dk, Dv] fp32, or NULL for zeros (read)
 *   S_in   [B * P, H, Dk, Dv] fp32 (written)
 */
kda_status kda_compose_segments(const float* M, const float* E, const float* S0, float* S_in, int B, int P, int H,
                                int Dk, int Dv, void* hip_stream);

/* Static text for a status code. */
const char* kda_status_string(kda_status status);

/* Detail of the last non-OK status returned on the calling thread ("" if none). */
const char* kda_last_error(void);

/* Library version, major * 10000 + minor * 100 + patch. */
int kda_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H */
