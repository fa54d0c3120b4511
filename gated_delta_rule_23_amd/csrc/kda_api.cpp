/*
 * kda_api.cpp -- the C ABI declared in include/kda.h: argument checks,
 * dispatch to the gfx950 kernels, and per-thread error text.
 */
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>

#include <atomic>

#include "kda.h"
#include "kda_internal.h"

namespace {

thread_local char g_last_error[512] = "";

kda_status fail(kda_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
kda_status fail(kda_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return s;
}

kda_status ok() { return KDA_OK; }

constexpr int kMaxPrefillHeads = 65536;
// Sequences (B * H) per call: kernels form unit indices up to the count plus
// one grid stride in 32-bit arithmetic, so the count keeps 2^20 of headroom.
constexpr int64_t kMaxUnits = (1ll << 31) - (1ll << 20);

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

/* Shared checks of dtype, head sizes and batch/head counts. */
kda_status check_common(const char* fn, int B, int H, int Dk, int Dv, kda_dtype dtype) {
  if (dtype != KDA_F32 && dtype != KDA_BF16) return fail(KDA_ERR_INVALID_ARGUMENT, "%s: unknown dtype %d", fn, (int)dtype);
  if (B < 0 || H < 0) return fail(KDA_ERR_INVALID_ARGUMENT, "%s: negative size (B=%d, H=%d)", fn, B, H);
  if (Dk <= 0 || Dv <= 0) return fail(KDA_ERR_INVALID_ARGUMENT, "%s: head sizes must be positive (Dk=%d, Dv=%d)", fn, Dk, Dv);
  if (Dk != 128 || Dv != 128)
    return fail(KDA_ERR_UNSUPPORTED, "%s: only Dk = Dv = 128 is implemented (got Dk=%d, Dv=%d)", fn, Dk, Dv);
  if ((int64_t)B * H > kMaxUnits)
    return fail(KDA_ERR_INVALID_ARGUMENT, "%s: B*H=%lld exceeds the limit of %lld sequences", fn, (long long)B * H,
                (long long)kMaxUnits);
  return KDA_OK;
}

kda_status check_ptr(const char* fn, const char* name, const void* p) {
  if (!p) return fail(KDA_ERR_INVALID_ARGUMENT, "%s: %s is NULL", fn, name);
  if (!aligned16(p)) return fail(KDA_ERR_INVALID_ARGUMENT, "%s: %s is not 16-byte aligned", fn, name);
  return KDA_OK;
}

#define KDA_TRY(expr)              \
  do {                             \
    kda_status _s = (expr);        \
    if (_s != KDA_OK) return _s;   \
  } while (0)

}  // namespace

namespace kda {

hipError_t device_cu_count(hipStream_t stream, int* cus) {
  static std::atomic<int> cache[64];
  int dev = 0;
  hipError_t err = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev >= 0 && dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) {
      *cus = c;
      return hipSuccess;
    }
  }
  err = hipDeviceGetAttribute(cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (err == hipSuccess && dev >= 0 && dev < 64) cache[dev].store(*cus, std::memory_order_relaxed);
  return err;
}

}  // namespace kda

namespace {

bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

/* The gate logits a: per key channel (16-byte aligned rows), one fp32 value
 * per token and head (4-byte aligned), or not read. */
kda_status check_gate(const char* fn, kda_gate gate, const void* a) {
  switch (gate) {
    case KDA_GATE_CHANNEL: return check_ptr(fn, "a", a);
    case KDA_GATE_SCALAR:
      if (!a) return fail(KDA_ERR_INVALID_ARGUMENT, "%s: a is NULL", fn);
      if (!aligned4(a)) return fail(KDA_ERR_INVALID_ARGUMENT, "%s: a is not 4-byte aligned", fn);
      return KDA_OK;
    case KDA_GATE_NONE: return KDA_OK;
  }
  return fail(KDA_ERR_INVALID_ARGUMENT, "%s: unknown gate %d", fn, (int)gate);
}

kda_status chunk_fwd_impl(const char* fn, const void* q, const void* k, const void* v, const void* a,
                          const float* beta, const float* initial_state, void* o, float* final_state,
                          const kda::PrefillOptions& opt, int B, int T, int H, int Dk, int Dv, kda_dtype dtype,
                          void* hip_stream) {
  KDA_TRY(check_common(fn, B, H, Dk, Dv, dtype));
  if (T < 0) return fail(KDA_ERR_INVALID_ARGUMENT, "%s: negative size (T=%d)", fn, T);
  if (opt.gate != KDA_GATE_CHANNEL && opt.gate != KDA_GATE_SCALAR && opt.gate != KDA_GATE_NONE)
    return fail(KDA_ERR_INVALID_ARGUMENT, "%s: unknown gate %d", fn, opt.gate);
  if (opt.z && !(opt.eps >= 0.0f && opt.eps <= 1.0e30f))
    return fail(KDA_ERR_INVALID_ARGUMENT, "%s: eps must be finite and >= 0", fn);
  const int64_t units = (int64_t)B * H;
  if (units == 0) return ok();
  // a chunk of one tensor (16 tokens x H x 128 elements) is addressed with 32-bit byte offsets
  if (H > kMaxPrefillHeads)
    return fail(KDA_ERR_UNSUPPORTED, "%s: H=%d exceeds the prefill limit of %d heads", fn, H, kMaxPrefillHeads);
  // every element index (b, t, h, channel) must fit in 63 bits: B*T*H*128 < 2^62
  // (packed sequences share the T rows: T*H*128)
  if ((opt.cu_seqlens ? 1.0 : (double)B) * (double)T * (double)H * 128.0 > 4.0e18)
    return fail(KDA_ERR_INVALID_ARGUMENT, "%s: B*T*H*128 overflows the index range", fn);
  KDA_TRY(check_ptr(fn, "final_state", final_state));
  if (initial_state) KDA_TRY(check_ptr(fn, "initial_state", initial_state));
  if (T > 0) {
    KDA_TRY(check_ptr(fn, "q", q));
    KDA_TRY(check_ptr(fn, "k", k));
    KDA_TRY(check_ptr(fn, "v", v));
    KDA_TRY(check_gate(fn, static_cast<kda_gate>(opt.gate), a));
    KDA_TRY(check_ptr(fn, "beta", beta));
    KDA_TRY(check_ptr(fn, "o", o));
    if (opt.z) KDA_TRY(check_ptr(fn, "z", opt.z));
  }
  if (opt.states || opt.state_every) {
    if (opt.state_every <= 0 || opt.state_every % 16 != 0)
      return fail(KDA_ERR_INVALID_ARGUMENT, "%s: state_every=%d must be a positive multiple of 16", fn,
                  opt.state_every);
    if (T / opt.state_every > 0) KDA_TRY(check_ptr(fn, "states", opt.states));
  }
  hipError_t e = kda::launch_chunk_fwd(q, k, v, a, beta, initial_state, o, final_state, B, T, H, dtype == KDA_BF16,
                                       static_cast<hipStream_t>(hip_stream), opt);
  if (e != hipSuccess) return fail(KDA_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return ok();
}

kda_status decode_impl(const char* fn, const void* q, const void* k, const void* v, const void* a, const float* beta,
                       float* state, void* o, int B, int H, int Dk, int Dv, kda_dtype dtype, kda_gate gate,
                       void* hip_stream) {
  KDA_TRY(check_common(fn, B, H, Dk, Dv, dtype));
  if (gate != KDA_GATE_CHANNEL && gate != KDA_GATE_SCALAR && gate != KDA_GATE_NONE)
    return fail(KDA_ERR_INVALID_ARGUMENT, "%s: unknown gate %d", fn, (int)gate);
  const int64_t units = (int64_t)B * H;
  if (units == 0) return ok();
  KDA_TRY(check_ptr(fn, "q", q));
  KDA_TRY(check_ptr(fn, "k", k));
  KDA_TRY(check_ptr(fn, "v", v));
  KDA_TRY(check_gate(fn, gate, a));
  KDA_TRY(check_ptr(fn, "beta", beta));
  KDA_TRY(check_ptr(fn, "state", state));
  KDA_TRY(check_ptr(fn, "o", o));
  hipError_t e = kda::launch_decode(q, k, v, a, beta, state, o, (int)units, dtype == KDA_BF16, (int)gate,
                                    static_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess) return fail(KDA_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return ok();
}

kda_status decode_multi_impl(const char* fn, const void* q, const void* k, const void* v, const void* a,
                             const float* beta, float* state, void* o, const int* n_commit, int B, int K, int H,
                             int Dk, int Dv, kda_dtype dtype, kda_gate gate, void* hip_stream) {
  KDA_TRY(check_common(fn, B, H, Dk, Dv, dtype));
  if (gate != KDA_GATE_CHANNEL && gate != KDA_GATE_SCALAR && gate != KDA_GATE_NONE)
    return fail(KDA_ERR_INVALID_ARGUMENT, "%s: unknown gate %d", fn, (int)gate);
  if (K < 0) return fail(KDA_ERR_INVALID_ARGUMENT, "%s: negative size (K=%d)", fn, K);
  const int64_t units = (int64_t)B * H;
  if (units == 0 || K == 0) return ok();
  if ((double)B * (double)K * (double)H * 128.0 > 4.0e18)
    return fail(KDA_ERR_INVALID_ARGUMENT, "%s: B*K*H*128 overflows the index range", fn);
  // the K rows of one (b, h) in one tensor are addressed with 32-bit byte offsets
  if ((int64_t)K * H * 128 * 4 > INT32_MAX)
    return fail(KDA_ERR_UNSUPPORTED, "%s: K*H=%lld exceeds the limit of %d", fn, (long long)K * H, INT32_MAX / 512);
  KDA_TRY(check_ptr(fn, "q", q));
  KDA_TRY(check_ptr(fn, "k", k));
  KDA_TRY(check_ptr(fn, "v", v));
  KDA_TRY(check_gate(fn, gate, a));
  KDA_TRY(check_ptr(fn, "beta", beta));
  KDA_TRY(check_ptr(fn, "state", state));
  KDA_TRY(check_ptr(fn, "o", o));
  if (n_commit && !aligned4(n_commit))
    return fail(KDA_ERR_INVALID_ARGUMENT, "%s: n_commit is not 4-byte aligned", fn);
  hipError_t e = kda::launch_decode_multi(q, k, v, a, beta, state, o, n_commit, (int)units, H, K, dtype == KDA_BF16,
                                          (int)gate, static_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess) return fail(KDA_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return ok();
}

/* Segments of the split: whole chunks of seg_len tokens, P of them covering T. */
void split_shape(int T, int segments, int* P, int* seg_len) {
  if (segments <= 1 || T <= 16) {
    *P = 1;
    *seg_len = T;
    return;
  }
  int L = (T + segments - 1) / segments;
  L = (L + 15) / 16 * 16;
  *seg_len = L;
  *P = (T + L - 1) / L;
}

}  // namespace

extern "C" {

kda_status kda_chunk_fwd(const void* q, const void* k, const void* v, const void* a, const float* beta,
                         const float* initial_state, void* o, float* final_state, int B, int T, int H, int Dk,
                         int Dv, kda_dtype dtype, void* hip_stream) {
  return chunk_fwd_impl("kda_chunk_fwd", q, k, v, a, beta, initial_state, o, final_state, kda::PrefillOptions(), B, T,
                        H, Dk, Dv, dtype, hip_stream);
}

kda_status kda_chunk_fwd_gated(const void* q, const void* k, const void* v, const void* a, const float* beta,
                               const float* initial_state, void* o, float* final_state, int B, int T, int H, int Dk,
                               int Dv, kda_dtype dtype, kda_gate gate, void* hip_stream) {
  kda::PrefillOptions opt;
  opt.gate = (int)gate;
  return chunk_fwd_impl("kda_chunk_fwd_gated", q, k, v, a, beta, initial_state, o, final_state, opt, B, T, H, Dk, Dv,
                        dtype, hip_stream);
}

kda_status kda_chunk_fwd_norm(const void* q, const void* k, const void* v, const void* a, const float* beta,
                              const float* initial_state, const void* z, float eps, void* y, float* final_state, int B,
                              int T, int H, int Dk, int Dv, kda_dtype dtype, void* hip_stream) {
  static const char* fn = "kda_chunk_fwd_norm";
  if (T > 0 && B > 0 && H > 0 && !z) return fail(KDA_ERR_INVALID_ARGUMENT, "%s: z is NULL", fn);
  kda::PrefillOptions opt;
  opt.z = z;
  opt.eps = eps;
  return chunk_fwd_impl(fn, q, k, v, a, beta, initial_state, y, final_state, opt, B, T, H, Dk, Dv, dtype, hip_stream);
}

kda_status kda_chunk_fwd_states(const void* q, const void* k, const void* v, const void* a, const float* beta,
                                const float* initial_state, void* o, float* final_state, float* states,
                                int state_every, int B, int T, int H, int Dk, int Dv, kda_dtype dtype,
                                void* hip_stream) {
  kda::PrefillOptions opt;
  opt.states = states;
  opt.state_every = state_every;
  return chunk_fwd_impl("kda_chunk_fwd_states", q, k, v, a, beta, initial_state, o, final_state, opt, B, T, H, Dk,
                        Dv, dtype, hip_stream);
}

kda_status kda_chunk_fwd_varlen(const void* q, const void* k, const void* v, const void* a, const float* beta,
                                const int* cu_seqlens, const float* initial_state, void* o, float* final_state, int N,
                                int T, int H, int Dk, int Dv, kda_dtype dtype, void* hip_stream) {
  static const char* fn = "kda_chunk_fwd_varlen";
  if (!cu_seqlens) return fail(KDA_ERR_INVALID_ARGUMENT, "%s: cu_seqlens is NULL", fn);
  if (!aligned4(cu_seqlens)) return fail(KDA_ERR_INVALID_ARGUMENT, "%s: cu_seqlens is not 4-byte aligned", fn);
  kda::PrefillOptions opt;
  opt.cu_seqlens = cu_seqlens;
  return chunk_fwd_impl(fn, q, k, v, a, beta, initial_state, o, final_state, opt, N, T, H, Dk, Dv, dtype, hip_stream);
}

size_t kda_chunk_fwd_split_workspace(int B, int T, int H, int segments) {
  if (B <= 0 || T <= 0 || H <= 0) return 0;
  int P = 1, L = 0;
  split_shape(T, segments, &P, &L);
  return kda::split_workspace_bytes(B, P, H);
}

kda_status kda_chunk_fwd_split(const void* q, const void* k, const void* v, const void* a, const float* beta,
                               const float* initial_state, void* o, float* final_state, int segments,
                               void* workspace, size_t workspace_bytes, int B, int T, int H, int Dk, int Dv,
                               kda_dtype dtype, void* hip_stream) {
  static const char* fn = "kda_chunk_fwd_split";
  if (segments < 1) return fail(KDA_ERR_INVALID_ARGUMENT, "%s: segments=%d must be at least 1", fn, segments);
  int P = 1, L = 0;
  split_shape(T, segments, &P, &L);
  // the same checks as the plain prefill, over B sequences of T tokens
  KDA_TRY(check_common(fn, B, H, Dk, Dv, dtype));
  if (T < 0) return fail(KDA_ERR_INVALID_ARGUMENT, "%s: negative size (T=%d)", fn, T);
  if ((int64_t)B * H * P > kMaxUnits)
    return fail(KDA_ERR_INVALID_ARGUMENT, "%s: B*H*segments exceeds the limit of %lld sequences", fn,
                (long long)kMaxUnits);
  if (P == 1 || (int64_t)B * H == 0)
    return chunk_fwd_impl(fn, q, k, v, a, beta, initial_state, o, final_state, kda::PrefillOptions(), B, T, H, Dk, Dv,
                          dtype, hip_stream);
  const size_t need = kda::split_workspace_bytes(B, P, H);
  if (!workspace) return fail(KDA_ERR_INVALID_ARGUMENT, "%s: workspace is NULL (%zu bytes needed)", fn, need);
  if (!aligned16(workspace)) return fail(KDA_ERR_INVALID_ARGUMENT, "%s: workspace is not 16-byte aligned", fn);
  if (workspace_bytes < need)
    return fail(KDA_ERR_INVALID_ARGUMENT, "%s: workspace of %zu bytes, %zu needed", fn, workspace_bytes, need);
  if (H > kMaxPrefillHeads)
    return fail(KDA_ERR_UNSUPPORTED, "%s: H=%d exceeds the prefill limit of %d heads", fn, H, kMaxPrefillHeads);
  if ((double)B * (double)T * (double)H * 128.0 > 4.0e18)
    return fail(KDA_ERR_INVALID_ARGUMENT, "%s: B*T*H*128 overflows the index range", fn);
  KDA_TRY(check_ptr(fn, "final_state", final_state));
  if (initial_state) KDA_TRY(check_ptr(fn, "initial_state", initial_state));
  KDA_TRY(check_ptr(fn, "q", q));
  KDA_TRY(check_ptr(fn, "k", k));
  KDA_TRY(check_ptr(fn, "v", v));
  KDA_TRY(check_ptr(fn, "a", a));
  KDA_TRY(check_ptr(fn, "beta", beta));
  KDA_TRY(check_ptr(fn, "o", o));
  hipError_t e = kda::launch_split(q, k, v, a, beta, initial_state, o, final_state, B, T, H, P, L, dtype == KDA_BF16,
                                   workspace, static_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess) return fail(KDA_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return ok();
}

kda_status kda_chunk_fwd_split_noalloc(const void* q, const void* k, const void* v, const void* a, const float* beta,
                                       const float* initial_state, void* o, float* final_state, int segments, int B,
                                       int T, int H, int Dk, int Dv, kda_dtype dtype, void* hip_stream) {
  static const char* fn = "kda_chunk_fwd_split_noalloc";
  if (segments < 1) return fail(KDA_ERR_INVALID_ARGUMENT, "%s: segments=%d must be at least 1", fn, segments);
  KDA_TRY(check_common(fn, B, H, Dk, Dv, dtype));
  if (T < 0) return fail(KDA_ERR_INVALID_ARGUMENT, "%s: negative size (T=%d)", fn, T);
  int P = 1, L = 0;
  split_shape(T, segments, &P, &L);
  if ((int64_t)B * H * P > kMaxUnits)
    return fail(KDA_ERR_INVALID_ARGUMENT, "%s: B*H*segments exceeds the limit of %lld sequences", fn,
                (long long)kMaxUnits);
  const size_t need = kda::split_workspace_bytes(B, P, H);
  if (need > kda::kSplitScratchBytes)
    return fail(KDA_ERR_INVALID_ARGUMENT,
                "%s: the split needs %zu bytes of scratch (B*H = %lld, %d segments), more than the %zu bytes the "
                "library holds; use fewer segments or kda_chunk_fwd_split with a workspace",
                fn, need, (long long)B * H, P, kda::kSplitScratchBytes);
  void* work = nullptr;  // the device address of the library's scratch array
  if (need > 0 && (int64_t)B * H > 0 && T > 0) {
    const hipError_t e = kda::split_noalloc_scratch(static_cast<hipStream_t>(hip_stream), &work);
    if (e != hipSuccess) return fail(KDA_ERR_HIP, "%s: scratch lookup failed: %s", fn, hipGetErrorString(e));
  }
  return kda_chunk_fwd_split(q, k, v, a, beta, initial_state, o, final_state, segments, work, need, B, T, H, Dk, Dv,
                             dtype, hip_stream);
}

kda_status kda_decode_step(const void* q, const void* k, const void* v, const void* a, const float* beta,
                           float* state, void* o, int B, int H, int Dk, int Dv, kda_dtype dtype, void* hip_stream) {
  return decode_impl("kda_decode_step", q, k, v, a, beta, state, o, B, H, Dk, Dv, dtype, KDA_GATE_CHANNEL, hip_stream);
}

kda_status kda_decode_step_gated(const void* q, const void* k, const void* v, const void* a, const float* beta,
                                 float* state, void* o, int B, int H, int Dk, int Dv, kda_dtype dtype, kda_gate gate,
                                 void* hip_stream) {
  return decode_impl("kda_decode_step_gated", q, k, v, a, beta, state, o, B, H, Dk, Dv, dtype, gate, hip_stream);
}

kda_status kda_decode_multi(const void* q, const void* k, const void* v, const void* a, const float* beta,
                            float* state, void* o, const int* n_commit, int B, int K, int H, int Dk, int Dv,
                            kda_dtype dtype, void* hip_stream) {
  return decode_multi_impl("kda_decode_multi", q, k, v, a, beta, state, o, n_commit, B, K, H, Dk, Dv, dtype,
                           KDA_GATE_CHANNEL, hip_stream);
}

kda_status kda_decode_multi_gated(const void* q, const void* k, const void* v, const void* a, const float* beta,
                                  float* state, void* o, const int* n_commit, int B, int K, int H, int Dk, int Dv,
                                  kda_dtype dtype, kda_gate gate, void* hip_stream) {
  return decode_multi_impl("kda_decode_multi_gated", q, k, v, a, beta, state, o, n_commit, B, K, H, Dk, Dv, dtype,
                           gate, hip_stream);
}

kda_status kda_output_gate_norm(const void* o, const void* z, void* y, int64_t rows, int Dv, float eps,
                                kda_dtype dtype, void* hip_stream) {
  static const char* fn = "kda_output_gate_norm";
  if (dtype != KDA_F32 && dtype != KDA_BF16) return fail(KDA_ERR_INVALID_ARGUMENT, "%s: unknown dtype %d", fn, (int)dtype);
  if (rows < 0) return fail(KDA_ERR_INVALID_ARGUMENT, "%s: negative size (rows=%lld)", fn, (long long)rows);
  if (Dv <= 0) return fail(KDA_ERR_INVALID_ARGUMENT, "%s: head size must be positive (Dv=%d)", fn, Dv);
  if (Dv != 128) return fail(KDA_ERR_UNSUPPORTED, "%s: only Dv = 128 is implemented (got Dv=%d)", fn, Dv);
  if (!(eps >= 0.0f) || eps > 1.0e30f) return fail(KDA_ERR_INVALID_ARGUMENT, "%s: eps must be finite and >= 0", fn);
  if (rows > ((int64_t)1 << 40)) return fail(KDA_ERR_INVALID_ARGUMENT, "%s: rows=%lld is too large", fn, (long long)rows);
  if (rows == 0) return ok();
  KDA_TRY(check_ptr(fn, "o", o));
  KDA_TRY(check_ptr(fn, "z", z));
  KDA_TRY(check_ptr(fn, "y", y));
  hipError_t e = kda::launch_output_gate_norm(o, z, y, rows, eps, dtype == KDA_BF16, static_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess) return fail(KDA_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return ok();
}

kda_status kda_compose_segments(const float* M, const float* E, const float* S0, float* S_in, int B, int P, int H,
                                int Dk, int Dv, void* hip_stream) {
  static const char* fn = "kda_compose_segments";
  KDA_TRY(check_common(fn, B, H, Dk, Dv, KDA_F32));
  if (P < 0) return fail(KDA_ERR_INVALID_ARGUMENT, "%s: negative size (P=%d)", fn, P);
  if ((int64_t)B * H * P > kMaxUnits)
    return fail(KDA_ERR_INVALID_ARGUMENT, "%s: B*H*P exceeds the limit of %lld states", fn, (long long)kMaxUnits);
  if ((int64_t)B * H == 0 || P == 0) return ok();
  if (P > 1) {
    KDA_TRY(check_ptr(fn, "M", M));
    KDA_TRY(check_ptr(fn, "E", E));
  }
  if (S0) KDA_TRY(check_ptr(fn, "S0", S0));
  KDA_TRY(check_ptr(fn, "S_in", S_in));
  hipError_t e = kda::launch_compose(M, E, S0, S_in, B, P, H, P, static_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess) return fail(KDA_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return ok();
}

const char* kda_status_string(kda_status status) {
  switch (status) {
    case KDA_OK: return "KDA_OK";
    case KDA_ERR_INVALID_ARGUMENT: return "KDA_ERR_INVALID_ARGUMENT";
    case KDA_ERR_UNSUPPORTED: return "KDA_ERR_UNSUPPORTED";
    case KDA_ERR_HIP: return "KDA_ERR_HIP";
  }
  return "KDA_ERR_UNKNOWN";
}

const char* kda_last_error(void) { return g_last_error; }

int kda_version(void) { return 100; }

}  // extern "C"
