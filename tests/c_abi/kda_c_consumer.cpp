/*
 * kda_c_consumer.cpp -- a plain C++ caller of the library's C ABI
 * (include/kda.h): no Python, no torch.  Device memory comes from hipMalloc,
 * inputs from a seeded host generator, and the outputs are checked against
 * the fp64 oracle (oracle/libkda_oracle.so, test infrastructure) at the
 * tolerances of the Python parity tests: relative L2 1e-5 for fp32 I/O, 2e-2
 * for bf16 I/O.
 *
 * Cases: kda_chunk_fwd over B = 2 sequences of T = 77 tokens (four whole
 * chunks and a ragged one) and H = 3 heads, fp32 and bf16 I/O, with and
 * without an initial state; kda_decode_step on the resulting states; a
 * request the library does not implement (Dk = 64), which must return
 * KDA_ERR_UNSUPPORTED with a reason in kda_last_error().
 *
 *   kda_c_consumer            all cases (needs a GPU)
 *   kda_c_consumer --abi-only the status and version calls and argument
 *                             checks that return before any HIP call
 *
 * Prints one line per case and exits 0 when every case passes.
 */
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "kda.h"

// The oracle's entry point (oracle/kda_oracle.c): per (batch, head) unit,
// q, k, a [n][T][dk]; v, o [n][T][dv]; beta [n][T]; states [n][dk][dv].
extern "C" int kda_oracle_forward(int n_units, int T, int dk, int dv, const double* q, const double* k,
                                  const double* v, const double* gate, int gate_is_logit, const double* beta,
                                  const double* s0, double* o, double* s_final, int n_threads);

namespace {

constexpr int B = 2, T = 77, H = 3, D = 128;
int failures = 0;

// splitmix64: a seeded stream of uniform doubles in [0, 1)
struct Rng {
  uint64_t s;
  double next() {
    uint64_t z = (s += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    z ^= z >> 31;
    return (double)(z >> 11) * (1.0 / 9007199254740992.0);
  }
  double uni(double lo, double hi) { return lo + (hi - lo) * next(); }
};

// bf16 bits of x, round to nearest even (inputs here are finite)
uint16_t to_bf16(float x) {
  uint32_t u;
  std::memcpy(&u, &x, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
float from_bf16(uint16_t b) {
  const uint32_t u = (uint32_t)b << 16;
  float x;
  std::memcpy(&x, &u, 4);
  return x;
}

double rel_l2(const std::vector<double>& x, const std::vector<double>& ref) {
  double num = 0, den = 0;
  for (size_t i = 0; i < x.size(); ++i) {
    num += (x[i] - ref[i]) * (x[i] - ref[i]);
    den += ref[i] * ref[i];
  }
  return std::sqrt(num / (den > 0 ? den : 1));
}

void report(const char* name, bool ok, const char* detail) {
  std::printf("%s %s %s\n", ok ? "PASS" : "FAIL", name, detail);
  if (!ok) ++failures;
}

#define HIP_OK(call)                                                                   \
  do {                                                                                 \
    hipError_t e_ = (call);                                                            \
    if (e_ != hipSuccess) {                                                            \
      std::printf("FAIL %s: %s\n", #call, hipGetErrorString(e_));                      \
      std::exit(1);                                                                    \
    }                                                                                  \
  } while (0)

// Inputs in the ABI layout: q, k, v, a [B, T, H, D]; beta [B, T, H]; s0 [B, H, D, D].
struct Inputs {
  std::vector<float> q, k, v, a, beta, s0;
};

Inputs draw(uint64_t seed) {
  Rng r{seed};
  Inputs in;
  const size_t n = (size_t)B * T * H * D;
  in.q.resize(n);
  in.k.resize(n);
  in.v.resize(n);
  in.a.resize(n);
  in.beta.resize((size_t)B * T * H);
  in.s0.resize((size_t)B * H * D * D);
  for (size_t row = 0; row < (size_t)B * T * H; ++row) {
    double kk = 0;
    for (int c = 0; c < D; ++c) {
      const size_t i = row * D + c;
      in.q[i] = (float)r.uni(-1, 1) * 0.1f;
      in.k[i] = (float)r.uni(-1, 1);
      kk += (double)in.k[i] * in.k[i];
      in.v[i] = (float)r.uni(-1, 1);
      in.a[i] = (float)r.uni(-10, -4);  // log-decay -5 sigmoid(a) in (-0.09, -0.0002): S0 persists to the end
    }
    const double inv = 1.0 / std::sqrt(kk);  // unit-norm keys, as the delta rule assumes
    for (int c = 0; c < D; ++c) in.k[row * D + c] = (float)(in.k[row * D + c] * inv);
    in.beta[row] = (float)r.uni(0, 1);
  }
  for (auto& x : in.s0) x = (float)r.uni(-0.5, 0.5);
  return in;
}

// The oracle on the ABI layout: units u = b H + h.
void oracle(const Inputs& in, bool with_s0, std::vector<double>& o, std::vector<double>& S) {
  const int n = B * H;
  std::vector<double> q((size_t)n * T * D), k(q.size()), v(q.size()), a(q.size()), beta((size_t)n * T);
  for (int b = 0; b < B; ++b)
    for (int t = 0; t < T; ++t)
      for (int h = 0; h < H; ++h) {
        const int u = b * H + h;
        beta[(size_t)u * T + t] = in.beta[((size_t)b * T + t) * H + h];
        for (int c = 0; c < D; ++c) {
          const size_t src = (((size_t)b * T + t) * H + h) * D + c, dst = ((size_t)u * T + t) * D + c;
          q[dst] = in.q[src];
          k[dst] = in.k[src];
          v[dst] = in.v[src];
          a[dst] = in.a[src];
        }
      }
  std::vector<double> s0(in.s0.begin(), in.s0.end()), ou((size_t)n * T * D);
  S.assign((size_t)n * D * D, 0.0);
  if (kda_oracle_forward(n, T, D, D, q.data(), k.data(), v.data(), a.data(), 1, beta.data(),
                         with_s0 ? s0.data() : nullptr, ou.data(), S.data(), 4) != 0) {
    report("oracle", false, "kda_oracle_forward failed");
    return;
  }
  o.assign(ou.size(), 0.0);  // back to [B, T, H, D]
  for (int b = 0; b < B; ++b)
    for (int t = 0; t < T; ++t)
      for (int h = 0; h < H; ++h)
        for (int c = 0; c < D; ++c)
          o[(((size_t)b * T + t) * H + h) * D + c] = ou[(((size_t)(b * H + h)) * T + t) * D + c];
}

template <typename T_>
void* upload(const std::vector<T_>& x) {
  void* p = nullptr;
  HIP_OK(hipMalloc(&p, x.size() * sizeof(T_)));
  HIP_OK(hipMemcpy(p, x.data(), x.size() * sizeof(T_), hipMemcpyHostToDevice));
  return p;
}

std::vector<uint16_t> to_bf16(const std::vector<float>& x) {
  std::vector<uint16_t> y(x.size());
  for (size_t i = 0; i < x.size(); ++i) y[i] = to_bf16(x[i]);
  return y;
}

// kda_chunk_fwd in one dtype against the oracle on the inputs that dtype sees
void prefill_case(const Inputs& in32, kda_dtype dtype, bool with_s0) {
  Inputs in = in32;
  if (dtype == KDA_BF16)  // the oracle runs on the bf16-rounded inputs
    for (auto* t : {&in.q, &in.k, &in.v, &in.a})
      for (auto& x : *t) x = from_bf16(to_bf16(x));
  const size_t n = (size_t)B * T * H * D;
  void *dq, *dk, *dv, *da;
  if (dtype == KDA_BF16) {
    dq = upload(to_bf16(in.q));
    dk = upload(to_bf16(in.k));
    dv = upload(to_bf16(in.v));
    da = upload(to_bf16(in.a));
  } else {
    dq = upload(in.q);
    dk = upload(in.k);
    dv = upload(in.v);
    da = upload(in.a);
  }
  float* dbeta = static_cast<float*>(upload(in.beta));
  float* ds0 = with_s0 ? static_cast<float*>(upload(in.s0)) : nullptr;
  const size_t osz = n * (dtype == KDA_BF16 ? 2 : 4);
  void* dout = nullptr;
  float* dS = nullptr;
  HIP_OK(hipMalloc(&dout, osz));
  HIP_OK(hipMalloc(reinterpret_cast<void**>(&dS), (size_t)B * H * D * D * sizeof(float)));
  const kda_status st = kda_chunk_fwd(dq, dk, dv, da, dbeta, ds0, dout, dS, B, T, H, D, D, dtype, nullptr);
  HIP_OK(hipDeviceSynchronize());
  std::vector<double> o(n), S((size_t)B * H * D * D);
  if (dtype == KDA_BF16) {
    std::vector<uint16_t> ob(n);
    HIP_OK(hipMemcpy(ob.data(), dout, osz, hipMemcpyDeviceToHost));
    for (size_t i = 0; i < n; ++i) o[i] = from_bf16(ob[i]);
  } else {
    std::vector<float> of(n);
    HIP_OK(hipMemcpy(of.data(), dout, osz, hipMemcpyDeviceToHost));
    for (size_t i = 0; i < n; ++i) o[i] = of[i];
  }
  std::vector<float> Sf(S.size());
  HIP_OK(hipMemcpy(Sf.data(), dS, Sf.size() * sizeof(float), hipMemcpyDeviceToHost));
  for (size_t i = 0; i < S.size(); ++i) S[i] = Sf[i];
  std::vector<double> o_ref, S_ref, o_zero, S_zero;
  oracle(in, with_s0, o_ref, S_ref);
  // the case's own check: the initial state changes the result well beyond the tolerance
  double s0_effect = 1.0;
  if (with_s0) {
    oracle(in, false, o_zero, S_zero);
    s0_effect = std::min(rel_l2(o_zero, o_ref), rel_l2(S_zero, S_ref));
  }
  const double eo = rel_l2(o, o_ref), es = rel_l2(S, S_ref), tol = dtype == KDA_BF16 ? 2e-2 : 1e-5;
  char msg[200];
  std::snprintf(msg, sizeof msg, "status %d, rel L2 o %.2e, S %.2e (tolerance %.0e)", (int)st, eo, es, tol);
  if (with_s0) {
    const size_t len = std::strlen(msg);
    std::snprintf(msg + len, sizeof msg - len, "; S0 moves the result by %.2e", s0_effect);
  }
  char name[64];
  std::snprintf(name, sizeof name, "kda_chunk_fwd %s%s", dtype == KDA_BF16 ? "bf16" : "fp32",
                with_s0 ? " with S0" : "");
  report(name, st == KDA_OK && eo <= tol && es <= tol && s0_effect > 0.1, msg);
  for (void* p : {dq, dk, dv, da, static_cast<void*>(dbeta), static_cast<void*>(ds0), dout, static_cast<void*>(dS)})
    if (p) HIP_OK(hipFree(p));
}

// kda_decode_step (fp32 I/O): one more token on top of the prefill's states
void decode_case(const Inputs& in) {
  // the states after the prefill (oracle), then one token of fresh inputs
  std::vector<double> o_ref, S_ref;
  oracle(in, true, o_ref, S_ref);
  Rng r{99};
  std::vector<float> q((size_t)B * H * D), k(q.size()), v(q.size()), a(q.size()), beta((size_t)B * H);
  for (size_t row = 0; row < (size_t)B * H; ++row) {
    double kk = 0;
    for (int c = 0; c < D; ++c) {
      q[row * D + c] = (float)r.uni(-0.1, 0.1);
      k[row * D + c] = (float)r.uni(-1, 1);
      kk += (double)k[row * D + c] * k[row * D + c];
      v[row * D + c] = (float)r.uni(-1, 1);
      a[row * D + c] = (float)r.uni(-10, -4);
    }
    for (int c = 0; c < D; ++c) k[row * D + c] = (float)(k[row * D + c] / std::sqrt(kk));
    beta[row] = (float)r.uni(0, 1);
  }
  std::vector<float> S0(S_ref.begin(), S_ref.end());
  float* dS = static_cast<float*>(upload(S0));
  void *dq = upload(q), *dk = upload(k), *dv = upload(v), *da = upload(a);
  float* dbeta = static_cast<float*>(upload(beta));
  void* dout = nullptr;
  HIP_OK(hipMalloc(&dout, q.size() * sizeof(float)));
  const kda_status st = kda_decode_step(dq, dk, dv, da, dbeta, dS, dout, B, H, D, D, KDA_F32, nullptr);
  HIP_OK(hipDeviceSynchronize());
  std::vector<float> of(q.size()), Sf(S0.size());
  HIP_OK(hipMemcpy(of.data(), dout, of.size() * sizeof(float), hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(Sf.data(), dS, Sf.size() * sizeof(float), hipMemcpyDeviceToHost));
  // the oracle's step: one token from the fp32-rounded states the kernel started from
  std::vector<double> qd(q.begin(), q.end()), kd(k.begin(), k.end()), vd(v.begin(), v.end()), ad(a.begin(), a.end()),
      bd(beta.begin(), beta.end()), s0d(S0.begin(), S0.end()), od(q.size()), Sd(S0.size());
  if (kda_oracle_forward(B * H, 1, D, D, qd.data(), kd.data(), vd.data(), ad.data(), 1, bd.data(), s0d.data(),
                         od.data(), Sd.data(), 4) != 0) {
    report("kda_decode_step fp32", false, "kda_oracle_forward failed");
  } else {
    const double eo = rel_l2(std::vector<double>(of.begin(), of.end()), od);
    const double es = rel_l2(std::vector<double>(Sf.begin(), Sf.end()), Sd);
    char msg[160];
    std::snprintf(msg, sizeof msg, "status %d, rel L2 o %.2e, S %.2e (tolerance 1e-05)", (int)st, eo, es);
    report("kda_decode_step fp32", st == KDA_OK && eo <= 1e-5 && es <= 1e-5, msg);
  }
  for (void* p : {dq, dk, dv, da, static_cast<void*>(dbeta), static_cast<void*>(dS), dout}) HIP_OK(hipFree(p));
}

// Calls that the library rejects before any HIP call (fake, never-dereferenced pointers).
void abi_case() {
  char msg[200];
  std::snprintf(msg, sizeof msg, "version %d, KDA_OK is \"%s\"", kda_version(), kda_status_string(KDA_OK));
  report("kda_version / kda_status_string", kda_version() >= 100 && std::strcmp(kda_status_string(KDA_OK), "KDA_OK") == 0,
         msg);
  void* p = reinterpret_cast<void*>(0x10000);
  float* pf = reinterpret_cast<float*>(0x10000);
  const kda_status s1 = kda_chunk_fwd(p, p, p, p, pf, nullptr, p, pf, 1, 16, 1, 64, 128, KDA_BF16, nullptr);
  std::snprintf(msg, sizeof msg, "Dk = 64: status %d (%s), \"%s\"", (int)s1, kda_status_string(s1), kda_last_error());
  report("unsupported head size", s1 == KDA_ERR_UNSUPPORTED && kda_last_error()[0] != '\0', msg);
  const kda_status s2 = kda_chunk_fwd(nullptr, p, p, p, pf, nullptr, p, pf, 1, 16, 1, 128, 128, KDA_BF16, nullptr);
  std::snprintf(msg, sizeof msg, "q = NULL: status %d (%s), \"%s\"", (int)s2, kda_status_string(s2), kda_last_error());
  report("null input", s2 == KDA_ERR_INVALID_ARGUMENT, msg);
}

}  // namespace

int main(int argc, char** argv) {
  const bool abi_only = argc > 1 && std::strcmp(argv[1], "--abi-only") == 0;
  abi_case();
  if (!abi_only) {
    const Inputs in = draw(2024);
    prefill_case(in, KDA_F32, false);
    prefill_case(in, KDA_F32, true);
    prefill_case(in, KDA_BF16, false);
    prefill_case(in, KDA_BF16, true);
    decode_case(in);
  }
  std::printf("%s: %d failure(s)\n", failures ? "FAILED" : "OK", failures);
  return failures ? 1 : 0;
}
