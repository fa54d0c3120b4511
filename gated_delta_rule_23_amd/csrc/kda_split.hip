/*
 * kda_split.hip -- the sequence split on one device: the page "Kimi K3：从三条
 * 信息流到完整系统", section "FlashKDA 与 KCP", eq. (17).  Eq. (1) is affine
 * in the state, so a segment of a sequence acts on the state it enters with
 * as S -> M S + E, with M the segment's transition (its state run from
 * S = I with v = 0) and E its fragment (its state run from zero).  Cutting
 * each of B sequences into P segments of seg_len tokens (whole chunks; the
 * last one takes the rest) gives P times the independent work:
 *
 *   1. transition and fragment runs, one launch: the first P - 1 segments
 *      of every sequence from the identity with v not read (the
 *      transitions), and the same segments from zero (the fragments), no o
 *      written                             -> M [B, P - 1, H, 128, 128],
 *                                             E [B, P - 1, H, 128, 128]
 *   2. composition: S_in[0] = S0, S_in[j + 1] = M_j S_in[j] + E_j
 *                                           -> S_in [B, P, H, 128, 128]
 *   3. final run: all P segments from S_in, writing o and, from each
 *      sequence's last segment, its final state.
 *
 * The prefill kernels run steps 1 and 3 (segments are sequences whose rows
 * start at b T + j seg_len, found from the unit index, so no offsets array is
 * needed) and the composition kernel runs step 2.  Three passes of the state
 * path instead of one, for P times the (sequence, head) parallelism; the
 * first two share a launch, so that together they fill the device as one.
 * The caller's workspace holds M, E (right after M) and S_in.
 */
#include <mutex>

#include "kda_common.h"
#include "kda_internal.h"

namespace kda {

namespace {

/* The workspace of kda_chunk_fwd_split_noalloc: a file-scope device array,
 * allocated with the library's code object on every GPU it runs on and held
 * until the process ends.  Host code never uses its name as an address: the
 * device address comes from hipGetSymbolAddress, once per device, and is
 * kept in scratch_ptr. */
constexpr size_t kScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_ptr[kMaxDevices] = {};

}  // namespace

const size_t kSplitScratchBytes = kScratchBytes;

hipError_t split_noalloc_scratch(hipStream_t stream, void** ptr) {
  int dev = 0;
  hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_ptr[dev]) {
    // with the stream's device current: each device holds its own copy of the array
    int cur = 0;
    e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    const hipError_t back = cur != dev ? hipSetDevice(cur) : hipSuccess;
    if (e != hipSuccess) return e;
    if (back != hipSuccess) return back;
    scratch_ptr[dev] = p;
  }
  *ptr = scratch_ptr[dev];
  return hipSuccess;
}

size_t split_workspace_bytes(int B, int P, int H) {
  if (P <= 1) return 0;
  const size_t state = (size_t)kD * kD * sizeof(float);
  return (size_t)B * H * state * (size_t)(2 * (P - 1) + P);
}

hipError_t launch_split(const void* q, const void* k, const void* v, const void* a, const float* beta,
                        const float* initial_state, void* o, float* final_state, int B, int T, int H, int P,
                        int seg_len, bool bf16_io, void* workspace, hipStream_t stream) {
  if (P <= 1) return launch_chunk_fwd(q, k, v, a, beta, initial_state, o, final_state, B, T, H, bf16_io, stream);
  const size_t per_seg = (size_t)B * H * kD * kD;  // floats per segment index over all (b, h)
  float* M = static_cast<float*>(workspace);
  float* E = M + per_seg * (P - 1);
  float* S_in = E + per_seg * (P - 1);

  PrefillOptions frag;
  frag.seg_len = seg_len;
  frag.seg_count = P - 1;
  frag.mode = kModeTransFrag;  // the transitions into M, the fragments into E = M + per_seg (P - 1)
  hipError_t e = launch_chunk_fwd(q, k, v, a, beta, nullptr, nullptr, M, B, T, H, bf16_io, stream, frag);
  if (e != hipSuccess) return e;
  e = launch_compose(M, E, initial_state, S_in, B, P, H, P - 1, stream);
  if (e != hipSuccess) return e;
  PrefillOptions fin;
  fin.seg_len = seg_len;
  fin.seg_count = P;
  fin.last_only = true;
  fin.mode = kModePacked;
  return launch_chunk_fwd(q, k, v, a, beta, S_in, o, final_state, B, T, H, bf16_io, stream, fin);
}

}  // namespace kda
