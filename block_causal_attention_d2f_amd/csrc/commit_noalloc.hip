// The commit pass without a caller-supplied workspace, for callers that
// cannot allocate device memory (code under stream capture, tight serving
// loops, harnesses that forbid hipMalloc).
//
// d2f_confidence_commit_noalloc runs exactly the kernels of
// d2f_confidence_commit; its per-(row, chunk) partials go to `scratch`, an
// array of this file that every device the library runs on holds from the
// loading of the library's code until the process ends.  The host never
// uses the array's name as an address (on the host it only names the
// symbol): its device address is looked up once per device, with that
// device current, and kept.  All calls on one device share its array, so
// calls that overlap on one device (two streams, or two host threads) race;
// nothing in the array needs to start at zero (every partial a decision
// reads was written by the same call).
#include <mutex>

#include "d2f_internal.h"

namespace d2f {
namespace {

constexpr size_t kScratchBytes = D2F_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch`, per device

// Device address of `scratch` on device dev (looked up on first use, with dev
// current, then kept).
d2f_status_t scratch_on(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices)
    return fail(D2F_ERR_UNSUPPORTED, "device %d is outside the %d devices the scratch table holds",
                dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    int cur = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return hip_fail(e, "hipSetDevice");
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess && e2 != hipSuccess) e = e2;
    }
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (p == nullptr) return fail(D2F_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return D2F_OK;
}

}  // namespace
}  // namespace d2f

using namespace d2f;

extern "C" {

d2f_status_t d2f_confidence_commit_noalloc(const float* logits, int64_t ld, int32_t n_rows,
                                           int32_t vocab, uint8_t* mask_state, int32_t* tokens,
                                           const uint8_t* block_phase, int32_t block_size,
                                           float tau, int32_t k_aggr, int32_t mask_token_id,
                                           float* conf_out, int32_t* argmax_out,
                                           int32_t* n_committed, uint8_t* block_complete,
                                           d2f_stream_t stream) {
  size_t need = 0;
  d2f_status_t st = d2f_confidence_commit_workspace_size(n_rows, vocab, &need);
  if (st != D2F_OK) return st;
  if (need > kScratchBytes)
    return fail(D2F_ERR_WORKSPACE,
                "%d rows x vocab %d need %zu bytes of scratch; the no-allocation pass holds "
                "%zu (use d2f_confidence_commit with a workspace)",
                n_rows, vocab, need, kScratchBytes);
  if (n_rows == 0) return D2F_OK;
  // The kernels run on the stream's device: its copy of the array is used.
  int dev = 0;
  hipError_t e = stream == nullptr ? hipGetDevice(&dev)
                                   : hipStreamGetDevice((hipStream_t)stream, &dev);
  if (e != hipSuccess) return hip_fail(e, "device of the stream");
  void* ws = nullptr;
  if ((st = scratch_on(dev, &ws)) != D2F_OK) return st;
  return d2f_confidence_commit(logits, ld, n_rows, vocab, mask_state, tokens, block_phase,
                               block_size, tau, k_aggr, mask_token_id, conf_out, argmax_out,
                               n_committed, block_complete, ws, kScratchBytes, stream);
}

}  // extern "C"
