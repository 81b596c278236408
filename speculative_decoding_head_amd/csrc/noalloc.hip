// The verify pass without a caller's workspace, for callers that cannot allocate device
// memory (code under HIP graph capture, serving loops that must not call hipMalloc).
//
// The verify kernels need scratch memory beyond their inputs and outputs: a completion
// ticket, one drafted-id logit per hidden row and the per-block partial results (at most
// 256 blocks x 128 hidden rows x 48 bytes).  Here that scratch is a file-scope device array
// of the largest size any valid call needs; each GPU holds its own copy, at its own
// address, for the life of the process.  Its address comes from hipGetSymbolAddress once
// per device (the array's name in host code is only a host-side stand-in), and the ticket
// is cleared then by a small kernel; every call leaves the ticket at zero again, as with a
// caller's workspace.  All calls on one GPU share the array: calls that overlap on one GPU
// (two streams, two host threads) race and must be ordered by the caller.
#include <mutex>

#include "../../include/mtp.h"
#include "kernels.hpp"

namespace mtp {
namespace {

// lmhead_ws_bytes(128 rows, any vocabulary): the ticket and drafted-id slots, then 256
// blocks x 128 rows of 48-byte partials
constexpr size_t kScratchBytes = 768 + (size_t)256 * kLmheadMaxWideRows * kPartialBytes;
constexpr int kMaxDevices = 64;

__device__ __attribute__((aligned(256))) unsigned char scratch[kScratchBytes];

__global__ void clear_words_kernel(uint32_t* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

std::once_flag g_once[kMaxDevices];
void* g_ptr[kMaxDevices];
hipError_t g_err[kMaxDevices];

// The device address of the scratch array of the device the stream runs on (the current
// device for the null stream), or nullptr on failure.  The first call on a device resolves
// the address with that device current (restoring the caller's current device after) and
// clears the ticket on the stream.
void* device_scratch(hipStream_t stream) {
  int dev = -1;
  const hipError_t q = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (q != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::call_once(g_once[dev], [dev, stream]() {
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e == hipSuccess && cur != dev) e = hipSetDevice(dev);
    void* ptr = nullptr;
    if (e == hipSuccess) e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e == hipSuccess && ptr != nullptr) {
      // the completion ticket and the drafted-id slots (the first 768 bytes) start at zero
      hipLaunchKernelGGL(clear_words_kernel, dim3(1), dim3(256), 0, stream, static_cast<uint32_t*>(ptr), 192);
      e = hipGetLastError();
    }
    if (cur >= 0 && cur != dev) {
      const hipError_t r = hipSetDevice(cur);
      if (e == hipSuccess) e = r;
    }
    g_err[dev] = e;
    g_ptr[dev] = e == hipSuccess ? ptr : nullptr;
  });
  return g_ptr[dev];
}

}  // namespace
}  // namespace mtp

extern "C" {

int mtp_verify_logits_noalloc(const mtp_head* head, const void* hidden, int32_t htype, int32_t B, int32_t k,
                              const int32_t* draft_tokens, int32_t k_max, const mtp_sampling* smp,
                              mtp_row_stats* row_stats, float* logits, void* stream) {
  // every argument is checked, and sizes beyond the scratch array are rejected, before
  // any device call
  mtp::VerifyPlan plan;
  const int st = mtp::verify_logits_prepare(head, hidden, htype, B, k, draft_tokens, k_max, smp, row_stats, logits,
                                            &plan);
  if (st != MTP_OK) return st;
  if (plan.ws_need > mtp::kScratchBytes) return MTP_ERR_WORKSPACE;
  void* ptr = mtp::device_scratch(static_cast<hipStream_t>(stream));
  if (!ptr) return MTP_ERR_HIP;
  return mtp::verify_logits_run(plan, ptr, mtp::kScratchBytes, stream);
}

}  // extern "C"
