// The L1 image loss without allocation: gs_loss_l1 with its per-workgroup partial sums in a static
// device array instead of a caller-provided workspace, for callers that cannot allocate device
// memory (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
//
// `scratch` is a file-scope __device__ array: every GPU the library runs on holds its own copy, at
// its own address, until the process ends.  In host code the name `scratch` is a host-side
// stand-in, not a device address; the kernels get the address hipGetSymbolAddress reports for the
// current device, looked up once per device with that device current.  Every call on one GPU shares
// that GPU's copy and leaves its partial sums there, so calls that overlap on one GPU (on two
// streams, or from two host threads) race; nothing in it must start at zero, since each call writes
// every partial sum it reads.
#include <mutex>

#include "gsmi_internal.h"

namespace gsmi {
namespace {

constexpr int64_t kLossBlockElems = 4096;        // elements per partial sum of the L1 kernels
constexpr int64_t kScratchPartials = 65536;      // 256 KiB per GPU
constexpr int64_t kNoAllocMax = kScratchPartials * kLossBlockElems;  // 268,435,456 elements

__device__ __align__(256) float scratch[kScratchPartials];

// The device address of `scratch` on the current device (looked up once per device).
hipError_t scratch_on_device(float** out) {
  static std::mutex mu;
  static float* addr[64] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = static_cast<float*>(p);
  }
  *out = addr[dev];
  return hipSuccess;
}

}  // namespace
}  // namespace gsmi

using namespace gsmi;

extern "C" int gs_loss_l1_noalloc(int64_t count, const float* image, const float* target, float* loss,
                                  float* dL_dimage, hipStream_t stream) {
  if (count < 0) return fail_status(GS_ERR_INVALID_ARGUMENT, "count < 0");
  if (count > kNoAllocMax)
    return fail_status(GS_ERR_CAPACITY,
                       "count %lld exceeds the %lld elements the no-allocation L1 loss serves (its static scratch "
                       "holds %lld partial sums of %lld elements); use gs_loss_l1 with a workspace",
                       (long long)count, (long long)kNoAllocMax, (long long)kScratchPartials,
                       (long long)kLossBlockElems);
  if (!loss || (count > 0 && (!image || !target || !dL_dimage)))
    return fail_status(GS_ERR_INVALID_ARGUMENT, "a required pointer is null");
  if (loss_workspace_bytes(count) > sizeof(float) * (size_t)kScratchPartials)
    return fail_status(GS_ERR_CAPACITY, "the L1 loss needs %zu bytes of partial sums, more than the static scratch",
                       loss_workspace_bytes(count));
  float* part = nullptr;
  hipError_t e = scratch_on_device(&part);
  if (e == hipSuccess) e = launch_loss_l1(count, image, target, loss, dL_dimage, part, stream);
  return e == hipSuccess ? ok_status() : hip_status(e, "gs_loss_l1_noalloc");
}
