// rr_scratch.hip -- the all-reduce entry point that allocates nothing.
//
// rr_all_reduce_ex takes its workspace (the staged ring's float32 partials
// of 16-bit types, the staged hierarchy's group partials) from the caller.
// rr_all_reduce_ex_noalloc serves callers that cannot allocate device memory
// at the call (code under graph capture, tight serving loops, harnesses that
// forbid allocation): its workspace is `scratch`, a fixed array of
// RR_NOALLOC_SCRATCH_BYTES in the library's own device memory, which every
// GPU the library runs on holds from the moment the library's code is loaded
// there until the process ends.
//
// In host code the array's name is only a host-side stand-in: its device
// address comes from hipGetSymbolAddress, taken once per device (with that
// device current) at the entry point's first call on the device and kept;
// kernels only ever receive that address.  Every call on a GPU shares the
// GPU's array and finds whatever the previous call left there; the staged
// algorithms write every workspace element they read before reading it
// within the call, so nothing needs clearing.  Calls that overlap in time on
// one GPU (different streams, or different host threads without ordering)
// race on the array.
#include <hip/hip_runtime.h>
#include <stdio.h>

#include <mutex>

#include "rr.h"

static __device__ __align__(256) unsigned char scratch[RR_NOALLOC_SCRATCH_BYTES];

namespace rr {

// Records the message rr_last_error() returns (rr_api.cpp).
rr_status_t record_failure(rr_status_t st, const char* msg);

namespace {

constexpr int kMaxDevices = 64;

struct ScratchDevice {
  std::mutex mu;
  void* ptr = nullptr;  // the device address of `scratch` on this device, once taken
};

ScratchDevice g_scratch[kMaxDevices];

// The device address of `scratch` on device `dev`: hipGetSymbolAddress with
// `dev` current, the first time (a failure is reported and tried again at
// the next call), the kept address afterwards.
hipError_t scratch_address(int dev, void** out) {
  ScratchDevice& d = g_scratch[dev];
  std::lock_guard<std::mutex> lock(d.mu);
  if (!d.ptr) {
    int cur = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    d.ptr = p;
  }
  *out = d.ptr;
  return hipSuccess;
}

}  // namespace

}  // namespace rr

extern "C" rr_status_t rr_all_reduce_ex_noalloc(const void* const* sendbufs, void* const* recvbufs, int p, size_t n,
                                                rr_dtype_t dtype, rr_op_t op, rr_algo_t algo, int group_size,
                                                rr_stream_t stream) {
  char msg[256];
  if (algo == RR_ALGO_RING_PERSISTENT)
    return rr::record_failure(RR_ERROR_UNSUPPORTED,
                              "rr_all_reduce_ex_noalloc: the persistent executor is not offered without allocation "
                              "(its first launch on a stream creates a completion event)");
  const size_t need = rr_workspace_size(algo, p, group_size, n, dtype);
  if (need > static_cast<size_t>(RR_NOALLOC_SCRATCH_BYTES)) {
    snprintf(msg, sizeof(msg),
             "rr_all_reduce_ex_noalloc: algo %d needs %zu bytes of workspace, more than the library's fixed "
             "scratch of %llu bytes; use rr_all_reduce_ex with a caller workspace",
             static_cast<int>(algo), need, static_cast<unsigned long long>(RR_NOALLOC_SCRATCH_BYTES));
    return rr::record_failure(RR_ERROR_INVALID_ARGUMENT, msg);
  }
  // No workspace needed (the fused algorithms, 4-byte staged ring, n == 0)
  // or invalid arguments, which rr_all_reduce_ex reports before any launch.
  if (need == 0) return rr_all_reduce_ex(sendbufs, recvbufs, p, n, dtype, op, algo, group_size, nullptr, 0, stream);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  int dev = 0;
  hipError_t e = s ? hipStreamGetDevice(s, &dev) : hipGetDevice(&dev);
  if (e == hipSuccess && (dev < 0 || dev >= rr::kMaxDevices)) e = hipErrorInvalidDevice;
  void* ws = nullptr;
  if (e == hipSuccess) e = rr::scratch_address(dev, &ws);
  if (e != hipSuccess) {
    snprintf(msg, sizeof(msg), "rr_all_reduce_ex_noalloc: the scratch address of device %d: HIP error %d (%s)", dev,
             static_cast<int>(e), hipGetErrorString(e));
    return rr::record_failure(RR_ERROR_HIP, msg);
  }
  return rr_all_reduce_ex(sendbufs, recvbufs, p, n, dtype, op, algo, group_size, ws,
                          static_cast<size_t>(RR_NOALLOC_SCRATCH_BYTES), stream);
}
