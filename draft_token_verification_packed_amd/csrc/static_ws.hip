// Greedy verification without any allocation: the workspace is a
// file-scope device array of fixed size instead of a caller buffer, for
// callers that cannot allocate device memory (code under HIP graph capture,
// tight serving loops, harnesses that forbid allocation).
//
// Each GPU holds its own copy of `scratch` at its own address. In host code
// the array's name is only a host-side stand-in, so the device address is
// looked up once per device (hipGetSymbolAddress, with that device current)
// and only that address is ever passed to kernels. The array is zero-filled
// on the first call on a device (on that call's stream, before its
// verification kernel); after that every call leaves it ready for the next,
// as any workspace. Every call on a device shares that device's array, so
// calls that may overlap in time on one device race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kernels.hpp"

namespace {

// Largest batch (packed rows) the array serves, and its size in bytes:
// the greedy workspace of that many rows, about 0.95 MiB.
constexpr int32_t kStaticRows = VSV_STATIC_MAX_ROWS;
constexpr size_t kStaticBytes = vsv::ws_bytes(0, kStaticRows, 0);

static __device__ __align__(256) unsigned char scratch[kStaticBytes];

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
void* g_ptr[kMaxDevices];
hipError_t g_err[kMaxDevices];

// Device address of this device's array, zero-filled on `stream` the first
// time; nullptr if the lookup or the fill failed.
void* device_scratch(int dev, hipStream_t stream) {
  std::call_once(g_once[dev], [&]() {
    void* p = nullptr;
    hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e == hipSuccess && p == nullptr) e = hipErrorInvalidSymbol;
    if (e == hipSuccess) e = vsv::launch_zero(p, kStaticBytes, stream);
    g_err[dev] = e;
    g_ptr[dev] = e == hipSuccess ? p : nullptr;
  });
  return g_ptr[dev];
}

}  // namespace

extern "C" {

vsv_status vsv_verify_greedy_static(const vsv_batch* batch, int32_t relaxed_topk, const vsv_outputs* out,
                                    hipStream_t stream) {
  if (!batch) return VSV_EINVAL;
  if (batch->num_rows > kStaticRows || batch->num_rows < 0) return VSV_ELIMIT;
  if (vsv::ws_bytes(batch->num_requests, batch->num_rows, 0) > kStaticBytes) return VSV_ELIMIT;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return VSV_EHIP;
  void* ws = device_scratch(dev, stream);
  if (!ws) return VSV_EHIP;
  return vsv_verify_greedy(batch, relaxed_topk, out, ws, kStaticBytes, stream);
}

}  // extern "C"
