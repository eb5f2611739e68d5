// noalloc.hip -- dsa_forward without a caller workspace, for callers that
// cannot allocate device memory (code under HIP graph capture, serving loops
// that forbid allocation).  The workspace is a file-scope device array of
// kScratchBytes that every device holds from the library's first use on it
// until the process ends.  Its device address is taken once per device with
// hipGetSymbolAddress and kept; host code only ever passes that address on
// (the array's own name in host code is a host-side stand-in, not a device
// address).  The call enqueues the same kernels as dsa_forward, so the
// results are identical.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/libdsa.h"

namespace dsa {
// api.hip: record the thread's last error and return the status
dsa_status report_error(dsa_status s, const char* fmt, ...);
}  // namespace dsa

namespace {
constexpr size_t kScratchBytes = size_t(128) << 20;  // 128 MiB per device
constexpr int kMaxDevices = 64;
}  // namespace

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {
void* g_scratch[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];
std::once_flag g_scratch_once[kMaxDevices];
}  // namespace

extern "C" dsa_status dsa_forward_noalloc(const dsa_forward_params* p, dsa_stream_t stream) {
  size_t need = 0;
  // argument checks and the workspace plan of dsa_forward (host only)
  if (dsa_status s = dsa_forward_workspace_size(p, &need)) return s;
  if (need > kScratchBytes)
    return dsa::report_error(DSA_ERR_WORKSPACE,
                             "dsa_forward_noalloc: this batch needs %zu bytes of workspace, the static scratch "
                             "holds %zu (use dsa_forward with a caller workspace)",
                             need, kScratchBytes);
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return dsa::report_error(DSA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return dsa::report_error(DSA_ERR_UNSUPPORTED, "device ordinal %d out of range", dev);
  // once per device, with that device current: the device address of its copy
  std::call_once(g_scratch_once[dev], [dev] {
    void* ptr = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    g_scratch[dev] = g_scratch_err[dev] == hipSuccess ? ptr : nullptr;
  });
  if (g_scratch_err[dev] != hipSuccess || !g_scratch[dev])
    return dsa::report_error(DSA_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                             hipGetErrorString(g_scratch_err[dev]));
  return dsa_forward(p, g_scratch[dev], kScratchBytes, stream);
}
