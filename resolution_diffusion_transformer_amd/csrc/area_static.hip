// area_window_plan_static: the Phase II window plan with the library's own
// device scratch instead of a caller workspace, for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops).
//
// The scratch is one file-scope device array per GPU, resolved once per
// device with hipGetSymbolAddress; the array's name is a host-side stand-in
// and is never passed to a kernel.  Every call on a GPU shares that GPU's
// array: calls that overlap on one GPU (different streams without ordering)
// race.  No region of the plan's scratch needs to start at zero (each kernel
// writes every word it later reads), so nothing is cleared.
#include <hip/hip_runtime.h>

#include <mutex>
#include <string>

#include "area_internal.h"

namespace {

constexpr size_t kScratchBytes = (size_t)16 << 20;  // 16 MiB per GPU, held until the process ends
__device__ __attribute__((aligned(256))) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
void* g_ptr[kMaxDevices];
hipError_t g_status[kMaxDevices];

}  // namespace

extern "C" int area_window_plan_static(const area_problem* p, int step, const int32_t* energy_q, const void* k,
                                       int32_t* plan, int32_t* wsum, int32_t* bridge_idx, void* stream) {
  int rc = area_validate(p);
  if (rc) return rc;
  const size_t need = area_workspace_bytes(p, AREA_OP_PLAN);
  if (need > kScratchBytes)
    return area::fail(AREA_E_WORKSPACE, "the plan needs " + std::to_string(need) +
                                             " bytes of scratch; the static scratch holds " +
                                             std::to_string(kScratchBytes) + " (use area_window_plan)");
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return area::fail(AREA_E_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return area::fail(AREA_E_UNSUPPORTED, "device index above 63");
  std::call_once(g_once[dev], [dev] {
    void* ptr = nullptr;
    g_status[dev] = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    g_ptr[dev] = ptr;
  });
  if (g_status[dev] != hipSuccess || !g_ptr[dev])
    return area::fail(AREA_E_HIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(g_status[dev]));
  return area_window_plan(p, step, energy_q, k, plan, wsum, bridge_idx, g_ptr[dev], kScratchBytes, stream);
}
