// The allocation-free MuonH step: muonh_step_noalloc runs the step of
// muonh_step (same plan, same kernels, same launch order) for callers that
// cannot allocate device memory, with every buffer the step needs beyond the
// caller's W, G and M inside one statically sized device array of this
// library, `scratch`.
//
// The array is a file-scope __device__ variable, so each GPU the library runs
// on holds its own copy, at its own address, until the process ends.  Host
// code never passes the array's name to a kernel or a copy (on the host it is
// only a stand-in symbol): the first call on a device looks up that device's
// address with hipGetSymbolAddress, with the device current, and every later
// call on the device uses that address.  Calls share the array and it keeps
// the last call's contents; each call uploads its own tables and clears the
// Newton-Schulz buffers, so only calls that overlap in time on one GPU (on
// different streams, or from different threads) race.

#include <hip/hip_runtime.h>

#include <cstring>
#include <mutex>
#include <string>

#include "internal.h"

namespace muonh {
namespace {

// 64 MiB (MUONH_NOALLOC_MAX_WORKSPACE): a single 2048 x 2048 matrix, four
// 1024 x 1024 or dozens of 256-wide ones with bf16 Newton-Schulz
// (muonh_workspace_size gives a plan's need).
constexpr size_t kScratchBytes = MUONH_NOALLOC_MAX_WORKSPACE;
static_assert(kScratchBytes % 256 == 0, "the workspace layout is 256-byte aligned");

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;

struct DeviceSlot {
  bool ready = false;
  uint8_t* ptr = nullptr;          // this device's address of `scratch`
  InWorkspaceHost host;            // upload staging of this device
};

std::mutex g_setup_mu;
DeviceSlot g_slots[kMaxDevices];

// Per-device set-up, once: the array's device address and the upload event.
int device_slot(int dev, DeviceSlot** out) {
  if (dev < 0 || dev >= kMaxDevices)
    return set_last_error(MUONH_ENODEV, "device index beyond the allocation-free step's table");
  std::lock_guard<std::mutex> lock(g_setup_mu);
  DeviceSlot& s = g_slots[dev];
  if (!s.ready) {
    hipDeviceProp_t prop;
    hipError_t e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess)
      return set_last_error(MUONH_EHIP, (std::string("hipGetDeviceProperties: ") + hipGetErrorString(e)).c_str());
    if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
      return set_last_error(MUONH_ENODEV, (std::string("device is ") + prop.gcnArchName +
                                           ", library is built for gfx950").c_str());
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return set_last_error(MUONH_EHIP, (std::string("hipGetSymbolAddress(scratch): ") +
                                         hipGetErrorString(e)).c_str());
    e = hipEventCreateWithFlags(&s.host.uploaded, hipEventDisableTiming);
    if (e != hipSuccess)
      return set_last_error(MUONH_EHIP, (std::string("hipEventCreate: ") + hipGetErrorString(e)).c_str());
    s.ptr = reinterpret_cast<uint8_t*>(p);
    s.ready = true;
  }
  *out = &s;
  return MUONH_OK;
}

}  // namespace
}  // namespace muonh

extern "C" int muonh_step_noalloc(const muonh_matrix_desc* mats, int32_t n, const muonh_options* opt,
                                  const muonh_step_args* args, void* stream) {
  using namespace muonh;
  if (!opt || !args || !mats) return set_last_error(MUONH_EINVAL, "null argument");
  // Host-only checks first: nothing touches a device for a call that cannot run.
  if (opt->workspace)
    return set_last_error(MUONH_EINVAL, "options.workspace must be NULL: this step uses the library's static buffer");
  for (int32_t i = 0; i < n; ++i)
    if (!(mats[i].radius > 0.0f))
      return set_last_error(MUONH_EINVAL, (std::string("matrix ") + std::to_string(i) +
                                           ": the allocation-free step needs the radius R (> 0)").c_str());
  size_t need = 0;
  int rc = muonh_workspace_size(mats, n, opt, &need);
  if (rc) return rc;
  if (need > kScratchBytes)
    return set_last_error(MUONH_ENOMEM, (std::string("the plan needs ") + std::to_string(need) +
                                         " bytes of workspace; the allocation-free step's static "
                                         "buffer holds " + std::to_string(kScratchBytes) + " per device")
                                            .c_str());
  int dev = 0;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess)
    return set_last_error(MUONH_EHIP, (std::string("hipGetDevice: ") + hipGetErrorString(e)).c_str());
  DeviceSlot* slot = nullptr;
  if ((rc = device_slot(dev, &slot))) return rc;
  return run_step_in_workspace(mats, n, *opt, *args, reinterpret_cast<hipStream_t>(stream), slot->ptr,
                               kScratchBytes, slot->host);
}
