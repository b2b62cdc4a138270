// Host-side runtime pieces shared by every entry point: status strings, the
// per-thread last-HIP-error slot and the once-per-device gfx950 check.
#include <atomic>
#include <cstring>

#include "common.hpp"

namespace {
thread_local int32_t t_last_hip_error = 0;
constexpr int kMaxDevices = 64;
// 0 = unknown, 1 = gfx950, 2 = other architecture; cu count cached beside it.
std::atomic<int> g_arch_state[kMaxDevices];
std::atomic<int> g_cu_count[kMaxDevices];
}  // namespace

namespace nvfp4host {

void set_hip_error(hipError_t e) { t_last_hip_error = (int32_t)e; }

nvfp4_status check_device() {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    set_hip_error(e);
    return NVFP4_EHIP;
  }
  if (dev < 0 || dev >= kMaxDevices) return NVFP4_ENOTSUP;
  int st = g_arch_state[dev].load(std::memory_order_acquire);
  if (st == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) {
      set_hip_error(e);
      return NVFP4_EHIP;
    }
    st = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_cu_count[dev].store(prop.multiProcessorCount, std::memory_order_relaxed);
    g_arch_state[dev].store(st, std::memory_order_release);
  }
  return st == 1 ? NVFP4_OK : NVFP4_ENOTSUP;
}

int num_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  const int n = g_cu_count[dev].load(std::memory_order_relaxed);
  return n > 0 ? n : 256;
}

}  // namespace nvfp4host

extern "C" {

int32_t nvfp4_abi_version(void) { return NVFP4_ABI_VERSION; }

const char* nvfp4_status_string(nvfp4_status status) {
  switch (status) {
    case NVFP4_OK: return "NVFP4_OK";
    case NVFP4_EINVAL: return "NVFP4_EINVAL: invalid argument";
    case NVFP4_EALIGN: return "NVFP4_EALIGN: tensor pointer not 16-byte aligned";
    case NVFP4_EWORKSPACE: return "NVFP4_EWORKSPACE: workspace missing or too small";
    case NVFP4_ENOTSUP: return "NVFP4_ENOTSUP: unsupported device or flag";
    case NVFP4_EHIP: return "NVFP4_EHIP: HIP runtime error";
    case NVFP4_ETIMEOUT: return "NVFP4_ETIMEOUT: a bounded cross-workgroup wait gave up";
    default: return "NVFP4: unknown status";
  }
}

int32_t nvfp4_last_hip_error(void) { return t_last_hip_error; }

}  // extern "C"
