// Library-wide entry points: status text, version, device check.
#include <string.h>

#include "common.h"

namespace moe {

namespace {
constexpr int kMaxDevices = 64;
// 0 = not checked yet, >0 = CU count of a gfx950 device, <0 = moe_status.
int g_dev_state[kMaxDevices];
}  // namespace

int device_cus() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
    int s = __atomic_load_n(&g_dev_state[dev], __ATOMIC_ACQUIRE);
    if (s != 0) return s;
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return MOE_ERR_HIP;
    if (strncmp(prop.gcnArchName, "gfx950", 6) != 0) {
        s = MOE_ERR_UNSUPPORTED;
    } else {
        s = prop.multiProcessorCount > 0 ? prop.multiProcessorCount : 256;
    }
    __atomic_store_n(&g_dev_state[dev], s, __ATOMIC_RELEASE);
    return s;
}

}  // namespace moe

extern "C" {

const char* moe_status_string(moe_status s) {
    switch (s) {
        case MOE_OK: return "ok";
        case MOE_ERR_INVALID_ARG: return "invalid argument";
        case MOE_ERR_UNSUPPORTED: return "unsupported device or mode (gfx950 only)";
        case MOE_ERR_WORKSPACE: return "workspace too small";
        case MOE_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

int moe_abi_version(void) { return 1; }

moe_status moe_init(int device) {
    int cur = 0;
    if (hipGetDevice(&cur) != hipSuccess) return MOE_ERR_HIP;
    if (device != cur && hipSetDevice(device) != hipSuccess) return MOE_ERR_HIP;
    int r = moe::device_cus();
    if (device != cur) (void)hipSetDevice(cur);
    return r < 0 ? (moe_status)r : MOE_OK;
}

}  // extern "C"
