// host.hip -- host-side helpers shared by the launchers: the current device and
// set-up that must run once per device (kernel attributes), thread-safe.
#include <mutex>

#include "kernels.h"

namespace w4a16 {

namespace {

std::mutex g_once_mu;
hipError_t g_once_status[kOnceSlots][kMaxDevices];
bool g_once_done[kOnceSlots][kMaxDevices];

} // namespace

hipError_t current_device(int *dev)
{
    const hipError_t e = hipGetDevice(dev);
    if (e != hipSuccess)
        return e;
    return (*dev >= 0 && *dev < kMaxDevices) ? hipSuccess : hipErrorInvalidDevice;
}

hipError_t once_per_device(int slot, hipError_t (*init)(int dev))
{
    int dev = 0;
    const hipError_t e = current_device(&dev);
    if (e != hipSuccess)
        return e;
    std::lock_guard<std::mutex> lock(g_once_mu);
    if (!g_once_done[slot][dev]) {
        g_once_status[slot][dev] = init(dev);
        g_once_done[slot][dev] = true;
    }
    return g_once_status[slot][dev];
}

} // namespace w4a16
