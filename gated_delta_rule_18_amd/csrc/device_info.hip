// Per-device facts the launch plans need: compute units and XCDs, asked of the device.
#include <atomic>

#include "kla_launch.h"

namespace kla {

namespace {

constexpr int kMaxDevices = 64;
// One entry per device ordinal: 0 until queried, then (cus << 8) | xcds.
std::atomic<uint32_t> g_info[kMaxDevices];

}  // namespace

DeviceInfo device_info() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return DeviceInfo{256, 8};
  const uint32_t c = g_info[dev].load(std::memory_order_relaxed);
  if (c) return DeviceInfo{(int)(c >> 8), (int)(c & 0xff)};
  int cus = 0, xcds = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
  // gfx950 has 32 compute units per XCD; a partition of the chip exposes whole XCDs.
  if (hipDeviceGetAttribute(&xcds, hipDeviceAttributeNumberOfXccs, dev) != hipSuccess || xcds <= 0)
    xcds = cus >= 32 ? cus / 32 : 1;
  if (xcds > 255) xcds = 255;
  g_info[dev].store(((uint32_t)cus << 8) | (uint32_t)xcds, std::memory_order_relaxed);
  return DeviceInfo{cus, xcds};
}

}  // namespace kla
