// Host-side facts about the current HIP device, queried once per device.
//
// The library keeps no other state between calls.  Each cache below is an
// array of atomics indexed by device ordinal: the first call on a device
// queries the runtime and publishes the answer; concurrent first calls on one
// device compute the same value, so the race is benign, and no call ever
// reads another device's entry.
#pragma once

#include <hip/hip_runtime.h>

#include <atomic>

namespace moe {

constexpr int kMaxDevices = 64;

// Ordinal of the calling thread's current device (0 if the query fails).
inline int current_device() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
    return dev;
}

// Positive int cached per device: slot[dev] holds 0 until the first call on
// dev stores compute() (clamped to at least 1).  Devices past kMaxDevices
// are queried on every call.
template <typename F>
inline int per_device_int(std::atomic<int> (&slot)[kMaxDevices], F&& compute) {
    const int dev = current_device();
    if (dev >= kMaxDevices) {
        const int v = compute();
        return v < 1 ? 1 : v;
    }
    int v = slot[dev].load(std::memory_order_acquire);
    if (v > 0) return v;
    v = compute();
    if (v < 1) v = 1;
    slot[dev].store(v, std::memory_order_release);
    return v;
}

// Compute units of the current device (256 on an MI355X).
inline int cu_count() {
    static std::atomic<int> slot[kMaxDevices];
    return per_device_int(slot, [] {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, current_device()) != hipSuccess ||
            n < 1)
            n = 256;
        return n;
    });
}

}  // namespace moe
