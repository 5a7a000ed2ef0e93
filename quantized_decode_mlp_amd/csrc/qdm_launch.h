// Host-side launch helpers shared by the kernel files.
#pragma once

#include <hip/hip_runtime.h>

#include <map>
#include <mutex>
#include <tuple>

namespace qdm {

inline int gshift_of(int group) { return group == 32 ? 5 : group == 64 ? 6 : group == 128 ? 7 : 0; }

// Resident blocks of a kernel on the current device (queried once per
// (device, kernel, dynamic LDS) and kept).
template <typename K>
inline int resident_blocks(K kernel, int threads, size_t lds) {
    static std::mutex mu;
    static std::map<std::tuple<int, const void*, size_t>, int> cache;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return -1;
    const auto key = std::make_tuple(dev, reinterpret_cast<const void*>(kernel), lds);
    {
        std::lock_guard<std::mutex> lk(mu);
        auto it = cache.find(key);
        if (it != cache.end()) return it->second;
    }
    int per_cu = 0, cus = 0;
    if (lds > 65536 &&
        hipFuncSetAttribute(reinterpret_cast<const void*>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                            static_cast<int>(lds)) != hipSuccess)
        return -1;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, lds) != hipSuccess) return -1;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return -1;
    const int n = (per_cu > 0 ? per_cu : 0) * (cus > 0 ? cus : 1);
    std::lock_guard<std::mutex> lk(mu);
    cache[key] = n;
    return n;
}


}  // namespace qdm
