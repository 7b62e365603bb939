// Host side of the persistent launches: how many workgroups the GPU holds at
// once (hand-offs between workgroups of one launch need every workgroup
// resident).
#include <mutex>

#include "handoff.hpp"

namespace w4 {

int resident_per_cu(const void* kern, int threads, size_t lds, int dev) {
    struct Entry {
        const void* kern;
        int threads;
        size_t lds;
        int dev, n;
    };
    static std::mutex mu;
    static Entry cache[64];
    static int used = 0;
    std::lock_guard<std::mutex> lock(mu);
    for (int i = 0; i < used; ++i)
        if (cache[i].kern == kern && cache[i].threads == threads && cache[i].lds == lds &&
            cache[i].dev == dev)
            return cache[i].n;
    hipFuncAttributes attr{};
    int n = 0;
    if (hipFuncGetAttributes(&attr, kern) != hipSuccess || attr.localSizeBytes > 0) n = 0;
    else if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kern, threads, lds) != hipSuccess) n = 0;
    if (used < 64) cache[used++] = Entry{kern, threads, lds, dev, n};
    return n;
}

int persistent_grid(const void* kern, int threads, size_t lds, int items, hipError_t* err) {
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) {
        *err = e;
        return 0;
    }
    const int per_cu = resident_per_cu(kern, threads, lds, dev);
    if (per_cu < 1 || cus < 1) {
        *err = hipErrorNotSupported;
        return 0;
    }
    *err = hipSuccess;
    return items < per_cu * cus ? items : per_cu * cus;
}

}  // namespace w4
