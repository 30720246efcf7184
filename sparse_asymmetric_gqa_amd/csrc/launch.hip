// Host-side launch caches shared by the kernels' launchers: the device's
// compute-unit count, resident workgroups per CU of a kernel at a given block
// and LDS size, and the one-time opt-in to more than 64 KiB of dynamic LDS.
// Every cache is keyed by the calling thread's current device and guarded by
// a mutex, so concurrent host threads and several GPUs may use the library
// at once. The queries themselves allocate nothing.
#include "saga_internal.h"

#include <mutex>
#include <tuple>
#include <vector>

namespace saga {
namespace {

std::mutex g_mu;
struct Occ {
    int dev;
    const void* kern;
    int threads;
    size_t lds;
    int blocks;
};
std::vector<Occ> g_occ;
struct LdsOk {
    int dev;
    const void* kern;
    size_t lds;
};
std::vector<LdsOk> g_lds_ok;
int g_cus[kMaxDevices] = {0};

int current_device() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return -1;
    return dev;
}

}  // namespace

int cu_count() {
    const int dev = current_device();
    if (dev < 0) return 256;
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_cus[dev]) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            n <= 0)
            n = 256;
        g_cus[dev] = n;
    }
    return g_cus[dev];
}

int blocks_per_cu(const void* kern, int threads, size_t lds) {
    const int dev = current_device();
    std::lock_guard<std::mutex> lk(g_mu);
    for (const Occ& o : g_occ)
        if (o.dev == dev && o.kern == kern && o.threads == threads && o.lds == lds) return o.blocks;
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, threads, lds) != hipSuccess ||
        per_cu <= 0)
        per_cu = 1;
    g_occ.push_back(Occ{dev, kern, threads, lds, per_cu});
    return per_cu;
}

hipError_t allow_dynamic_lds(const void* kern, size_t lds) {
    const int dev = current_device();
    std::lock_guard<std::mutex> lk(g_mu);
    LdsOk* have = nullptr;
    for (LdsOk& p : g_lds_ok)
        if (p.dev == dev && p.kern == kern) have = &p;
    if (have && have->lds >= lds) return hipSuccess;
    // the largest LDS a workgroup of this kernel may request on this device
    const hipError_t e =
        hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    if (have) have->lds = lds;
    else g_lds_ok.push_back(LdsOk{dev, kern, lds});
    return hipSuccess;
}

}  // namespace saga
