// ve_muon_static.hip -- Muon's Newton-Schulz iteration for callers that
// cannot allocate device memory (code under HIP graph capture, tight
// serving loops, harnesses that forbid hipMalloc): the same launch sequence
// as ve_muon_newton_schulz, with its workspace in a file-scope device array
// instead of a caller buffer.
//
// The array is `scratch`, kScratchBytes long; every GPU the library runs on
// holds its own copy until the process ends.  Its device address is looked
// up once per device (hipGetSymbolAddress, with that device current) and
// kept; host code never passes the array's name itself to a kernel or a
// copy.  Every call on a GPU shares that GPU's copy, so calls that overlap
// on one GPU (two streams, two threads) race; nothing in it has to start at
// zero (each kernel of the sequence writes what it later reads).

#include <hip/hip_runtime.h>

#include <mutex>

#include "ve.h"
#include "ve_internal.h"

// 200 MiB: the workspace of 2048 x 7168 (DeepSeek-V3's routed experts) or
// 3,400 x 3,400, split-product slices included.
static constexpr int64_t kScratchBytes = int64_t(200) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices];  // per device: the array's device address, once looked up

}  // namespace

extern "C" ve_status ve_muon_newton_schulz_noalloc(const uint16_t* G, uint16_t* out, int64_t rows, int64_t cols,
                                                   int32_t steps, float eps, void* stream) {
    int64_t need = 0;
    ve_status st = ve_muon_workspace_bytes(rows, cols, &need);
    if (st != VE_OK) return st;
    if (need > kScratchBytes)
        return ve::fail(VE_ERR_UNSUPPORTED,
                        "%lld x %lld needs %lld bytes of workspace; the static scratch holds %lld "
                        "(use ve_muon_newton_schulz with a workspace)",
                        (long long)rows, (long long)cols, (long long)need, (long long)kScratchBytes);
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return ve::fail(VE_ERR_DEVICE, "no current device (or device %d beyond %d)", dev, kMaxDevices);
    void* ptr = nullptr;
    {
        std::lock_guard<std::mutex> lock(g_mu);
        ptr = g_scratch[dev];
        if (!ptr) {
            const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
            if (e != hipSuccess || !ptr)
                return ve::fail(VE_ERR_DEVICE, "device %d: address of the static scratch: %s", dev,
                                hipGetErrorString(e));
            g_scratch[dev] = ptr;
        }
    }
    return ve_muon_newton_schulz(G, out, rows, cols, steps, eps, ptr, kScratchBytes, stream);
}
