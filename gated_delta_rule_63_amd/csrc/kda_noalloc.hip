// kda_noalloc.hip -- kda_fwd for callers that cannot allocate device memory.
//
// kda_fwd needs a workspace only on its slice routes for few long chains. When
// the caller passes none, it takes the three-slice route and allocates that
// route's four fp32 states per sequence and head on the stream.
// kda_fwd_noalloc instead points the workspace at `scratch`, a static device
// array of fixed size, and never calls an allocator: kda_fwd then takes the
// one-pass slice route when its workspace fits there, else the three-slice route.
#include "../../include/kda.h"
#include "kda_launch.h"

#include <hip/hip_runtime.h>

#include <mutex>

namespace {

// 8 MiB: the three-slice workspace of 32 (sequence, head) chains, e.g. one
// sequence of 32 heads (the long-context workload T = 131072, H = 32), or the
// one-pass workspace of short enough ones (T = 12288, H = 1, three slices:
// 4.4 MiB).
constexpr size_t kScratchBytes = size_t(8) << 20;

// Each GPU the library runs on holds its own copy until the process ends.
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
struct DeviceScratch {
    std::once_flag once;
    void* ptr = nullptr;   // device address of this device's copy of `scratch`
};
DeviceScratch g_scratch[kMaxDevices];

// Address of the current device's copy, looked up once per device. Host code
// never passes `scratch` itself to a kernel or a copy: in host code that name
// is a stand-in, not a device address.
void* scratch_address(int dev) {
    if (dev < 0 || dev >= kMaxDevices) return nullptr;
    DeviceScratch& d = g_scratch[dev];
    std::call_once(d.once, [&d] {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) == hipSuccess) d.ptr = p;
        else (void)hipGetLastError();
    });
    return d.ptr;
}

}  // namespace

extern "C" {

size_t kda_fwd_noalloc_max_workspace(void) { return kScratchBytes; }

kda_status_t kda_fwd_noalloc(const void* q, const void* k, const void* v, const float* g,
                             const float* beta, const int32_t* cu_seqlens, const float* h0, void* o,
                             float* hT, const kda_desc_t* desc, void* stream) {
    if (!desc) return KDA_ERR_NULL;
    // 0 for an invalid descriptor too: kda_fwd then reports the argument error.
    // Variable-length batches never take the slice route.
    const size_t need = cu_seqlens ? 0 : kda::fwd_workspace_bytes(desc, true);
    if (need > kScratchBytes) return KDA_ERR_WORKSPACE;
    kda_desc_t d = *desc;
    d.workspace = nullptr;
    d.workspace_bytes = 0;
    if (need > 0) {
        int dev = -1;
        if (hipGetDevice(&dev) != hipSuccess) return KDA_ERR_HIP;
        void* p = scratch_address(dev);
        if (!p) return KDA_ERR_HIP;
        d.workspace = p;
        d.workspace_bytes = kScratchBytes;
    }
    // with a large enough workspace kda_fwd allocates nothing; the slice route
    // writes every workspace state before it reads it, so nothing is cleared
    return kda_fwd(q, k, v, g, beta, cu_seqlens, h0, o, hT, &d, stream);
}

}  // extern "C"
