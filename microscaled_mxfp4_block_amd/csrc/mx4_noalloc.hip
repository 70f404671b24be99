// mx4_noalloc.hip -- mx_gemm_noalloc: mx_gemm for callers that cannot
// allocate (code under HIP graph capture, tight serving loops, harnesses that
// forbid hipMalloc).  The workspace mx_gemm takes from its caller (per-tile
// arrival counters, the pre-quantised activation, the split-K partials) is
// instead a file-scope device array of kScratchBytes per GPU, held by the
// process until it ends.
//
// The array's name is a host-side stand-in in host code, not a device
// address, so it is never passed to a kernel or a copy: once per device, with
// that device current, hipGetSymbolAddress gives the array's address on that
// device, which is kept per device and used from then on.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/mx4.h"
#include "mx4_internal.h"

namespace mx4 {

constexpr size_t kScratchBytes = (size_t)MX_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0 && kScratchBytes >= kCounterBytes, "scratch size");

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
void* g_scratch[kMaxDevices];   // this device's address of `scratch`, once set up
std::mutex g_setup;

// Zero the arrival counters at the start of the scratch array: a workspace's
// counters must be zero before its first use (every completed call leaves
// them zero).  A kernel, not hipMemsetAsync, so that a first call made under
// graph capture records a plain kernel node.
__global__ void __launch_bounds__(256) clear_counters_kernel(uint32_t* counters, int n) {
    const int i = (int)(blockIdx.x * 256u + threadIdx.x);
    if (i < n) counters[i] = 0u;
}

// This device's scratch address; on the first call for a device, looks it up
// and clears the counters on `stream`.  Returns nullptr if a HIP call fails.
void* device_scratch(hipStream_t stream) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_setup);
    if (g_scratch[dev]) return g_scratch[dev];
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return nullptr;
    const int n = (int)(kCounterBytes / 4);
    if (launch_kernel(clear_counters_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                      (uint32_t*)ptr, n) != hipSuccess)
        return nullptr;
    g_scratch[dev] = ptr;
    return ptr;
}

}  // namespace
}  // namespace mx4

extern "C" int mx_gemm_noalloc(const void* A_dev, int M, int K, int lda, const void* packed_dev, int N, void* C_dev,
                               int ldc, void* stream) {
    size_t need = 0;
    int rc = mx_gemm_workspace_bytes(M, N, K, &need);   // host only: validates the shape
    if (rc) return rc;
    if (need > mx4::kScratchBytes) return MX_ESPACE;
    void* ws = mx4::device_scratch((hipStream_t)stream);
    if (!ws) return MX_EHIP;
    return mx_gemm(A_dev, M, K, lda, packed_dev, N, C_dev, ldc, ws, mx4::kScratchBytes, stream);
}
