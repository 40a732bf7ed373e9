// Static device scratch for jpa_forward_scratch, the attention entry point
// that allocates nothing and takes no workspace.  The partial results of work
// items cut between key ranges (fp32 O and log2 LSE per piece, the same
// layout a jpa_forward_ws workspace holds) go to this array instead of a
// caller buffer.  Every device the library runs on holds its own copy from
// the time the library's code is loaded there until the process ends.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "jpa.h"
#include "jpa_params.h"
#include "jpa_scratch.h"

// Partial outputs [2 * JPA_SCRATCH_MAX_WGS][JPA_BLOCK_M][128] fp32, then the
// partial LSE [2 * JPA_SCRATCH_MAX_WGS][JPA_BLOCK_M] fp32: the workspace of
// JPA_SCRATCH_MAX_WGS key ranges at head_dim 128 (64.5 MiB).
static constexpr size_t kScratchBytes =
    (size_t)2 * JPA_SCRATCH_MAX_WGS * JPA_BLOCK_M * 128 * sizeof(float) +
    (size_t)2 * JPA_SCRATCH_MAX_WGS * JPA_BLOCK_M * sizeof(float);

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

size_t jpa_scratch_bytes() { return kScratchBytes; }

// Device address of the current device's scratch.  In host code `scratch`
// names a host-side stand-in, never device memory, so its address is looked
// up with hipGetSymbolAddress once per device (with that device current) and
// kept; kernels get that address as an argument.
int jpa_scratch_address(void** ptr) {
    constexpr int kMaxDevices = 64;
    static std::atomic<void*> addr[kMaxDevices];
    static std::mutex mu;
    *ptr = nullptr;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return (int)e;
    if (dev < 0 || dev >= kMaxDevices) return (int)hipErrorInvalidDevice;
    void* p = addr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(mu);
        p = addr[dev].load(std::memory_order_relaxed);
        if (!p) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess || !p) return e != hipSuccess ? (int)e : (int)hipErrorInvalidSymbol;
            addr[dev].store(p, std::memory_order_release);
        }
    }
    *ptr = p;
    return (int)hipSuccess;
}
