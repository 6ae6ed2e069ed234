// chunk_dr_fwd_noalloc: the forward with its workspace in a static device array, for callers
// that cannot allocate device memory (code under graph capture, serving loops, harnesses that
// forbid allocation).  Declared in chunk_dr.h.
//
// The array lives in this file's device code object.  Its device address is looked up once per
// device, with that device current, on the first call there (hipGetSymbolAddress); the address
// is what the kernels receive, exactly as they receive a caller's workspace.  Host code never
// passes the array's own name anywhere: on the host it names a stand-in, not device memory.
#include <atomic>
#include <mutex>

#include "chunk_dr.h"
#include "cdr_common.h"

namespace {

// the workspace: CDR_NOALLOC_SCRATCH_BYTES per device that runs the entry point, held until the
// process ends
__device__ __align__(256) unsigned char scratch[CDR_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// device address of `scratch` on the current device (nullptr on failure)
void* scratch_address(int dev) {
    void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p != nullptr) return p;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
        void* addr = nullptr;
        if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess || addr == nullptr) return nullptr;
        g_scratch_ptr[dev].store(addr, std::memory_order_release);
        p = addr;
    }
    return p;
}

}  // namespace

extern "C" cdr_status chunk_dr_fwd_noalloc(const cdr_problem* p, const void* q, const void* k, const void* v,
                                           const float* g, const float* beta, const float* initial_state,
                                           const int32_t* cu_seqlens, void* o, float* final_state,
                                           void* stream) {
    const cdr_status st = cdr_check(p);
    if (st != CDR_OK) return st;
    if (cdr_workspace_bytes(p) > (size_t)CDR_NOALLOC_SCRATCH_BYTES) return CDR_ERR_SCRATCH_LIMIT;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return CDR_ERR_HIP;
    void* ws = scratch_address(dev);
    if (ws == nullptr) return CDR_ERR_HIP;
    return chunk_dr_fwd(p, q, k, v, g, beta, initial_state, cu_seqlens, o, final_state, ws,
                        (size_t)CDR_NOALLOC_SCRATCH_BYTES, stream);
}
