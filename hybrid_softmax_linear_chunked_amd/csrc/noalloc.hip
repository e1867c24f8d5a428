// noalloc.hip -- rehyat_forward_parallel_noalloc: the chunk-parallel forward with its workspace in
// a static device array instead of a caller buffer, for callers that cannot allocate device
// memory (code under graph capture, tight serving loops, harnesses that forbid allocation).
//
// The array `scratch` is a module-global of this library: every GPU the library runs on holds
// its own copy (kScratchBytes each) until the process ends.  Host code never uses its name as
// an address: the device address of this GPU's copy is looked up once per device with that
// device current (hipGetSymbolAddress) and kept.  The call runs exactly the kernels of
// rehyat_forward_parallel on that memory.  Everything the kernels read from the workspace is
// written earlier in the same call (per-frame partials, state images), so the contents a
// previous call left do not matter.  Calls that overlap on one GPU (on different streams, or
// from different host threads) share the array and race; calls in stream order do not.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/rehyat.h"

namespace {

constexpr size_t kScratchBytes = size_t(64) << 20;  // 64 MiB per GPU
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

void* g_scratch[kMaxDevices] = {};
std::mutex g_scratch_lock;

// Device address of the current device's copy of `scratch`.
rehyat_status scratch_address(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return REHYAT_EHIP;
    std::lock_guard<std::mutex> guard(g_scratch_lock);
    if (!g_scratch[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return REHYAT_EHIP;
        g_scratch[dev] = ptr;
    }
    *out = g_scratch[dev];
    return REHYAT_OK;
}

}  // namespace

extern "C" rehyat_status rehyat_forward_parallel_noalloc(const rehyat_params* p, const void* q, const void* k,
                                                         const void* v, const void* wq, const void* wk,
                                                         const float* bq, const float* bk, void* out,
                                                         hipStream_t stream) {
    // parameter errors first (a zero size also stands for invalid parameters), then the size
    // limit, then the pointer checks and the launches of rehyat_forward_parallel
    const size_t need = rehyat_workspace_bytes(p);
    if (need == 0) return rehyat_forward_parallel(p, q, k, v, wq, wk, bq, bk, out, nullptr, 0, stream);
    if (need > kScratchBytes) return REHYAT_ESCRATCH;
    void* ws = nullptr;
    const rehyat_status st = scratch_address(&ws);
    if (st != REHYAT_OK) return st;
    return rehyat_forward_parallel(p, q, k, v, wq, wk, bq, bk, out, ws, kScratchBytes, stream);
}
