// lora_linear for callers that cannot allocate device memory (code under HIP
// graph capture, tight serving loops, harnesses that forbid hipMalloc): the
// same kernels, with the workspace taken from a file-scope device array
// instead of a caller buffer.
//
// `scratch` exists once per GPU the library runs on (each GPU holds its own
// copy, at its own address, until the process ends). In host code its name
// is only a stand-in for the device symbol, so the device address of the
// current GPU's copy is looked up with hipGetSymbolAddress on the first call
// on that GPU and kept; every launch gets that address. Nothing is allocated
// and nothing is freed here.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/lora.h"

namespace {

constexpr size_t kScratchBytes = LORA_NOALLOC_MAX_WORKSPACE;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// Device address of the current GPU's scratch array.
int scratch_address(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return LORA_EHIP;
    std::lock_guard<std::mutex> g(g_mu);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return LORA_EHIP;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return LORA_OK;
}

}  // namespace

extern "C" int lora_linear_noalloc(const lora_pool* pool, const void* x, const void* W, const int32_t* token_order,
                                   const int32_t* slot_indptr, const int32_t* work, const lora_plan_info* info,
                                   void* y, void* stream) {
    if (!pool || !info || info->T < 0) return LORA_EINVAL;
    if (lora_workspace_bytes(pool, info->T) > kScratchBytes) return LORA_ESPACE;
    void* ws = nullptr;
    const int rc = scratch_address(&ws);
    if (rc != LORA_OK) return rc;
    return lora_linear(pool, x, W, token_order, slot_indptr, work, info, y, ws, kScratchBytes, stream);
}
