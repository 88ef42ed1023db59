// kdt_tree_verify_attn_noalloc: the verify attention with its workspace in a static device
// array instead of a caller-supplied buffer, for callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
//
// The array lives in this file, `scratch`, kScratchBytes bytes on every device the library
// runs on, held until the process ends.  Host code never uses the array's name as an address
// (on the host it is only a stand-in for the symbol): the device address is looked up once per
// device with hipGetSymbolAddress, with that device current, and kept in g_scratch[device].
// Every call on a device shares that device's array, so calls that overlap on one device (two
// streams, two threads) race; nothing in the array has to start at zero (the plan rewrites
// every field the attention reads before it reads it).
#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

#include "kdt_internal.h"
#include "kdt_noalloc.h"

namespace {

constexpr size_t kScratchBytes = KDT_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void *g_scratch[kMaxDevices];

// Device address of this device's scratch array (looked up on the first call per device).
int scratch_of_current_device(void **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return kdt::set_error(KDT_ERR_HIP, "hipGetDevice failed");
    if (dev < 0 || dev >= kMaxDevices) return kdt::set_error(KDT_ERR_HIP, "device id out of range");
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            char msg[160];
            snprintf(msg, sizeof(msg), "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
            return kdt::set_error(KDT_ERR_HIP, msg);
        }
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return KDT_OK;
}

}  // namespace

extern "C" {

int kdt_tree_verify_attn_noalloc(const void *q_lat, const void *q_rope, const void *ckv_cache,
                                 const void *krope_cache, const void *tree_ckv, const void *tree_krope,
                                 const uint64_t *bitmask, const int32_t *cache_lens, float scale, float *out,
                                 const kdt_verify_desc *desc, int32_t *dev_status, void *stream) {
    const size_t need = kdt_tree_verify_workspace_size(desc);
    if (need == 0) return kdt_last_status();             // invalid desc: the error is already set
    if (need > kScratchBytes) {
        char msg[200];
        snprintf(msg, sizeof(msg),
                 "this batch needs %zu bytes of workspace; the static scratch array holds %zu (use "
                 "kdt_tree_verify_attn with a workspace of that size)",
                 need, kScratchBytes);
        return kdt::set_error(KDT_ERR_WORKSPACE, msg);
    }
    void *ws = nullptr;
    const int rc = scratch_of_current_device(&ws);
    if (rc != KDT_OK) return rc;
    return kdt_tree_verify_attn(q_lat, q_rope, ckv_cache, krope_cache, tree_ckv, tree_krope, bitmask, cache_lens,
                                scale, out, desc, ws, kScratchBytes, dev_status, stream);
}

}  // extern "C"
