// static_ws.hip -- zero1_mta_step_static: the whole step with its workspace in
// a static device array of the library, for callers that cannot allocate
// (code under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc).  It runs the same kernels as zero1_mta_step, which it calls with
// this array as the workspace.
//
// The array (`scratch`) holds the norm info, the per-workgroup fp64 partials
// and the fp32 g of the store-g design for shards of up to
// ZERO1_STATIC_MAX_G_ELEMS elements: 64 MiB + 64.25 KiB, held on every GPU the
// library runs on until the process ends.  In host code `scratch` is only a
// host-side stand-in for the symbol: the device address of each GPU's copy
// comes from hipGetSymbolAddress, taken once per device (on the entry point's
// first call with that device current) and kept; only that address is ever
// passed to the kernels.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

#include "../../include/zero1.h"
#include "internal.h"

namespace {

constexpr size_t kStaticBytes = z1::kGOffset + (size_t)ZERO1_STATIC_MAX_G_ELEMS * sizeof(float);
static_assert(kStaticBytes % 256 == 0, "scratch size");
constexpr int kMaxDevices = 64;

}  // namespace

static __device__ __align__(256) unsigned char scratch[kStaticBytes];

namespace {

std::mutex g_mu;
void* g_scratch[kMaxDevices];   // device address of `scratch` on each device, once looked up

// The device address of the current device's copy of `scratch`.
zero1_status scratch_address(void** out)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    char msg[256];
    if (e != hipSuccess) {
        std::snprintf(msg, sizeof msg, "hipGetDevice failed: %s", hipGetErrorString(e));
        return (zero1_status)z1::set_error(ZERO1_EHIP, msg);
    }
    if (dev < 0 || dev >= kMaxDevices) {
        std::snprintf(msg, sizeof msg, "device index %d out of range", dev);
        return (zero1_status)z1::set_error(ZERO1_ENOTSUPPORTED, msg);
    }
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            std::snprintf(msg, sizeof msg, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev,
                          hipGetErrorString(e));
            return (zero1_status)z1::set_error(ZERO1_EHIP, msg);
        }
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return ZERO1_OK;
}

}  // namespace

extern "C" zero1_status zero1_mta_step_static(const uint16_t* const* grads, int W, int64_t begin,
                                              const zero1_plan* plan, const zero1_hparams* hp,
                                              double* rank_sumsq, int n_ranks, int my_rank, uint32_t flags,
                                              zero1_norm_info* info_out, void* stream)
{
    // the size limit first, before any device call: a store-g step needs
    // 4 bytes of g per shard element
    if (plan && !((flags & ZERO1_STORE_G) && (flags & ZERO1_RECOMPUTE_G))) {
        const size_t need = zero1_mta_workspace_bytes(plan, W, flags);
        if (need > kStaticBytes) {
            char msg[320];
            std::snprintf(msg, sizeof msg,
                          "zero1_mta_step_static: the store-g step of a %lld-element shard needs %zu bytes of "
                          "workspace; the static scratch holds %zu (shards of up to %d elements): pass "
                          "ZERO1_RECOMPUTE_G or call zero1_mta_step with a workspace",
                          (long long)plan->shard_len, need, kStaticBytes, (int)ZERO1_STATIC_MAX_G_ELEMS);
            return (zero1_status)z1::set_error(ZERO1_EINVAL, msg);
        }
    }
    void* ws = nullptr;
    if (zero1_status st = scratch_address(&ws)) return st;
    return zero1_mta_step(grads, W, begin, plan, hp, rank_sumsq, n_ranks, my_rank, flags, info_out, ws,
                          kStaticBytes, stream);
}
