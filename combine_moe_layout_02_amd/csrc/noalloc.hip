// moe_dispatch_noalloc (include/moe.h): moe_dispatch_ws with the planned pack's record lists in a
// fixed device array of this library instead of a caller workspace, for callers that cannot
// allocate. The array's device address is looked up once per device with hipGetSymbolAddress and
// kept; host code never uses the array's own name as an address (in host code that name is a
// host-side stand-in, not device memory).

#include <mutex>

#include "moe_internal.h"

namespace moe {
namespace {

// The planned pack's record lists of the latest call on this GPU (every call overwrites all the
// records its pack kernel reads).
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;

struct ScratchAddress {
    std::once_flag once;
    void *ptr = nullptr;
    hipError_t err = hipSuccess;
};

ScratchAddress g_scratch[kMaxDevices];

// Device address of `scratch` on device `dev`, looked up once with that device current; nullptr
// (and *err set) on failure.
void *scratch_address(int dev, hipError_t *err) {
    if (dev < 0 || dev >= kMaxDevices) {
        *err = hipErrorInvalidDevice;
        return nullptr;
    }
    ScratchAddress &slot = g_scratch[dev];
    std::call_once(slot.once, [&slot, dev] {
        int cur = -1;
        slot.err = hipGetDevice(&cur);
        if (slot.err != hipSuccess) return;
        if (cur != dev && (slot.err = hipSetDevice(dev)) != hipSuccess) return;
        void *p = nullptr;
        slot.err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (slot.err == hipSuccess) slot.ptr = p;
        if (cur != dev) {
            const hipError_t back = hipSetDevice(cur);
            if (slot.err == hipSuccess) slot.err = back;
        }
    });
    *err = slot.err;
    return slot.err == hipSuccess ? slot.ptr : nullptr;
}

}  // namespace
}  // namespace moe

extern "C" int moe_dispatch_noalloc(const void *x, const int32_t *slot_idx, int32_t S, int32_t H,
                                    int32_t K, int32_t quant, int32_t src_rank, void *window,
                                    int64_t window_bytes, hipStream_t stream) {
    const int st = moe::check_dispatch(x, slot_idx, S, H, K, quant, window, window_bytes);
    if (st != MOE_OK) return st;
    if (!moe::pack_planned_used(S, K, quant))
        return moe::launch_pack(x, slot_idx, S, H, K, quant, src_rank, window, stream) == hipSuccess
                   ? MOE_OK
                   : MOE_ERR_HIP;
    if (moe::pack_plan_bytes(S, K) > MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_SCRATCH;
    int dev = 0;
    if (hipStreamGetDevice(stream, &dev) != hipSuccess) return MOE_ERR_HIP;
    hipError_t err = hipSuccess;
    void *ptr = moe::scratch_address(dev, &err);
    if (!ptr) return MOE_ERR_HIP;
    return moe::launch_pack_planned(x, slot_idx, S, H, K, src_rank, window, ptr, stream) == hipSuccess
               ? MOE_OK
               : MOE_ERR_HIP;
}
