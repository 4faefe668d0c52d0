// moet_moe_forward_noalloc: the layer forward with its scratch (the h and y
// rows the kernels pass between launches) in a static device array of this
// library instead of a caller workspace, for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops, hosts
// that forbid allocation).  It runs the same kernels as moet_moe_forward.
//
// The array holds kNoallocScratchBytes per GPU for as long as the process
// runs.  In host code its name is only a host-side stand-in: the device
// address is looked up once per device (hipGetSymbolAddress, with that
// device current) and only that address is handed to the kernels.  Every
// call on one GPU shares its array: calls that overlap in time on one GPU
// (other streams, other threads) race on it and must be ordered by the
// caller.  Nothing in it needs clearing: every row the kernels read was
// written earlier in the same call.
#include <mutex>

#include "moet_common.h"

namespace moet {

constexpr size_t kNoallocScratchBytes = MOET_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) uint8_t scratch[kNoallocScratchBytes];

static std::mutex g_scratch_mutex;
static void *g_scratch_ptr[kMaxDevices];

// Device address of the current device's scratch array (looked up on the first call per device).
static int device_scratch(void **ptr)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(MOET_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(MOET_EUNSUPPORTED, "device %d beyond the %d this library tracks", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) return fail(MOET_EHIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return MOET_OK;
}

}  // namespace moet

using namespace moet;

extern "C" {

moet_status moet_moe_forward_noalloc(const moet_layer *L, const uint16_t *x, int32_t T, int32_t top_k,
                             const int32_t *topk_ids, const float *topk_w, const int32_t *expert_offsets,
                             const int32_t *sorted_pairs, const uint8_t *gate_flags, uint16_t *out,
                             int32_t *miss_count, void *stream)
{
    set_error("%s", "");
    int rc = check_forward(L, x, T, top_k, topk_ids, topk_w, expert_offsets, sorted_pairs, gate_flags, out, miss_count);
    if (rc != MOET_OK) return (moet_status)(rc);
    const size_t need = forward_workspace_bytes(L, T, top_k);
    if (need > kNoallocScratchBytes)
        return (moet_status)fail(MOET_EWORKSPACE, "this batch needs %zu bytes of scratch; the static scratch of "
                                 "moet_moe_forward_noalloc holds %zu (use moet_moe_forward with a "
                                 "workspace)",
                                 need, kNoallocScratchBytes);
    void *ws = nullptr;
    rc = device_scratch(&ws);
    if (rc != MOET_OK) return (moet_status)(rc);
    return (moet_status)dispatch_forward(L, x, T, top_k, topk_ids, topk_w, expert_offsets, sorted_pairs, gate_flags, out,
                                         miss_count, ws, kNoallocScratchBytes, (hipStream_t)stream);
}

}  // extern "C"
