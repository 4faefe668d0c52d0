// Measurement helpers of libmoet (declared in include/moet_instrument.h): a
// plain streaming read of a device buffer, the achievable HBM read rate that
// the weight-streaming kernels are compared with.  Nothing on the layer's path
// calls it.
#include "moet_common.h"
#include "moet_instrument.h"

namespace moet {

// 1024 workgroups of 4 waves, one 16-byte load per lane and iteration in a
// grid-stride loop: the fastest of the shapes measured on MI355X (1024 to
// 16384 workgroups; 1, 2, 4 or 8 loads in flight per lane, strided or per-
// workgroup chunks, with and without non-temporal loads), 6.2-6.5 TB/s over
// 1 GiB.  Each wave's 64 lanes read 1 KiB of consecutive bytes; the xor of
// what a wave read goes to its sink word so that the loads cannot be dropped.
constexpr int kProbeBlocks = 1024;
static_assert(kProbeBlocks * 4 <= MOET_PROBE_SINK_WORDS, "sink too small");

__global__ __launch_bounds__(256) void probe_read_kernel(const uint4 *__restrict__ src, size_t n16,
                                                         uint32_t *__restrict__ sink)
{
    const size_t stride = (size_t)gridDim.x * 256;
    uint32_t acc = 0;
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += stride) {
        const uint4 a = src[i];
        acc ^= a.x ^ a.y ^ a.z ^ a.w;
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, off, 64);
    if ((threadIdx.x & 63) == 0) sink[blockIdx.x * 4 + (threadIdx.x >> 6)] = acc;
}

}  // namespace moet

using namespace moet;

extern "C" int moet_probe_read(const void *src, size_t bytes, uint32_t *sink, void *stream)
{
    set_error("%s", "");
    if (!aligned16(src) || !aligned16(sink)) return fail(MOET_EINVAL, "src and sink must be non-NULL and 16-byte aligned");
    if (bytes == 0 || bytes % 16) return fail(MOET_EINVAL, "bytes (%zu) must be a positive multiple of 16", bytes);
    hipLaunchKernelGGL(probe_read_kernel, dim3(kProbeBlocks), dim3(256), 0, (hipStream_t)stream,
                       (const uint4 *)src, bytes / 16, sink);
    return check_launch("probe_read_kernel");
}
