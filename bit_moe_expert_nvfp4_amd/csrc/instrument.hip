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

// Tight-loop peaks.  Every wave runs `iters` rounds of 4 independent chains
// (so no instruction waits on the previous one of its chain) and writes one
// word of its results so that nothing can be dropped; no memory traffic
// inside the loop.  4 waves per workgroup, 4 workgroups per CU.
constexpr int kPeakBlocks = 1024;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(256) void probe_mfma_kernel(int iters, uint32_t *__restrict__ sink)
{
    bf16x8_t a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = (__bf16)(float)((threadIdx.x + i) & 7);
        b[i] = (__bf16)(float)((threadIdx.x * 3 + i) & 7);
    }
    f32x16_t c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int it = 0; it < iters; ++it) {
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
    }
    float r = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) r += c0[i] + c1[i] + c2[i] + c3[i];
    if ((threadIdx.x & 63) == 0) sink[blockIdx.x * 4 + (threadIdx.x >> 6)] = __float_as_uint(r);
}

__global__ __launch_bounds__(256) void probe_dot2_kernel(int iters, uint32_t *__restrict__ sink)
{
    const uint32_t x = 0x3F803F80u + threadIdx.x, y = 0x3F003F00u ^ threadIdx.x;
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = (float)i;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = dot2_bf16(x + i, y, acc[i]);
    }
    float r = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) r += acc[i];
    if ((threadIdx.x & 63) == 0) sink[blockIdx.x * 4 + (threadIdx.x >> 6)] = __float_as_uint(r);
}

}  // namespace moet

using namespace moet;

extern "C" moet_status moet_probe_read(const void *src, size_t bytes, uint32_t *sink, void *stream)
{
    set_error("%s", "");
    if (!aligned16(src) || !aligned16(sink))
        return (moet_status)(fail(MOET_EINVAL, "src and sink must be non-NULL and 16-byte aligned"));
    if (bytes == 0 || bytes % 16)
        return (moet_status)(fail(MOET_EINVAL, "bytes (%zu) must be a positive multiple of 16", bytes));
    hipLaunchKernelGGL(probe_read_kernel, dim3(kProbeBlocks), dim3(256), 0, (hipStream_t)stream,
                       (const uint4 *)src, bytes / 16, sink);
    return (moet_status)(check_launch("probe_read_kernel"));
}

extern "C" moet_status moet_probe_peak(int kind, int32_t iters, uint32_t *sink, void *stream)
{
    set_error("%s", "");
    if (!aligned16(sink)) return (moet_status)(fail(MOET_EINVAL, "sink must be non-NULL and 16-byte aligned"));
    if (iters < 1) return (moet_status)(fail(MOET_EINVAL, "iters (%d) must be >= 1", iters));
    static_assert(kPeakBlocks * 4 <= MOET_PROBE_SINK_WORDS, "sink too small");
    if (kind == MOET_PROBE_MFMA_BF16)
        hipLaunchKernelGGL(probe_mfma_kernel, dim3(kPeakBlocks), dim3(256), 0, (hipStream_t)stream, iters, sink);
    else if (kind == MOET_PROBE_DOT2_BF16)
        hipLaunchKernelGGL(probe_dot2_kernel, dim3(kPeakBlocks), dim3(256), 0, (hipStream_t)stream, iters, sink);
    else
        return (moet_status)(fail(MOET_EINVAL, "unknown probe kind %d", kind));
    return (moet_status)(check_launch("probe peak kernel"));
}
