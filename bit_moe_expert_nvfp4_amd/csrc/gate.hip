// Confidence gate: flags the tokens whose next-token distribution is not
// confident enough, so the layer forward adds the FP4 delta for them.
//
// Method: README "Frontier MoE on consumer Blackwell (SM120)", section "How it
// fits — 2-bit experts at FP4 quality" (a confidence gate re-runs
// low-confidence steps with the FP4 delta; tau = 0.60 in the benchmark table).
// The statistic is the largest softmax probability of the token's logits,
// 1 / sum_v exp(l_v - l_max), decided in float64 (l_v - l_max is exact there).
//
// One workgroup per token row streams the row twice (max, then the sum of
// exponentials): V floats per row, a few MB per step, HBM-bound.  Reductions go
// through wavefront shuffles and LDS in a fixed order, so the result is
// bitwise repeatable.
#include "moet_common.h"

namespace moet {

constexpr int kGateThreads = 1024;

__device__ __forceinline__ float wave_max(float v)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
    return v;
}

__device__ __forceinline__ double wave_sum(double v)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

__global__ __launch_bounds__(kGateThreads) void gate_kernel(const float *__restrict__ logits, int V, float tau,
                                                          uint8_t *__restrict__ flags, float *__restrict__ conf)
{
    __shared__ float s_max[kGateThreads / 64];
    __shared__ double s_sum[kGateThreads / 64];
    const int t = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const float *row = logits + (size_t)t * V;
    const bool vec = (V % 4) == 0;   // rows start 16-byte aligned
    float m = -INFINITY;
    if (vec) {
        const float4 *r4 = reinterpret_cast<const float4 *>(row);
        for (int i = tid; i < V / 4; i += kGateThreads) {
            const float4 q = r4[i];
            m = fmaxf(m, fmaxf(fmaxf(q.x, q.y), fmaxf(q.z, q.w)));
        }
    } else {
        for (int i = tid; i < V; i += kGateThreads) m = fmaxf(m, row[i]);
    }
    m = wave_max(m);
    if (lane == 0) s_max[wave] = m;
    __syncthreads();
    m = s_max[0];
#pragma unroll
    for (int w = 1; w < kGateThreads / 64; ++w) m = fmaxf(m, s_max[w]);
    const double md = (double)m;
    double s = 0.0;
    if (vec) {
        const float4 *r4 = reinterpret_cast<const float4 *>(row);
        for (int i = tid; i < V / 4; i += kGateThreads) {
            const float4 q = r4[i];
            s += exp((double)q.x - md) + exp((double)q.y - md) + exp((double)q.z - md) + exp((double)q.w - md);
        }
    } else {
        for (int i = tid; i < V; i += kGateThreads) s += exp((double)row[i] - md);
    }
    s = wave_sum(s);
    if (lane == 0) s_sum[wave] = s;
    __syncthreads();
    if (tid == 0) {
        double tot = 0.0;
#pragma unroll
        for (int w = 0; w < kGateThreads / 64; ++w) tot += s_sum[w];
        const double c = 1.0 / tot;
        flags[t] = (c < (double)tau) ? 1 : 0;
        if (conf) conf[t] = (float)c;
    }
}

int launch_gate(const float *logits, int T, int V, float tau, uint8_t *flags, float *conf, hipStream_t stream)
{
    hipLaunchKernelGGL(gate_kernel, dim3(T), dim3(kGateThreads), 0, stream, logits, V, tau, flags, conf);
    return check_launch("gate_kernel");
}

}  // namespace moet
