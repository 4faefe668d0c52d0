// Confidence gate: flags the tokens whose next-token distribution is not
// confident enough, so the layer forward adds the FP4 delta for them.
//
// Method: README "Frontier MoE on consumer Blackwell (SM120)", section "How it
// fits — 2-bit experts at FP4 quality" (a confidence gate re-runs
// low-confidence steps with the FP4 delta; tau = 0.60 in the benchmark table).
// The statistic is the largest softmax probability of the token's logits,
// 1 / sum_v exp(l_v - l_max), decided in float64 (l_v - l_max is exact there).
//
// Few rows (a decode step, a handful of streams): each row is cut into chunks
// of at least 2048 logits, about 1024 workgroups in all, so the whole chip
// shares the float64 exponentials.  A chunk workgroup writes its maximum m_c
// and sum s_c = sum exp(l - m_c) to the caller's workspace; one wavefront per
// row then forms sum_c s_c exp(m_c - M) with M = max_c m_c.  Many rows (one
// chunk each): one workgroup per row streams it twice (max, then the sum of
// exponentials), no workspace.  Every reduction (wavefront shuffles, LDS, the
// chunk combine) runs in a fixed order, so results are bitwise repeatable.
#include <algorithm>

#include "moet_common.h"

namespace moet {

constexpr int kGateThreads = 1024;

__device__ __forceinline__ float wave_max(float v)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
    return v;
}

__device__ __forceinline__ double wave_max_d(double v)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v = fmax(v, __shfl_xor(v, off, 64));
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

// ---------------------------------------------------------------------------
// Split rows: chunk partials, then a per-row combine.
// ---------------------------------------------------------------------------
constexpr int kPartThreads = 256;
constexpr int kChunkMin = 2048;     // logits per chunk, at least
constexpr int kGateTargetWG = 1024; // chunk workgroups aimed at over all rows

struct GatePart {
    double m;   // chunk maximum (-inf: every logit of the chunk is masked)
    double s;   // sum over the chunk of exp(l - m), 0 for a masked chunk
};

// chunks per row and logits per chunk (a multiple of 4, so float4 rows stay aligned)
int gate_chunks(int T, int V, int *len)
{
    const int64_t by_v = ((int64_t)V + kChunkMin - 1) / kChunkMin, by_t = (kGateTargetWG + (int64_t)T - 1) / T;
    const int64_t c0 = std::max<int64_t>(1, std::min(by_v, by_t));
    if (c0 == 1) {
        *len = V;
        return 1;
    }
    const int64_t L = ((((int64_t)V + c0 - 1) / c0) + 3) & ~(int64_t)3;
    *len = (int)L;
    return (int)(((int64_t)V + L - 1) / L);
}

size_t gate_workspace_bytes(int T, int V)
{
    int len;
    const int C = gate_chunks(T, V, &len);
    return C > 1 ? (size_t)T * C * sizeof(GatePart) : 0;
}

__global__ __launch_bounds__(kPartThreads) void gate_partial_kernel(const float *__restrict__ logits, int V, int L,
                                                                  int C, GatePart *__restrict__ part)
{
    __shared__ float s_max[kPartThreads / 64];
    __shared__ double s_sum[kPartThreads / 64];
    const int c = blockIdx.x, t = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const float *row = logits + (size_t)t * V;
    const int b = c * L, e = (int)min((int64_t)V, (int64_t)b + L);
    const bool vec = (V % 4) == 0;   // b and e are then multiples of 4
    float m = -INFINITY;
    if (vec) {
        const float4 *r4 = reinterpret_cast<const float4 *>(row);
        for (int i = b / 4 + tid; i < e / 4; i += kPartThreads) {
            const float4 q = r4[i];
            m = fmaxf(m, fmaxf(fmaxf(q.x, q.y), fmaxf(q.z, q.w)));
        }
    } else {
        for (int i = b + tid; i < e; i += kPartThreads) m = fmaxf(m, row[i]);
    }
    m = wave_max(m);
    if (lane == 0) s_max[wave] = m;
    __syncthreads();
    m = s_max[0];
#pragma unroll
    for (int w = 1; w < kPartThreads / 64; ++w) m = fmaxf(m, s_max[w]);
    const double md = (double)m;
    double s = 0.0;
    if (m != -INFINITY) {   // a fully masked chunk contributes nothing
        if (vec) {
            const float4 *r4 = reinterpret_cast<const float4 *>(row);
            for (int i = b / 4 + tid; i < e / 4; i += kPartThreads) {
                const float4 q = r4[i];
                s += exp((double)q.x - md) + exp((double)q.y - md) + exp((double)q.z - md) + exp((double)q.w - md);
            }
        } else {
            for (int i = b + tid; i < e; i += kPartThreads) s += exp((double)row[i] - md);
        }
    }
    s = wave_sum(s);
    if (lane == 0) s_sum[wave] = s;
    __syncthreads();
    if (tid == 0) {
        double tot = 0.0;
#pragma unroll
        for (int w = 0; w < kPartThreads / 64; ++w) tot += s_sum[w];
        part[(size_t)t * C + c] = GatePart{md, tot};
    }
}

// one wavefront per row: confidence = 1 / sum_c s_c exp(m_c - M), M = max_c m_c (finite)
__global__ __launch_bounds__(64) void gate_combine_kernel(const GatePart *__restrict__ part, int C, float tau,
                                                          uint8_t *__restrict__ flags, float *__restrict__ conf)
{
    const int t = blockIdx.x, lane = threadIdx.x;
    const GatePart *pr = part + (size_t)t * C;
    double M = -INFINITY;
    for (int c = lane; c < C; c += 64) M = fmax(M, pr[c].m);
    M = wave_max_d(M);
    double S = 0.0;
    for (int c = lane; c < C; c += 64) {
        const GatePart q = pr[c];
        if (q.s > 0.0) S += q.s * exp(q.m - M);
    }
    S = wave_sum(S);
    if (lane == 0) {
        const double cf = 1.0 / S;
        flags[t] = (cf < (double)tau) ? 1 : 0;
        if (conf) conf[t] = (float)cf;
    }
}

int launch_gate(const float *logits, int T, int V, float tau, uint8_t *flags, float *conf, void *workspace,
                hipStream_t stream)
{
    int L;
    const int C = gate_chunks(T, V, &L);
    if (C == 1) {
        hipLaunchKernelGGL(gate_kernel, dim3(T), dim3(kGateThreads), 0, stream, logits, V, tau, flags, conf);
        return check_launch("gate_kernel");
    }
    GatePart *part = static_cast<GatePart *>(workspace);
    hipLaunchKernelGGL(gate_partial_kernel, dim3(C, T), dim3(kPartThreads), 0, stream, logits, V, L, C, part);
    const int rc = check_launch("gate_partial_kernel");
    if (rc) return rc;
    hipLaunchKernelGGL(gate_combine_kernel, dim3(T), dim3(64), 0, stream, part, C, tau, flags, conf);
    return check_launch("gate_combine_kernel");
}

}  // namespace moet
