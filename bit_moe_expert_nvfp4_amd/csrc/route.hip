// Router top-k, routing weights and the token -> expert permutation.
//
// Method: README "Frontier MoE on consumer Blackwell (SM120)", sections
// "How it fits — 2-bit experts at FP4 quality" (routed experts per token) and
// "When the model doesn't fit at all — the GPU as an expert cache" (a
// descriptor step groups the step's routings per expert before the GEMMs).
//
// Selection uses the raw fp32 logits (largest first, equal logits -> lower id;
// softmax and sigmoid are monotonic).  One 64-lane wavefront owns one token:
// each lane holds up to 16 logits (e = lane + 64 i) and top_k rounds of
// shuffle reductions pick the winners.  The permutation is stable by pair id:
//  - small batches (T*top_k <= 1024): one workgroup does top-k, counts,
//    scan and ranks in LDS (one launch);
//  - large batches: a top-k kernel, then one workgroup per expert that scans
//    all pair ids twice (count of smaller ids -> offset, then a ballot-ordered
//    compaction of its own pairs).
#include <float.h>

#include "moet_common.h"

namespace moet {

constexpr int kMaxE = 1024;
constexpr int kMaxPerLane = kMaxE / 64;
constexpr int kSmallPairs = 1024;

__device__ __forceinline__ bool better(float v, int id, float bv, int bid)
{
    return v > bv || (v == bv && id < bid);
}

// Top-k of one token by one wavefront; writes ids / weights of token t.
__device__ void topk_token(const float *__restrict__ logits, int t, int E, int k, int fn, int renorm, float rscale,
                           int32_t *__restrict__ ids, float *__restrict__ w, int32_t *lds_ids)
{
    const int lane = threadIdx.x & 63;
    float v[kMaxPerLane];
    const float *row = logits + (size_t)t * E;
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i) {
        const int e = lane + 64 * i;
        v[i] = (e < E) ? row[e] : -FLT_MAX;
    }
    uint32_t used = 0;
    float my_val = 0.f;
    int my_id = 0;
    for (int j = 0; j < k; ++j) {
        float bv = -FLT_MAX;
        int bid = 0x7FFFFFFF;
#pragma unroll
        for (int i = 0; i < kMaxPerLane; ++i) {
            const int e = lane + 64 * i;
            if (e < E && !((used >> i) & 1u) && better(v[i], e, bv, bid)) {
                bv = v[i];
                bid = e;
            }
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) {
            const float ov = __shfl_xor(bv, off, 64);
            const int oid = __shfl_xor(bid, off, 64);
            if (better(ov, oid, bv, bid)) {
                bv = ov;
                bid = oid;
            }
        }
        if ((bid & 63) == lane) used |= 1u << (bid >> 6);
        if (lane == j) {
            my_val = bv;
            my_id = bid;
        }
    }
    // weights: lane j < k holds selected logit j (descending)
    const float lmax = __shfl(my_val, 0, 64);
    float s;
    if (fn == MOET_SOFTMAX) s = expf(my_val - lmax);
    else s = 1.0f / (1.0f + expf(-my_val));
    float part = (lane < k) ? s : 0.f;
    float denom;
    if (renorm) {
        denom = part;
    } else if (fn == MOET_SOFTMAX) {
        denom = 0.f;
#pragma unroll
        for (int i = 0; i < kMaxPerLane; ++i) {
            const int e = lane + 64 * i;
            if (e < E) denom += expf(v[i] - lmax);
        }
    } else {
        denom = 0.f;
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) denom += __shfl_xor(denom, off, 64);
    float wt = (fn == MOET_SIGMOID && !renorm) ? s : s / denom;
    wt *= rscale;
    if (lane < k) {
        ids[(size_t)t * k + lane] = my_id;
        w[(size_t)t * k + lane] = wt;
        if (lds_ids) lds_ids[t * k + lane] = my_id;
    }
}

__global__ __launch_bounds__(1024) void route_small_kernel(const float *__restrict__ logits, int T, int E, int k, int fn,
                                                           int renorm, float rscale, int32_t *__restrict__ ids,
                                                           float *__restrict__ w, int32_t *__restrict__ offsets,
                                                           int32_t *__restrict__ sorted)
{
    __shared__ int32_t s_ids[kSmallPairs];
    __shared__ int32_t s_cnt[kMaxE + 1];
    const int tid = threadIdx.x, nthr = blockDim.x;
    const int wave = tid >> 6, nwaves = nthr >> 6;
    for (int e = tid; e <= E; e += nthr) s_cnt[e] = 0;
    for (int t = wave; t < T; t += nwaves) topk_token(logits, t, E, k, fn, renorm, rscale, ids, w, s_ids);
    __syncthreads();
    const int P = T * k;
    for (int p = tid; p < P; p += nthr) atomicAdd(&s_cnt[s_ids[p]], 1);
    __syncthreads();
    // exclusive scan of s_cnt[0..E) by wave 0, 64 entries per step
    if (wave == 0) {
        const int lane = tid & 63;
        int carry = 0;
        for (int base = 0; base < E; base += 64) {
            const int e = base + lane;
            const int c = (e < E) ? s_cnt[e] : 0;
            int incl = c;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const int o = __shfl_up(incl, off, 64);
                if (lane >= off) incl += o;
            }
            if (e < E) s_cnt[e] = carry + incl - c;
            carry += __shfl(incl, 63, 64);
        }
        if (lane == 0) s_cnt[E] = carry;
    }
    __syncthreads();
    for (int e = tid; e <= E; e += nthr) offsets[e] = s_cnt[e];
    for (int p = tid; p < P; p += nthr) {
        const int e = s_ids[p];
        int rank = 0;
        for (int q = 0; q < p; ++q) rank += (s_ids[q] == e) ? 1 : 0;
        sorted[s_cnt[e] + rank] = p;
    }
}

__global__ __launch_bounds__(256) void route_topk_kernel(const float *__restrict__ logits, int T, int E, int k, int fn,
                                                         int renorm, float rscale, int32_t *__restrict__ ids,
                                                         float *__restrict__ w)
{
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t < T) topk_token(logits, t, E, k, fn, renorm, rscale, ids, w, nullptr);
}

// One workgroup per expert e: offset = #pairs with id < e, then its pairs in order.
__global__ __launch_bounds__(256) void route_permute_kernel(const int32_t *__restrict__ ids, int P, int E,
                                                            int32_t *__restrict__ offsets,
                                                            int32_t *__restrict__ sorted)
{
    __shared__ int s_wave[4];
    const int e = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int lt = 0;
    for (int p = tid; p < P; p += 256) lt += (ids[p] < e) ? 1 : 0;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) lt += __shfl_xor(lt, off, 64);
    if (lane == 0) s_wave[wave] = lt;
    __syncthreads();
    const int off_e = s_wave[0] + s_wave[1] + s_wave[2] + s_wave[3];
    if (tid == 0) {
        offsets[e] = off_e;
        if (e == E - 1) offsets[E] = P;
    }
    __syncthreads();
    int base = 0;
    for (int start = 0; start < P; start += 256) {
        const int p = start + tid;
        const bool eq = (p < P) && (ids[p] == e);
        const uint64_t bal = __ballot(eq);
        const int before = __popcll(bal & ((1ull << lane) - 1ull));
        __syncthreads();
        if (lane == 0) s_wave[wave] = __popcll(bal);
        __syncthreads();
        int wbase = base;
        for (int i = 0; i < wave; ++i) wbase += s_wave[i];
        if (eq) sorted[off_e + wbase + before] = p;
        base += s_wave[0] + s_wave[1] + s_wave[2] + s_wave[3];
    }
}

int launch_route(const float *logits, int T, int E, int k, int fn, int renorm, float rscale, int32_t *ids, float *w,
                 int32_t *offsets, int32_t *sorted, hipStream_t stream)
{
    const int P = T * k;
    if (P <= kSmallPairs) {
        int threads = ((T + 0) * 64);
        if (threads > 1024) threads = 1024;
        if (threads < 256) threads = 256;
        hipLaunchKernelGGL(route_small_kernel, dim3(1), dim3(threads), 0, stream, logits, T, E, k, fn, renorm, rscale,
                           ids, w, offsets, sorted);
        return check_launch("route_small_kernel");
    }
    hipLaunchKernelGGL(route_topk_kernel, dim3((T + 3) / 4), dim3(256), 0, stream, logits, T, E, k, fn, renorm, rscale,
                       ids, w);
    int rc = check_launch("route_topk_kernel");
    if (rc != MOET_OK) return rc;
    hipLaunchKernelGGL(route_permute_kernel, dim3(E), dim3(256), 0, stream, (const int32_t *)ids, P, E, offsets, sorted);
    return check_launch("route_permute_kernel");
}

}  // namespace moet
