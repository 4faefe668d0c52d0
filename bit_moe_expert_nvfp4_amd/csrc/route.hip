// Router top-k, routing weights and the token -> expert permutation.
//
// Method: README "Frontier MoE on consumer Blackwell (SM120)", sections
// "How it fits — 2-bit experts at FP4 quality" (routed experts per token) and
// "When the model doesn't fit at all — the GPU as an expert cache" (a
// descriptor step groups the step's routings per expert before the GEMMs).
//
// Selection uses the raw fp32 logits (largest first, equal logits -> lower id;
// softmax and sigmoid are monotonic).  One 64-lane wavefront owns one token:
// each lane holds up to 16 logits (e = lane + 64 i); the k-th largest is found
// by a 32-step bisection over order-preserving integer keys with ballot
// counts, so no cross-lane shuffles sit on the critical path.  The
// permutation is stable by pair id:
//  - small batches (T*top_k <= 1024): one workgroup does top-k, then every
//    thread counts the offset of one expert and the rank of one pair in LDS
//    (one launch);
//  - large batches: a top-k kernel, then one workgroup per expert that scans
//    all pair ids twice (count of smaller ids -> offset, then a ballot-ordered
//    compaction of its own pairs).
#include <float.h>

#include "moet_common.h"

namespace moet {

constexpr int kMaxE = 1024;
constexpr int kSmallPairs = 1024;

// monotonic map float -> uint32 (larger float -> larger key); inputs are finite
__device__ __forceinline__ uint32_t fkey(float f)
{
    const uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Top-k of one token by one wavefront; writes ids / weights of token t.
// The k-th largest key is found by bisection on its 32 bits, counting with
// ballots (no cross-lane shuffles); ties at the threshold are filled in
// increasing expert id; the k winners are then ordered by (key desc, id asc).
template <int NPL>
__device__ __forceinline__ void topk_token(const float *__restrict__ logits, int t, int E, int k, int fn, int renorm, float rscale,
                           int32_t *__restrict__ ids, float *__restrict__ w, int32_t *lds_ids, uint32_t *scratch)
{
    const int lane = threadIdx.x & 63;
    uint32_t key[NPL];
    float v[NPL];
    const float *row = logits + (size_t)t * E;
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
        const int e = lane + 64 * i;
        v[i] = (e < E) ? row[e] : 0.f;
        key[i] = (e < E) ? fkey(v[i]) : 0u;   // key 0 is below every finite value
    }
    uint32_t thr = 0;
    for (int b = 31; b >= 0; --b) {
        const uint32_t cand = thr | (1u << b);
        int c = 0;
#pragma unroll
        for (int i = 0; i < NPL; ++i) c += __popcll(__ballot(key[i] >= cand));
        if (c >= k) thr = cand;
        // exactly k keys >= cand: they are the top k (ties at thr below are then
        // all selected, since k - #{key > thr} = #{key == thr})
        if (c == k) break;
    }
    int c_gt = 0;
#pragma unroll
    for (int i = 0; i < NPL; ++i) c_gt += __popcll(__ballot(key[i] > thr));
    const int need_eq = k - c_gt;   // >= 1
    // selected flags: key > thr, or key == thr among the first need_eq in id order
    bool sel[NPL];
    int eq_before = 0;
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
        const bool eq = (lane + 64 * i < E) && key[i] == thr;
        const uint64_t be = __ballot(eq);
        const int rank_eq = eq_before + __popcll(be & lt_mask);
        sel[i] = key[i] > thr || (eq && rank_eq < need_eq);
        eq_before += __popcll(be);
    }
    // compact the k winners (key, id) into scratch[0..k) in (i, lane) order
    int before = 0;
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
        const uint64_t bs = __ballot(sel[i]);
        if (sel[i]) {
            const int pos = before + __popcll(bs & lt_mask);
            scratch[2 * pos] = key[i];
            scratch[2 * pos + 1] = (uint32_t)(lane + 64 * i);
        }
        before += __popcll(bs);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");   // LDS writes done before other lanes read them
    __builtin_amdgcn_wave_barrier();
    uint32_t my_key = 0, my_id = 0;
    if (lane < k) {
        my_key = scratch[2 * lane];
        my_id = scratch[2 * lane + 1];
    }
    // rank among the k winners by (key desc, id asc): the other winners are read
    // from their lanes (wave-uniform loop, no memory round trips)
    int rank = 0;
    for (int j = 0; j < k; ++j) {
        const uint32_t kj = __builtin_amdgcn_readlane(my_key, j), ij = __builtin_amdgcn_readlane(my_id, j);
        rank += (kj > my_key || (kj == my_key && ij < my_id)) ? 1 : 0;
    }
    // the winner's logit from the lane that loaded it (no second read of the row)
    float my_val = 0.f;
    {
        const int src = (int)(my_id & 63u), slot = (int)(my_id >> 6);
#pragma unroll
        for (int i = 0; i < NPL; ++i) {
            const float vi = __shfl(v[i], src, 64);
            if (slot == i) my_val = vi;
        }
        if (lane >= k) my_val = 0.f;
    }
    // largest selected logit (rank 0)
    const uint64_t r0 = __ballot(lane < k && rank == 0);
    const float lmax = __shfl(my_val, (int)__builtin_ctzll(r0), 64);
    float s;
    if (fn == MOET_SOFTMAX) s = expf(my_val - lmax);
    else s = 1.0f / (1.0f + expf(-my_val));
    float denom;
    if (renorm) {
        denom = (lane < k) ? s : 0.f;
    } else if (fn == MOET_SOFTMAX) {
        denom = 0.f;
#pragma unroll
        for (int i = 0; i < NPL; ++i)
            if (lane + 64 * i < E) denom += expf(v[i] - lmax);
    } else {
        denom = 0.f;
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) denom += __shfl_xor(denom, off, 64);
    float wt = (fn == MOET_SIGMOID && !renorm) ? s : s / denom;
    wt *= rscale;
    if (lane < k) {
        ids[(size_t)t * k + rank] = (int32_t)my_id;
        w[(size_t)t * k + rank] = wt;
        if (lds_ids) lds_ids[t * k + rank] = (int32_t)my_id;
    }
}

// NPL = logits per lane (E <= 64 NPL), chosen on the host so that one top-k
// body is inlined per kernel
template <int NPL>
__global__ __launch_bounds__(1024) void route_small_kernel(const float *__restrict__ logits, int T, int E, int k, int fn,
                                                           int renorm, float rscale, int32_t *__restrict__ ids,
                                                           float *__restrict__ w, int32_t *__restrict__ offsets,
                                                           int32_t *__restrict__ sorted)
{
    __shared__ __align__(16) int32_t s_ids[kSmallPairs + 8];
    __shared__ int32_t s_off[kMaxE + 1];
    __shared__ uint32_t s_scr[16][32];
    const int tid = threadIdx.x, nthr = blockDim.x;
    const int wave = tid >> 6, nwaves = nthr >> 6;
    for (int t = wave; t < T; t += nwaves) topk_token<NPL>(logits, t, E, k, fn, renorm, rscale, ids, w, s_ids, s_scr[wave]);
    __syncthreads();
    const int P = T * k;
    // offsets[e] = number of pairs routed to experts < e (LDS reads in unrolled
    // groups of 8 so their latencies overlap; s_ids is padded with E)
    for (int p = P + tid; p < ((P + 7) & ~7); p += nthr) s_ids[p] = E;
    __syncthreads();
    const int4 *ids4 = reinterpret_cast<const int4 *>(s_ids);
    for (int e = tid; e <= E; e += nthr) {
        int c = 0;
        for (int p = 0; p < P; p += 8) {   // two 16-byte LDS reads per group of 8 ids
            const int4 a = ids4[p >> 2], b = ids4[(p >> 2) + 1];
            c += (a.x < e) + (a.y < e) + (a.z < e) + (a.w < e) + (b.x < e) + (b.y < e) + (b.z < e) + (b.w < e);
        }
        s_off[e] = c;
        offsets[e] = c;
    }
    __syncthreads();
    for (int p = tid; p < P; p += nthr) {
        const int e = s_ids[p];
        int rank = 0;
        for (int q = 0; q < p; q += 8) {
            const int4 a = ids4[q >> 2], b = ids4[(q >> 2) + 1];
            rank += (q + 0 < p && a.x == e) + (q + 1 < p && a.y == e) + (q + 2 < p && a.z == e) +
                    (q + 3 < p && a.w == e) + (q + 4 < p && b.x == e) + (q + 5 < p && b.y == e) +
                    (q + 6 < p && b.z == e) + (q + 7 < p && b.w == e);
        }
        sorted[s_off[e] + rank] = p;
    }
}

template <int NPL>
__global__ __launch_bounds__(256) void route_topk_kernel(const float *__restrict__ logits, int T, int E, int k, int fn,
                                                         int renorm, float rscale, int32_t *__restrict__ ids,
                                                         float *__restrict__ w)
{
    __shared__ uint32_t s_scr[4][32];
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t < T) topk_token<NPL>(logits, t, E, k, fn, renorm, rscale, ids, w, nullptr, s_scr[threadIdx.x >> 6]);
}

template <int NPL>
static int launch_route_n(const float *logits, int T, int E, int k, int fn, int renorm, float rscale, int32_t *ids,
                          float *w, int32_t *offsets, int32_t *sorted, hipStream_t stream);

// One workgroup per expert e: offset = #pairs with id < e, then its pairs in
// pair order.  Wavefront w of 8 owns a contiguous eighth of the pairs and reads
// it in 1 KiB steps (lane l takes ids 4l .. 4l + 3 of a step, one 16-byte load, 8
// steps in flight), so every load is coalesced.  One pass counts the ids below
// e and ranks the matches of e in pair order with one ballot per id of a lane
// (earlier lanes, then the lane's own earlier ids), appending their positions
// to the wave's list in LDS.  A block-wide sum gives the offset and every wave
// its first output slot, and the lists are copied out, so the order is stable.
// A wave with more matches than its list holds reads its range again.
constexpr int kPermWaves = 8;
constexpr int kPermList = 1024;   // positions per wave list (4 KiB)

__global__ __launch_bounds__(64 * kPermWaves) void route_permute_kernel(const int32_t *__restrict__ ids, int P,
                                                                       int E, int32_t *__restrict__ offsets,
                                                                       int32_t *__restrict__ sorted)
{
    __shared__ int s_lt[kPermWaves], s_eq[kPermWaves];
    __shared__ int s_list[kPermWaves][kPermList];
    const int e = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int range = (((P + kPermWaves - 1) / kPermWaves) + 255) & ~255;   // whole 1 KiB steps
    const int q0 = min(wave * range, P), q1 = min(q0 + range, P);
    const uint64_t below = (1ull << lane) - 1ull;
    // ids [p, p + 4) of this lane at step base b (beyond q1: INT_MAX, neither e nor below it)
    auto load4 = [&](int b, int v[4]) {
        const int p = b + 4 * lane;
        if (p + 4 <= q1) {
            const int4 x = *reinterpret_cast<const int4 *>(ids + p);   // ids is 16-byte aligned, p % 4 == 0
            v[0] = x.x;
            v[1] = x.y;
            v[2] = x.z;
            v[3] = x.w;
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] = (p + i < q1) ? ids[p + i] : 0x7FFFFFFF;
        }
    };
    // rank this step's matches after the wave's `cnt` earlier ones; emit(slot, position)
    auto rank_step = [&](int b, const int v[4], int &cnt, auto emit) {
        uint64_t m[4];
        int tot = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            m[i] = __ballot(v[i] == e);
            tot += __popcll(m[i]);
        }
        if (tot == 0) return;   // wave-uniform
        int r = cnt;
#pragma unroll
        for (int i = 0; i < 4; ++i) r += __popcll(m[i] & below);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (v[i] == e) emit(r++, b + 4 * lane + i);
        cnt += tot;
    };
    int lt = 0, cnt = 0;
    for (int b0 = q0; b0 < q1; b0 += 8 * 256) {
        int v[8][4];
#pragma unroll
        for (int u = 0; u < 8; ++u) load4(b0 + 256 * u, v[u]);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
#pragma unroll
            for (int i = 0; i < 4; ++i) lt += (v[u][i] < e) ? 1 : 0;
            rank_step(b0 + 256 * u, v[u], cnt, [&](int slot, int pos) {
                if (slot < kPermList) s_list[wave][slot] = pos;
            });
        }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) lt += __shfl_xor(lt, off, 64);
    if (lane == 0) {
        s_lt[wave] = lt;
        s_eq[wave] = cnt;
    }
    __syncthreads();
    int off_e = 0;
    for (int i = 0; i < kPermWaves; ++i) off_e += s_lt[i];
    int base = off_e;   // this wave's first output slot
    for (int i = 0; i < wave; ++i) base += s_eq[i];
    if (tid == 0) {
        offsets[e] = off_e;
        if (e == E - 1) offsets[E] = P;
    }
    if (cnt <= kPermList) {   // wave-uniform
        for (int i = lane; i < cnt; i += 64) sorted[base + i] = s_list[wave][i];
        return;
    }
    int c2 = 0;
    for (int b = q0; b < q1; b += 256) {
        int v[4];
        load4(b, v);
        rank_step(b, v, c2, [&](int slot, int pos) { sorted[base + slot] = pos; });
    }
}

template <int NPL>
static int launch_route_n(const float *logits, int T, int E, int k, int fn, int renorm, float rscale, int32_t *ids,
                          float *w, int32_t *offsets, int32_t *sorted, hipStream_t stream)
{
    const int P = T * k;
    if (P <= kSmallPairs) {
        int threads = T * 64;
        if (threads > 1024) threads = 1024;
        if (threads < 256) threads = 256;
        hipLaunchKernelGGL(route_small_kernel<NPL>, dim3(1), dim3(threads), 0, stream, logits, T, E, k, fn, renorm,
                           rscale, ids, w, offsets, sorted);
        return check_launch("route_small_kernel");
    }
    hipLaunchKernelGGL(route_topk_kernel<NPL>, dim3((T + 3) / 4), dim3(256), 0, stream, logits, T, E, k, fn, renorm,
                       rscale, ids, w);
    int rc = check_launch("route_topk_kernel");
    if (rc != MOET_OK) return rc;
    hipLaunchKernelGGL(route_permute_kernel, dim3(E), dim3(64 * kPermWaves), 0, stream, (const int32_t *)ids, P, E, offsets, sorted);
    return check_launch("route_permute_kernel");
}

int launch_route(const float *logits, int T, int E, int k, int fn, int renorm, float rscale, int32_t *ids, float *w,
                 int32_t *offsets, int32_t *sorted, hipStream_t stream)
{
    if (E <= 64) return launch_route_n<1>(logits, T, E, k, fn, renorm, rscale, ids, w, offsets, sorted, stream);
    if (E <= 128) return launch_route_n<2>(logits, T, E, k, fn, renorm, rscale, ids, w, offsets, sorted, stream);
    if (E <= 256) return launch_route_n<4>(logits, T, E, k, fn, renorm, rscale, ids, w, offsets, sorted, stream);
    if (E <= 512) return launch_route_n<8>(logits, T, E, k, fn, renorm, rscale, ids, w, offsets, sorted, stream);
    return launch_route_n<16>(logits, T, E, k, fn, renorm, rscale, ids, w, offsets, sorted, stream);
}

}  // namespace moet
