// Other checkpoint flavours loaded into the same sign-symmetric 2-bit planes.
//
// README "Frontier MoE on consumer Blackwell (SM120)", section "How it fits —
// 2-bit experts at FP4 quality": FP4 experts are loaded by remapping their
// codes, FP8 block-quantised experts are requantised at load in float64.
//
// MXFP4 codes remap.  The codebook {-4,-1,1,4} is a subset of the e2m1 grid,
// so every e2m1 code goes to the nearest of those values in units of its
// block's e8m0 scale (magnitudes 0..2 -> 1, 3..6 -> 4; no ties exist), and the
// scales carry over: with Emax the largest exponent over blocks that hold a
// non-zero code, the tensor scale is 2^(Emax - 135) and a block's e4m3 scale
// is 2^(E - Emax + 8), exact down to e4m3's smallest subnormal 2^-9; blocks
// below that, and blocks of zeros, get scale 0.  Emax comes from an integer
// atomic max over 64 workgroups per matrix.
//
// FP8 block-quant requant.  e4m3fn weights with one fp32 scale per 128 x 128
// block.  The tensor scale is the power of two S = 2^p, p >= -149 smallest
// with 4 * 448 * S >= amax; per 32 weights along K the e4m3 block scale t
// minimises sum_i min((y_i - a)^2, (y_i - 4a)^2), a = e4m3(t) * S, over every
// finite code, ties to the smaller code.  Unlike the NVFP4 case the weights are
// not integer multiples of one unit (each 128 x 128 block has its own fp32
// scale), so the error is a float64 sum: y_i and a are exact in float64, and
// the squares and the sum are rounded in a fixed order (k order, no
// contraction into FMAs), which makes the decision reproducible bit for bit.
// All 127 candidates are scanned: a window argument only holds for the exact
// error, not for its rounded value.
#include "moet_common.h"

namespace moet {

namespace {

// 2^e as a float32, e in [-149, 127]
__device__ __forceinline__ float pow2f(int e)
{
    return e >= -126 ? __uint_as_float((uint32_t)(e + 127) << 23) : __uint_as_float(1u << (e + 149));
}

template <int NT>
__device__ __forceinline__ int block_max_i32(int v)
{
    __shared__ int red[NT / 64];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v = max(v, __shfl_xor(v, off));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    v = red[0];
#pragma unroll
    for (int i = 1; i < NT / 64; ++i) v = max(v, red[i]);
    return v;
}

template <int NT>
__device__ __forceinline__ double block_max_f64(double v)
{
    __shared__ double red[NT / 64];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v = fmax(v, __shfl_xor(v, off));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    v = red[0];
#pragma unroll
    for (int i = 1; i < NT / 64; ++i) v = fmax(v, red[i]);
    return v;
}

// e4m3fn value of code t (0x00..0x7E) as a float64, exact
__device__ __forceinline__ double e4m3_f64(int t) { return (double)e4m3_x512(t) * (1.0 / 512.0); }

constexpr int kScanThreads = 512;

}  // namespace

// ---------------------------------------------------------------------------
// MXFP4
// ---------------------------------------------------------------------------

// Tensor scale from the largest live block exponent, in three steps that keep
// the int in the scale2 output slot: -1, then an integer atomic max over
// workgroup maxima (kMxSlices workgroups per matrix), then (after the remap has
// read it) the float 2^(Emax - 135).
constexpr int kMxSlices = 64;

__global__ void mx_emax_init_kernel(int32_t *emax, int64_t n_mat)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n_mat) emax[i] = -1;
}

__global__ __launch_bounds__(kScanThreads) void mx_emax_kernel(const uint8_t *__restrict__ codes,
                                                               const uint8_t *__restrict__ escales, int N, int K,
                                                               int32_t *__restrict__ emax_out)
{
    const size_t mat = blockIdx.x;
    const size_t nblk = (size_t)N * (K / 32);
    const size_t per = (nblk + kMxSlices - 1) / kMxSlices;
    const size_t b0 = per * blockIdx.y, b1 = b0 + per < nblk ? b0 + per : nblk;
    const uint4 *c = reinterpret_cast<const uint4 *>(codes + mat * nblk * 16);
    const uint8_t *e = escales + mat * nblk;
    int emax = -1;
    for (size_t i = b0 + threadIdx.x; i < b1; i += kScanThreads) {
        const uint4 w = c[i];
        if (((w.x | w.y | w.z | w.w) & 0x77777777u) != 0u) emax = max(emax, (int)e[i]);
    }
    emax = block_max_i32<kScanThreads>(emax);
    if (threadIdx.x == 0 && emax >= 0) atomicMax(emax_out + mat, emax);
}

__global__ void mx_scale_final_kernel(float *ws2, int64_t n_mat)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n_mat) {
        const int emax = __float_as_int(ws2[i]);
        ws2[i] = emax < 0 ? 1.0f : pow2f(emax - 135);
    }
}

// one thread per 32-weight block
__global__ __launch_bounds__(256) void mx_remap_kernel(const uint8_t *__restrict__ codes,
                                                       const uint8_t *__restrict__ escales, int64_t n_mat, int N, int K,
                                                       const int32_t *__restrict__ emax_in, int balance,
                                                       uint32_t *__restrict__ wcodes, uint8_t *__restrict__ wscales)
{
    const int nb = K / 32;
    const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (size_t)n_mat * N * nb) return;
    const int b = (int)(idx % nb);
    const size_t rg = idx / nb;
    const int n = (int)(rg % N);
    const size_t mat = rg / N;

    const uint4 cw = reinterpret_cast<const uint4 *>(codes)[idx];  // blocks are 16 contiguous bytes
    const int E = escales[idx];
    const uint32_t words[4] = {cw.x, cw.y, cw.z, cw.w};
    int tau = 0;
    if (((cw.x | cw.y | cw.z | cw.w) & 0x77777777u) != 0u) {
        const int emax = emax_in[mat];   // >= 0: this block is live
        const int d = E - (emax - 8);                     // block scale 2^d, d <= 8
        if (d >= -6) tau = (d + 7) << 3;                  // normal: exponent field d + 7
        else if (d >= -9) tau = 1 << (d + 9);             // subnormal: mantissa 2^(d + 9)
    }
    uint32_t out[2] = {0, 0};
    int zeros = 0;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const uint32_t nib = (words[2 * half + (e >> 3)] >> (4 * (e & 7))) & 15u;
            const uint32_t mag = nib & 7u;
            const uint32_t m = mag >= 5u ? 1u : 0u;       // |e2m1| in {3, 4, 6}
            const uint32_t s = (balance && mag == 0u) ? (uint32_t)(zeros++ & 1) : nib >> 3;
            out[half] |= (m << mbit(e)) | (s << sbit(e));
        }
    }
    store_w2_block(wcodes, wscales, mat, N, K, n, b, out, tau);
}

// ---------------------------------------------------------------------------
// FP8 block-quant
// ---------------------------------------------------------------------------

// Tensor scale 2^p.  p(amax) (smallest p >= -149 with 1792 * 2^p >= amax) is
// monotone in amax, so the largest p over workgroup maxima is p of the tensor
// maximum: each of kMxSlices workgroups per matrix finds its own p exactly in
// float64 and takes an integer atomic max into the scale2 slot (kNoP first:
// no positive weight seen), and the requant reads that int before the last
// step turns it into the float scale.
constexpr int kNoP = -1000;

__global__ void fp8_p_init_kernel(int32_t *pmax, int64_t n_mat)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n_mat) pmax[i] = kNoP;
}

__global__ __launch_bounds__(kScanThreads) void fp8_p_kernel(const uint8_t *__restrict__ w,
                                                             const float *__restrict__ bs, int N, int K,
                                                             int32_t *__restrict__ pmax)
{
    const size_t mat = blockIdx.x;
    const int KB = K / 128, NB = (N + 127) / 128;
    const size_t nchunk = (size_t)N * (K / 16);
    const size_t per = (nchunk + kMxSlices - 1) / kMxSlices;
    const size_t c0 = per * blockIdx.y, c1 = c0 + per < nchunk ? c0 + per : nchunk;
    const uint4 *c = reinterpret_cast<const uint4 *>(w + mat * (size_t)N * K);
    const float *s = bs + mat * (size_t)NB * KB;
    double amax = 0.0;
    for (size_t i = c0 + threadIdx.x; i < c1; i += kScanThreads) {
        const uint4 q = c[i];
        const uint32_t words[4] = {q.x, q.y, q.z, q.w};
        int mx = 0;
#pragma unroll
        for (int j = 0; j < 16; ++j) mx = max(mx, (int)((words[j >> 2] >> (8 * (j & 3))) & 0x7Fu));
        const int n = (int)(i / (K / 16)), k = (int)(i % (K / 16)) * 16;
        amax = fmax(amax, e4m3_f64(mx) * (double)s[(size_t)(n / 128) * KB + k / 128]);
    }
    amax = block_max_f64<kScanThreads>(amax);
    if (threadIdx.x == 0 && amax > 0.0) {
        int p = -149;
        while (1792.0 * ldexp(1.0, p) < amax) ++p;
        atomicMax(pmax + mat, p);
    }
}

__device__ __forceinline__ float scale_of_p(int p) { return p == kNoP ? 1.0f : pow2f(p); }

__global__ void fp8_scale_final_kernel(float *ws2, int64_t n_mat)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n_mat) ws2[i] = scale_of_p(__float_as_int(ws2[i]));
}

// one thread per 32-weight block: the float64 scan over all 127 block scales
__global__ __launch_bounds__(256) void fp8_requant_kernel(const uint8_t *__restrict__ w, const float *__restrict__ bs,
                                                          int64_t n_mat, int N, int K, const int32_t *__restrict__ pmax,
                                                          int balance, uint32_t *__restrict__ wcodes,
                                                          uint8_t *__restrict__ wscales)
{
#pragma clang fp contract(off)
    const int nb = K / 32, KB = K / 128, NB = (N + 127) / 128;
    const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (size_t)n_mat * N * nb) return;
    const int b = (int)(idx % nb);
    const size_t rg = idx / nb;
    const int n = (int)(rg % N);
    const size_t mat = rg / N;

    const uint4 *src = reinterpret_cast<const uint4 *>(w + idx * 32);  // rows are K contiguous bytes
    const uint4 q0 = src[0], q1 = src[1];
    const uint32_t words[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
    const double sb = (double)bs[mat * (size_t)NB * KB + (size_t)(n / 128) * KB + (32 * b) / 128];
    const double S = (double)scale_of_p(pmax[mat]);
    double y[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) y[i] = e4m3_f64((int)((words[i >> 2] >> (8 * (i & 3))) & 0x7Fu)) * sb;

    // The per-element term is min(fl((y-a)^2), fl((y-4a)^2)).  Rounding is
    // monotone, so that minimum is the rounded square of whichever difference is
    // smaller exactly, and y > 2.5a (exact: y and a have few significant bits)
    // says which: one difference and one square instead of two, same bits.
    int best_t = 0;
    double best_err = -1.0;
    for (int t = 0; t < 127; ++t) {
        const double a = e4m3_f64(t) * S;
        const double a4 = 4.0 * a, a25 = 2.5 * a;
        double err = 0.0;
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            const double d = y[i] - (y[i] > a25 ? a4 : a);
            err = err + d * d;
        }
        if (best_err < 0.0 || err < best_err) {
            best_err = err;
            best_t = t;
        }
    }
    const double a = e4m3_f64(best_t) * S;
    uint32_t out[2] = {0, 0};
    int zeros = 0;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
        const uint32_t byte = (words[i >> 2] >> (8 * (i & 3))) & 0xFFu;
        const uint32_t m = (2.0 * y[i] > 5.0 * a) ? 1u : 0u;
        const uint32_t s = (balance && y[i] == 0.0) ? (uint32_t)(zeros++ & 1) : byte >> 7;
        const int e = i & 15;
        out[i >> 4] |= (m << mbit(e)) | (s << sbit(e));
    }
    store_w2_block(wcodes, wscales, mat, N, K, n, b, out, best_t);
}

// ---------------------------------------------------------------------------
// NVFP4 -> FP4 layout (values unchanged)
// ---------------------------------------------------------------------------

// one thread per (matrix, row, 32-k chunk); the thread of every fourth chunk
// also moves the row's eight block scales of that 128-k group
__global__ __launch_bounds__(256) void pack_nvfp4_kernel(const uint8_t *__restrict__ codes,
                                                         const uint8_t *__restrict__ scales,
                                                         const float *__restrict__ s2in, int64_t n_mat, int N, int K,
                                                         uint8_t *__restrict__ dcodes, uint8_t *__restrict__ dscales,
                                                         float *__restrict__ ds2)
{
    const int nc = K / 32;
    const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (size_t)n_mat * N * nc) return;
    const int c = (int)(idx % nc);
    const size_t rg = idx / nc;
    const int n = (int)(rg % N);
    const size_t mat = rg / N;
    if (n == 0 && c == 0) ds2[mat] = s2in[mat];
    const int tile = n / 64, r = n % 64;
    const uint4 v = reinterpret_cast<const uint4 *>(codes)[idx];   // chunk c of row n: 16 contiguous bytes
    reinterpret_cast<uint4 *>(dcodes + mat * (size_t)N * (K / 2))[fp4_chunk_idx(tile, c, r, K)] = v;
    if ((c & 3) == 0) {
        const uint2 sv = reinterpret_cast<const uint2 *>(scales)[idx / 4];   // 8 scales of group c / 4
        reinterpret_cast<uint2 *>(dscales + mat * (size_t)N * (K / 16))[fp4_scale_idx(tile, c / 4, r, K)] = sv;
    }
}

int launch_pack_nvfp4(const uint8_t *codes, const uint8_t *scales, const float *s2, int64_t n_mat, int N, int K,
                      uint8_t *dc, uint8_t *ds, float *ds2, hipStream_t stream)
{
    const size_t total = (size_t)n_mat * N * (K / 32);
    hipLaunchKernelGGL(pack_nvfp4_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream, codes, scales,
                       s2, n_mat, N, K, dc, ds, ds2);
    return check_launch("pack_nvfp4_kernel");
}

int launch_remap_mxfp4(const uint8_t *codes, const uint8_t *escales, int64_t n_mat, int N, int K, int balance,
                       uint32_t *wc, uint8_t *wsc, float *ws2, hipStream_t stream)
{
    int32_t *emax = reinterpret_cast<int32_t *>(ws2);   // the int lives in the output slot until the last step
    const unsigned mb = (unsigned)((n_mat + 255) / 256);
    hipLaunchKernelGGL(mx_emax_init_kernel, dim3(mb), dim3(256), 0, stream, emax, n_mat);
    int rc = check_launch("mx_emax_init_kernel");
    if (rc != MOET_OK) return rc;
    hipLaunchKernelGGL(mx_emax_kernel, dim3((unsigned)n_mat, kMxSlices), dim3(kScanThreads), 0, stream, codes, escales,
                       N, K, emax);
    rc = check_launch("mx_emax_kernel");
    if (rc != MOET_OK) return rc;
    const size_t total = (size_t)n_mat * N * (K / 32);
    hipLaunchKernelGGL(mx_remap_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream, codes, escales,
                       n_mat, N, K, (const int32_t *)emax, balance, wc, wsc);
    rc = check_launch("mx_remap_kernel");
    if (rc != MOET_OK) return rc;
    hipLaunchKernelGGL(mx_scale_final_kernel, dim3(mb), dim3(256), 0, stream, ws2, n_mat);
    return check_launch("mx_scale_final_kernel");
}

int launch_requant_fp8(const uint8_t *w, const float *bs, int64_t n_mat, int N, int K, int balance, uint32_t *wc,
                       uint8_t *wsc, float *ws2, hipStream_t stream)
{
    int32_t *pmax = reinterpret_cast<int32_t *>(ws2);   // the int lives in the output slot until the last step
    const unsigned mb = (unsigned)((n_mat + 255) / 256);
    hipLaunchKernelGGL(fp8_p_init_kernel, dim3(mb), dim3(256), 0, stream, pmax, n_mat);
    int rc = check_launch("fp8_p_init_kernel");
    if (rc != MOET_OK) return rc;
    hipLaunchKernelGGL(fp8_p_kernel, dim3((unsigned)n_mat, kMxSlices), dim3(kScanThreads), 0, stream, w, bs, N, K, pmax);
    rc = check_launch("fp8_p_kernel");
    if (rc != MOET_OK) return rc;
    const size_t total = (size_t)n_mat * N * (K / 32);
    hipLaunchKernelGGL(fp8_requant_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream, w, bs, n_mat,
                       N, K, (const int32_t *)pmax, balance, wc, wsc);
    rc = check_launch("fp8_requant_kernel");
    if (rc != MOET_OK) return rc;
    hipLaunchKernelGGL(fp8_scale_final_kernel, dim3(mb), dim3(256), 0, stream, ws2, n_mat);
    return check_launch("fp8_scale_final_kernel");
}

}  // namespace moet
