// Load-time NVFP4 -> sign-symmetric 2-bit requantisation and FP4 delta build.
//
// Method: README "Frontier MoE on consumer Blackwell (SM120)", sections
// "GLM-5.2 (753B) — the headline model" (modelopt NVFP4 experts requantised
// at load, exactly) and "How it fits — 2-bit experts at FP4 quality"
// (codebook {-4,-1,1,4}; FP4 delta for cached experts).
//
// Every NVFP4 value is an integer multiple of u = 2^-10 * scale_2:
// |Y| = (2|e2m1|) * (e4m3 * 2^9) < 2^22.  With the output tensor scale
// 2 * scale_2, a candidate e4m3 block scale t has level-1 magnitude
// a = 4 * (e4m3(t) * 2^9) in the same unit, so the block error
//   Err(t) = sum_i min((|Y_i| - a)^2, (|Y_i| - 4a)^2)
// is an integer below 2^51 and float64 evaluates it exactly.
//
// Search window: Err is continuous and piecewise quadratic in a; for
// a > amax every term is (|Y|-a)^2 and increases, and for a < amax/128 the
// largest element's slope -8(amax - 4a) outweighs the at most 31*12a of the
// others, so Err decreases.  The exact minimiser over the grid therefore lies
// between the last grid point <= amax/128 and the first grid point >= amax,
// and strict monotonicity outside keeps the "smallest scale on ties" rule.
// One thread handles one 32-weight block; the 32 magnitudes collapse to at
// most 16 distinct values (two 16-blocks x 8 e2m1 magnitudes), counted with
// nibble SWAR tricks.
//
// Per-tensor codebook pick (README "How it fits": nearly every tensor picks
// {-4,-1,1,4}): codebook c has level magnitudes {lo_c, hi_c} times the block
// scale and tensor scale 2^j_c * scale_2 -- c = 0: {1, 4}, j = 1; c = 1:
// {1/2, 3}, j = 1; c = 2: {0, 2}, j = 2 -- so in units of u the levels of
// scale code t are LO = lo2_c * T << j_c and HI = hi2_c * T << j_c (T =
// e4m3(t) * 2^9, lo2/hi2 = 2 lo / 2 hi), an element takes HI iff
// 2|Y| > LO + HI, and the block error is exact in float64 as above.  With
// MOET_PICK_CODEBOOK a first pass sums every block's smallest error per
// codebook per matrix (exact integer sums: workgroup sums below 2^60, split
// into 32-bit halves and added with 64-bit integer atomics into the head of
// the matrix's output code plane, which the requant pass overwrites), a
// second pass picks the codebook with the smallest total (ties to the lower
// index), and the requant pass writes the codes of each matrix's codebook.
// Each codebook has its own search window, by the argument above: below the
// window the largest element's slope, -2 hi (amax - HI) in units of the
// scale, outweighs the at most 31 max(2 lo^2, hi (hi - lo)) of the others
// (codebook 0: below amax/50; 1: amax/41; 2: amax/33, taken with margin as
// the code with a <= amax/128, amax/64, amax/64, a = 4 T, 4 T, 8 T), so Err
// falls there; above it every element sits on LO and Err rises (LO >= amax,
// codebooks 0 and 1) or is constant at sum y^2 (HI >= 2 amax, codebook 2,
// whose LO is 0), which the smallest-scale tie rule settles at the window's
// end.  Windows in T: [amax/512, amax/4], [amax/256, amax/2], [amax/512,
// amax/8].
#include "moet_common.h"

namespace moet {

constexpr int kNumCodebooks = 3;
__device__ __forceinline__ int cb_lo2(int c) { return c == 0 ? 2 : c == 1 ? 1 : 0; }
__device__ __forceinline__ int cb_hi2(int c) { return c == 0 ? 8 : c == 1 ? 6 : 4; }
__device__ __forceinline__ int cb_j(int c) { return c == 2 ? 2 : 1; }

__device__ __forceinline__ int e4m3_floor_code(int u)  // largest t with e4m3_x512(t) <= u, u >= 0
{
    if (u >= 448 * 512) return 126;
    if (u < 8) return u;
    int ef = 31 - __clz(u);
    int e = ef - 2;
    int m = (u >> (e - 1)) - 8;
    return 8 * e + m;
}

__device__ __forceinline__ int e4m3_ceil_code(int u)   // smallest t with e4m3_x512(t) >= u
{
    int t = e4m3_floor_code(u);
    if (e4m3_x512(t) < u && t < 126) ++t;
    return t;
}

// number of nibbles of w (magnitudes only, bit 3 cleared) equal to L
__device__ __forceinline__ int count_nibbles_eq(uint32_t mags, uint32_t L)
{
    uint32_t x = mags ^ (L * 0x11111111u);               // zero nibble <=> equal
    uint32_t nz = ((x & 0x77777777u) + 0x77777777u) | x;  // bit 3 set iff nibble != 0
    return __popc(~nz & 0x88888888u);
}

__device__ __forceinline__ int mag2_of(int L)  // 2*|e2m1| for magnitude code L in 0..7
{
    return L < 2 ? L : ((2 + (L & 1)) << ((L >> 1) - 1));
}


// The 32 magnitudes of one block as at most 14 distinct non-zero bins (value in
// units of u, count) plus the zero count, and the largest magnitude.
struct BlockBins {
    int yv[14], cc[14], cy[14];
    double y2;              // sum c*y^2 (< 2^49, exact)
    int stot, ctot, nzero, amax;
};

__device__ __forceinline__ void block_bins(const uint32_t words[4], const int S9[2], BlockBins &bb)
{
    int cnt[2][8];
    bb.amax = 0;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const uint32_t m0 = words[2 * h] & 0x77777777u, m1 = words[2 * h + 1] & 0x77777777u;
#pragma unroll
        for (int L = 1; L < 8; ++L) {
            cnt[h][L] = count_nibbles_eq(m0, L) + count_nibbles_eq(m1, L);
            if (cnt[h][L]) bb.amax = max(bb.amax, mag2_of(L) * S9[h]);
        }
        cnt[h][0] = 16;
#pragma unroll
        for (int L = 1; L < 8; ++L) cnt[h][0] -= cnt[h][L];
    }
    bb.y2 = 0.0;
    bb.stot = bb.ctot = 0;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int L = 1; L < 8; ++L) {
            const int i = 7 * h + L - 1;
            bb.yv[i] = mag2_of(L) * S9[h];                    // < 2^22
            bb.cc[i] = cnt[h][L];
            bb.cy[i] = bb.cc[i] * bb.yv[i];                   // < 2^27
            bb.y2 = fma((double)bb.cy[i], (double)bb.yv[i], bb.y2);
            bb.stot += bb.cy[i];
            bb.ctot += bb.cc[i];
        }
    bb.nzero = cnt[0][0] + cnt[1][0];
}

// Err for levels LO = lo2 a, HI = hi2 a (a = T << j) with the bins split at the
// level boundary: a bin (value y, count c) sits on LO iff 2y <= LO + HI (then
// (y-LO)^2 <= (y-HI)^2), so with S_lo, C_lo the sums of c*y and c over the LO
// bins and S_hi, C_hi over the HI bins,
//   Err = sum c*y^2 - 2a (lo2 S_lo + hi2 S_hi) + a^2 (lo2^2 (zeros + C_lo) + hi2^2 C_hi),
// the same exact integer as the per-bin sum: the two bracketed sums are
// integers (< 2^30 and <= 2048) and every product and partial sum is an
// integer below 2^53, so float64 holds it exactly.
template <int C>
__device__ __forceinline__ double block_err(const BlockBins &bb, int a)
{
    constexpr int lo2 = C == 0 ? 2 : C == 1 ? 1 : 0, hi2 = C == 0 ? 8 : C == 1 ? 6 : 4;
    int slo = 0, clo = 0;
#pragma unroll
    for (int i = 0; i < 14; ++i) {
        const bool l = 2 * bb.yv[i] <= (lo2 + hi2) * a;
        slo += l ? bb.cy[i] : 0;
        clo += l ? bb.cc[i] : 0;
    }
    const int lin = lo2 * slo + hi2 * (bb.stot - slo);                                  // < 2^30
    const int quad = lo2 * lo2 * (bb.nzero + clo) + hi2 * hi2 * (bb.ctot - clo);        // <= 2048
    const double ad = (double)a;                                                        // < 2^20
    return fma(ad * ad, (double)quad, fma(-2.0 * ad, (double)lin, bb.y2));
}

// Smallest-error scale code of codebook C (ties: the smaller code) and its error.
template <int C>
__device__ __forceinline__ int block_best(const BlockBins &bb, double &best_err)
{
    best_err = 0.0;
    if (bb.amax == 0) return 0;   // every level of scale 0 is exact
    int t_lo, t_hi;
    if constexpr (C == 0) {
        t_lo = e4m3_floor_code(bb.amax / 512);
        t_hi = e4m3_ceil_code((bb.amax + 3) / 4);
    } else if constexpr (C == 1) {
        t_lo = e4m3_floor_code(bb.amax / 256);
        t_hi = e4m3_ceil_code((bb.amax + 1) / 2);
    } else {
        t_lo = e4m3_floor_code(bb.amax / 512);
        t_hi = e4m3_ceil_code((bb.amax + 7) / 8);
    }
    constexpr int j = C == 2 ? 2 : 1;
    int best_t = t_lo;
    best_err = -1.0;
    for (int t = t_lo; t <= t_hi; ++t) {
        const double err = block_err<C>(bb, e4m3_x512(t) << j);
        if (best_err < 0.0 || err < best_err) {   // ascending scan: ties keep the smaller scale
            best_err = err;
            best_t = t;
        }
    }
    return best_t;
}

__device__ __forceinline__ int block_best_of(const BlockBins &bb, int c, double &err)
{
    if (c == 0) return block_best<0>(bb, err);
    if (c == 1) return block_best<1>(bb, err);
    return block_best<2>(bb, err);
}

__device__ __forceinline__ void load_block(const uint8_t *codes, const uint8_t *scales, size_t mat, int N, int K, int n,
                                           int b, uint32_t words[4], int S9[2])
{
    const uint4 cw = *reinterpret_cast<const uint4 *>(codes + (mat * N + n) * (size_t)(K / 2) + 16 * (size_t)b);
    const uint32_t sw = *reinterpret_cast<const uint16_t *>(scales + (mat * N + n) * (size_t)(K / 16) + 2 * (size_t)b);
    S9[0] = e4m3_x512(sw & 0x7F);
    S9[1] = e4m3_x512((sw >> 8) & 0x7F);
    words[0] = cw.x;
    words[1] = cw.y;
    words[2] = cw.z;
    words[3] = cw.w;
}

// the per-matrix error sums of the pick, in the head of the matrix's output code plane:
// [codebook][lo 32 bits, hi bits] as uint64
__device__ __forceinline__ unsigned long long *pick_sums(uint32_t *wcodes, size_t mat, int N, int K)
{
    return reinterpret_cast<unsigned long long *>(wcodes + mat * (size_t)N * (K / 16));
}

__global__ __launch_bounds__(256) void pick_clear_kernel(uint32_t *__restrict__ wcodes, int64_t n_mat, int N, int K)
{
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (size_t)n_mat * 2 * kNumCodebooks) return;
    pick_sums(wcodes, i / (2 * kNumCodebooks), N, K)[i % (2 * kNumCodebooks)] = 0ull;
}

// every block's smallest error per codebook, summed per matrix (a workgroup's 256 blocks lie in
// one matrix: N * K / 32 is a multiple of 256)
__global__ __launch_bounds__(256) void pick_err_kernel(const uint8_t *__restrict__ codes,
                                                       const uint8_t *__restrict__ scales, int64_t n_mat, int N, int K,
                                                       uint32_t *__restrict__ wcodes)
{
    __shared__ unsigned long long part[4][kNumCodebooks];
    const int nb = K / 32;
    const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
    const size_t total = (size_t)n_mat * N * nb;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    unsigned long long e[kNumCodebooks] = {0ull, 0ull, 0ull};
    size_t mat = 0;
    if (idx < total) {
        const int b = (int)(idx % nb);
        const size_t rg = idx / nb;
        const int n = (int)(rg % N);
        mat = rg / N;
        uint32_t words[4];
        int S9[2];
        load_block(codes, scales, mat, N, K, n, b, words, S9);
        BlockBins bb;
        block_bins(words, S9, bb);
        double err;
        block_best<0>(bb, err);
        e[0] = (unsigned long long)err;   // exact integers < 2^51
        block_best<1>(bb, err);
        e[1] = (unsigned long long)err;
        block_best<2>(bb, err);
        e[2] = (unsigned long long)err;
    }
#pragma unroll
    for (int c = 0; c < kNumCodebooks; ++c) {
        unsigned long long v = e[c];
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
        if (lane == 0) part[wave][c] = v;
    }
    __syncthreads();
    if (threadIdx.x < kNumCodebooks && (size_t)blockIdx.x * 256 < total) {
        const int c = threadIdx.x;
        const unsigned long long v = part[0][c] + part[1][c] + part[2][c] + part[3][c];   // < 2^59
        const size_t m = ((size_t)blockIdx.x * 256) / nb / N;
        unsigned long long *sum = pick_sums(wcodes, m, N, K);
        atomicAdd(sum + 2 * c, v & 0xFFFFFFFFull);
        atomicAdd(sum + 2 * c + 1, v >> 32);
    }
}

// codebook of each matrix: the smallest total (sum = hi * 2^32 + lo, compared exactly), ties lower
__global__ __launch_bounds__(256) void pick_choose_kernel(const uint32_t *__restrict__ wcodes, int64_t n_mat, int N,
                                                          int K, uint8_t *__restrict__ cbook)
{
    const size_t m = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (m >= (size_t)n_mat) return;
    const unsigned long long *sum =
        reinterpret_cast<const unsigned long long *>(wcodes + m * (size_t)N * (K / 16));
    int best = 0;
    unsigned long long bhi = 0, blo = 0;
    for (int c = 0; c < kNumCodebooks; ++c) {
        // normalise lo < 2^32 (the carries of the lo sums into hi)
        const unsigned long long lo = sum[2 * c] & 0xFFFFFFFFull, hi = sum[2 * c + 1] + (sum[2 * c] >> 32);
        if (c == 0 || hi < bhi || (hi == bhi && lo < blo)) {
            best = c;
            bhi = hi;
            blo = lo;
        }
    }
    cbook[m] = (uint8_t)best;
}

// PICK: each matrix's codebook comes from cbook (else codebook 0 everywhere)
template <bool PICK>
__global__ __launch_bounds__(256) void requant_kernel(const uint8_t *__restrict__ codes,
                                                      const uint8_t *__restrict__ scales,
                                                      const float *__restrict__ s2in, int64_t n_mat, int N, int K,
                                                      uint32_t *__restrict__ wcodes, uint8_t *__restrict__ wscales,
                                                      float *__restrict__ ws2, const uint8_t *__restrict__ cbook,
                                                      int balance)
{
    const int nb = K / 32;
    const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
    const size_t total = (size_t)n_mat * N * nb;
    if (idx >= total) return;
    const int b = (int)(idx % nb);
    const size_t rg = idx / nb;
    const int n = (int)(rg % N);
    const size_t mat = rg / N;
    const int c = PICK ? min((int)cbook[mat], kNumCodebooks - 1) : 0;
    if (n == 0 && b == 0) ws2[mat] = (float)(1 << cb_j(c)) * s2in[mat];

    uint32_t words[4];
    int S9[2];
    load_block(codes, scales, mat, N, K, n, b, words, S9);
    BlockBins bb;
    block_bins(words, S9, bb);
    double err;
    const int best_t = PICK ? block_best_of(bb, c, err) : block_best<0>(bb, err);
    const int T = e4m3_x512(best_t);
    const int lo = (cb_lo2(c) * T) << cb_j(c), hi = (cb_hi2(c) * T) << cb_j(c);

    // element codes -> two output words (k = 32b .. 32b+31 = words 2b, 2b+1)
    uint32_t out[2] = {0, 0};
    int zeros = 0;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const uint32_t nib = (words[2 * half + (e >> 3)] >> (4 * (e & 7))) & 15u;
            const int y = mag2_of(nib & 7) * S9[half];
            const uint32_t m = (2 * y > lo + hi) ? 1u : 0u;
            const uint32_t s = (balance && y == 0) ? (uint32_t)(zeros++ & 1) : nib >> 3;
            out[half] |= (m << mbit(e)) | (s << sbit(e));
        }
    }
    store_w2_block(wcodes, wscales, mat, N, K, n, b, out, best_t);
}

// FP4 re-encoding of the exact residual D = Y_nvfp4 - Y_2bit (units of u).
__global__ __launch_bounds__(256) void delta_kernel(const uint8_t *__restrict__ codes,
                                                    const uint8_t *__restrict__ scales,
                                                    const float *__restrict__ s2in, int64_t n_mat, int N, int K,
                                                    const uint32_t *__restrict__ wcodes,
                                                    const uint8_t *__restrict__ wscales,
                                                    const uint8_t *__restrict__ cbook,
                                                    const int32_t *__restrict__ sel, int64_t n_sel,
                                                    uint8_t *__restrict__ dcodes, uint8_t *__restrict__ dscales,
                                                    float *__restrict__ ds2)
{
    const int nb = K / 32;
    const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
    const size_t total = (size_t)n_sel * N * nb;
    if (idx >= total) return;
    const int b = (int)(idx % nb);
    const size_t rg = idx / nb;
    const int n = (int)(rg % N);
    const size_t slot = rg / N;
    const int mat = sel[slot];
    if (mat < 0 || mat >= n_mat) return;
    if (n == 0 && b == 0) ds2[slot] = s2in[mat];

    const uint4 cw = *reinterpret_cast<const uint4 *>(codes + ((size_t)mat * N + n) * (size_t)(K / 2) + 16 * (size_t)b);
    const uint32_t sw = *reinterpret_cast<const uint16_t *>(scales + ((size_t)mat * N + n) * (size_t)(K / 16) + 2 * (size_t)b);
    const uint32_t words[4] = {cw.x, cw.y, cw.z, cw.w};
    const int tile = n / 64, r = n % 64;
    const uint32_t *wmat = wcodes + (size_t)mat * N * (K / 16);
    const uint32_t w2w[2] = {wmat[(((size_t)tile * (K / 64) + (2 * b) / 4) * 64 + r) * 4 + (2 * b) % 4],
                             wmat[(((size_t)tile * (K / 64) + (2 * b + 1) / 4) * 64 + r) * 4 + (2 * b + 1) % 4]};
    const int tau = wscales[(size_t)mat * N * (K / 32) + (((size_t)tile * (K / 128) + b / 4) * 64 + r) * 4 + (b % 4)];
    const int c = cbook ? min((int)cbook[mat], kNumCodebooks - 1) : 0;
    const int lo = (cb_lo2(c) * e4m3_x512(tau)) << cb_j(c), hi = (cb_hi2(c) * e4m3_x512(tau)) << cb_j(c);

    uint32_t out[4] = {0, 0, 0, 0};
    uint32_t sbytes = 0;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        const int S9 = e4m3_x512((sw >> (8 * half)) & 0x7F);
        int D[16];
        int M = 0;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const uint32_t nib = (words[2 * half + (e >> 3)] >> (4 * (e & 7))) & 15u;
            int y = mag2_of(nib & 7) * S9;
            if (nib & 8) y = -y;
            const uint32_t w = w2w[half];
            const int m = (w >> mbit(e)) & 1, s = (w >> sbit(e)) & 1;
            int lvl = m ? hi : lo;
            if (s) lvl = -lvl;
            D[e] = y - lvl;
            M = max(M, abs(D[e]));
        }
        // block scale: e4m3 nearest to M / 12 (in units of 2^-9), ties to the even code
        int ts = e4m3_floor_code(M / 12);
        if (ts < 126) {
            const int d0 = abs(M - 12 * e4m3_x512(ts)), d1 = abs(M - 12 * e4m3_x512(ts + 1));
            if (d1 < d0 || (d1 == d0 && ((ts + 1) & 1) == 0)) ++ts;
        }
        sbytes |= (uint32_t)ts << (8 * half);
        const int T = e4m3_x512(ts);
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            uint32_t code = 0;
            if (T > 0 && D[e] != 0) {
                const int ad2 = 2 * abs(D[e]);
                int i = 0;
                i += (ad2 > 1 * T) ? 1 : 0;                       // ties at even j stay below
                i += (ad2 >= 3 * T) ? 1 : 0;                      // ties at odd j go up
                i += (ad2 > 5 * T) ? 1 : 0;
                i += (ad2 >= 7 * T) ? 1 : 0;
                i += (ad2 > 10 * T) ? 1 : 0;
                i += (ad2 >= 14 * T) ? 1 : 0;
                i += (ad2 > 20 * T) ? 1 : 0;
                code = (uint32_t)i | (D[e] < 0 ? 8u : 0u);
            }
            const int kk = 16 * half + e;  // position in the 32-k chunk
            out[kk >> 3] |= code << (4 * (kk & 7));
        }
    }
    uint8_t *dmat = dcodes + slot * (size_t)N * (K / 2);
    *reinterpret_cast<uint4 *>(dmat + (((size_t)tile * (K / 32) + b) * 64 + r) * 16) = make_uint4(out[0], out[1], out[2], out[3]);
    uint8_t *smat = dscales + slot * (size_t)N * (K / 16);
    *reinterpret_cast<uint16_t *>(smat + (((size_t)tile * (K / 128) + b / 4) * 64 + r) * 8 + 2 * (b % 4)) = (uint16_t)sbytes;
}

__global__ __launch_bounds__(256) void cbook_fill_kernel(uint8_t *__restrict__ cbook, int64_t n_mat)
{
    const size_t m = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (m < (size_t)n_mat) cbook[m] = 0;
}

int launch_requant(const uint8_t *codes, const uint8_t *scales, const float *s2, int64_t n_mat, int N, int K,
                   uint32_t *wc, uint8_t *wsc, float *ws2, uint8_t *cbook, const int32_t *sel, int64_t n_sel,
                   uint8_t *dc, uint8_t *ds, float *ds2, int balance, int pick, hipStream_t stream)
{
    const size_t total = (size_t)n_mat * N * (K / 32);
    const size_t blocks = (total + 255) / 256;
    int rc;
    if (pick) {
        const size_t nsum = (size_t)n_mat * 2 * kNumCodebooks;
        hipLaunchKernelGGL(pick_clear_kernel, dim3((unsigned)((nsum + 255) / 256)), dim3(256), 0, stream, wc, n_mat, N, K);
        rc = check_launch("pick_clear_kernel");
        if (rc != MOET_OK) return rc;
        hipLaunchKernelGGL(pick_err_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, codes, scales, n_mat, N, K, wc);
        rc = check_launch("pick_err_kernel");
        if (rc != MOET_OK) return rc;
        hipLaunchKernelGGL(pick_choose_kernel, dim3((unsigned)((n_mat + 255) / 256)), dim3(256), 0, stream,
                           (const uint32_t *)wc, n_mat, N, K, cbook);
        rc = check_launch("pick_choose_kernel");
        if (rc != MOET_OK) return rc;
    } else if (cbook) {
        // no pick: every matrix takes codebook 0
        hipLaunchKernelGGL(cbook_fill_kernel, dim3((unsigned)((n_mat + 255) / 256)), dim3(256), 0, stream, cbook, n_mat);
        rc = check_launch("cbook_fill_kernel");
        if (rc != MOET_OK) return rc;
    }
    if (pick)
        hipLaunchKernelGGL(requant_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, stream, codes, scales, s2, n_mat,
                           N, K, wc, wsc, ws2, (const uint8_t *)cbook, balance);
    else
        hipLaunchKernelGGL(requant_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, stream, codes, scales, s2, n_mat,
                           N, K, wc, wsc, ws2, (const uint8_t *)nullptr, balance);
    rc = check_launch("requant_kernel");
    if (rc != MOET_OK || n_sel == 0) return rc;
    const size_t dtotal = (size_t)n_sel * N * (K / 32);
    const size_t dblocks = (dtotal + 255) / 256;
    hipLaunchKernelGGL(delta_kernel, dim3((unsigned)dblocks), dim3(256), 0, stream, codes, scales, s2, n_mat, N, K,
                       (const uint32_t *)wc, (const uint8_t *)wsc, (const uint8_t *)(pick ? cbook : nullptr), sel, n_sel,
                       dc, ds, ds2);
    return check_launch("delta_kernel");
}

}  // namespace moet
