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
#include "moet_common.h"

namespace moet {

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


__global__ __launch_bounds__(256) void requant_kernel(const uint8_t *__restrict__ codes,
                                                      const uint8_t *__restrict__ scales,
                                                      const float *__restrict__ s2in, int64_t n_mat, int N, int K,
                                                      uint32_t *__restrict__ wcodes, uint8_t *__restrict__ wscales,
                                                      float *__restrict__ ws2, int balance)
{
    const int nb = K / 32;
    const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
    const size_t total = (size_t)n_mat * N * nb;
    if (idx >= total) return;
    const int b = (int)(idx % nb);
    const size_t rg = idx / nb;
    const int n = (int)(rg % N);
    const size_t mat = rg / N;
    if (n == 0 && b == 0) ws2[mat] = 2.0f * s2in[mat];

    const uint4 cw = *reinterpret_cast<const uint4 *>(codes + (mat * N + n) * (size_t)(K / 2) + 16 * (size_t)b);
    const uint32_t sw = *reinterpret_cast<const uint16_t *>(scales + (mat * N + n) * (size_t)(K / 16) + 2 * (size_t)b);
    const int S9[2] = {e4m3_x512(sw & 0x7F), e4m3_x512((sw >> 8) & 0x7F)};
    const uint32_t words[4] = {cw.x, cw.y, cw.z, cw.w};

    // histogram of magnitudes per 16-half
    int cnt[2][8];
    int amax = 0;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const uint32_t m0 = words[2 * h] & 0x77777777u, m1 = words[2 * h + 1] & 0x77777777u;
#pragma unroll
        for (int L = 1; L < 8; ++L) {
            cnt[h][L] = count_nibbles_eq(m0, L) + count_nibbles_eq(m1, L);
            if (cnt[h][L]) amax = max(amax, mag2_of(L) * S9[h]);
        }
        cnt[h][0] = 16;
#pragma unroll
        for (int L = 1; L < 8; ++L) cnt[h][0] -= cnt[h][L];
    }

    // Err(a) with the bins split at the level boundary: a bin (value y, count
    // c) sits on level 1 iff 2y <= 5a (then (y-a)^2 <= (y-4a)^2), so with
    // S1, C1 the sums of c*y and c over level-1 bins and S4, C4 over level-4
    // bins,
    //   Err(a) = sum c*y^2 - 2a (S1 + 4 S4) + a^2 (zeros + C1 + 16 C4),
    // the same exact integer as the per-bin sum (every product and partial
    // sum is an integer below 2^53, so float64 holds it exactly).
    int best_t = 0;
    if (amax > 0) {
        const int t_lo = e4m3_floor_code(amax / 512);
        const int t_hi = e4m3_ceil_code((amax + 3) / 4);
        int yv[14], cy[14], cc[14];
        double y2 = 0.0;
        int stot = 0, ctot = 0;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int L = 1; L < 8; ++L) {
                const int i = 7 * h + L - 1;
                yv[i] = mag2_of(L) * S9[h];                    // < 2^22
                cc[i] = cnt[h][L];
                cy[i] = cc[i] * yv[i];                         // < 2^27
                y2 = fma((double)cy[i], (double)yv[i], y2);    // < 2^49, exact
                stot += cy[i];
                ctot += cc[i];
            }
        const int nzero = cnt[0][0] + cnt[1][0];
        double best_err = -1.0;
        for (int t = t_lo; t <= t_hi; ++t) {
            const int ai = 4 * e4m3_x512(t);                   // < 2^20
            int s1 = 0, c1 = 0;
#pragma unroll
            for (int i = 0; i < 14; ++i) {
                const bool l1 = 2 * yv[i] <= 5 * ai;
                s1 += l1 ? cy[i] : 0;
                c1 += l1 ? cc[i] : 0;
            }
            const int lin = s1 + 4 * (stot - s1);              // < 2^29
            const int quad = nzero + c1 + 16 * (ctot - c1);    // <= 512
            const double ad = (double)ai;
            const double err = fma(ad * ad, (double)quad, fma(-2.0 * ad, (double)lin, y2));
            if (best_err < 0.0 || err < best_err) {   // ascending scan: ties keep the smaller scale
                best_err = err;
                best_t = t;
            }
        }
    }
    const int a = 4 * e4m3_x512(best_t);

    // element codes -> two output words (k = 32b .. 32b+31 = words 2b, 2b+1)
    uint32_t out[2] = {0, 0};
    int zeros = 0;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const uint32_t nib = (words[2 * half + (e >> 3)] >> (4 * (e & 7))) & 15u;
            const int y = mag2_of(nib & 7) * S9[half];
            const uint32_t m = (2 * y > 5 * a) ? 1u : 0u;
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
    const int a = 4 * e4m3_x512(tau);

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
            int lvl = m ? 4 * a : a;
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

int launch_requant(const uint8_t *codes, const uint8_t *scales, const float *s2, int64_t n_mat, int N, int K,
                   uint32_t *wc, uint8_t *wsc, float *ws2, const int32_t *sel, int64_t n_sel, uint8_t *dc,
                   uint8_t *ds, float *ds2, int balance, hipStream_t stream)
{
    const size_t total = (size_t)n_mat * N * (K / 32);
    const size_t blocks = (total + 255) / 256;
    hipLaunchKernelGGL(requant_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, codes, scales, s2, n_mat, N, K,
                       wc, wsc, ws2, balance);
    int rc = check_launch("requant_kernel");
    if (rc != MOET_OK || n_sel == 0) return rc;
    const size_t dtotal = (size_t)n_sel * N * (K / 32);
    const size_t dblocks = (dtotal + 255) / 256;
    hipLaunchKernelGGL(delta_kernel, dim3((unsigned)dblocks), dim3(256), 0, stream, codes, scales, s2, n_mat, N, K,
                       (const uint32_t *)wc, (const uint8_t *)wsc, sel, n_sel, dc, ds, ds2);
    return check_launch("delta_kernel");
}

}  // namespace moet
