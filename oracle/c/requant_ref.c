/*
 * Exact reference for the load-time NVFP4 -> sign-symmetric 2-bit
 * requantisation and for the FP4 delta (oracle; test infrastructure only).
 *
 * Sources (public description of vLLM-Moet):
 *  - README "Frontier MoE on consumer Blackwell (SM120)", section
 *    "GLM-5.2 (753B) — the headline model": NVFP4 experts (e2m1 values,
 *    e4m3 scale per 16 weights, fp32 per-tensor scale_2) are requantised at
 *    load time to sign-symmetric 2-bit planes, exactly in float64.
 *  - same README, section "How it fits — 2-bit experts at FP4 quality": the
 *    codebook is {-4,-1,1,4}, chosen at equal L2 error; an FP4 delta restores
 *    precision for experts held in a delta cache.
 *  - same README, section "Kimi-K2.7-Code (1T MoE) on 4x RTX PRO 6000": zeros
 *    exported only as +0 skew the result, so a zero takes its level from its
 *    own sign bit.
 *
 * Readings (the pages leave these open):
 *  - every NVFP4 value is an integer multiple of u = 2^-10 * scale_2:
 *    |Y| = (2|e2m1|) * (e4m3 * 2^9), |Y| < 2^22;
 *  - output per-tensor scale = 2 * scale_2; per-block e4m3 scale over
 *    B = 32 consecutive weights along K (B is a parameter here so that tiny
 *    blocks can be brute-forced); the level-1 magnitude of candidate scale code
 *    t is a = 4 * (e4m3(t) * 2^9) in units of u;
 *  - the block scale minimises the exact L2 error
 *        Err(t) = sum_i min((|Y_i| - a)^2, (|Y_i| - 4a)^2)
 *    over all finite non-negative e4m3 codes t = 0x00..0x7E, ties -> smaller t;
 *  - element code = (s << 1) | m with s = the NVFP4 sign bit (also for -0) and
 *    m = 1 iff 2|Y| > 5a (a tie keeps magnitude 1); levels: 0:+1 1:+4 2:-1 3:-4;
 *  - zero-sign balancing (same README, section "Kimi-K2.7-Code (1T MoE) on
 *    4x RTX PRO 6000": an export that writes every exact zero as +0 biases the
 *    2-bit weights, and the fix balances the zero signs): when asked for, the
 *    zeros of a block take alternating signs in k order, the first one +, and
 *    the source sign bit of a zero is ignored.  Zeros cost a^2 whatever their
 *    sign, so the block scale does not change;
 *  - per-tensor codebook pick (same README, section "How it fits": the
 *    sign-symmetric {-4,-1,1,4} is picked by nearly every tensor): a tensor
 *    may instead use one of two other sign-symmetric four-level codebooks whose
 *    levels are FP4 values.  Codebook c has magnitudes {lo_c, hi_c} times the
 *    block scale and tensor scale 2^j_c * scale_2:
 *        c = 0: {1, 4}, j = 1;   c = 1: {1/2, 3}, j = 1;   c = 2: {0, 2}, j = 2
 *    (j_c is the smallest power of two with hi_c * 448 * 2^j_c >= 6 * 448, so
 *    the largest NVFP4 value stays in range).  In units of u the two level
 *    magnitudes of scale code t are LO = lo2_c * T9[t] << j_c and
 *    HI = hi2_c * T9[t] << j_c with lo2/hi2 = 2 lo / 2 hi = (2, 8), (1, 6),
 *    (0, 4); the block error is sum_i min((|Y_i| - LO)^2, (|Y_i| - HI)^2) and
 *    an element takes HI iff 2|Y| > LO + HI.  Codebook 0 is the method's
 *    default; the tensor-level pick (smallest exact total error, ties to the
 *    lower c) is made by the caller from the per-block errors;
 *  - delta D = Y_nvfp4 - Y_2bit (exact integer in units of u), re-encoded as
 *    NVFP4 with the source scale_2: block-16 scale = e4m3 nearest (ties to the
 *    even code, saturating at 448) to max|D| / (6 * 2^10); element = e2m1
 *    nearest (ties to the even code, saturating at 6) to D / (2 * e4m3*2^9);
 *    a value rounding to zero keeps the sign of D; D == 0 gives +0.
 *
 * All arithmetic is int64 and exact.  OpenMP parallelises over rows only.
 */
#include <stdint.h>
#include <math.h>
#include <stdlib.h>

/* e4m3fn value * 2^9 for the finite non-negative codes 0x00..0x7E. */
static int64_t e4m3_x512(int t)
{
    int e = (t >> 3) & 15, m = t & 7;
    if (e == 0)
        return m;                       /* m/8 * 2^-6 * 2^9 */
    return (int64_t)(8 + m) << (e - 1); /* (1 + m/8) * 2^(e-7) * 2^9 */
}

/* 2 * |e2m1| for the magnitude bits of a 4-bit code. */
static int64_t e2m1_mag2(int c)
{
    int e = (c >> 1) & 3, m = c & 1;
    if (e == 0)
        return m;                       /* 0 or 0.5, doubled */
    return (int64_t)(2 + m) << (e - 1); /* (1 + m/2) * 2^(e-1), doubled */
}

static inline int nib(const uint8_t *row, int64_t k)
{
    uint8_t b = row[k >> 1];
    return (k & 1) ? (b >> 4) : (b & 15);
}

/* level magnitudes (doubled) and tensor-scale exponent of codebook c */
static const int64_t CB_LO2[3] = {2, 1, 0}, CB_HI2[3] = {8, 6, 4};
static const int CB_J[3] = {1, 1, 2};

/* Returns 0 on success, -1 if a block scale byte is negative or NaN or the
 * codebook index is not 0, 1 or 2. */
int oracle_requant(const uint8_t *codes, const uint8_t *scales, int64_t N, int64_t K,
                   int64_t B, int balance, int cb, uint8_t *codes2, uint8_t *tau, int64_t *err_out)
{
    if (cb < 0 || cb > 2)
        return -1;
    int64_t T9[127];
    for (int t = 0; t < 127; ++t)
        T9[t] = e4m3_x512(t);
    const int64_t lo2 = CB_LO2[cb], hi2 = CB_HI2[cb];
    const int j = CB_J[cb];
    int bad = 0;
    const int64_t nb = K / B;
#pragma omp parallel for schedule(dynamic, 4) reduction(| : bad)
    for (int64_t n = 0; n < N; ++n) {
        const uint8_t *crow = codes + n * (K / 2);
        const uint8_t *srow = scales + n * (K / 16);
        int64_t *y = (int64_t *)malloc(sizeof(int64_t) * B);
        for (int64_t b = 0; b < nb; ++b) {
            for (int64_t i = 0; i < B; ++i) {
                int64_t k = b * B + i;
                int sb = srow[k / 16];
                if (sb >= 0x7F) { bad = 1; sb = 0; }
                y[i] = e2m1_mag2(nib(crow, k) & 7) * T9[sb];
            }
            int best_t = 0;
            int64_t best_err = -1;
            for (int t = 0; t < 127; ++t) {
                int64_t lo = (lo2 * T9[t]) << j, hi = (hi2 * T9[t]) << j;
                int64_t e = 0;
                for (int64_t i = 0; i < B; ++i) {
                    int64_t d1 = y[i] - lo, d4 = y[i] - hi;
                    int64_t q1 = d1 * d1, q4 = d4 * d4;
                    e += q1 < q4 ? q1 : q4;
                }
                if (best_err < 0 || e < best_err) {
                    best_err = e;
                    best_t = t;
                }
            }
            tau[n * nb + b] = (uint8_t)best_t;
            if (err_out)
                err_out[n * nb + b] = best_err;
            int64_t lo = (lo2 * T9[best_t]) << j, hi = (hi2 * T9[best_t]) << j;
            int zeros = 0;
            for (int64_t i = 0; i < B; ++i) {
                int64_t k = b * B + i;
                int s = (nib(crow, k) >> 3) & 1;
                if (balance && y[i] == 0)
                    s = (zeros++) & 1;
                int m = (2 * y[i] > lo + hi) ? 1 : 0;
                codes2[n * K + k] = (uint8_t)((s << 1) | m);
            }
        }
        free(y);
    }
    return bad ? -1 : 0;
}

/* FP4 re-encoding of the exact residual; dcodes gets one 4-bit code per weight.
 * cb: the codebook the 2-bit codes use. */
int oracle_delta(const uint8_t *codes, const uint8_t *scales, int64_t N, int64_t K, int64_t B, int cb,
                 const uint8_t *codes2, const uint8_t *tau, uint8_t *dcodes, uint8_t *dscales)
{
    if (cb < 0 || cb > 2)
        return -1;
    const int64_t lo2 = CB_LO2[cb], hi2 = CB_HI2[cb];
    const int j = CB_J[cb];
    int64_t T9[127];
    for (int t = 0; t < 127; ++t)
        T9[t] = e4m3_x512(t);
    static const int64_t thr2[7] = {1, 3, 5, 7, 10, 14, 20}; /* 2 * e2m1 midpoints, doubled */
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 4) reduction(| : bad)
    for (int64_t n = 0; n < N; ++n) {
        const uint8_t *crow = codes + n * (K / 2);
        const uint8_t *srow = scales + n * (K / 16);
        int64_t D[16];
        for (int64_t g = 0; g < K / 16; ++g) {
            int64_t M = 0;
            for (int i = 0; i < 16; ++i) {
                int64_t k = g * 16 + i;
                int c = nib(crow, k);
                int sb = srow[k / 16];
                if (sb >= 0x7F) { bad = 1; sb = 0; }
                int64_t y = e2m1_mag2(c & 7) * T9[sb];
                if (c & 8)
                    y = -y;
                int c2 = codes2[n * K + k];
                int64_t T = T9[tau[n * (K / B) + k / B]];
                int64_t lvl = ((c2 & 1) ? hi2 * T : lo2 * T) << j;   /* level magnitude in units of u */
                if (c2 & 2)
                    lvl = -lvl;
                D[i] = y - lvl;
                int64_t ad = D[i] < 0 ? -D[i] : D[i];
                if (ad > M)
                    M = ad;
            }
            /* nearest e4m3 to M / (6 * 2^10): compare M with 12 * T9 (same units) */
            int ts = 0;
            int64_t bd = -1;
            for (int t = 0; t < 127; ++t) {
                int64_t d = M - 12 * T9[t];
                if (d < 0)
                    d = -d;
                if (bd < 0 || d < bd || (d == bd && (t & 1) == 0 && (ts & 1) == 1)) {
                    bd = d;
                    ts = t;
                }
            }
            dscales[n * (K / 16) + g] = (uint8_t)ts;
            int64_t T = T9[ts];
            for (int i = 0; i < 16; ++i) {
                int64_t k = g * 16 + i;
                int code = 0;
                if (T > 0 && D[i] != 0) {
                    int64_t ad2 = 2 * (D[i] < 0 ? -D[i] : D[i]);
                    int idx = 0;
                    for (int j = 0; j < 7; ++j)
                        if (ad2 > thr2[j] * T || (ad2 == thr2[j] * T && (j & 1)))
                            idx = j + 1;
                    code = idx | (D[i] < 0 ? 8 : 0);
                }
                dcodes[n * K + k] = (uint8_t)code;
            }
        }
    }
    return bad ? -1 : 0;
}

/*
 * FP8 block-quantised source (README "Frontier MoE on consumer Blackwell
 * (SM120)", section "How it fits — 2-bit experts at FP4 quality": FP8
 * block-quant checkpoints are requantised to the same sign-symmetric codebook
 * at load, in float64).  Readings taken where the pages say no more:
 *  - source: e4m3fn weights [N][K] and one fp32 scale per 128 x 128 block,
 *    [ceil(N/128)][K/128]; weight = e4m3(code) * scale;
 *  - the 2-bit tensor scale is a power of two, S = 2^p with p the smallest
 *    integer >= -149 (so that S is a float32) such that 4 * 448 * S >= amax
 *    (the largest level at the largest e4m3 block scale covers the largest
 *    weight), S = 1 for an all-zero tensor;
 *  - per block of B weights along K the e4m3 scale t minimises
 *        Err(t) = sum_i min((y_i - a)^2, (y_i - 4a)^2),  a = e4m3(t) * S,
 *    y_i = |weight|, evaluated in float64 in this order: d1 = y - a,
 *    d4 = y - 4a, q = min(d1*d1, d4*d4), Err += q for i = 0..B-1 in k order,
 *    over every finite code t = 0x00..0x7E, ties -> smaller t.  y_i and a are
 *    exact in float64; the squares and the sum are rounded, so the decision is
 *    the one this float64 evaluation makes;
 *  - element code as for NVFP4: m = 1 iff 2y > 5a (exact), sign from the e4m3
 *    sign bit, or balanced zeros when asked for.
 * Returns 0, or -1 for a NaN weight code or a negative / non-finite block
 * scale.  Compile with -ffp-contract=off.
 */
static double e4m3_f64(int t) { return (double)e4m3_x512(t) / 512.0; }

int oracle_requant_fp8(const uint8_t *w, const float *bscale, int64_t N, int64_t K, int64_t B,
                       int balance, uint8_t *codes2, uint8_t *tau, float *scale2_out)
{
    const int64_t KB = K / 128;
    double amax = 0.0;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            int c = w[n * K + k] & 0x7F;
            float s = bscale[(n / 128) * KB + k / 128];
            if (c == 0x7F || !(s >= 0.0f) || s > 3.4028235e38f)
                return -1;
            double y = e4m3_f64(c) * (double)s;
            if (y > amax)
                amax = y;
        }
    int p = 0;
    if (amax > 0.0) {
        p = -149;
        while (1792.0 * ldexp(1.0, p) < amax)
            ++p;
    }
    const double S = ldexp(1.0, p);
    *scale2_out = (float)S;
    const int64_t nb = K / B;
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t n = 0; n < N; ++n) {
        double *y = (double *)malloc(sizeof(double) * B);
        for (int64_t b = 0; b < nb; ++b) {
            for (int64_t i = 0; i < B; ++i) {
                int64_t k = b * B + i;
                y[i] = e4m3_f64(w[n * K + k] & 0x7F) * (double)bscale[(n / 128) * KB + k / 128];
            }
            int best_t = 0;
            double best_err = -1.0;
            for (int t = 0; t < 127; ++t) {
                double a = e4m3_f64(t) * S;
                double a4 = 4.0 * a;
                double e = 0.0;
                for (int64_t i = 0; i < B; ++i) {
                    double d1 = y[i] - a, d4 = y[i] - a4;
                    double q1 = d1 * d1, q4 = d4 * d4;
                    e += q1 < q4 ? q1 : q4;
                }
                if (best_err < 0.0 || e < best_err) {
                    best_err = e;
                    best_t = t;
                }
            }
            tau[n * nb + b] = (uint8_t)best_t;
            double a = e4m3_f64(best_t) * S;
            int zeros = 0;
            for (int64_t i = 0; i < B; ++i) {
                int64_t k = b * B + i;
                int s = (w[n * K + k] >> 7) & 1;
                if (balance && y[i] == 0.0)
                    s = (zeros++) & 1;
                int m = (2.0 * y[i] > 5.0 * a) ? 1 : 0;
                codes2[n * K + k] = (uint8_t)((s << 1) | m);
            }
        }
        free(y);
    }
    return 0;
}
