// Decode-sized MoE layer forward: GEMV kernels streaming the packed 2-bit
// (and FP4 delta) planes from HBM.
//
// Method: README "Frontier MoE on consumer Blackwell (SM120)", section
// "How it fits — 2-bit experts at FP4 quality": decode is bound by HBM
// bandwidth, the experts run from the 2-bit planes with an in-register decode,
// and the FP4 delta GEMM adds the residual of delta-cache experts on tokens
// the confidence gate flags.
//
// Kernel shape (MI355X): one 64-lane wavefront owns one 64-row storage tile,
// one row per lane, so every 16-byte load of a wavefront is one contiguous
// 1 KiB segment of the tiled planes and every lane works on the same k at the
// same time.  The activations of the (up to 4) tokens handled together are
// therefore wave-uniform: they are staged once in LDS and read with broadcast
// loads (scalar loads would drain on every wait, since they return out of
// order).  Eight
// wavefronts split K and are reduced in LDS in a fixed order; each keeps the
// next 128-k group's loads in flight while it decodes the current one.
//
//  fc1: grid (I/64 tiles, slots); a slot is the first sorted pair of an
//       expert (its whole run of tokens) or the shared expert.  Each lane
//       computes gate row j and up row j of its tile for every token of the
//       slot, adds the FP4 delta for flagged tokens of resident experts and
//       writes h = bf16(silu(gate) * up).
//  fc2: grid (H/64 tiles, slots); y = W2 h (+ D2 h) per pair into an fp32
//       buffer.
//  combine: out = bf16(sum_j w_tj * y_(t,j) + y_shared) in slot order:
//       deterministic, no float atomics.  (A last-workgroup combine inside fc2
//       needs an agent-scope release per workgroup, which on this chip's
//       per-XCD L2s costs far more than one more launch.)
#include <algorithm>

#include "moet_common.h"

namespace moet {

struct DecodeParams {
    const uint16_t *x;
    int T, k, H, I, E;
    const int32_t *ids;
    const float *w;
    const int32_t *offsets;
    const int32_t *sorted;
    const uint8_t *gate;
    moet_w2 w13, w2, sh13, sh2;
    int has_shared;
    int n_slots;
    const int32_t *slot_of_expert;
    moet_fp4 d13, d2;
    float swiglu_limit;
    uint16_t *h;        // [P + T][I] bf16
    float *ypart;       // [P + T][H] fp32
    uint16_t *out;      // [T][H] bf16
};

struct SlotInfo {
    int e, pbeg, pend, dslot;
    bool shared;
};

__device__ __forceinline__ bool resolve_slot(const DecodeParams &p, int s, SlotInfo &si)
{
    const int P = p.T * p.k;
    if (s < P) {
        const int pair = p.sorted[s];
        if (pair < 0 || pair >= P) return false;
        const int e = p.ids[pair];
        if (e < 0 || e >= p.E) return false;
        if (p.offsets[e] != s) return false;
        si.e = e;
        si.pbeg = s;
        si.pend = min(p.offsets[e + 1], P);
        si.shared = false;
        int ds = -1;
        if (p.n_slots > 0 && p.gate != nullptr) {
            ds = p.slot_of_expert[e];
            if (ds >= p.n_slots) ds = -1;
        }
        si.dslot = ds;
        return si.pend > si.pbeg;
    }
    if (p.has_shared && s == P) {
        si.e = -1;
        si.pbeg = 0;
        si.pend = p.T;
        si.shared = true;
        si.dslot = -1;
        return true;
    }
    return false;
}

// token / h-row / delta flag of entry i of a slot's run
__device__ __forceinline__ void slot_token(const DecodeParams &p, const SlotInfo &si, int i, int &t, int &hrow, bool &flag)
{
    if (si.shared) {
        t = i;
        hrow = p.T * p.k + i;
        flag = false;
    } else {
        const int P = p.T * p.k;
        const int pair = min(max(p.sorted[i], 0), P - 1);  // guards reads/writes against malformed input
        t = pair / p.k;
        hrow = pair;
        flag = si.dslot >= 0 && p.gate[t] != 0;
    }
}

// ---------------------------------------------------------------------------
// Inner products.  Activations of the tokens handled together are staged in
// LDS once per pass; every lane of a wavefront reads the same address
// (broadcast), so each block of 32 k costs 4 ds_read_b128 per token.
// ---------------------------------------------------------------------------

// x pairs [kp, kp + 16) of token row xl (LDS) into 16 dwords
__device__ __forceinline__ void lds_x16(const uint32_t *xl, int kp, uint32_t xv[16])
{
    const uint4 *q = reinterpret_cast<const uint4 *>(xl + kp);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint4 v = q[i];
        xv[4 * i + 0] = v.x;
        xv[4 * i + 1] = v.y;
        xv[4 * i + 2] = v.z;
        xv[4 * i + 3] = v.w;
    }
}

// decode constants: the and-mask lives in an SGPR, the or-constant in a VGPR
struct W2Consts {
    uint32_t sm, vb;
};

__device__ __forceinline__ W2Consts w2_consts()
{
    W2Consts c;
    c.sm = __builtin_amdgcn_readfirstlane(0x81008100u);
    c.vb = 0x3E803E80u;
    asm volatile("" : "+v"(c.vb));
    return c;
}

__device__ __forceinline__ void decode_w2_block(uint32_t w0, uint32_t w1, uint32_t pr[16], W2Consts k)
{
    const uint32_t sm = k.sm, vb = k.vb;
    pr[0] = w2_pair<0>(w0, sm, vb);
    pr[1] = w2_pair<1>(w0, sm, vb);
    pr[2] = w2_pair<2>(w0, sm, vb);
    pr[3] = w2_pair<3>(w0, sm, vb);
    pr[4] = w2_pair<4>(w0, sm, vb);
    pr[5] = w2_pair<5>(w0, sm, vb);
    pr[6] = w2_pair<6>(w0, sm, vb);
    pr[7] = w2_pair<7>(w0, sm, vb);
    pr[8] = w2_pair<0>(w1, sm, vb);
    pr[9] = w2_pair<1>(w1, sm, vb);
    pr[10] = w2_pair<2>(w1, sm, vb);
    pr[11] = w2_pair<3>(w1, sm, vb);
    pr[12] = w2_pair<4>(w1, sm, vb);
    pr[13] = w2_pair<5>(w1, sm, vb);
    pr[14] = w2_pair<6>(w1, sm, vb);
    pr[15] = w2_pair<7>(w1, sm, vb);
}

// One 32-k block (2-bit words w0, w1; first bf16 pair index kp) of NM matrices
// for TT tokens; the activations are read once and shared by all matrices.
template <int TT, int NM, int BLK>
__device__ __forceinline__ void w2_block(const uint32_t w0[NM], const uint32_t w1[NM], const uint32_t sc[NM],
                                         const uint32_t *const xl[TT], int kp, float acc[NM][TT], W2Consts kc)
{
    uint32_t xv[TT][16];
#pragma unroll
    for (int t = 0; t < TT; ++t) lds_x16(xl[t], kp, xv[t]);
#pragma unroll
    for (int m = 0; m < NM; ++m) {
        uint32_t pr[16];
        decode_w2_block(w0[m], w1[m], pr, kc);
        const float s = e4m3_byte<BLK>(sc[m]);
#pragma unroll
        for (int t = 0; t < TT; ++t) {
            float bs = 0.f;
#pragma unroll
            for (int i = 0; i < 16; ++i) bs = dot2_bf16(pr[i], xv[t][i], bs);
            acc[m][t] = fmaf(bs, s, acc[m][t]);
        }
    }
}

template <int NM>
struct W2Group {
    uint4 c0[NM], c1[NM];
    uint32_t sc[NM];
};

template <int NM>
__device__ __forceinline__ void w2_load(W2Group<NM> &G, const uint4 *const c4[NM], const uint32_t *const s4[NM], int tile,
                                        int lane, int K, int g)
{
#pragma unroll
    for (int m = 0; m < NM; ++m) {
        G.c0[m] = c4[m][w2_chunk_idx(tile, 2 * g, lane, K)];
        G.c1[m] = c4[m][w2_chunk_idx(tile, 2 * g + 1, lane, K)];
        G.sc[m] = s4[m][w2_scale_idx(tile, g, lane, K)];
    }
}

template <int TT, int NM>
__device__ __forceinline__ void w2_group(const W2Group<NM> &G, int g, const uint32_t *const xl[TT], float acc[NM][TT],
                                         W2Consts kc)
{
    const int kp = 64 * g;
    uint32_t a[NM], b[NM];
#pragma unroll
    for (int m = 0; m < NM; ++m) a[m] = G.c0[m].x, b[m] = G.c0[m].y;
    w2_block<TT, NM, 0>(a, b, G.sc, xl, kp + 0, acc, kc);
    __builtin_amdgcn_sched_barrier(0);  // keep each block's activations short-lived
#pragma unroll
    for (int m = 0; m < NM; ++m) a[m] = G.c0[m].z, b[m] = G.c0[m].w;
    w2_block<TT, NM, 1>(a, b, G.sc, xl, kp + 16, acc, kc);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int m = 0; m < NM; ++m) a[m] = G.c1[m].x, b[m] = G.c1[m].y;
    w2_block<TT, NM, 2>(a, b, G.sc, xl, kp + 32, acc, kc);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int m = 0; m < NM; ++m) a[m] = G.c1[m].z, b[m] = G.c1[m].w;
    w2_block<TT, NM, 3>(a, b, G.sc, xl, kp + 48, acc, kc);
    __builtin_amdgcn_sched_barrier(0);
}

// NM 2-bit matrices of one 64-row tile, groups [g0, g1) of 128 k, TT tokens.
// acc[m][t] receives sum over k of (level/4) * scale * x.  Two register
// buffers alternate so that the loads of the next group are in flight while
// the current one is decoded (no copies between them, so no early drain).
template <int TT, int NM>
__device__ __forceinline__ void w2_gemv(const uint4 *const c4[NM], const uint32_t *const s4[NM], int tile, int lane, int K,
                                        int g0, int g1, const uint32_t *const xl[TT], float acc[NM][TT])
{
    const W2Consts kc = w2_consts();
    if (g0 >= g1) return;
    W2Group<NM> A, B;
    w2_load<NM>(A, c4, s4, tile, lane, K, g0);
    for (int g = g0; g < g1; g += 2) {
        if (g + 1 < g1) w2_load<NM>(B, c4, s4, tile, lane, K, g + 1);
        w2_group<TT, NM>(A, g, xl, acc, kc);
        if (g + 1 >= g1) break;
        if (g + 2 < g1) w2_load<NM>(A, c4, s4, tile, lane, K, g + 2);
        w2_group<TT, NM>(B, g + 1, xl, acc, kc);
    }
}

// FP4 16-block: words w0, w1 = k .. k+15 (first pair index kp), scale s
template <int TT>
__device__ __forceinline__ void fp4_block(uint32_t w0, uint32_t w1, float s, const uint32_t *const xl[TT], int kp,
                                          float acc[TT])
{
    uint32_t pr[8];
    pr[0] = fp4_pair<0>(w0);
    pr[1] = fp4_pair<1>(w0);
    pr[2] = fp4_pair<2>(w0);
    pr[3] = fp4_pair<3>(w0);
    pr[4] = fp4_pair<0>(w1);
    pr[5] = fp4_pair<1>(w1);
    pr[6] = fp4_pair<2>(w1);
    pr[7] = fp4_pair<3>(w1);
#pragma unroll
    for (int t = 0; t < TT; ++t) {
        const uint4 *q = reinterpret_cast<const uint4 *>(xl[t] + kp);
        const uint4 v0 = q[0], v1 = q[1];
        const uint32_t xv[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
        float bs = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) bs = dot2_bf16(pr[i], xv[i], bs);
        acc[t] = fmaf(bs, s, acc[t]);
    }
}

template <int TT, int NM>
__device__ __forceinline__ void fp4_gemv(const uint4 *const c4[NM], const uint2 *const s8[NM], int tile, int lane, int K,
                                         int g0, int g1, const uint32_t *const xl[TT], float acc[NM][TT])
{
    for (int g = g0; g < g1; ++g) {
        uint2 sc[NM];
        uint4 c[NM][4];
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            sc[m] = s8[m][fp4_scale_idx(tile, g, lane, K)];
#pragma unroll
            for (int j = 0; j < 4; ++j) c[m][j] = c4[m][fp4_chunk_idx(tile, 4 * g + j, lane, K)];
        }
        const int kp = 64 * g;
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            __builtin_amdgcn_sched_barrier(0);
            fp4_block<TT>(c[m][0].x, c[m][0].y, e4m3_byte<0>(sc[m].x), xl, kp + 0, acc[m]);
            fp4_block<TT>(c[m][0].z, c[m][0].w, e4m3_byte<1>(sc[m].x), xl, kp + 8, acc[m]);
            __builtin_amdgcn_sched_barrier(0);
            fp4_block<TT>(c[m][1].x, c[m][1].y, e4m3_byte<2>(sc[m].x), xl, kp + 16, acc[m]);
            fp4_block<TT>(c[m][1].z, c[m][1].w, e4m3_byte<3>(sc[m].x), xl, kp + 24, acc[m]);
            __builtin_amdgcn_sched_barrier(0);
            fp4_block<TT>(c[m][2].x, c[m][2].y, e4m3_byte<0>(sc[m].y), xl, kp + 32, acc[m]);
            fp4_block<TT>(c[m][2].z, c[m][2].w, e4m3_byte<1>(sc[m].y), xl, kp + 40, acc[m]);
            __builtin_amdgcn_sched_barrier(0);
            fp4_block<TT>(c[m][3].x, c[m][3].y, e4m3_byte<2>(sc[m].y), xl, kp + 48, acc[m]);
            fp4_block<TT>(c[m][3].z, c[m][3].w, e4m3_byte<3>(sc[m].y), xl, kp + 56, acc[m]);
        }
    }
}

// Row pointers and scales of the matrices one slot uses.
struct Mats {
    const uint4 *c4[2];
    const uint32_t *s4[2];
    float s2[2];
    const uint4 *dc4[2];
    const uint2 *ds8[2];
    float ds2[2];
};

// One chunk of TT tokens: per-wave partial pre-activations (2-bit + delta) for NM matrices.
template <int TT, int NM>
__device__ __forceinline__ void chunk_partials(const Mats &M, int tile, int lane, int K, int g0, int g1,
                                               const uint32_t *const xl[TT], const bool flag[TT], bool any_flag,
                                               float out[NM][TT])
{
    float acc[NM][TT];
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int t = 0; t < TT; ++t) acc[m][t] = 0.f;
    w2_gemv<TT, NM>(M.c4, M.s4, tile, lane, K, g0, g1, xl, acc);
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int t = 0; t < TT; ++t) out[m][t] = 4.0f * M.s2[m] * acc[m][t];
    if (any_flag) {
        float dacc[NM][TT];
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
            for (int t = 0; t < TT; ++t) dacc[m][t] = 0.f;
        fp4_gemv<TT, NM>(M.dc4, M.ds8, tile, lane, K, g0, g1, xl, dacc);
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
            for (int t = 0; t < TT; ++t)
                if (flag[t]) out[m][t] += M.ds2[m] * dacc[m][t];
    }
}

constexpr int kTT = 2;   // tokens per pass (more would cost occupancy)
constexpr int kWaves = 8;

template <int NM>
__device__ void slot_pass(const Mats &M, int tile, int lane, int wave, int K, const uint32_t *const xl[kTT],
                          const bool flag[kTT], int n, float part[NM][kTT])
{
    const int G = K / 128;
    const int g0 = wave * G / kWaves, g1 = (wave + 1) * G / kWaves;
    bool any_flag = false;
#pragma unroll
    for (int t = 0; t < kTT; ++t) any_flag |= (t < n) && flag[t];
    if (n == 1) {
        float q[NM][1];
        chunk_partials<1, NM>(M, tile, lane, K, g0, g1, xl, flag, any_flag, q);
#pragma unroll
        for (int m = 0; m < NM; ++m) part[m][0] = q[m][0];
    } else {
        chunk_partials<2, NM>(M, tile, lane, K, g0, g1, xl, flag, any_flag, part);
    }
}

// Copy n token rows of K bf16 (16-byte units) from global src rows into LDS dst
// rows of stride K; all threads of the workgroup take part.
__device__ __forceinline__ void stage_rows(uint32_t *dst, const uint16_t *const src[kTT], int n, int K)
{
    const int per_row = K / 8;  // uint4 per row
    for (int i = threadIdx.x; i < n * per_row; i += blockDim.x) {
        const int t = i / per_row, c = i - t * per_row;
        reinterpret_cast<uint4 *>(dst + (size_t)t * (K / 2))[c] = reinterpret_cast<const uint4 *>(src[t])[c];
    }
}

__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(4))) void fc1_decode_kernel(DecodeParams p)
{
    extern __shared__ __align__(16) uint32_t smem[];   // x rows [kTT][H/2], reused for the reduction
    const int tile = blockIdx.x, s = blockIdx.y;
    SlotInfo si;
    if (!resolve_slot(p, s, si)) return;
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int I = p.I, H = p.H;
    const size_t wmat = (size_t)I * H / 16, smat = (size_t)I * H / 32;
    const moet_w2 &W = si.shared ? p.sh13 : p.w13;
    const int m0 = si.shared ? 0 : 2 * si.e;
    Mats M;
#pragma unroll
    for (int m = 0; m < 2; ++m) {
        M.c4[m] = reinterpret_cast<const uint4 *>(W.codes + (m0 + m) * wmat);
        M.s4[m] = reinterpret_cast<const uint32_t *>(W.scales + (m0 + m) * smat);
        M.s2[m] = W.scale2[m0 + m];
        M.dc4[m] = nullptr;
        M.ds8[m] = nullptr;
        M.ds2[m] = 0.f;
    }
    if (si.dslot >= 0) {
        const size_t dmat = (size_t)I * H / 2, dsmat = (size_t)I * H / 16;
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            M.dc4[m] = reinterpret_cast<const uint4 *>(p.d13.codes + (2 * si.dslot + m) * dmat);
            M.ds8[m] = reinterpret_cast<const uint2 *>(p.d13.scales + (2 * si.dslot + m) * dsmat);
            M.ds2[m] = p.d13.scale2[2 * si.dslot + m];
        }
    }
    float(*red)[2][kTT][64] = reinterpret_cast<float(*)[2][kTT][64]>(smem);
    for (int i0 = si.pbeg; i0 < si.pend; i0 += kTT) {
        const int n = min(kTT, si.pend - i0);
        const uint16_t *src[kTT];
        const uint32_t *xl[kTT];
        bool flag[kTT];
        int hrow[kTT];
#pragma unroll
        for (int j = 0; j < kTT; ++j) {
            int t;
            slot_token(p, si, i0 + (j < n ? j : 0), t, hrow[j], flag[j]);
            src[j] = p.x + (size_t)t * H;
            xl[j] = smem + (size_t)(j < n ? j : 0) * (H / 2);
        }
        stage_rows(smem, src, n, H);
        __syncthreads();
        float part[2][kTT];
        slot_pass<2>(M, tile, lane, wave, H, xl, flag, n, part);
        __syncthreads();
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int t = 0; t < kTT; ++t)
                if (t < n) red[wave][m][t][lane] = part[m][t];
        __syncthreads();
        if (wave < n) {
            const int j = wave;
            float ug = 0.f, uu = 0.f;
#pragma unroll
            for (int v = 0; v < kWaves; ++v) {
                ug += red[v][0][j][lane];
                uu += red[v][1][j][lane];
            }
            if (p.swiglu_limit > 0.f) {
                ug = fminf(ug, p.swiglu_limit);
                uu = fminf(fmaxf(uu, -p.swiglu_limit), p.swiglu_limit);
            }
            const float hv = silu_f32(ug) * uu;
            p.h[(size_t)hrow[j] * I + tile * 64 + lane] = (uint16_t)f32_to_bf16_rne(hv);
        }
        __syncthreads();
    }
}

__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(4))) void fc2_decode_kernel(DecodeParams p)
{
    extern __shared__ __align__(16) uint32_t smem[];   // h rows [kTT][I/2], reused for the reduction
    const int tile = blockIdx.x, s = blockIdx.y;
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int I = p.I, H = p.H;
    SlotInfo si;
    if (!resolve_slot(p, s, si)) return;
    const moet_w2 &W = si.shared ? p.sh2 : p.w2;
    const int m0 = si.shared ? 0 : si.e;
    const size_t wmat = (size_t)H * I / 16, smat = (size_t)H * I / 32;
    Mats M;
    M.c4[0] = reinterpret_cast<const uint4 *>(W.codes + m0 * wmat);
    M.s4[0] = reinterpret_cast<const uint32_t *>(W.scales + m0 * smat);
    M.s2[0] = W.scale2[m0];
    M.dc4[0] = nullptr;
    M.ds8[0] = nullptr;
    M.ds2[0] = 0.f;
    if (si.dslot >= 0) {
        const size_t dmat = (size_t)H * I / 2, dsmat = (size_t)H * I / 16;
        M.dc4[0] = reinterpret_cast<const uint4 *>(p.d2.codes + si.dslot * dmat);
        M.ds8[0] = reinterpret_cast<const uint2 *>(p.d2.scales + si.dslot * dsmat);
        M.ds2[0] = p.d2.scale2[si.dslot];
    }
    float(*red)[1][kTT][64] = reinterpret_cast<float(*)[1][kTT][64]>(smem);
    for (int i0 = si.pbeg; i0 < si.pend; i0 += kTT) {
        const int n = min(kTT, si.pend - i0);
        const uint16_t *src[kTT];
        const uint32_t *xl[kTT];
        bool flag[kTT];
        int hrow[kTT];
#pragma unroll
        for (int j = 0; j < kTT; ++j) {
            int t;
            slot_token(p, si, i0 + (j < n ? j : 0), t, hrow[j], flag[j]);
            src[j] = p.h + (size_t)hrow[j] * I;
            xl[j] = smem + (size_t)(j < n ? j : 0) * (I / 2);
        }
        stage_rows(smem, src, n, I);
        __syncthreads();
        float part[1][kTT];
        slot_pass<1>(M, tile, lane, wave, I, xl, flag, n, part);
        __syncthreads();
#pragma unroll
        for (int t = 0; t < kTT; ++t)
            if (t < n) red[wave][0][t][lane] = part[0][t];
        __syncthreads();
        if (wave < n) {
            const int j = wave;
            float y = 0.f;
#pragma unroll
            for (int v = 0; v < kWaves; ++v) y += red[v][0][j][lane];
            p.ypart[(size_t)hrow[j] * H + tile * 64 + lane] = y;
        }
        __syncthreads();
    }
}

// out[t][n] = bf16(sum_j w[t][j] * y[(t, j)][n] + y_shared[t][n]), j in slot order
__global__ __launch_bounds__(256) void combine_kernel(DecodeParams p)
{
    const int n = blockIdx.x * 256 + threadIdx.x;
    const int t = blockIdx.y;
    if (n >= p.H) return;
    const int P = p.T * p.k;
    float acc = 0.f;
    for (int j = 0; j < p.k; ++j) {
        const int pair = t * p.k + j;
        const int e = p.ids[pair];
        if (e >= 0 && e < p.E) acc = fmaf(p.w[pair], p.ypart[(size_t)pair * p.H + n], acc);
    }
    if (p.has_shared) acc += p.ypart[(size_t)(P + t) * p.H + n];
    p.out[(size_t)t * p.H + n] = (uint16_t)f32_to_bf16_rne(acc);
}

// ---------------------------------------------------------------------------
// Standalone FP4 delta GEMV: acc[r][n] += D_slot[n][:] . act[r][:]
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(512) void delta_gemv_kernel(moet_fp4 D, int n_slots, int N, int K,
                                                         const uint16_t *__restrict__ act,
                                                         const int32_t *__restrict__ row_slot,
                                                         float *__restrict__ acc)
{
    extern __shared__ __align__(16) uint32_t smem[];   // act row [K/2], then the reduction
    const int tile = blockIdx.x, r = blockIdx.y;
    const int slot = row_slot[r];
    if (slot < 0 || slot >= n_slots) return;
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int G = K / 128;
    const int g0 = wave * G / kWaves, g1 = (wave + 1) * G / kWaves;
    const uint16_t *src[kTT] = {act + (size_t)r * K, nullptr};
    stage_rows(smem, src, 1, K);
    __syncthreads();
    const uint4 *c4[1] = {reinterpret_cast<const uint4 *>(D.codes + (size_t)slot * N * K / 2)};
    const uint2 *s8[1] = {reinterpret_cast<const uint2 *>(D.scales + (size_t)slot * N * K / 16)};
    const uint32_t *xl[1] = {smem};
    float a[1][1] = {{0.f}};
    fp4_gemv<1, 1>(c4, s8, tile, lane, K, g0, g1, xl, a);
    __syncthreads();
    float *red = reinterpret_cast<float *>(smem);
    red[wave * 64 + lane] = a[0][0];
    __syncthreads();
    if (wave == 0) {
        float v = 0.f;
#pragma unroll
        for (int u = 0; u < kWaves; ++u) v += red[u * 64 + lane];
        v *= D.scale2[slot];
        float *dst = acc + (size_t)r * N + tile * 64 + lane;
        *dst = *dst + v;
    }
}

// ---------------------------------------------------------------------------
// Host launchers
// ---------------------------------------------------------------------------
size_t decode_workspace_bytes(int T, int k, int H, int I)
{
    const size_t rows = (size_t)T * k + T;
    auto al = [](size_t b) { return (b + 255) & ~(size_t)255; };
    return al(rows * I * 2) + al(rows * H * 4);
}

int launch_decode(const moet_layer *L, const uint16_t *x, int T, int k, const int32_t *ids, const float *w,
                  const int32_t *offsets, const int32_t *sorted, const uint8_t *gate, uint16_t *out, void *ws,
                  hipStream_t stream)
{
    DecodeParams p;
    p.x = x;
    p.T = T;
    p.k = k;
    p.H = L->H;
    p.I = L->I;
    p.E = L->E;
    p.ids = ids;
    p.w = w;
    p.offsets = offsets;
    p.sorted = sorted;
    p.gate = gate;
    p.w13 = L->w13;
    p.w2 = L->w2;
    p.has_shared = L->has_shared ? 1 : 0;
    p.sh13 = L->shared13;
    p.sh2 = L->shared2;
    p.n_slots = L->n_slots;
    p.slot_of_expert = L->slot_of_expert;
    p.d13 = L->d13;
    p.d2 = L->d2;
    p.swiglu_limit = L->swiglu_limit;
    const size_t rows = (size_t)T * k + T;
    auto al = [](size_t b) { return (b + 255) & ~(size_t)255; };
    char *base = static_cast<char *>(ws);
    p.h = reinterpret_cast<uint16_t *>(base);
    p.ypart = reinterpret_cast<float *>(base + al(rows * L->I * 2));
    p.out = out;
    const int slots = T * k + p.has_shared;
    timing_start(stream);
    const int tt = T < kTT ? T : kTT;
    const size_t red1 = (size_t)kWaves * 2 * kTT * 64 * 4, red2 = (size_t)kWaves * kTT * 64 * 4;
    const size_t lds1 = std::max((size_t)tt * L->H * 2, red1), lds2 = std::max((size_t)tt * L->I * 2, red2);
    hipLaunchKernelGGL(fc1_decode_kernel, dim3(L->I / 64, slots), dim3(64 * kWaves), lds1, stream, p);
    timing_stop(stream);
    int rc = check_launch("fc1_decode_kernel");
    if (rc != MOET_OK) return rc;
    hipLaunchKernelGGL(fc2_decode_kernel, dim3(L->H / 64, slots), dim3(64 * kWaves), lds2, stream, p);
    rc = check_launch("fc2_decode_kernel");
    if (rc != MOET_OK) return rc;
    hipLaunchKernelGGL(combine_kernel, dim3((L->H + 255) / 256, T), dim3(256), 0, stream, p);
    return check_launch("combine_kernel");
}

int launch_delta(const moet_fp4 *D, int n_slots, int N, int K, const uint16_t *act, const int32_t *row_slot, int R,
                 float *acc, hipStream_t stream)
{
    if (R == 0) return MOET_OK;
    const size_t lds = std::max((size_t)K * 2, (size_t)kWaves * 64 * 4);
    hipLaunchKernelGGL(delta_gemv_kernel, dim3(N / 64, R), dim3(64 * kWaves), lds, stream, *D, n_slots, N, K, act, row_slot, acc);
    return check_launch("delta_gemv_kernel");
}

}  // namespace moet
