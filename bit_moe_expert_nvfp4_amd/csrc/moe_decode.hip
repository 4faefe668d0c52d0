// Decode-sized MoE layer forward: GEMV kernels streaming the packed 2-bit
// (and FP4 delta) planes from HBM.
//
// Method: README "Frontier MoE on consumer Blackwell (SM120)", section
// "How it fits — 2-bit experts at FP4 quality": decode is bound by HBM
// bandwidth, the experts run from the 2-bit planes with an in-register decode,
// and the FP4 delta GEMM adds the residual of delta-cache experts on tokens
// the confidence gate flags.
//
// Kernel shape (MI355X).  Every lane owns one row of one matrix and every
// lane of a wavefront works on the same k at the same time, so each 16-byte
// load of a wavefront covers contiguous 512 B / 1 KiB segments of the tiled
// planes and the activations are wave-uniform: they are read with scalar
// loads into SGPRs, one 64-k chunk per wait, because scalar loads return out
// of order and every wait drains all of them.  Weights of the next group are
// loaded into a second register set while the current group is decoded
// (ping-pong, no copies).  A code word of 16 weights becomes 8 bf16 pairs
// with 3 and-or/shift operations and 8 FP4 -> bf16 conversions, so a weight
// costs about 0.7 VALU operations to decode plus one dot2 per pair and token;
// that is about as long as streaming the planes from HBM, so work is cut
// into many small workgroups for load balance.
//
//  fc1: grid (I/32 half-tiles, entries), 4 wavefronts splitting K.  Lanes
//       0-31 hold 32 gate rows, lanes 32-63 the same 32 up rows, so SwiGLU
//       pairs lane j with lane j+32 after the cross-wave reduction in LDS.  An
//       entry is one pass over up to two tokens of one routed expert (two
//       consecutive sorted pairs of its run) or over one shared-expert token,
//       so workgroups do nearly the same work (a two-token shared entry was
//       the longest one and set the tail); the shared expert's entries come
//       first in the grid so the hardware dispatches them first.  FP4 delta
//       rows are added for flagged tokens of resident experts.  Writes
//       h = bf16(silu(gate) * up).
//  fc2: grid (H/64 tiles, entries), 2 wavefronts splitting K; y = W2 h
//       (+ D2 h) per pair into an fp32 buffer.
//  Both run at 8 wavefronts per SIMD (<= 64 VGPRs) so the whole grid of a
//  decode step is resident at once.
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
    const int32_t *base_slot;   // expert -> cache slot of w13/w2 (null: expert e at e)
    int n_base_slots;
    int32_t *miss_count;        // routings to missing experts (null: not counted)
    int shared_fp4;             // the shared expert is NVFP4 (shf13 / shf2) instead of 2-bit
    moet_fp4 shf13, shf2;
    uint16_t *h;        // [P + T][I] bf16
    float *ypart;       // [P + T][H] fp32
    uint16_t *out;      // [T][H] bf16
};

struct SlotInfo {
    int e, ws, pbeg, pend, dslot;   // expert, its slot in w13/w2, sorted pairs [pbeg, pend), delta slot
    bool shared;
    bool sole;                      // no other entry of this call reads the same planes
};

// cache slot of expert e's 2-bit planes, or -1 when it is missing from the expert cache
__device__ __forceinline__ int weight_slot(const DecodeParams &p, int e)
{
    if (!p.base_slot) return e;
    const int ws = p.base_slot[e];
    return (ws >= 0 && ws < p.n_base_slots) ? ws : -1;
}

constexpr int kTT = 2;     // tokens per pass (more would cost SGPRs / occupancy)

// Number of grid entries (blockIdx.y) of the GEMV kernels: the shared
// expert's tokens come first (one entry each), so that their workgroups are
// dispatched first, then one entry per sorted pair position.
__host__ __device__ __forceinline__ int decode_entries(int T, int k, int has_shared)
{
    return (has_shared ? T : 0) + T * k;
}

// Entry s -> one pass over at most kTT tokens of one expert.  Entries below
// nsh = T cover shared-expert token s.  Entry nsh + q covers
// sorted positions [q, q + kTT) of expert e when q starts a group of kTT
// inside e's run [offsets[e], offsets[e+1]); e is the number of experts whose
// run ends at or before q.  One round of loads over offsets[1..E] (ballot
// counts) finds it, instead of a chain through the permutation and the ids.
// Every workgroup therefore does exactly one pass of equal length.
__device__ __forceinline__ bool resolve_slot(const DecodeParams &p, int s, SlotInfo &si)
{
    const int P = p.T * p.k;
    const int nsh = p.has_shared ? p.T : 0;
    if (s < nsh) {
        si.e = -1;
        si.ws = 0;
        si.pbeg = s;
        si.pend = s + 1;
        si.shared = true;
        si.sole = p.T == 1;   // the T shared entries all read the shared planes
        si.dslot = -1;
        return true;
    }
    const int q = s - nsh;
    if (q >= P) return false;
    const int lane = threadIdx.x & 63;
    int e = 0;
    if (p.E <= 256) {   // the common sizes: one round of at most 4 loads
        int v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int j = 1 + lane + 64 * i;
            v[i] = (j <= p.E) ? p.offsets[j] : 0x7FFFFFFF;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) e += __popcll(__ballot(v[i] <= q));
    } else {
        int v[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int j = 1 + lane + 64 * i;
            v[i] = (j <= p.E) ? p.offsets[j] : 0x7FFFFFFF;
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) e += __popcll(__ballot(v[i] <= q));
    }
    e = __builtin_amdgcn_readfirstlane(e);
    if (e >= p.E) return false;
    const int o0 = p.offsets[e], o1 = p.offsets[e + 1];
    if (q < o0 || q >= o1 || (q - o0) % kTT != 0) return false;
    const int ws = weight_slot(p, e);
    if (ws < 0) return false;   // missing expert: no work, the combine skips its routings
    si.e = e;
    si.ws = ws;
    si.pbeg = q;
    si.pend = min(min(q + kTT, o1), P);
    si.shared = false;
    si.sole = o1 - o0 <= kTT;
    int ds = -1;
    if (p.n_slots > 0 && p.gate != nullptr) {
        ds = p.slot_of_expert[e];
        if (ds >= p.n_slots) ds = -1;
    }
    si.dslot = ds;
    return true;
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
// 2-bit decode constants: the and-mask lives in an SGPR, the or-constant (the
// lane's codebook) in a VGPR
struct W2Consts {
    uint32_t sm, vb;
};

__device__ __forceinline__ W2Consts w2_consts(uint32_t orc)
{
    W2Consts c;
    c.sm = __builtin_amdgcn_readfirstlane(kW2Mask);
    c.vb = orc;
    asm volatile("" : "+v"(c.vb));
    return c;
}

// bs[t] += sum over one 16-weight word of level * x, x pairs x[t][o .. o+7]
// dot2 that starts a new sum (the zero is an inline constant, so no register
// has to be cleared first)
__device__ __forceinline__ float dot2_bf16_new(uint32_t a, uint32_t b)
{
    float r;
    asm("v_dot2_f32_bf16 %0, %1, %2, 0" : "=v"(r) : "v"(a), "s"(b));
    return r;
}

// FIRST: bs[] holds no sum yet (the word opens a 32-k block)
template <int TT, bool FIRST, typename XT>
__device__ __forceinline__ void w2_word(uint32_t w, const XT *x, int o, float bs[TT], W2Consts k)
{
    const uint32_t fa = w2_fp4_lo(w, k.sm, k.vb), fb = w2_fp4_hi(w, k.sm, k.vb);
    uint32_t pr[8];
    pr[0] = fp4_pair<0>(fa);
    pr[1] = fp4_pair<1>(fa);
    pr[2] = fp4_pair<2>(fa);
    pr[3] = fp4_pair<3>(fa);
    pr[4] = fp4_pair<0>(fb);
    pr[5] = fp4_pair<1>(fb);
    pr[6] = fp4_pair<2>(fb);
    pr[7] = fp4_pair<3>(fb);
#pragma unroll
    for (int t = 0; t < TT; ++t) {
        if constexpr (FIRST)
            bs[t] = dot2_bf16_new(pr[0], x[t][o]);
        else
            bs[t] = dot2_bf16(pr[0], x[t][o], bs[t]);
#pragma unroll
        for (int i = 1; i < 8; ++i) bs[t] = dot2_bf16(pr[i], x[t][o + i], bs[t]);
    }
}

// per-lane view of the one row this lane computes
// The 2-bit planes are addressed as a wave-uniform base plus a 32-bit per-lane
// offset, so the loads use scalar base registers and the per-group advance
// is scalar arithmetic.
struct LaneRow {
    const uint8_t *cb;    // wave-uniform: 2-bit codes of the wave's first matrix
    const uint8_t *sb;    // wave-uniform: its block scales
    uint32_t co, so;      // this lane's byte offsets (codes of 64-k chunk 0, scale dword of group 0)
    uint32_t orc;         // or-constant of this lane's matrix's codebook
    const uint4 *dc4;     // FP4 delta codes (or null)
    const uint2 *ds8;     // FP4 delta scales
    int tile, rt;         // storage tile and row within it
};

// per-lane offsets of row (tile, rt) of matrix `mat` (relative to the wave's first matrix)
__device__ __forceinline__ void lane_offsets(LaneRow &L, int mat, int tile, int rt, int N, int K)
{
    L.co = (uint32_t)mat * (uint32_t)(N * (K / 4)) + (uint32_t)(tile * (K / 64) + 0) * 1024u + (uint32_t)rt * 16u;
    L.so = (uint32_t)mat * (uint32_t)(N * (K / 32)) + (uint32_t)(tile * (K / 128)) * 256u + (uint32_t)rt * 4u;
    L.tile = tile;
    L.rt = rt;
}

struct W2Buf {
    uint4 c0, c1;
    uint32_t sc;
};

// NT: the planes are read by this workgroup alone, so the loads are
// non-temporal (streamed past the caches instead of displacing lines that
// other workgroups still read)
template <bool NT>
__device__ __forceinline__ void w2_load(W2Buf &B, const LaneRow &L, int K, int g)
{
    (void)K;
    // the opaque copies keep the group advance in the scalar base (scalar base +
    // 32-bit lane offset addressing) instead of being folded into lane pointers
    typedef uint32_t v4u __attribute__((ext_vector_type(4)));
    typedef const uint8_t __attribute__((address_space(1))) gu8;
    typedef const v4u __attribute__((address_space(1))) gv4;
    typedef const uint32_t __attribute__((address_space(1))) gu32;
    gu8 *c = (gu8 *)(uintptr_t)(L.cb + (size_t)g * 2048);   // 64-k chunks 2g, 2g+1 of the row: 1 KiB apart
    gu8 *sc = (gu8 *)(uintptr_t)(L.sb + (size_t)g * 256);
    asm volatile("" : "+s"(c), "+s"(sc));
    v4u a, b;
    if constexpr (NT) {
        a = __builtin_nontemporal_load((gv4 *)(c + L.co));
        b = __builtin_nontemporal_load((gv4 *)(c + (L.co + 1024u)));
        B.sc = __builtin_nontemporal_load((gu32 *)(sc + L.so));
    } else {
        a = *(gv4 *)(c + L.co);
        b = *(gv4 *)(c + (L.co + 1024u));
        B.sc = *(gu32 *)(sc + L.so);
    }
    B.c0 = make_uint4(a.x, a.y, a.z, a.w);
    B.c1 = make_uint4(b.x, b.y, b.z, b.w);
}

// activations of one 64-k chunk (32 bf16 pairs) of token rows xr[t] (scalar loads)
template <int TT>
__device__ __forceinline__ void load_x_chunk(const cu32 *const xr[TT], int kp, uint32_t (*x)[32])
{
#pragma unroll
    for (int t = 0; t < TT; ++t)
#pragma unroll
        for (int i = 0; i < 32; ++i) x[t][i] = xr[t][kp + i];
}

// Activations of one code word (16 k = 8 bf16 pairs) of one token travel by
// one scalar load into SGPRs.  The loads are issued from inline asm one word
// ahead and waited explicitly (the wait names the buffer, so no use of it can
// move above the wait): scalar loads return out of order and every wait
// drains all of them, so the compiler would otherwise wait for the
// prefetched word together with the current one.  Every prefetch issued is
// waited before the loop ends.
typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));

// `sum` is tied to the load so that the arithmetic that follows in program
// order (which updates it) cannot be hoisted above the load's issue
__device__ __forceinline__ void xload(u32x8 &v, const cu32 *p, float &sum)
{
    asm volatile("s_load_dwordx8 %0, %2, 0x0" : "=s"(v), "+v"(sum) : "s"(p));
}

// The wait also names the running sums, so the previous word's arithmetic
// stays above it and the prefetch it follows has that long to land.
template <int TT>
__device__ __forceinline__ void xwait(u32x8 (&v)[TT], float bs[TT], float acc[TT])
{
    if constexpr (TT == 1)
        asm volatile("s_waitcnt lgkmcnt(0)" : "+s"(v[0]), "+v"(bs[0]), "+v"(acc[0]));
    else
        asm volatile("s_waitcnt lgkmcnt(0)" : "+s"(v[0]), "+s"(v[1]), "+v"(bs[0]), "+v"(bs[1]), "+v"(acc[0]),
                     "+v"(acc[1]));
}

// word j (0..7) of group g: wait for its activations (in `cur`), prefetch word
// j + 1 (clamped to the wave's last word `wl`) into `nxt`, then decode and dot
template <int TT>
__device__ __forceinline__ void xwait_acc(u32x8 (&v)[TT], float acc[TT])
{
    if constexpr (TT == 1)
        asm volatile("s_waitcnt lgkmcnt(0)" : "+s"(v[0]), "+v"(acc[0]));
    else
        asm volatile("s_waitcnt lgkmcnt(0)" : "+s"(v[0]), "+s"(v[1]), "+v"(acc[0]), "+v"(acc[1]));
}

// FIRST: the word opens a 32-k block (its running sums are still zero, so the
// wait orders it after the previous block's accumulation instead)
template <int TT, bool FIRST>
__device__ __forceinline__ void w2_step(uint32_t w, int word, const cu32 *const xr[TT], int wl, u32x8 (&cur)[TT],
                                        u32x8 (&nxt)[TT], float bs[TT], float acc[TT], W2Consts k)
{
    if constexpr (FIRST) {
        xwait_acc<TT>(cur, acc);
#pragma unroll
        for (int t = 0; t < TT; ++t) xload(nxt[t], xr[t] + 8 * min(word + 1, wl), acc[t]);
    } else {
        xwait<TT>(cur, bs, acc);
#pragma unroll
        for (int t = 0; t < TT; ++t) xload(nxt[t], xr[t] + 8 * min(word + 1, wl), bs[t]);
    }
    w2_word<TT, FIRST>(w, cur, 0, bs, k);
}

template <int TT>
__device__ __forceinline__ void block_done(float bs[TT], float s, float acc[TT])
{
#pragma unroll
    for (int t = 0; t < TT; ++t) {
        acc[t] = fmaf(bs[t], s, acc[t]);
        bs[t] = 0.f;
    }
}

// the 8 code words of group g; word buffers alternate xa (even words), xb (odd)
template <int TT>
__device__ __forceinline__ void w2_group(const W2Buf &B, int g, const cu32 *const xr[TT], int wl, u32x8 (&xa)[TT],
                                         u32x8 (&xb)[TT], float acc[TT], W2Consts k)
{
    const int w0 = 8 * g;
    float bs[TT];
#pragma unroll
    for (int t = 0; t < TT; ++t) bs[t] = 0.f;
    w2_step<TT, true>(B.c0.x, w0 + 0, xr, wl, xa, xb, bs, acc, k);
    w2_step<TT, false>(B.c0.y, w0 + 1, xr, wl, xb, xa, bs, acc, k);
    block_done<TT>(bs, e4m3_byte<0>(B.sc), acc);
    w2_step<TT, true>(B.c0.z, w0 + 2, xr, wl, xa, xb, bs, acc, k);
    w2_step<TT, false>(B.c0.w, w0 + 3, xr, wl, xb, xa, bs, acc, k);
    block_done<TT>(bs, e4m3_byte<1>(B.sc), acc);
    w2_step<TT, true>(B.c1.x, w0 + 4, xr, wl, xa, xb, bs, acc, k);
    w2_step<TT, false>(B.c1.y, w0 + 5, xr, wl, xb, xa, bs, acc, k);
    block_done<TT>(bs, e4m3_byte<2>(B.sc), acc);
    w2_step<TT, true>(B.c1.z, w0 + 6, xr, wl, xa, xb, bs, acc, k);
    w2_step<TT, false>(B.c1.w, w0 + 7, xr, wl, xb, xa, bs, acc, k);
    block_done<TT>(bs, e4m3_byte<3>(B.sc), acc);
}

#ifndef MOET_DECODE_WAVES
#define MOET_DECODE_WAVES 8
#endif
#ifndef MOET_DECODE_PF
#define MOET_DECODE_PF 1
#endif
constexpr int kPF = MOET_DECODE_PF;   // weight groups loaded ahead of the one being computed

// acc[t] += sum over groups [g0, g1) of level * scale * x for this lane's row.
// Weights run kPF groups ahead of the group being computed, in a ring of
// kPF + 1 register sets; a load is issued for every group computed (past the
// end it re-loads the final group) so that the outstanding-load count, and
// with it the compiler's wait, is the same on every path.  xr[] must be
// wave-uniform.
template <int TT, bool NT>
__device__ __forceinline__ void w2_gemv(const LaneRow &L, int K, int g0, int g1, const cu32 *const xr[TT], float acc[TT])
{
    if (g0 >= g1) return;
    const W2Consts kc = w2_consts(L.orc);
    const int wl = 8 * g1 - 1;
    W2Buf buf[kPF + 1];
    u32x8 xa[TT], xb[TT];
#pragma unroll
    for (int d = 0; d < kPF; ++d) w2_load<NT>(buf[d], L, K, min(g0 + d, g1 - 1));
#pragma unroll
    for (int t = 0; t < TT; ++t) xload(xa[t], xr[t] + 8 * (8 * g0), acc[t]);
    for (int g = g0; g < g1; g += kPF + 1) {
#pragma unroll
        for (int u = 0; u <= kPF; ++u) {
            if (g + u < g1) {
                w2_load<NT>(buf[(u + kPF) % (kPF + 1)], L, K, min(g + u + kPF, g1 - 1));
                w2_group<TT>(buf[u], g + u, xr, wl, xa, xb, acc, kc);
            }
        }
    }
    float bs[TT];
#pragma unroll
    for (int t = 0; t < TT; ++t) bs[t] = 0.f;
    xwait<TT>(xa, bs, acc);   // drain the last prefetch
}

// FP4 delta planes: a 64-k half group of a row is two 32-k chunks (16 B each,
// 8 e2m1 codes per word) and four e4m3 block scales (one per 16 k, one dword).
struct FP4Buf {
    uint4 c0, c1;
    uint32_t sc;
};

// half group hg = 64-k chunk pair hg of the row (NT as for w2_load)
template <bool NT>
__device__ __forceinline__ void fp4_load(FP4Buf &B, const LaneRow &L, int K, int hg)
{
    typedef uint32_t v4u __attribute__((ext_vector_type(4)));
    const v4u *c = reinterpret_cast<const v4u *>(L.dc4);
    const uint32_t *sc = reinterpret_cast<const uint32_t *>(L.ds8) + 2 * fp4_scale_idx(L.tile, hg >> 1, L.rt, K) + (hg & 1);
    const int i0 = fp4_chunk_idx(L.tile, 2 * hg, L.rt, K), i1 = fp4_chunk_idx(L.tile, 2 * hg + 1, L.rt, K);
    v4u a, b;
    if constexpr (NT) {
        a = __builtin_nontemporal_load(c + i0);
        b = __builtin_nontemporal_load(c + i1);
        B.sc = __builtin_nontemporal_load(sc);
    } else {
        a = c[i0];
        b = c[i1];
        B.sc = *sc;
    }
    B.c0 = make_uint4(a.x, a.y, a.z, a.w);
    B.c1 = make_uint4(b.x, b.y, b.z, b.w);
}

template <int TT>
__device__ __forceinline__ void fp4_step(uint32_t w0, uint32_t w1, float s, int word, const cu32 *const xr[TT], int wl,
                                         u32x8 (&cur)[TT], u32x8 (&nxt)[TT], float acc[TT])
{
    xwait_acc<TT>(cur, acc);
#pragma unroll
    for (int t = 0; t < TT; ++t) xload(nxt[t], xr[t] + 8 * min(word + 1, wl), acc[t]);
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
        float bs = dot2_bf16_new(pr[0], cur[t][0]);
#pragma unroll
        for (int i = 1; i < 8; ++i) bs = dot2_bf16(pr[i], cur[t][i], bs);
        acc[t] = fmaf(bs, s, acc[t]);
    }
}

template <int TT>
__device__ __forceinline__ void fp4_half(const FP4Buf &B, int hg, const cu32 *const xr[TT], int wl, u32x8 (&xa)[TT],
                                         u32x8 (&xb)[TT], float acc[TT])
{
    const int w0 = 4 * hg;   // 16-k words of this half group
    fp4_step<TT>(B.c0.x, B.c0.y, e4m3_byte<0>(B.sc), w0 + 0, xr, wl, xa, xb, acc);
    fp4_step<TT>(B.c0.z, B.c0.w, e4m3_byte<1>(B.sc), w0 + 1, xr, wl, xb, xa, acc);
    fp4_step<TT>(B.c1.x, B.c1.y, e4m3_byte<2>(B.sc), w0 + 2, xr, wl, xa, xb, acc);
    fp4_step<TT>(B.c1.z, B.c1.w, e4m3_byte<3>(B.sc), w0 + 3, xr, wl, xb, xa, acc);
}

// acc[t] += sum over groups [g0, g1) of e2m1 * scale * x for this lane's FP4 row
// (same prefetching as the 2-bit GEMV: weights one 64-k half group ahead,
// activations one 16-k block ahead; xr[] wave-uniform)
template <int TT, bool NT>
__device__ __forceinline__ void fp4_gemv(const LaneRow &L, int K, int g0, int g1, const cu32 *const xr[TT], float acc[TT])
{
    if (g0 >= g1) return;
    const int h0 = 2 * g0, h1 = 2 * g1;
    const int wl = 8 * g1 - 1;
    FP4Buf A, B;
    u32x8 xa[TT], xb[TT];
    fp4_load<NT>(A, L, K, h0);
#pragma unroll
    for (int t = 0; t < TT; ++t) xload(xa[t], xr[t] + 8 * (8 * g0), acc[t]);
    for (int hg = h0; hg < h1; hg += 2) {   // h1 - h0 is even
        fp4_load<NT>(B, L, K, hg + 1);
        fp4_half<TT>(A, hg, xr, wl, xa, xb, acc);
        fp4_load<NT>(A, L, K, min(hg + 2, h1 - 1));
        fp4_half<TT>(B, hg + 1, xr, wl, xa, xb, acc);
    }
    xwait_acc<TT>(xa, acc);   // drain the last prefetch
}

constexpr int kW1 = 4;     // wavefronts per fc1 workgroup (K split)
constexpr int kW2 = 2;     // wavefronts per fc2 workgroup (K split)

// One pass over up to kTT tokens: this lane's partial pre-activation per token
// (2-bit part scaled by s2 plus the delta part scaled by ds2 for flagged tokens).
template <bool NT>
__device__ __forceinline__ void lane_pass(const LaneRow &L, float s2, float ds2, int K, int g0, int g1,
                                          const cu32 *const xr[kTT], const bool flag[kTT], int n, float part[kTT])
{
    bool any_flag = false;
#pragma unroll
    for (int t = 0; t < kTT; ++t) any_flag |= (t < n) && flag[t];
    float acc[kTT] = {0.f, 0.f}, dacc[kTT] = {0.f, 0.f};
    if (n == 1) {
        w2_gemv<1, NT>(L, K, g0, g1, xr, acc);
        if (any_flag) fp4_gemv<1, NT>(L, K, g0, g1, xr, dacc);
    } else {
        w2_gemv<2, NT>(L, K, g0, g1, xr, acc);
        if (any_flag) fp4_gemv<2, NT>(L, K, g0, g1, xr, dacc);
    }
#pragma unroll
    for (int t = 0; t < kTT; ++t) part[t] = s2 * acc[t] + ((any_flag && flag[t]) ? ds2 * dacc[t] : 0.f);
}

// The same for an NVFP4 shared expert: FP4 planes only, scaled by their scale2.
template <bool NT>
__device__ __forceinline__ void lane_pass_fp4(const LaneRow &L, float s2, int K, int g0, int g1,
                                              const cu32 *const xr[kTT], int n, float part[kTT])
{
    float acc[kTT] = {0.f, 0.f};
    if (n == 1) fp4_gemv<1, NT>(L, K, g0, g1, xr, acc);
    else fp4_gemv<2, NT>(L, K, g0, g1, xr, acc);
#pragma unroll
    for (int t = 0; t < kTT; ++t) part[t] = s2 * acc[t];
}

__global__ __launch_bounds__(64 * kW1) __attribute__((amdgpu_waves_per_eu(MOET_DECODE_WAVES))) void fc1_decode_kernel(DecodeParams p)
{
    if (p.miss_count && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) *p.miss_count = 0;   // counted by the combine
    __shared__ float red[kW1][kTT][64];
    const int half = blockIdx.x, s = blockIdx.y;   // rows [32 half, 32 half + 32) of gate and of up
    SlotInfo si;
    if (!resolve_slot(p, s, si)) return;
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int I = p.I, H = p.H;
    const int mat = lane >> 5;                      // 0: gate, 1: up
    const int row = 32 * half + (lane & 31);
    const moet_w2 &W = si.shared ? p.sh13 : p.w13;
    const int m0 = si.shared ? 0 : 2 * si.ws;
    LaneRow L;
    L.cb = reinterpret_cast<const uint8_t *>(W.codes + (size_t)m0 * I * H / 16);
    L.sb = W.scales + (size_t)m0 * I * H / 32;
    lane_offsets(L, mat, row >> 6, row & 63, I, H);
    const float s2 = (si.shared && p.shared_fp4) ? 0.f : W.scale2[m0 + mat];
    L.orc = (si.shared && p.shared_fp4) ? kW2Or : w2_or_of(w2_codebook(W, m0 + mat));
    float ds2 = 0.f;
    L.dc4 = nullptr;
    L.ds8 = nullptr;
    if (si.dslot >= 0) {
        const int dm = 2 * si.dslot + mat;
        L.dc4 = reinterpret_cast<const uint4 *>(p.d13.codes + (size_t)dm * I * H / 2);
        L.ds8 = reinterpret_cast<const uint2 *>(p.d13.scales + (size_t)dm * I * H / 16);
        ds2 = p.d13.scale2[dm];
    }
    const bool fp4_shared = si.shared && p.shared_fp4;
    if (fp4_shared) {
        L.dc4 = reinterpret_cast<const uint4 *>(p.shf13.codes + (size_t)mat * I * H / 2);
        L.ds8 = reinterpret_cast<const uint2 *>(p.shf13.scales + (size_t)mat * I * H / 16);
        ds2 = p.shf13.scale2[mat];
    }
    const int G = H / 128;
    const int g0 = wave * G / kW1, g1 = (wave + 1) * G / kW1;
    for (int i0 = si.pbeg; i0 < si.pend; i0 += kTT) {
        const int n = min(kTT, si.pend - i0);
        const cu32 *xr[kTT];
        bool flag[kTT];
        int hrow[kTT];
#pragma unroll
        for (int j = 0; j < kTT; ++j) {
            int t;
            slot_token(p, si, i0 + (j < n ? j : 0), t, hrow[j], flag[j]);
            t = __builtin_amdgcn_readfirstlane(t);
            xr[j] = as_const(p.x + (size_t)t * H);
        }
        float part[kTT];
        if (fp4_shared) {
            if (si.sole) lane_pass_fp4<true>(L, ds2, H, g0, g1, xr, n, part);
            else lane_pass_fp4<false>(L, ds2, H, g0, g1, xr, n, part);
        } else if (si.sole) {
            lane_pass<true>(L, s2, ds2, H, g0, g1, xr, flag, n, part);
        } else {
            lane_pass<false>(L, s2, ds2, H, g0, g1, xr, flag, n, part);
        }
#pragma unroll
        for (int t = 0; t < kTT; ++t)
            if (t < n) red[wave][t][lane] = part[t];
        __syncthreads();
        if (wave < n && lane < 32) {
            const int j = wave;
            float ug = 0.f, uu = 0.f;
#pragma unroll
            for (int v = 0; v < kW1; ++v) {
                ug += red[v][j][lane];
                uu += red[v][j][lane + 32];
            }
            if (p.swiglu_limit > 0.f) {
                ug = fminf(ug, p.swiglu_limit);
                uu = fminf(fmaxf(uu, -p.swiglu_limit), p.swiglu_limit);
            }
            const float hv = silu_f32(ug) * uu;
            p.h[(size_t)hrow[j] * I + row] = (uint16_t)f32_to_bf16_rne(hv);
        }
        __syncthreads();
    }
}

__global__ __launch_bounds__(64 * kW2) __attribute__((amdgpu_waves_per_eu(MOET_DECODE_WAVES))) void fc2_decode_kernel(DecodeParams p)
{
    __shared__ float red[kW2][kTT][64];
    const int tile = blockIdx.x, s = blockIdx.y;
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int I = p.I, H = p.H;
    SlotInfo si;
    if (!resolve_slot(p, s, si)) return;
    const moet_w2 &W = si.shared ? p.sh2 : p.w2;
    const int m0 = si.shared ? 0 : si.ws;
    const bool fp4_shared = si.shared && p.shared_fp4;
    LaneRow L;
    L.cb = reinterpret_cast<const uint8_t *>(W.codes + (size_t)m0 * H * I / 16);
    L.sb = W.scales + (size_t)m0 * H * I / 32;
    lane_offsets(L, 0, tile, lane, H, I);
    const float s2 = fp4_shared ? 0.f : W.scale2[m0];
    L.orc = fp4_shared ? kW2Or : w2_or_of(w2_codebook(W, m0));
    float ds2 = 0.f;
    L.dc4 = nullptr;
    L.ds8 = nullptr;
    if (si.dslot >= 0) {
        L.dc4 = reinterpret_cast<const uint4 *>(p.d2.codes + (size_t)si.dslot * H * I / 2);
        L.ds8 = reinterpret_cast<const uint2 *>(p.d2.scales + (size_t)si.dslot * H * I / 16);
        ds2 = p.d2.scale2[si.dslot];
    }
    if (fp4_shared) {
        L.dc4 = reinterpret_cast<const uint4 *>(p.shf2.codes);
        L.ds8 = reinterpret_cast<const uint2 *>(p.shf2.scales);
        ds2 = p.shf2.scale2[0];
    }
    const int G = I / 128;
    const int g0 = wave * G / kW2, g1 = (wave + 1) * G / kW2;
    for (int i0 = si.pbeg; i0 < si.pend; i0 += kTT) {
        const int n = min(kTT, si.pend - i0);
        const cu32 *xr[kTT];
        bool flag[kTT];
        int hrow[kTT];
#pragma unroll
        for (int j = 0; j < kTT; ++j) {
            int t;
            slot_token(p, si, i0 + (j < n ? j : 0), t, hrow[j], flag[j]);
            hrow[j] = __builtin_amdgcn_readfirstlane(hrow[j]);
            xr[j] = as_const(p.h + (size_t)hrow[j] * I);
        }
        float part[kTT];
        if (fp4_shared) {
            if (si.sole) lane_pass_fp4<true>(L, ds2, I, g0, g1, xr, n, part);
            else lane_pass_fp4<false>(L, ds2, I, g0, g1, xr, n, part);
        } else if (si.sole) {
            lane_pass<true>(L, s2, ds2, I, g0, g1, xr, flag, n, part);
        } else {
            lane_pass<false>(L, s2, ds2, I, g0, g1, xr, flag, n, part);
        }
#pragma unroll
        for (int t = 0; t < kTT; ++t)
            if (t < n) red[wave][t][lane] = part[t];
        __syncthreads();
        if (wave < n) {
            const int j = wave;
            float y = 0.f;
#pragma unroll
            for (int v = 0; v < kW2; ++v) y += red[v][j][lane];
            p.ypart[(size_t)hrow[j] * H + tile * 64 + lane] = y;
        }
        __syncthreads();
    }
}

// out[t][n] = bf16(sum_j w[t][j] * y[(t, j)][n] + y_shared[t][n]), j in slot order;
// routings to experts missing from the expert cache contribute nothing and are
// counted once per token (by the first column block).  The token's ids and
// weights are wave-uniform (scalar loads); its y loads do not depend on them
// and are issued first, so the kernel pays about one memory round trip.
constexpr int kCombineMaxK = 16;

__global__ __launch_bounds__(256) void combine_kernel(DecodeParams p)
{
    const int n = blockIdx.x * 256 + threadIdx.x;
    const int t = blockIdx.y;
    const int P = p.T * p.k;
    const bool in = n < p.H;
    // the y rows sit at fixed positions (pair t*k + j, shared P + t): their loads
    // go out before the ids and weights arrive, so the two round trips overlap
    float y[kCombineMaxK];
#pragma unroll
    for (int j = 0; j < kCombineMaxK; ++j) y[j] = (j < p.k && in) ? p.ypart[(size_t)(t * p.k + j) * p.H + n] : 0.f;
    const float ysh = (p.has_shared && in) ? p.ypart[(size_t)(P + t) * p.H + n] : 0.f;
    const cu32 *idr = as_const(p.ids + (size_t)t * p.k);
    const cu32 *wr = as_const(p.w + (size_t)t * p.k);
    int e[kCombineMaxK];
    float wt[kCombineMaxK];
#pragma unroll
    for (int j = 0; j < kCombineMaxK; ++j) {
        e[j] = (j < p.k) ? (int)idr[j] : -1;
        wt[j] = (j < p.k) ? __uint_as_float(wr[j]) : 0.f;
    }
    bool live[kCombineMaxK];
    int miss = 0;
#pragma unroll
    for (int j = 0; j < kCombineMaxK; ++j) {
        const bool valid = e[j] >= 0 && e[j] < p.E;
        live[j] = valid && weight_slot(p, e[j]) >= 0;
        miss += (valid && !live[j]) ? 1 : 0;
    }
    if (p.miss_count && blockIdx.x == 0 && threadIdx.x == 0 && miss) atomicAdd(p.miss_count, miss);
    if (!in) return;
    float acc = 0.f;   // rows of missing experts were not written this call: selected out, never used
#pragma unroll
    for (int j = 0; j < kCombineMaxK; ++j)
        if (live[j]) acc = fmaf(wt[j], y[j], acc);
    if (p.has_shared) acc += ysh;
    p.out[(size_t)t * p.H + n] = (uint16_t)f32_to_bf16_rne(acc);
}

// ---------------------------------------------------------------------------
// Standalone FP4 delta GEMV: acc[r][n] += D_slot[n][:] . act[r][:]
// ---------------------------------------------------------------------------
constexpr int kWd = 4;

__global__ __launch_bounds__(64 * kWd) void delta_gemv_kernel(moet_fp4 D, int n_slots, int N, int K,
                                                              const uint16_t *__restrict__ act,
                                                              const int32_t *__restrict__ row_slot,
                                                              float *__restrict__ acc)
{
    __shared__ float red[kWd][64];
    const int tile = blockIdx.x, r = blockIdx.y;
    const int slot = row_slot[r];
    if (slot < 0 || slot >= n_slots) return;
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int G = K / 128;
    const int g0 = wave * G / kWd, g1 = (wave + 1) * G / kWd;
    LaneRow L;
    L.cb = nullptr;
    L.sb = nullptr;
    L.co = L.so = 0;
    L.dc4 = reinterpret_cast<const uint4 *>(D.codes + (size_t)slot * N * K / 2);
    L.ds8 = reinterpret_cast<const uint2 *>(D.scales + (size_t)slot * N * K / 16);
    L.tile = tile;
    L.rt = lane;
    const cu32 *xr[1] = {as_const(act + (size_t)r * K)};
    float a[1] = {0.f};
    fp4_gemv<1, false>(L, K, g0, g1, xr, a);
    red[wave][lane] = a[0];
    __syncthreads();
    if (wave == 0) {
        float v = 0.f;
#pragma unroll
        for (int u = 0; u < kWd; ++u) v += red[u][lane];
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
                  const int32_t *offsets, const int32_t *sorted, const uint8_t *gate, uint16_t *out, int32_t *miss_count,
                  void *ws, hipStream_t stream)
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
    p.base_slot = L->base_slot_of_expert;
    p.n_base_slots = L->n_base_slots;
    p.miss_count = miss_count;
    p.shared_fp4 = (L->has_shared && L->shared_fp4) ? 1 : 0;
    p.shf13 = L->shared13_fp4;
    p.shf2 = L->shared2_fp4;
    const size_t rows = (size_t)T * k + T;
    auto al = [](size_t b) { return (b + 255) & ~(size_t)255; };
    char *base = static_cast<char *>(ws);
    p.h = reinterpret_cast<uint16_t *>(base);
    p.ypart = reinterpret_cast<float *>(base + al(rows * L->I * 2));
    p.out = out;
    const int slots = decode_entries(T, k, p.has_shared);
    hipEvent_t ev0, ev1;
    if (timing_events(&ev0, &ev1))
        hipExtLaunchKernelGGL(fc1_decode_kernel, dim3(L->I / 32, slots), dim3(64 * kW1), 0, stream, ev0, ev1, 0, p);
    else
        hipLaunchKernelGGL(fc1_decode_kernel, dim3(L->I / 32, slots), dim3(64 * kW1), 0, stream, p);
    int rc = check_launch("fc1_decode_kernel");
    if (rc != MOET_OK) return rc;
    hipLaunchKernelGGL(fc2_decode_kernel, dim3(L->H / 64, slots), dim3(64 * kW2), 0, stream, p);
    rc = check_launch("fc2_decode_kernel");
    if (rc != MOET_OK) return rc;
    hipLaunchKernelGGL(combine_kernel, dim3((L->H + 255) / 256, T), dim3(256), 0, stream, p);
    return check_launch("combine_kernel");
}

int launch_delta(const moet_fp4 *D, int n_slots, int N, int K, const uint16_t *act, const int32_t *row_slot, int R,
                 float *acc, hipStream_t stream)
{
    if (R == 0) return MOET_OK;
    hipLaunchKernelGGL(delta_gemv_kernel, dim3(N / 64, R), dim3(64 * kWd), 0, stream, *D, n_slots, N, K, act, row_slot,
                       acc);
    return check_launch("delta_gemv_kernel");
}

}  // namespace moet
