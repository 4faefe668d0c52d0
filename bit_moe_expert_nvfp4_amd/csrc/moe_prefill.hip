// Prefill-sized MoE layer forward: grouped GEMM on the matrix cores.
//
// Method: README "Frontier MoE on consumer Blackwell (SM120)", section
// "How it fits — 2-bit experts at FP4 quality": prefill runs the same 2-bit
// expert GEMM as decode on many tokens per expert; the page notes that the
// prefill GEMM is limited by how fast operands are fed to the matrix units
// (one wide load per operand fragment), not by DRAM.
//
// MI355X design (bf16 v_mfma_f32_16x16x32, fp32 accumulation):
//  * Work item = (M-tile of up to 160 consecutive sorted pairs of one expert,
//    N-tile).  160 rows hold a whole expert at the usual prefill load
//    (T*k/E ~ 128 +- 11 rows), so the weights are staged and dequantised once
//    per expert instead of twice for about half of them; MFMAs are issued per
//    16-row block, so a tile pays for ceil(rows / 16) blocks.  A one-wave
//    kernel turns expert_offsets into the M-tile table on the device (largest
//    tiles first), so the routing never round-trips to the host and each
//    workgroup finds its tile with one load.  Linear workgroup ids are mapped so that every
//    N-tile of one M-tile lands on the same XCD (workgroups are dispatched
//    round-robin over the 8 XCDs): the gathered activation rows are then read
//    from that XCD's L2 by all of them.
//  * A (activations): up to 160 rows x 64 k bf16 per step (the tile's valid
//    32-row blocks), gathered by token (gate/up) or read from h in sorted
//    order (down), staged in LDS with an XOR swizzle of the 16-byte columns
//    (by row / 2) so each MFMA A fragment is one conflict-free ds_read_b128
//    (16-lane phases over 64 banks).  A, B codes and B scales of each 64-k
//    step travel by LDS-DMA into a 3-stage ring, so two steps are in flight
//    while one is computed and no registers are spent on prefetching.
//  * B (weights): each lane dequantises the 8 k-values its MFMA B fragment
//    needs from the staged 2-bit words into registers: one and-or makes their
//    e2m1 image, four FP4 -> bf16 conversions give the levels, and a packed
//    16-bit add of the scale's bf16 bits (less those of 1.0) multiplies by
//    the e4m3 block scale; bf16(level * scale) is exact (4 significant bits).
//    That add is a product only for levels +-1, +-4 (powers of two): a
//    workgroup whose matrices use codebook 1 ({1/2, 3}) or 2 ({0, 2}) takes
//    a second instantiation that converts e2m1 -> f32, multiplies by the scale
//    and rounds to bf16, exact as well (at most 5 significant bits).
//    The per-tensor scale2 is applied in the epilogue.
//  * The MFMAs take the dequantised B fragment as their first operand, so a
//    lane's result holds four consecutive features of one row, stored with one
//    8-byte (h) or 16-byte (y, pre-activations) access.
//  * gate/up kernel: wave w owns 32 gate columns and the same 32 up columns,
//    so SwiGLU is computed in registers and h = bf16(silu(g) * u) is written
//    in sorted-pair order (the down kernel reads it contiguously).
//  * down kernel: 256 output features per workgroup, y (fp32) scattered to
//    the pair's row for the shared combine kernel.
//  * FP4 operand (README "How it fits": FP4 delta GEMM for gate-flagged tokens
//    on delta-cache experts; a shared expert kept in NVFP4): a partition step
//    reorders each delta expert's run of pairs so that its gate-flagged pairs
//    come first.  The 2-bit kernels run every expert's whole run and leave the
//    fp32 pre-activations of the flagged rows; FP4 kernels of their own then
//    run only the flagged rows, 128 per tile, so no MFMA multiplies a row that
//    takes no delta: gate/up adds the delta and applies SwiGLU, down adds its
//    product to y.  A lane dequantises each 8 FP4 values as e2m1 -> f32 ->
//    * scale -> bf16, exact (e2m1 * e4m3 has at most 6 significant bits).  An
//    NVFP4 shared expert's tiles run only in the FP4 kernels.
#include <algorithm>

#include "moet_common.h"

namespace moet {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kPM = 160;    // rows per M-tile
constexpr int kPB = kPM / 16;     // 16-row MFMA blocks per M-tile (2-bit kernels)
constexpr int kASeg = kPM / 32;   // 8-row A segments each wavefront stages per step
constexpr int kPK = 64;     // k per pipeline step
constexpr int kPW = 4;      // wavefronts per workgroup

struct PrefillParams {
    const uint16_t *x;
    int T, k, H, I, E;
    const int32_t *ids;
    const float *w;
    const int32_t *offsets;
    const int32_t *sorted;
    moet_w2 w13, w2, sh13, sh2;
    int has_shared;
    float swiglu_limit;
    uint16_t *h;        // [P + T][I] bf16, rows in `order` (shared expert: P + t)
    float *ypart;       // [P + T][H] fp32, rows by pair id (shared expert: P + t)
    float *pre;         // [P][2I] fp32 gate/up pre-activations of flagged rows, rows in `order` (aliases ypart)
    uint16_t *out;
    const int32_t *order;   // the pairs in expert order, a delta expert's flagged pairs first (= sorted without delta)
    const int32_t *nflag;   // per expert: its flagged pairs at the head of its run in `order` (null: none)
    int n_mslots;       // upper bound on 160-row M-tiles (grid of the 2-bit kernels)
    int4 *tiles;        // [n_mslots] M-tile table: (expert, first row, rows, flagged end); rows 0 = no tile
    int n_ntiles;
    const int32_t *base_slot;   // expert -> cache slot of w13/w2 (null: expert e at e)
    int n_base_slots;
    int32_t *miss_count;        // routings to missing experts (null: not counted)
    const uint8_t *gate;        // confidence-gate flags per token (null: no delta)
    int n_slots;                // delta cache
    const int32_t *slot_of_expert;
    moet_fp4 d13, d2;
    int shared_fp4;             // the shared expert is NVFP4 (shf13 / shf2)
    moet_fp4 shf13, shf2;
};

// cache slot of expert e's 2-bit planes, or -1 when it is missing from the expert cache
__device__ __forceinline__ int weight_slot(const PrefillParams &p, int e)
{
    if (!p.base_slot) return e;
    const int ws = p.base_slot[e];
    return (ws >= 0 && ws < p.n_base_slots) ? ws : -1;
}

struct MTile {
    int e;        // expert, or -1 for the shared expert
    int row0;     // first row in `order` (shared: first token)
    int rows;     // valid rows (<= the tile size)
    int fl_end;   // rows of `order` below this take the FP4 delta (the flagged head of a delta expert's run)
};

// Expert e's run [o0, o1) of sorted pairs, clamped to [0, P]: the routing arrays
// come from the route call, and the clamp keeps every index derived from them
// in bounds if they do not.
__device__ __forceinline__ void expert_run(const PrefillParams &p, int e, int &o0, int &o1)
{
    const int P = p.T * p.k;
    o0 = min(max(p.offsets[e], 0), P);
    o1 = min(max(p.offsets[e + 1], o0), P);
}

// The M-tile table of the 2-bit kernels: slot ms -> (expert, first row in
// `order`, rows, flagged end).  Each expert's run (the 2-bit shared expert's
// T tokens after the routed experts) is cut into tiles of kPM rows, the last
// one partial.  The tiles are ordered by their 16-row block count, largest
// first (within a count, by expert), so the grid's last workgroups are its
// shortest and finish closer together; the slots after the last tile get
// rows = 0.  One wavefront writes
// the table once per forward (a pass counting the tiles of each block count,
// then a pass placing them: scans for the full tiles, one ballot per count for
// the partial ones), so each GEMM workgroup finds its tile with one load and the
// slots beyond the last tile exit at once.
__global__ __launch_bounds__(64) void mtile_table_kernel(PrefillParams p)
{
    constexpr int kCls = kPM / 16;   // classes 1 .. kCls (index = class - 1)
    const int lane = threadIdx.x;
    const uint64_t below = (1ull << lane) - 1ull;
    const bool sh = p.has_shared && !p.shared_fp4;
    // pass 1: tiles per class
    int ncls[kCls];
#pragma unroll
    for (int c = 0; c < kCls; ++c) ncls[c] = 0;
    for (int c0 = 0; c0 < p.E + 64; c0 += 64) {
        const int e = c0 + lane;
        int cnt = 0;
        if (e < p.E) {
            int o0, o1;
            expert_run(p, e, o0, o1);
            cnt = o1 - o0;
        } else if (sh && e == p.E) {
            cnt = p.T;   // the shared expert after the routed ones
        }
        const int full = cnt / kPM, rem = cnt - full * kPM;
        const int rc = rem ? (rem + 15) / 16 : 0;
        int fsum = full;
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) fsum += __shfl_xor(fsum, off, 64);
        ncls[kCls - 1] += fsum;
#pragma unroll
        for (int c = 0; c < kCls; ++c) ncls[c] += __popcll(__ballot(rc == c + 1));
        if (c0 >= p.E) break;
    }
    int base[kCls];   // first slot of each class, largest class first
    int acc = 0;
#pragma unroll
    for (int c = kCls - 1; c >= 0; --c) {
        base[c] = acc;
        acc += ncls[c];
    }
    // pass 2: write the tiles
    for (int c0 = 0; c0 < p.E + 64; c0 += 64) {
        const int e = c0 + lane;
        int cnt = 0, o0 = 0, fl = 0, ee = e;
        if (e < p.E) {
            int o1;
            expert_run(p, e, o0, o1);
            cnt = o1 - o0;
            fl = o0 + (p.nflag ? p.nflag[e] : 0);
        } else if (sh && e == p.E) {
            cnt = p.T;
            ee = -1;
        }
        const int full = cnt / kPM, rem = cnt - full * kPM;
        const int rc = rem ? (rem + 15) / 16 : 0;
        int incl = full;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int v = __shfl_up(incl, off, 64);
            if (lane >= off) incl += v;
        }
        for (int t = 0; t < full; ++t) {
            const int ms = base[kCls - 1] + incl - full + t;
            if (ms < p.n_mslots) p.tiles[ms] = make_int4(ee, o0 + t * kPM, kPM, fl);
        }
        base[kCls - 1] += __shfl(incl, 63, 64);
#pragma unroll
        for (int c = 0; c < kCls; ++c) {
            const uint64_t m = __ballot(rc == c + 1);
            if (rc == c + 1) {
                const int ms = base[c] + __popcll(m & below);
                if (ms < p.n_mslots) p.tiles[ms] = make_int4(ee, o0 + full * kPM, rem, fl);
            }
            base[c] += __popcll(m);
        }
        if (c0 >= p.E) break;
    }
    for (int ms = acc + lane; ms < p.n_mslots; ms += 64) p.tiles[ms] = make_int4(0, 0, 0, 0);
}

// slot ms of the M-tile table (false: no tile)
__device__ __forceinline__ bool lookup_mtile(const PrefillParams &p, int ms, MTile &mt)
{
    const int4 v = p.tiles[ms];
    mt.e = __builtin_amdgcn_readfirstlane(v.x);
    mt.row0 = __builtin_amdgcn_readfirstlane(v.y);
    mt.rows = __builtin_amdgcn_readfirstlane(v.z);
    mt.fl_end = __builtin_amdgcn_readfirstlane(v.w);
    return mt.rows > 0;
}

// XCD-aware decode of the linear workgroup id into (M-tile slot, N-tile)
__device__ __forceinline__ void decode_wg(int id, int n_ntiles, int &ms, int &nt)
{
    const int xcd = id & 7, local = id >> 3;
    nt = local % n_ntiles;
    ms = (local / n_ntiles) * 8 + xcd;
}

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// per (row, 32-k block) dequant constants from a scale byte: the and-mask and
// or-constant that turn a code word into e2m1 values (both 0 for a zero scale,
// which then yields +0), and the per-half bf16 bit offset that multiplies a
// level +-1 / +-4 by the scale: level and scale are exact bf16 with the level's
// mantissa 0, so adding bits(scale) - bits(1.0) to the level's bits adds the
// exponents and copies the scale's mantissa.
__device__ __forceinline__ void block_consts(uint32_t scale_word, int byte, uint32_t &mask, uint32_t &orc,
                                             uint32_t &sadd)
{
    const uint32_t b = (scale_word >> (8 * byte)) & 0xFFu;
    const float f = __builtin_amdgcn_cvt_f32_fp8(b, 0);
    const uint32_t d = ((__float_as_uint(f) >> 16) - 0x3F80u) & 0xFFFFu;
    sadd = b ? (d | (d << 16)) : 0u;
    mask = b ? kW2Mask : 0u;
    orc = b ? kW2Or : 0u;
}

// the same for any codebook (or-constant `cbor`): `sadd` carries the block scale as a float
__device__ __forceinline__ void block_consts_gen(uint32_t scale_word, int byte, uint32_t cbor, uint32_t &mask,
                                                 uint32_t &orc, uint32_t &sadd)
{
    const uint32_t b = (scale_word >> (8 * byte)) & 0xFFu;
    sadd = __float_as_uint(__builtin_amdgcn_cvt_f32_fp8(b, 0));
    mask = kW2Mask;
    orc = cbor;
}

typedef float f32x2 __attribute__((ext_vector_type(2)));

// e2m1 byte B of w (low nibble first) as two bf16 of value * sc (exact)
template <int B>
__device__ __forceinline__ void deq_fp4_pair(uint32_t w, float sc, bf16x8 &r)
{
    const f32x2 v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, B);
    r[2 * B] = (__bf16)(v.x * sc);
    r[2 * B + 1] = (__bf16)(v.y * sc);
}

// 8 bf16 of one row for one MFMA k-step from 8 e2m1 codes, times `sc` (exact)
__device__ __forceinline__ bf16x8 deq_fp4(uint32_t w, float sc)
{
    bf16x8 r;
    deq_fp4_pair<0>(w, sc, r);
    deq_fp4_pair<1>(w, sc, r);
    deq_fp4_pair<2>(w, sc, r);
    deq_fp4_pair<3>(w, sc, r);
    return r;
}

// 8 bf16 of one row for one MFMA k-step: elements 8h .. 8h+7 of code word w
// (sh = 2h selects the bit pair of each nibble), times the block scale
template <bool GEN>
__device__ __forceinline__ bf16x8 deq_frag(uint32_t w, uint32_t sh, uint32_t mask, uint32_t orc, uint32_t sadd)
{
    if constexpr (GEN) return deq_fp4(and_or_v(w << sh, mask, orc), __uint_as_float(sadd));

    const uint32_t f = and_or_v(w << sh, mask, orc);
    const u16x2 a = __builtin_bit_cast(u16x2, sadd);
    uint32_t q[4];
    q[0] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(u16x2, fp4_pair<0>(f)) + a);
    q[1] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(u16x2, fp4_pair<1>(f)) + a);
    q[2] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(u16x2, fp4_pair<2>(f)) + a);
    q[3] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(u16x2, fp4_pair<3>(f)) + a);
    return __builtin_bit_cast(bf16x8, make_uint4(q[0], q[1], q[2], q[3]));
}

// ---------------------------------------------------------------------------
// Pipeline: kPS-stage LDS ring filled by LDS-DMA (global_load_lds) so no
// registers are held for prefetch.  Per stage and wavefront: one A segment
// (1 KiB) per valid 32-row block of the tile (at most kASeg), 1 B chunk
// (1 KiB = 64 rows x 16 B), 1 scale dword per row of the B chunk (256 B).  The
// DMA is issued from inline asm, invisible to the compiler's wait-count pass,
// and waited explicitly (segments + 2 per stage).
// ---------------------------------------------------------------------------
constexpr int kPS = 3;                         // stages
constexpr int kStageA = kPM * 128;             // kPM rows x 64 k bf16
constexpr int kStageB = 4 * 1024;              // 256 B-rows x 16 B
constexpr int kStageS = 4 * 256;               // 256 rows x one scale dword
constexpr int kStage = kStageA + kStageB + kStageS;

__device__ __forceinline__ void dma16(const void *g, uint32_t lds_base)
{
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(lds_base) : "memory", "m0");
}

__device__ __forceinline__ void dma4(const void *g, uint32_t lds_base)
{
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" ::"v"(g), "s"(lds_base) : "memory", "m0");
}

// wait until at most n of this wave's LDS-DMA instructions are outstanding, then
// barrier (every wave's part of the stage has landed; the oldest buffer is free)
template <int N>
__device__ __forceinline__ void wait_barrier()
{
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}

// A tile in LDS: row r (128 B = 8 columns of 16 B) holds logical column c at
// physical column c ^ ((r >> 1) & 7).  A ds_read_b128 is served 16 lanes at a
// time over 64 four-byte banks (256 B); the 16 lanes of an A-fragment read
// cover 16 consecutive rows, and this swizzle puts them in 16 distinct 16-byte
// slots of a 256-byte window, so the read is conflict-free.
__device__ __forceinline__ int a_swz(int r) { return (r >> 1) & 7; }

__device__ __forceinline__ bf16x8 a_frag(const uint8_t *a, int r, int c)
{
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(a + r * 128 + ((c ^ a_swz(r)) << 4)));
}

// logical 16-byte column that lane `lane` fetches into its LDS slot of A segment g
// (rows 8g .. 8g + 7, row 8g + lane / 8, physical column lane % 8): the inverse of
// a_swz for those rows, whose (r >> 1) & 7 is 4 (g & 1) + lane / 16
__device__ __forceinline__ int a_dma_col(int lane, int g) { return (lane & 7) ^ (4 * (g & 1) + (lane >> 4)); }

struct PipeSrc {
    const uint8_t *arow[kASeg]; // this lane's A source rows, one per A segment it fetches
    const uint8_t *bsrc;        // this wave's B storage tile (codes), row = lane
    const uint8_t *ssrc;        // this wave's B storage tile (scales), row = lane
    int K;
};

// issue the DMA of pipeline step s into stage buffer `stage`.  Only the NSEG * 32
// rows of the tile's valid 32-row blocks are staged: wave w fetches A segments
// NSEG w .. NSEG w + NSEG - 1.
template <int NSEG>
__device__ __forceinline__ void issue_stage(const PipeSrc &src, uint8_t *smem, int stage, int s, int wave, int lane)
{
    const uint32_t base = (uint32_t)(uintptr_t)(smem + stage * kStage);
#pragma unroll
    for (int i = 0; i < NSEG; ++i)
        dma16(src.arow[i] + (size_t)s * 128 + a_dma_col(lane, NSEG * wave + i) * 16,
              base + (uint32_t)((NSEG * wave + i) * 1024));
    dma16(src.bsrc + ((size_t)s * 64 + lane) * 16, base + kStageA + wave * 1024);
    dma4(src.ssrc + ((size_t)(s >> 1) * 64 + lane) * 4, base + kStageA + kStageB + wave * 256);
}

// Main loop shared by both 2-bit kernels, on v_mfma_f32_16x16x32_bf16 so that an
// M-tile costs MFMAs for ceil(rows / 16) blocks of 16 rows.  acc[mb][nb] accumulates
// the 16 x 16 product of A rows 16 mb .. +15 and the dequantised B block nb, with the
// B fragment as the MFMA's first operand so that the result comes out transposed:
// lane l holds features 4 (l / 16) .. + 3 of tile row 16 mb + l % 16, which the
// epilogues store as one 16-byte (y) or 8-byte (h) write.  brow[nb] = index (0..255)
// of this lane's B row within the workgroup's 256 B-rows (lane l loads the fragment
// of feature l % 16 of each of its four 16-feature blocks).  The 32 k of one MFMA are split over the lane groups
// g = l / 16 so that lane group g always reads the same pair of 16-k code words of
// a 64-k step (words 2 (g / 2) and 2 (g / 2) + 1, i.e. one 32-k scale block): MFMA
// kc of the step takes word 2 (g / 2) + kc, elements 8 (g % 2) .. + 7, and the A
// fragment of the same 8 k.  NB = valid 16-row blocks; the tile's ceil(NB / 2)
// 32-row blocks are staged.
// GEN: the generic dequant, with the or-constant cbor[nb] of B row brow[nb]'s codebook
template <int NB, bool GEN>
__device__ __forceinline__ void gemm_pipe_n(const PipeSrc &src, uint8_t *smem, const int brow[4], f32x4 acc[kPB][4],
                                            const uint32_t cbor[4])
{
    constexpr int NSEG = (NB + 1) / 2;
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4;                 // k group of the MFMA fragment
    const int wsel = g >> 1;                 // this lane's word pair / scale block of a step
    const uint32_t sh = 2 * (g & 1);         // selects elements 8 (g % 2) .. + 7 of a code word
    const int nsteps = src.K / kPK;
#pragma unroll
    for (int st = 0; st < kPS - 1; ++st)
        if (st < nsteps) issue_stage<NSEG>(src, smem, st, st, wave, lane);
    for (int s = 0; s < nsteps; ++s) {
        // stages issued after s: min(kPS - 2, nsteps - 1 - s), NSEG + 2 DMAs each
        if (s + 1 < nsteps) wait_barrier<(NSEG + 2) * (kPS - 2)>();
        else wait_barrier<0>();
        if (s + kPS - 1 < nsteps) issue_stage<NSEG>(src, smem, (s + kPS - 1) % kPS, s + kPS - 1, wave, lane);
        const uint8_t *stg = smem + (s % kPS) * kStage;
        const uint8_t *aT = stg;
        const uint8_t *bT = stg + kStageA;
        const uint8_t *sT = stg + kStageA + kStageB;
        uint2 bw[4];
        uint32_t mask[4], orc[4], sadd[4];
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
            bw[nb] = *reinterpret_cast<const uint2 *>(bT + brow[nb] * 16 + 8 * wsel);
            const uint32_t sw = *reinterpret_cast<const uint32_t *>(sT + brow[nb] * 4);
            if constexpr (GEN) block_consts_gen(sw, 2 * (s & 1) + wsel, cbor[nb], mask[nb], orc[nb], sadd[nb]);
            else block_consts(sw, 2 * (s & 1) + wsel, mask[nb], orc[nb], sadd[nb]);
        }
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) {
            bf16x8 bfr[4];
#pragma unroll
            for (int nb = 0; nb < 4; ++nb)
                bfr[nb] = deq_frag<GEN>(kc ? bw[nb].y : bw[nb].x, sh, mask[nb], orc[nb], sadd[nb]);
#pragma unroll
            for (int mb = 0; mb < NB; ++mb) {
                const bf16x8 afr = a_frag(aT, 16 * mb + (lane & 15), 4 * wsel + 2 * kc + (g & 1));
#pragma unroll
                for (int nb = 0; nb < 4; ++nb)
                    acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bfr[nb], afr, acc[mb][nb], 0, 0, 0);
            }
        }
    }
}

template <bool GEN>
__device__ __forceinline__ void gemm_pipe_g(const PipeSrc &src, uint8_t *smem, const int brow[4], f32x4 acc[kPB][4],
                                            int nb16, const uint32_t cbor[4])
{
    switch (nb16) {
    case 1: gemm_pipe_n<1, GEN>(src, smem, brow, acc, cbor); break;
    case 2: gemm_pipe_n<2, GEN>(src, smem, brow, acc, cbor); break;
    case 3: gemm_pipe_n<3, GEN>(src, smem, brow, acc, cbor); break;
    case 4: gemm_pipe_n<4, GEN>(src, smem, brow, acc, cbor); break;
    case 5: gemm_pipe_n<5, GEN>(src, smem, brow, acc, cbor); break;
    case 6: gemm_pipe_n<6, GEN>(src, smem, brow, acc, cbor); break;
    case 7: gemm_pipe_n<7, GEN>(src, smem, brow, acc, cbor); break;
    case 8: gemm_pipe_n<8, GEN>(src, smem, brow, acc, cbor); break;
    case 9: gemm_pipe_n<9, GEN>(src, smem, brow, acc, cbor); break;
    default: gemm_pipe_n<10, GEN>(src, smem, brow, acc, cbor); break;
    }
}

// one instantiation per number of valid 16-row blocks and dequant kind, chosen once per
// workgroup; cb[nb]: codebook id of B row brow[nb]'s matrix
__device__ __forceinline__ void gemm_pipe(const PipeSrc &src, uint8_t *smem, const int brow[4], f32x4 acc[kPB][4],
                                          int nb16, const uint32_t cb[4])
{
    const uint32_t cbor[4] = {w2_or_of(cb[0]), w2_or_of(cb[1]), w2_or_of(cb[2]), w2_or_of(cb[3])};
    if ((cb[0] | cb[1] | cb[2] | cb[3]) == 0) gemm_pipe_g<false>(src, smem, brow, acc, nb16, cbor);
    else gemm_pipe_g<true>(src, smem, brow, acc, nb16, cbor);
}

// ---------------------------------------------------------------------------
// Partition of the delta experts' rows.  One workgroup per expert e: its run
// [offsets[e], offsets[e+1]) of sorted pairs is copied to `order`, with the
// pairs of gate-flagged tokens first when e takes the FP4 delta (both parts
// keep their order), and nflag[e] = the number of flagged pairs (0 when e
// takes no delta).  e takes the delta when it holds a delta-cache slot that no
// lower expert holds and its 2-bit planes are resident.  Each thread owns a
// contiguous range of the run: one pass counts its flagged pairs, a block-wide
// exclusive scan gives its first slots, a second pass writes its pairs.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int delta_slot_of(const PrefillParams &p, int e)
{
    const int lane = threadIdx.x & 63;
    const int ds = p.slot_of_expert[e];
    if (ds < 0 || ds >= p.n_slots || weight_slot(p, e) < 0) return -1;
    bool lower = false;
    for (int i = lane; i < e; i += 64) lower |= p.slot_of_expert[i] == ds;
    return __ballot(lower) ? -1 : ds;
}

__global__ __launch_bounds__(256) void partition_kernel(PrefillParams p, int32_t *__restrict__ order,
                                                        int32_t *__restrict__ nflag)
{
    __shared__ int s_cnt[4];
    __shared__ int s_delta;
    const int e = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int P = p.T * p.k;
    if (wave == 0) {
        const int ds = delta_slot_of(p, e);
        if (lane == 0) s_delta = ds >= 0;
    }
    __syncthreads();
    const bool delta = s_delta != 0;
    int o0, o1;
    expert_run(p, e, o0, o1);
    const int n = o1 - o0;
    const int per = (n + 255) / 256;
    const int b0 = o0 + min(tid * per, n), b1 = o0 + min(tid * per + per, n);
    int f = 0;
    if (delta)
        for (int i = b0; i < b1; ++i) f += p.gate[min(max(p.sorted[i], 0), P - 1) / p.k] != 0;
    int inc = f;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int v = __shfl_up(inc, off, 64);
        if (lane >= off) inc += v;
    }
    if (lane == 63) s_cnt[wave] = inc;
    __syncthreads();
    int before = inc - f;
    for (int w = 0; w < wave; ++w) before += s_cnt[w];
    const int F = s_cnt[0] + s_cnt[1] + s_cnt[2] + s_cnt[3];
    int fi = o0 + before, ui = o0 + F + (b0 - o0) - before;
    for (int i = b0; i < b1; ++i) {
        const int pr = p.sorted[i];
        const bool fl = delta && p.gate[min(max(pr, 0), P - 1) / p.k] != 0;
        if (fl) order[fi++] = pr;
        else order[ui++] = pr;
    }
    if (tid == 0) nflag[e] = F;
}

// gate/up + SwiGLU.  N-tile nt covers h columns [128 nt, 128 nt + 128); wave w
// owns gate rows and up rows [128 nt + 32 w, + 32).
__device__ __forceinline__ void fc1_prefill_body(const PrefillParams &p, uint8_t *smem)
{
    int ms, nt;
    decode_wg(blockIdx.x, p.n_ntiles, ms, nt);
    if (ms >= p.n_mslots) return;
    MTile mt;
    if (!lookup_mtile(p, ms, mt)) return;
    const int nb16 = (mt.rows + 15) / 16;
    const int nmb = (nb16 + 1) / 2;   // staged 32-row blocks
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int H = p.H, I = p.I, P = p.T * p.k;
    // A rows fetched by this lane: segment i of wave w holds rows 8(nmb w + i) .. +7; lane -> row + lane/8
    // (only the nmb valid 32-row blocks are staged)
    PipeSrc src;
    src.K = H;
#pragma unroll
    for (int i = 0; i < kASeg; ++i) {
        const int r = min(8 * (nmb * wave + i) + (lane >> 3), mt.rows - 1);
        int tok;
        if (mt.e >= 0) tok = min(max(p.order[mt.row0 + r], 0), P - 1) / p.k;
        else tok = mt.row0 + r;
        src.arow[i] = reinterpret_cast<const uint8_t *>(p.x + (size_t)tok * H);
    }
    // B: 256 rows = gate rows [128 nt, +128) then up rows [128 nt, +128); wave w fetches storage tile w
    const int ws = (mt.e >= 0) ? weight_slot(p, mt.e) : 0;
    if (ws < 0) return;   // missing expert: no work, the combine skips its routings
    // B rows of this lane's fragments: gate jl + 16 c, up 128 + jl + 16 c (c = 0, 1)
    const int jl = 32 * wave + (lane & 15);
    const int brow[4] = {jl, jl + 16, 128 + jl, 128 + jl + 16};
    f32x4 acc[kPB][4];
#pragma unroll
    for (int mb = 0; mb < kPB; ++mb)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[mb][nb][v] = 0.f;
    const moet_w2 &W = (mt.e >= 0) ? p.w13 : p.sh13;
    const int m0 = (mt.e >= 0) ? 2 * ws : 0;
    const int mat = m0 + (wave >> 1);
    const int tile = 2 * nt + (wave & 1);
    src.bsrc = reinterpret_cast<const uint8_t *>(W.codes + (size_t)mat * I * H / 16) + (size_t)tile * (H / 64) * 1024;
    src.ssrc = W.scales + (size_t)mat * I * H / 32 + (size_t)tile * (H / 128) * 256;
    const uint32_t cbg = w2_codebook(W, m0), cbu = w2_codebook(W, m0 + 1);
    const uint32_t cb[4] = {cbg, cbg, cbu, cbu};   // gate, gate, up, up
    gemm_pipe(src, smem, brow, acc, nb16, cb);
    const float sg = W.scale2[m0], su = W.scale2[m0 + 1];
    const int rowbase = (mt.e >= 0) ? mt.row0 : P + mt.row0;   // h row of tile row 0
    // acc[mb][nb][v]: tile row 16 mb + lane % 16, feature 4 (lane / 16) + v of B block nb
    const int r0 = lane & 15, f0 = 4 * (lane >> 4);
#pragma clang loop unroll(full)
    for (int mb = 0; mb < kPB; ++mb) {
        const int r = 16 * mb + r0;
        if (mb < nb16 && r < mt.rows) {
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                const int j = 128 * nt + 32 * wave + 16 * c + f0;   // h columns j .. j + 3
                float g[4], u[4];
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    g[v] = acc[mb][c][v] * sg;
                    u[v] = acc[mb][2 + c][v] * su;
                }
                if (rowbase + r < mt.fl_end) {   // flagged row: the FP4 kernel adds its delta, then SwiGLU
                    float *pre = p.pre + (size_t)(rowbase + r) * (2 * I) + j;
                    *reinterpret_cast<float4 *>(pre) = make_float4(g[0], g[1], g[2], g[3]);
                    *reinterpret_cast<float4 *>(pre + I) = make_float4(u[0], u[1], u[2], u[3]);
                    continue;
                }
                uint32_t hv[4];
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    if (p.swiglu_limit > 0.f) {
                        g[v] = fminf(g[v], p.swiglu_limit);
                        u[v] = fminf(fmaxf(u[v], -p.swiglu_limit), p.swiglu_limit);
                    }
                    hv[v] = f32_to_bf16_rne(silu_f32(g[v]) * u[v]);
                }
                *reinterpret_cast<uint2 *>(p.h + (size_t)(rowbase + r) * I + j) =
                    make_uint2(hv[0] | (hv[1] << 16), hv[2] | (hv[3] << 16));
            }
        }
    }
}

__global__ __launch_bounds__(64 * kPW) __attribute__((amdgpu_waves_per_eu(2))) void fc1_prefill_kernel(PrefillParams p)
{
    __shared__ __align__(1024) uint8_t smem[kPS * kStage];
    if (p.miss_count && blockIdx.x == 0 && threadIdx.x == 0) *p.miss_count = 0;   // counted by the combine
    fc1_prefill_body(p, smem);
}

// down: N-tile nt covers output features [256 nt, 256 nt + 256); wave w owns 64 of them.
__device__ __forceinline__ void fc2_prefill_body(const PrefillParams &p, uint8_t *smem)
{
    int ms, nt;
    decode_wg(blockIdx.x, p.n_ntiles, ms, nt);
    if (ms >= p.n_mslots) return;
    MTile mt;
    if (!lookup_mtile(p, ms, mt)) return;
    const int nb16 = (mt.rows + 15) / 16;
    const int nmb = (nb16 + 1) / 2;   // staged 32-row blocks
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int H = p.H, I = p.I, P = p.T * p.k;
    const int rowbase = (mt.e >= 0) ? mt.row0 : P + mt.row0;
    PipeSrc src;
    src.K = I;
#pragma unroll
    for (int i = 0; i < kASeg; ++i) {
        const int r = min(8 * (nmb * wave + i) + (lane >> 3), mt.rows - 1);
        src.arow[i] = reinterpret_cast<const uint8_t *>(p.h + (size_t)(rowbase + r) * I);
    }
    const int ws = (mt.e >= 0) ? weight_slot(p, mt.e) : 0;
    if (ws < 0) return;
    const int tile = 4 * nt + wave;
    const int bl = 64 * wave + (lane & 15);
    const int brow[4] = {bl, bl + 16, bl + 32, bl + 48};
    f32x4 acc[kPB][4];
#pragma unroll
    for (int mb = 0; mb < kPB; ++mb)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[mb][nb][v] = 0.f;
    const moet_w2 &W = (mt.e >= 0) ? p.w2 : p.sh2;
    const int m0 = (mt.e >= 0) ? ws : 0;
    src.bsrc = reinterpret_cast<const uint8_t *>(W.codes + (size_t)m0 * H * I / 16) + (size_t)tile * (I / 64) * 1024;
    src.ssrc = W.scales + (size_t)m0 * H * I / 32 + (size_t)tile * (I / 128) * 256;
    const uint32_t cbw = w2_codebook(W, m0);
    const uint32_t cb[4] = {cbw, cbw, cbw, cbw};
    gemm_pipe(src, smem, brow, acc, nb16, cb);
    const float s2 = W.scale2[m0];
    // acc[mb][nb][v]: tile row 16 mb + lane % 16, output feature 64 wave + 16 nb + 4 (lane / 16) + v
    const int r0 = lane & 15, f0 = 64 * wave + 4 * (lane >> 4);
#pragma clang loop unroll(full)
    for (int mb = 0; mb < kPB; ++mb) {
        const int r = 16 * mb + r0;
        if (mb < nb16 && r < mt.rows) {
            const int prow = (mt.e >= 0) ? min(max(p.order[mt.row0 + r], 0), P - 1) : P + mt.row0 + r;
            float *y = p.ypart + (size_t)prow * H + 256 * nt + f0;
#pragma unroll
            for (int nb = 0; nb < 4; ++nb)
                *reinterpret_cast<float4 *>(y + 16 * nb) =
                    make_float4(acc[mb][nb][0] * s2, acc[mb][nb][1] * s2, acc[mb][nb][2] * s2, acc[mb][nb][3] * s2);
        }
    }
}

__global__ __launch_bounds__(64 * kPW) __attribute__((amdgpu_waves_per_eu(2))) void fc2_prefill_kernel(PrefillParams p)
{
    __shared__ __align__(1024) uint8_t smem[kPS * kStage];
    fc2_prefill_body(p, smem);
}

// ---------------------------------------------------------------------------
// FP4 pass.  Delta tiles hold the gate-flagged rows of a delta expert (the
// head of its run in `order`), up to 128 per tile, so no MFMA multiplies a row
// that takes no delta; an NVFP4 shared expert's tiles hold 128 tokens.  Per
// stage and wavefront the LDS-DMA ring carries the tile's valid A segments and
// the wave's two 32-k FP4 chunks and FP4 scale dword.  gate/up adds the delta
// to the 2-bit pre-activations the 2-bit kernel left for these rows and
// applies SwiGLU; down adds its product to the 2-bit y.
// ---------------------------------------------------------------------------
#ifndef MOET_FP4_TILE
#define MOET_FP4_TILE 128
#endif
constexpr int kDM = MOET_FP4_TILE;            // rows per FP4 M-tile (64 or 128)
constexpr int kDB = kDM / 16;                 // 16-row MFMA blocks
constexpr int kDSeg = kDM / 32;               // 8-row A segments per wavefront (4 waves x kDSeg x 8 = kDM rows)
constexpr int kDStageA = kDM * 128;
constexpr int kDOffB4 = kDStageA;
constexpr int kDOffS4 = kDOffB4 + 8 * 1024;
constexpr int kDStage = kDOffS4 + 4 * 256;    // 25 KiB at 128 rows, 17 KiB at 64
constexpr int kDWaves = kDM == 64 ? 3 : 2;    // waves per SIMD: workgroups per CU the LDS ring allows

struct DeltaSrc {
    const uint8_t *arow[kDSeg];   // this lane's A source rows, one per A segment it fetches
    const uint8_t *b4, *s4;       // this wave's FP4 storage tile: codes, scales (row = lane)
    int K;
};

// DMA of pipeline step s into stage buffer `stage` (NSEG valid A segments per wave)
template <int NSEG>
__device__ __forceinline__ void issue_dstage(const DeltaSrc &src, uint8_t *smem, int stage, int s, int wave, int lane)
{
    const uint32_t base = (uint32_t)(uintptr_t)(smem + stage * kDStage);
#pragma unroll
    for (int i = 0; i < NSEG; ++i)
        dma16(src.arow[i] + (size_t)s * 128 + a_dma_col(lane, NSEG * wave + i) * 16,
              base + (uint32_t)((NSEG * wave + i) * 1024));
    dma16(src.b4 + ((size_t)(2 * s) * 64 + lane) * 16, base + kDOffB4 + wave * 2048);
    dma16(src.b4 + ((size_t)(2 * s + 1) * 64 + lane) * 16, base + kDOffB4 + wave * 2048 + 1024);
    dma4(src.s4 + ((size_t)(s >> 1) * 64 + lane) * 8 + (s & 1) * 4, base + kDOffS4 + wave * 256);
}

// block-16 scale byte Q of a scale dword as a float
template <int Q>
__device__ __forceinline__ float fp8_byte(uint32_t w) { return __builtin_amdgcn_cvt_f32_fp8(w, Q); }

// acc[mb][nb] accumulates the product of A rows 16 mb .. +15 and the dequantised
// FP4 B block nb on v_mfma_f32_16x16x32_bf16, transposed as in the 2-bit kernels
// (lane l loads the fragment of feature l % 16 of each of its four 16-feature
// blocks and holds features 4 (l / 16) .. + 3 of row 16 mb + l % 16).  MFMA kc of a 64-k step covers the step's 32-k FP4 chunk kc,
// lane group g = l / 16 taking its code dword g (8 k) and the A fragment of the
// same 8 k; that dword lies in block-16 2 kc + g / 2 of the row's scale dword.
// NB = valid 16-row blocks; ceil(NB / 2) 32-row blocks of A are staged.  The B of
// MFMA 1 is dequantised while the MFMAs of MFMA 0 run.
template <int NB>
__device__ __forceinline__ void fp4_pipe_n(const DeltaSrc &src, uint8_t *smem, const int brow[4], f32x4 acc[kDB][4])
{
    constexpr int NSEG = (NB + 1) / 2;
    constexpr int kDma = NSEG + 3;    // DMA instructions per wave per stage
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4;
    const int nsteps = src.K / kPK;
    int boff[4];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) boff[nb] = kDOffB4 + (brow[nb] >> 6) * 2048 + (brow[nb] & 63) * 16 + 4 * g;
#pragma unroll
    for (int st = 0; st < kPS - 1; ++st)
        if (st < nsteps) issue_dstage<NSEG>(src, smem, st, st, wave, lane);
    for (int s = 0; s < nsteps; ++s) {
        if (s + 1 < nsteps) wait_barrier<kDma * (kPS - 2)>();
        else wait_barrier<0>();
        if (s + kPS - 1 < nsteps) issue_dstage<NSEG>(src, smem, (s + kPS - 1) % kPS, s + kPS - 1, wave, lane);
        const uint8_t *stg = smem + (s % kPS) * kDStage;
        // every B word and scale of the step first, so one LDS round trip covers them
        uint32_t w0[4], w1[4], sw[4];
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
            w0[nb] = *reinterpret_cast<const uint32_t *>(stg + boff[nb]);
            w1[nb] = *reinterpret_cast<const uint32_t *>(stg + boff[nb] + 1024);
            sw[nb] = *reinterpret_cast<const uint32_t *>(stg + kDOffS4 + brow[nb] * 4) >> (8 * (g >> 1));
        }
        bf16x8 b0[4], b1[4];
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) b0[nb] = deq_fp4(w0[nb], fp8_byte<0>(sw[nb]));
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) b1[nb] = deq_fp4(w1[nb], fp8_byte<2>(sw[nb]));
#pragma unroll
        for (int mb = 0; mb < NB; ++mb) {
            const bf16x8 afr = a_frag(stg, 16 * mb + (lane & 15), g);
#pragma unroll
            for (int nb = 0; nb < 4; ++nb)
                acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b0[nb], afr, acc[mb][nb], 0, 0, 0);
        }
#pragma unroll
        for (int mb = 0; mb < NB; ++mb) {
            const bf16x8 afr = a_frag(stg, 16 * mb + (lane & 15), 4 + g);
#pragma unroll
            for (int nb = 0; nb < 4; ++nb)
                acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b1[nb], afr, acc[mb][nb], 0, 0, 0);
        }
    }
}

__device__ __forceinline__ void fp4_pipe(const DeltaSrc &src, uint8_t *smem, const int brow[4], f32x4 acc[kDB][4],
                                         int nb16)
{
    if constexpr (kDB == 4) {
        switch (nb16) {
        case 1: fp4_pipe_n<1>(src, smem, brow, acc); break;
        case 2: fp4_pipe_n<2>(src, smem, brow, acc); break;
        case 3: fp4_pipe_n<3>(src, smem, brow, acc); break;
        default: fp4_pipe_n<4>(src, smem, brow, acc); break;
        }
    } else {
        switch (nb16) {
        case 1: fp4_pipe_n<1>(src, smem, brow, acc); break;
        case 2: fp4_pipe_n<2>(src, smem, brow, acc); break;
        case 3: fp4_pipe_n<3>(src, smem, brow, acc); break;
        case 4: fp4_pipe_n<4>(src, smem, brow, acc); break;
        case 5: fp4_pipe_n<5>(src, smem, brow, acc); break;
        case 6: fp4_pipe_n<6>(src, smem, brow, acc); break;
        case 7: fp4_pipe_n<7>(src, smem, brow, acc); break;
        default: fp4_pipe_n<8>(src, smem, brow, acc); break;
        }
    }
}

// The FP4 tiles of a workgroup.  Delta mode (SHARED = false): blockIdx.y is a
// delta-cache slot; its expert is the lowest one holding it, and its tiles are
// the flagged rows at the head of its run in `order`, taken z, z + Z, ...
// (blockIdx.z, gridDim.z).  NVFP4 shared expert (SHARED = true): blockIdx.y is
// the tile of tokens [128 y, 128 y + 128).
struct DeltaTiles {
    int e, ds, row0, count;   // expert (-1: shared), delta slot, first row (in `order`, or token), rows
};

template <bool SHARED>
__device__ __forceinline__ bool delta_tiles(const PrefillParams &p, DeltaTiles &dt)
{
    if constexpr (SHARED) {
        dt.e = -1;
        dt.ds = -1;
        dt.row0 = kDM * blockIdx.y;
        dt.count = min(kDM, p.T - dt.row0);
        return dt.count > 0;
    } else {
        const int lane = threadIdx.x & 63, s = blockIdx.y;
        int e = -1;
        for (int c = 0; c < p.E && e < 0; c += 64) {
            const uint64_t b = __ballot(c + lane < p.E && p.slot_of_expert[c + lane] == s);
            if (b) e = c + __builtin_ctzll(b);
        }
        e = __builtin_amdgcn_readfirstlane(e);
        if (e < 0 || p.nflag[e] == 0) return false;   // nflag is 0 unless e takes the delta
        dt.e = e;
        dt.ds = s;
        int o1;
        expert_run(p, e, dt.row0, o1);
        dt.count = p.nflag[e];
        return true;
    }
}

template <bool SHARED>
__device__ __forceinline__ void fc1_delta_body(const PrefillParams &p, uint8_t *smem)
{
    DeltaTiles dt;
    if (!delta_tiles<SHARED>(p, dt)) return;
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int H = p.H, I = p.I, P = p.T * p.k, nt = blockIdx.x;
    // B rows of this lane's fragments: gate jl + 16 c, up 128 + jl + 16 c (c = 0, 1)
    const int jl = 32 * wave + (lane & 15);
    const int brow[4] = {jl, jl + 16, 128 + jl, 128 + jl + 16};
    const moet_fp4 &F = SHARED ? p.shf13 : p.d13;
    const int fm0 = SHARED ? 0 : 2 * dt.ds;
    const int mat = wave >> 1, tile = 2 * nt + (wave & 1);
    DeltaSrc src;
    src.K = H;
    src.b4 = F.codes + (size_t)(fm0 + mat) * I * H / 2 + (size_t)tile * (H / 32) * 1024;
    src.s4 = F.scales + (size_t)(fm0 + mat) * I * H / 16 + (size_t)tile * (H / 128) * 512;
    const float dsg = F.scale2[fm0], dsu = F.scale2[fm0 + 1];
    const int ntile = (dt.count + kDM - 1) / kDM;
    for (int it = SHARED ? 0 : (int)blockIdx.z; it < ntile; it += SHARED ? 1 : (int)gridDim.z) {
        const int r0 = dt.row0 + kDM * it, rows = min(kDM, dt.count - kDM * it);
        const int nb16 = (rows + 15) / 16;
        const int nmb = (nb16 + 1) / 2;   // staged 32-row blocks
#pragma unroll
        for (int i = 0; i < kDSeg; ++i) {
            const int r = min(8 * (nmb * wave + i) + (lane >> 3), rows - 1);
            const int tok = SHARED ? r0 + r : min(max(p.order[r0 + r], 0), P - 1) / p.k;
            src.arow[i] = reinterpret_cast<const uint8_t *>(p.x + (size_t)tok * H);
        }
        f32x4 acc[kDB][4];
#pragma unroll
        for (int mb = 0; mb < kDB; ++mb)
#pragma unroll
            for (int nb = 0; nb < 4; ++nb)
#pragma unroll
                for (int v = 0; v < 4; ++v) acc[mb][nb][v] = 0.f;
        fp4_pipe(src, smem, brow, acc, nb16);
        const int hbase = SHARED ? P + r0 : r0;
        // acc[mb][nb][v]: tile row 16 mb + lane % 16, feature 4 (lane / 16) + v of B block nb
        const int rl = lane & 15, f0 = 4 * (lane >> 4);
#pragma clang loop unroll(full)
        for (int mb = 0; mb < kDB; ++mb) {
            const int r = 16 * mb + rl;
            if (mb < nb16 && r < rows) {
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    const int j = 128 * nt + 32 * wave + 16 * c + f0;   // h columns j .. j + 3
                    float g[4], u[4];
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        g[v] = acc[mb][c][v] * dsg;
                        u[v] = acc[mb][2 + c][v] * dsu;
                    }
                    if (!SHARED) {   // plus the 2-bit pre-activations of this row
                        const float *pre = p.pre + (size_t)(r0 + r) * (2 * I) + j;
                        const float4 pg = *reinterpret_cast<const float4 *>(pre);
                        const float4 pu = *reinterpret_cast<const float4 *>(pre + I);
                        g[0] += pg.x; g[1] += pg.y; g[2] += pg.z; g[3] += pg.w;
                        u[0] += pu.x; u[1] += pu.y; u[2] += pu.z; u[3] += pu.w;
                    }
                    uint32_t hv[4];
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        if (p.swiglu_limit > 0.f) {
                            g[v] = fminf(g[v], p.swiglu_limit);
                            u[v] = fminf(fmaxf(u[v], -p.swiglu_limit), p.swiglu_limit);
                        }
                        hv[v] = f32_to_bf16_rne(silu_f32(g[v]) * u[v]);
                    }
                    *reinterpret_cast<uint2 *>(p.h + (size_t)(hbase + r) * I + j) =
                        make_uint2(hv[0] | (hv[1] << 16), hv[2] | (hv[3] << 16));
                }
            }
        }
        __syncthreads();   // every wave is done with the ring before the next tile refills it
    }
}

template <bool SHARED>
__device__ __forceinline__ void fc2_delta_body(const PrefillParams &p, uint8_t *smem, int *s_prow)
{
    DeltaTiles dt;
    if (!delta_tiles<SHARED>(p, dt)) return;
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int H = p.H, I = p.I, P = p.T * p.k, nt = blockIdx.x;
    const int bl = 64 * wave + (lane & 15);
    const int brow[4] = {bl, bl + 16, bl + 32, bl + 48};
    const moet_fp4 &F = SHARED ? p.shf2 : p.d2;
    const int fm = SHARED ? 0 : dt.ds;
    const int tile = 4 * nt + wave;
    DeltaSrc src;
    src.K = I;
    src.b4 = F.codes + (size_t)fm * H * I / 2 + (size_t)tile * (I / 32) * 1024;
    src.s4 = F.scales + (size_t)fm * H * I / 16 + (size_t)tile * (I / 128) * 512;
    const float ds2 = F.scale2[fm];
    const int ntile = (dt.count + kDM - 1) / kDM;
    for (int it = SHARED ? 0 : (int)blockIdx.z; it < ntile; it += SHARED ? 1 : (int)gridDim.z) {
        const int r0 = dt.row0 + kDM * it, rows = min(kDM, dt.count - kDM * it);
        const int nb16 = (rows + 15) / 16;
        const int nmb = (nb16 + 1) / 2;   // staged 32-row blocks
        const int hbase = SHARED ? P + r0 : r0;
#pragma unroll
        for (int i = 0; i < kDSeg; ++i) {
            const int r = min(8 * (nmb * wave + i) + (lane >> 3), rows - 1);
            src.arow[i] = reinterpret_cast<const uint8_t *>(p.h + (size_t)(hbase + r) * I);
        }
        // y row (pair id) of each tile row, staged once for the epilogue
        if (tid < rows) s_prow[tid] = SHARED ? P + r0 + tid : min(max(p.order[r0 + tid], 0), P - 1);
        __syncthreads();
        f32x4 acc[kDB][4];
#pragma unroll
        for (int mb = 0; mb < kDB; ++mb)
#pragma unroll
            for (int nb = 0; nb < 4; ++nb)
#pragma unroll
                for (int v = 0; v < 4; ++v) acc[mb][nb][v] = 0.f;
        fp4_pipe(src, smem, brow, acc, nb16);
        // acc[mb][nb][v]: tile row 16 mb + lane % 16, output feature 64 wave + 16 nb + 4 (lane / 16) + v
        const int rl = lane & 15, f0 = 64 * wave + 4 * (lane >> 4);
#pragma clang loop unroll(full)
        for (int mb = 0; mb < kDB; ++mb) {
            const int r = 16 * mb + rl;
            if (mb < nb16 && r < rows) {
                float *y = p.ypart + (size_t)s_prow[r] * H + 256 * nt + f0;
#pragma unroll
                for (int nb = 0; nb < 4; ++nb) {
                    float4 d = make_float4(acc[mb][nb][0] * ds2, acc[mb][nb][1] * ds2, acc[mb][nb][2] * ds2,
                                           acc[mb][nb][3] * ds2);
                    if (!SHARED) {   // delta: added to the 2-bit y
                        const float4 y2 = *reinterpret_cast<const float4 *>(y + 16 * nb);
                        d = make_float4(y2.x + d.x, y2.y + d.y, y2.z + d.z, y2.w + d.w);
                    }
                    *reinterpret_cast<float4 *>(y + 16 * nb) = d;
                }
            }
        }
        __syncthreads();
    }
}

template <bool SHARED>
__global__ __launch_bounds__(64 * kPW) __attribute__((amdgpu_waves_per_eu(kDWaves))) void fc1_prefill_delta_kernel(PrefillParams p)
{
    __shared__ __align__(1024) uint8_t smem[kPS * kDStage];
    fc1_delta_body<SHARED>(p, smem);
}

template <bool SHARED>
__global__ __launch_bounds__(64 * kPW) __attribute__((amdgpu_waves_per_eu(kDWaves))) void fc2_prefill_delta_kernel(PrefillParams p)
{
    __shared__ __align__(1024) uint8_t smem[kPS * kDStage];
    __shared__ int s_prow[kDM];
    fc2_delta_body<SHARED>(p, smem, s_prow);
}

// out[t][n] = bf16(sum_j w[t][j] * y[(t, j)][n] + y_shared[t][n]), j in slot order;
// routings to experts missing from the expert cache contribute nothing and are
// counted once per token (by the first column block).  The token's ids and
// weights are wave-uniform (scalar loads); its y loads do not depend on them
// and are issued first, so the kernel pays about one memory round trip.
constexpr int kCombineMaxK = 16;

// Four output features per thread (16-byte y loads, 8-byte stores): the
// kernel streams (k + 1) fp32 rows of H per token.
__global__ __launch_bounds__(256) void combine_prefill_kernel(PrefillParams p)
{
    const int n = 4 * (blockIdx.x * 256 + threadIdx.x);
    const int t = blockIdx.y;
    const int P = p.T * p.k;
    const bool in = n < p.H;   // H % 4 == 0
    // the y rows sit at fixed positions (pair t*k + j, shared P + t): their loads
    // go out before the ids and weights arrive, so the two round trips overlap
    float4 y[kCombineMaxK];
    typedef float f4v __attribute__((ext_vector_type(4)));
#pragma unroll
    for (int j = 0; j < kCombineMaxK; ++j) {
        if (j < p.k && in) {
            const f4v v = __builtin_nontemporal_load(reinterpret_cast<const f4v *>(p.ypart + (size_t)(t * p.k + j) * p.H + n));
            y[j] = make_float4(v.x, v.y, v.z, v.w);
        } else {
            y[j] = make_float4(0.f, 0.f, 0.f, 0.f);
        }
    }
    const float4 ysh = (p.has_shared && in) ? *reinterpret_cast<const float4 *>(p.ypart + (size_t)(P + t) * p.H + n)
                                            : make_float4(0.f, 0.f, 0.f, 0.f);
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
    float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;   // rows of missing experts: selected out, never used
#pragma unroll
    for (int j = 0; j < kCombineMaxK; ++j)
        if (live[j]) {
            a0 = fmaf(wt[j], y[j].x, a0);
            a1 = fmaf(wt[j], y[j].y, a1);
            a2 = fmaf(wt[j], y[j].z, a2);
            a3 = fmaf(wt[j], y[j].w, a3);
        }
    if (p.has_shared) {
        a0 += ysh.x;
        a1 += ysh.y;
        a2 += ysh.z;
        a3 += ysh.w;
    }
    const uint32_t lo = f32_to_bf16_rne(a0) | (f32_to_bf16_rne(a1) << 16);
    const uint32_t hi = f32_to_bf16_rne(a2) | (f32_to_bf16_rne(a3) << 16);
    *reinterpret_cast<uint2 *>(p.out + (size_t)t * p.H + n) = make_uint2(lo, hi);
}

size_t decode_workspace_bytes(int T, int k, int H, int I);
int launch_decode(const moet_layer *, const uint16_t *, int, int, const int32_t *, const float *, const int32_t *,
                  const int32_t *, const uint8_t *, uint16_t *, int32_t *, void *, hipStream_t);

size_t prefill_workspace_bytes(int T, int k, int H, int I, int E)
{
    const size_t rows = (size_t)T * k + T;
    auto al = [](size_t b) { return (b + 255) & ~(size_t)255; };
    // h rows, y rows (or the flagged rows' pre-activations before them), the reordered pairs, the
    // flagged count per expert
    // and the M-tile table
    const size_t mslots = ((size_t)T * k + kPM - 1) / kPM + E + ((size_t)T + kPM - 1) / kPM;
    return al(rows * I * 2) + al(rows * (size_t)std::max(H, 2 * I) * 4) + al((size_t)T * k * 4) + al((size_t)E * 4) +
           al(mslots * 16);
}

int launch_prefill(const moet_layer *L, const uint16_t *x, int T, int k, const int32_t *ids, const float *w,
                   const int32_t *offsets, const int32_t *sorted, const uint8_t *gate, uint16_t *out, int32_t *miss_count,
                   void *ws, hipStream_t stream)
{
    if (L->H % 256) {
        // the grouped GEMM tiles need H % 256 == 0 (and I % 128 == 0, which every layer has)
        if ((int64_t)T * k + (L->has_shared ? T : 0) > 65535)
            return fail(MOET_EUNSUPPORTED, "this batch needs the GEMV kernels (H %% 256 not 0), which take at most "
                                            "T*top_k (+ T with a shared expert) = 65535 work entries");
        return launch_decode(L, x, T, k, ids, w, offsets, sorted, gate, out, miss_count, ws, stream);
    }
    PrefillParams p;
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
    p.w13 = L->w13;
    p.w2 = L->w2;
    p.has_shared = L->has_shared ? 1 : 0;
    p.sh13 = L->shared13;
    p.sh2 = L->shared2;
    p.swiglu_limit = L->swiglu_limit;
    p.base_slot = L->base_slot_of_expert;
    p.n_base_slots = L->n_base_slots;
    p.miss_count = miss_count;
    p.gate = gate;
    p.n_slots = (gate != nullptr) ? L->n_slots : 0;
    p.slot_of_expert = L->slot_of_expert;
    p.d13 = L->d13;
    p.d2 = L->d2;
    p.shared_fp4 = (L->has_shared && L->shared_fp4) ? 1 : 0;
    p.shf13 = L->shared13_fp4;
    p.shf2 = L->shared2_fp4;
    const int P = T * k;
    const size_t rows = (size_t)P + T;
    auto al = [](size_t b) { return (b + 255) & ~(size_t)255; };
    char *base = static_cast<char *>(ws);
    p.h = reinterpret_cast<uint16_t *>(base);
    p.ypart = reinterpret_cast<float *>(base + al(rows * L->I * 2));
    p.pre = p.ypart;   // read by the FP4 gate/up kernel before the down kernels write y there
    int32_t *order = reinterpret_cast<int32_t *>(base + al(rows * L->I * 2) +
                                                 al(rows * (size_t)std::max(L->H, 2 * L->I) * 4));
    int32_t *nflag = reinterpret_cast<int32_t *>(reinterpret_cast<char *>(order) + al((size_t)P * 4));
    p.tiles = reinterpret_cast<int4 *>(reinterpret_cast<char *>(nflag) + al((size_t)L->E * 4));
    p.out = out;
    const bool delta = p.n_slots > 0;
    p.order = delta ? order : sorted;
    p.nflag = delta ? nflag : nullptr;
    int rc;
    if (delta) {
        // a delta expert's gate-flagged pairs to the head of its run
        hipLaunchKernelGGL(partition_kernel, dim3(L->E), dim3(256), 0, stream, p, order, nflag);
        rc = check_launch("partition_kernel");
        if (rc != MOET_OK) return rc;
    }
    const int mslots = (P + kPM - 1) / kPM + L->E + ((p.has_shared && !p.shared_fp4) ? (T + kPM - 1) / kPM : 0);
    p.n_mslots = mslots;
    const int ms8 = (mslots + 7) / 8 * 8;
    hipLaunchKernelGGL(mtile_table_kernel, dim3(1), dim3(64), 0, stream, p);
    rc = check_launch("mtile_table_kernel");
    if (rc != MOET_OK) return rc;
    // FP4 delta tiles: (N-tile, delta slot, 2 workgroups splitting the slot's tiles); NVFP4 shared
    // expert: (N-tile, 128-token tile)
    const dim3 dgrid1(L->I / 128, L->n_slots, 2), dgrid2(L->H / 256, L->n_slots, 2);
    const dim3 sgrid1(L->I / 128, (T + kDM - 1) / kDM), sgrid2(L->H / 256, (T + kDM - 1) / kDM);
    p.n_ntiles = L->I / 128;
    hipEvent_t ev0, ev1;
    if (timing_events(&ev0, &ev1))
        hipExtLaunchKernelGGL(fc1_prefill_kernel, dim3(ms8 * p.n_ntiles), dim3(64 * kPW), 0, stream, ev0, ev1, 0, p);
    else
        hipLaunchKernelGGL(fc1_prefill_kernel, dim3(ms8 * p.n_ntiles), dim3(64 * kPW), 0, stream, p);
    rc = check_launch("fc1_prefill_kernel");
    if (rc != MOET_OK) return rc;
    if (delta) {
        hipLaunchKernelGGL(fc1_prefill_delta_kernel<false>, dgrid1, dim3(64 * kPW), 0, stream, p);
        rc = check_launch("fc1_prefill_delta_kernel");
        if (rc != MOET_OK) return rc;
    }
    if (p.shared_fp4) {
        hipLaunchKernelGGL(fc1_prefill_delta_kernel<true>, sgrid1, dim3(64 * kPW), 0, stream, p);
        rc = check_launch("fc1_prefill_delta_kernel");
        if (rc != MOET_OK) return rc;
    }
    p.n_ntiles = L->H / 256;
    hipLaunchKernelGGL(fc2_prefill_kernel, dim3(ms8 * p.n_ntiles), dim3(64 * kPW), 0, stream, p);
    rc = check_launch("fc2_prefill_kernel");
    if (rc != MOET_OK) return rc;
    if (delta) {
        hipLaunchKernelGGL(fc2_prefill_delta_kernel<false>, dgrid2, dim3(64 * kPW), 0, stream, p);
        rc = check_launch("fc2_prefill_delta_kernel");
        if (rc != MOET_OK) return rc;
    }
    if (p.shared_fp4) {
        hipLaunchKernelGGL(fc2_prefill_delta_kernel<true>, sgrid2, dim3(64 * kPW), 0, stream, p);
        rc = check_launch("fc2_prefill_delta_kernel");
        if (rc != MOET_OK) return rc;
    }
    hipLaunchKernelGGL(combine_prefill_kernel, dim3((L->H + 1023) / 1024, T), dim3(256), 0, stream, p);
    return check_launch("combine_prefill_kernel");
}

}  // namespace moet
