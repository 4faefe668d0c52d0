/*
 * moet.h - C ABI of libmoet, a 2-bit + FP4-delta MoE expert layer for AMD
 * MI355X (gfx950).
 *
 * The operations follow the public description of the vLLM-Moet project
 * (README "Frontier MoE on consumer Blackwell (SM120)" as carried by the
 * pickgithub.com project payload; airanks.app "kacper-daftcode/vLLM-Moet"):
 *   moet_requant        load-time NVFP4 -> sign-symmetric 2-bit requantisation,
 *                       plus the FP4 delta of selected matrices
 *                       (README, "GLM-5.2 (753B) — the headline model" and
 *                       "How it fits — 2-bit experts at FP4 quality")
 *   moet_route          router top-k, routing weights and the token->expert
 *                       permutation the expert GEMMs consume
 *                       (README, "When the model doesn't fit at all — the GPU
 *                       as an expert cache": a descriptor step groups the
 *                       step's routings per expert)
 *   moet_moe_forward    the expert FFN on the 2-bit planes (gate/up + SwiGLU,
 *                       down + routing-weighted combine, optional shared
 *                       expert), with the FP4 delta added for tokens flagged by
 *                       the confidence gate on experts resident in the delta
 *                       cache (README, "How it fits"); optionally over a cache
 *                       that holds only some experts' 2-bit planes, zeroing and
 *                       counting routings to missing experts (README, "When the
 *                       model doesn't fit at all — the GPU as an expert cache")
 *   moet_delta_forward  the standalone FP4 delta GEMM/GEMV (README, "How it fits")
 *   moet_pack_nvfp4     NVFP4 matrices -> the FP4 layout (an NVFP4 shared
 *                       expert; README, "How it fits")
 *   moet_remap_mxfp4    FP4 (MXFP4) experts -> the same 2-bit planes by a
 *                       code remap (README, "How it fits")
 *   moet_requant_fp8    FP8 block-quantised experts -> the same 2-bit planes
 *                       (README, "How it fits")
 *   moet_confidence_gate  the confidence gate: flags low-confidence tokens for
 *                       the FP4 delta from their next-token logits (README,
 *                       "How it fits")
 *
 * Conventions (all entry points):
 *  - Every array argument is DEVICE memory owned by the caller (e.g. a torch
 *    tensor); only the moet_layer / moet_w2 / moet_fp4 structs themselves are
 *    host memory (holding device pointers).  The library never allocates or
 *    frees: scratch comes from the caller's workspace.
 *  - Every call enqueues work on `stream` (a hipStream_t; NULL = the null
 *    stream) and returns without synchronising the host.
 *  - Argument checks run on the host before any launch and return
 *    MOET_EINVAL / MOET_EUNSUPPORTED / MOET_EWORKSPACE without touching the
 *    GPU; a failed launch returns MOET_EHIP.  moet_last_error() gives a
 *    thread-local message for the last failure.  No C++ exception crosses
 *    the ABI.
 *  - Pointers must be 16-byte aligned.  Inputs must hold no NaN or Inf
 *    (undefined results otherwise).
 *  - Identical inputs give bitwise-identical outputs (no float atomics).
 *
 * Storage layouts (the library's own; every matrix is [N rows][K cols], K is
 * the reduction axis; N % 64 == 0 and K % 128 == 0):
 *  NVFP4 source (standard modelopt layout): codes uint8 [N][K/2], even k in the
 *    low nibble; block scales e4m3fn uint8 [N][K/16]; per-tensor scale_2 fp32.
 *  MXFP4 source (OCP microscaling): codes as NVFP4; block scales e8m0 uint8
 *    [N][K/32], value 2^(E-127); no tensor scale.
 *  FP8 block-quant source: weights e4m3fn uint8 [N][K]; one fp32 scale per
 *    128 x 128 block, [ceil(N/128)][K/128]; weight = e4m3 * scale.
 *  2-bit planes ("W2"): rows are grouped in tiles of 64;
 *    codes uint32 word index ((n/64 * K/64 + k/64) * 64 + n%64) * 4 + (k%64)/16;
 *    inside a word, element e = k%16 has code c = (s<<1)|m with m at bit
 *    4e+2 and s at bit 4e+3 for e < 8, and m at bit 4(e-8), s at bit
 *    4(e-8)+1 for e >= 8 (nibble j: element j in bits 2-3, element j+8 in
 *    bits 0-1);
 *    block scales e4m3fn, one per 32 along k, byte index
 *    ((n/64 * K/128 + k/128) * 64 + n%64) * 4 + (k%128)/32;
 *    per-tensor scale2 fp32; per-tensor codebook id (uint8, optional).
 *    Weight = level * e4m3(scale) * scale2 with level (code 0, 1, 2, 3) =
 *    codebook 0 (the default): +1, +4, -1, -4;  codebook 1: +1/2, +3, -1/2, -3;
 *    codebook 2: +0, +2, -0, -2.
 *    Storage: 2.25 bits per weight.
 *  FP4 delta planes ("FP4"): NVFP4 values in the same row tiling;
 *    code byte index ((n/64 * K/32 + k/32) * 64 + n%64) * 16 + (k%32)/2, even k
 *    in the low nibble; block scales one per 16 along k, byte index
 *    ((n/64 * K/128 + k/128) * 64 + n%64) * 8 + (k%128)/16; scale2 fp32.
 *  A stack of matrices is the concatenation of the per-matrix arrays.
 */
#ifndef MOET_H
#define MOET_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOET_OK = 0,
    MOET_EINVAL = 1,       /* bad shape, pointer, alignment or enum value */
    MOET_EUNSUPPORTED = 2, /* a valid request this library does not implement */
    MOET_EWORKSPACE = 3,   /* workspace missing or too small */
    MOET_EHIP = 4          /* a HIP launch or runtime call failed */
} moet_status;

enum { MOET_SOFTMAX = 0, MOET_SIGMOID = 1 };

/* Flags of the load-time conversions (moet_requant, moet_remap_mxfp4,
 * moet_requant_fp8).  MOET_BALANCE_ZERO_SIGNS: the zeros of each 32-weight
 * block take alternating signs in k order (+ first) instead of their source
 * sign bit, for checkpoints whose export wrote every zero as +0 (README
 * "Frontier MoE on consumer Blackwell (SM120)", section "Kimi-K2.7-Code (1T
 * MoE) on 4x RTX PRO 6000": such zeros would all land on +1 and bias the
 * layer).  Block scales are unaffected: a zero costs the same either way. */
enum { MOET_BALANCE_ZERO_SIGNS = 1 };

/* moet_requant only.  MOET_PICK_CODEBOOK: each matrix picks its codebook
 * (README "Frontier MoE on consumer Blackwell (SM120)", section "How it fits
 * — 2-bit experts at FP4 quality": a per-tensor pick, won by {-4,-1,1,4} for
 * nearly every tensor).  The candidates are the three sign-symmetric
 * four-level codebooks of the 2-bit layout (magnitudes {1, 4}, {1/2, 3},
 * {0, 2}); the pick is the one whose requantisation has the smallest exact
 * total L2 error over the matrix, ties to the lower id. */
enum { MOET_PICK_CODEBOOK = 2 };

/* Static string for a status code. */
const char *moet_status_str(moet_status status);
/* Thread-local detail of the last failed call on this thread ("" if none). */
const char *moet_last_error(void);
/* ABI version (bumped on any incompatible change). */
int moet_abi_version(void);

/*
 * moet_requant - NVFP4 -> sign-symmetric 2-bit planes for a stack of n_mat
 * equal-shape matrices [N][K], and optionally the FP4 delta of some of them.
 * (README "Frontier MoE on consumer Blackwell (SM120)", sections "GLM-5.2
 * (753B) — the headline model" and "How it fits — 2-bit experts at FP4
 * quality".)
 *
 * Per 32 consecutive weights along K the block scale is the e4m3fn value that
 * minimises the exact L2 error of the block against the codebook levels
 * * scale * scale2 (ties -> the smaller scale); each weight takes the nearest
 * level (a tie keeps the smaller magnitude) and its sign from the NVFP4 sign
 * bit, zeros included.  The search is exact.  Codebook 0 ({-4,-1,1,4}, scale2
 * = 2 * scale_2) unless flags hold MOET_PICK_CODEBOOK: then each matrix takes
 * the codebook of smallest total error (1: {-3,-1/2,1/2,3}, scale2 = 2 *
 * scale_2; 2: {-2,-0,+0,2}, scale2 = 4 * scale_2), and its id is written to
 * w2_codebook.
 *
 * Inputs: fp4_codes uint8 [n_mat][N][K/2], fp4_scales uint8 [n_mat][N][K/16]
 *   (finite, non-negative e4m3fn), fp4_scale2 fp32 [n_mat].
 * Outputs: w2_codes uint32 [n_mat][N*K/16], w2_scales uint8 [n_mat][N*K/32],
 *   w2_scale2 fp32 [n_mat], all in the 2-bit layout above; w2_codebook uint8
 *   [n_mat] (required with MOET_PICK_CODEBOOK; without it may be NULL, else
 *   it is filled with 0).
 * Delta (n_sel > 0): delta_sel int32 [n_sel] (device) lists matrix indices;
 *   the delta of matrix delta_sel[i] = W_nvfp4 - W_2bit, re-encoded as NVFP4
 *   with the source scale_2 (block-16 scale nearest to max|D|/6, ties to the
 *   even code; elements nearest e2m1, ties to even, a value rounding to zero
 *   keeps D's sign), is written at slot i of d_codes uint8 [n_sel][N*K/2],
 *   d_scales uint8 [n_sel][N*K/16], d_scale2 fp32 [n_sel] (FP4 layout).
 *   n_sel == 0: delta_sel and d_* may be NULL.
 * flags: 0 or a combination of MOET_BALANCE_ZERO_SIGNS (the delta then
 *   follows the balanced codes) and MOET_PICK_CODEBOOK (the delta is taken
 *   against the picked codebook).  With the pick, the first 48 bytes of each
 *   matrix's w2_codes hold its error sums until the requant pass overwrites
 *   them.
 * Errors: MOET_EINVAL for n_mat < 1, N % 64, K % 128, NULL or misaligned
 *   pointers, n_sel < 0 or n_sel > n_mat, unknown flags, NULL w2_codebook
 *   with MOET_PICK_CODEBOOK.  Out-of-range delta_sel entries are skipped by
 *   the kernel (their slots are left unwritten).
 */
moet_status moet_requant(const uint8_t *fp4_codes, const uint8_t *fp4_scales, const float *fp4_scale2,
                 int64_t n_mat, int64_t N, int64_t K,
                 uint32_t *w2_codes, uint8_t *w2_scales, float *w2_scale2, uint8_t *w2_codebook,
                 const int32_t *delta_sel, int64_t n_sel,
                 uint8_t *d_codes, uint8_t *d_scales, float *d_scale2,
                 uint32_t flags, void *stream);

/*
 * moet_pack_nvfp4 - a stack of n_mat modelopt NVFP4 matrices [N][K] in the
 * library's FP4 layout, unchanged in value (codes, block scales and scale_2
 * are moved, not re-encoded): the form the forward reads an NVFP4 shared
 * expert in.  (README "Frontier MoE on consumer Blackwell (SM120)", section
 * "How it fits — 2-bit experts at FP4 quality": only the routed experts are
 * compressed to 2 bits.)
 *
 * Inputs: fp4_codes uint8 [n_mat][N][K/2], fp4_scales uint8 [n_mat][N][K/16],
 *   fp4_scale2 fp32 [n_mat] (modelopt layout).
 * Outputs: d_codes uint8 [n_mat][N*K/2], d_scales uint8 [n_mat][N*K/16],
 *   d_scale2 fp32 [n_mat] (FP4 layout).
 * Errors: MOET_EINVAL for n_mat < 1, N % 64, K % 128, NULL or misaligned
 *   pointers.
 */
moet_status moet_pack_nvfp4(const uint8_t *fp4_codes, const uint8_t *fp4_scales, const float *fp4_scale2,
                    int64_t n_mat, int64_t N, int64_t K,
                    uint8_t *d_codes, uint8_t *d_scales, float *d_scale2, void *stream);

/*
 * moet_remap_mxfp4 - MXFP4 experts -> sign-symmetric 2-bit planes by a code
 * remap, for a stack of n_mat equal-shape matrices [N][K].  (README "Frontier
 * MoE on consumer Blackwell (SM120)", section "How it fits — 2-bit experts at
 * FP4 quality": FP4 experts load by remapping their codes.)
 *
 * {-4,-1,1,4} is a subset of the e2m1 grid, so each e2m1 code becomes the
 * nearest of those values in units of its block scale (magnitudes 0, 0.5, 1,
 * 1.5, 2 -> 1; 3, 4, 6 -> 4; sign from the code, or balanced zeros).  The
 * scales carry over exactly: with Emax the largest e8m0 exponent over the
 * blocks holding a non-zero code, w2_scale2 = 2^(Emax - 135) and a block's
 * e4m3 scale is 2^(E - Emax + 8); blocks with E < Emax - 17 (below e4m3's
 * range) and blocks with no non-zero code get scale 0.  A matrix with no
 * non-zero code gets w2_scale2 = 1 and scale 0 everywhere.  No search: a
 * reduction (64 workgroups per matrix, integer atomic max into the w2_scale2
 * slot), then one thread per 32-weight block, then the float scale.
 *
 * Inputs: mx_codes uint8 [n_mat][N][K/2], mx_scales uint8 [n_mat][N][K/32]
 *   (e8m0; 0xFF (NaN) gives undefined results).
 * Outputs: w2_codes, w2_scales, w2_scale2 as for moet_requant.
 * flags: 0 or MOET_BALANCE_ZERO_SIGNS.
 * Errors: MOET_EINVAL for n_mat < 1, N % 64, K % 128, NULL or misaligned
 *   pointers, unknown flags.
 */
moet_status moet_remap_mxfp4(const uint8_t *mx_codes, const uint8_t *mx_scales, int64_t n_mat, int64_t N, int64_t K,
                     uint32_t *w2_codes, uint8_t *w2_scales, float *w2_scale2, uint32_t flags, void *stream);

/*
 * moet_requant_fp8 - FP8 block-quantised experts -> sign-symmetric 2-bit
 * planes, for a stack of n_mat equal-shape matrices [N][K].  (README
 * "Frontier MoE on consumer Blackwell (SM120)", section "How it fits — 2-bit
 * experts at FP4 quality": FP8 block-quant checkpoints are requantised to the
 * same codebook at load, in float64.)
 *
 * w2_scale2 = 2^p, the smallest p >= -149 with 4 * 448 * 2^p >= max|weight|
 * (1 for an all-zero matrix).  Per 32 weights along K the e4m3 block scale t
 * minimises sum_i min((y_i - a)^2, (y_i - 4a)^2), y_i = |weight_i|,
 * a = e4m3(t) * w2_scale2, over all 127 finite codes (ties -> smaller t),
 * evaluated in float64 in k order without fused multiply-adds; each weight
 * takes the nearest level (2y > 5a -> magnitude 4; a tie keeps 1) and its
 * sign from the e4m3 sign bit, or balanced zeros.
 *
 * Inputs: fp8_w uint8 [n_mat][N][K] (e4m3fn; 0x7F / 0xFF (NaN) give undefined
 *   results), fp8_scales fp32 [n_mat][ceil(N/128)][K/128] (finite, >= 0).
 * Outputs: w2_codes, w2_scales, w2_scale2 as for moet_requant.
 * flags: 0 or MOET_BALANCE_ZERO_SIGNS.
 * Errors: MOET_EINVAL for n_mat < 1, N % 64, K % 128, NULL or misaligned
 *   pointers, unknown flags.
 */
moet_status moet_requant_fp8(const uint8_t *fp8_w, const float *fp8_scales, int64_t n_mat, int64_t N, int64_t K,
                     uint32_t *w2_codes, uint8_t *w2_scales, float *w2_scale2, uint32_t flags, void *stream);

/*
 * moet_route - router top-k and token permutation.
 * (README "Frontier MoE on consumer Blackwell (SM120)", sections "How it fits"
 * and "When the model doesn't fit at all — the GPU as an expert cache".)
 *
 * logits fp32 [T][E].  Per token the top_k largest logits are selected
 * (equal logits -> lower expert id first) into topk_ids int32 [T][top_k] in
 * descending order.  topk_w fp32 [T][top_k]: score_fn MOET_SOFTMAX ->
 * exp(l - l_max) normalised over the selected experts when renormalize != 0,
 * else over all E; MOET_SIGMOID -> sigmoid(l), divided by the selected sum
 * when renormalize != 0; then times route_scale.
 * expert_offsets int32 [E+1]: number of (token, slot) pairs routed to experts
 * < e; sorted_pairs int32 [T*top_k]: the pair ids p = t*top_k + j ordered by
 * (expert, p).
 * Limits: 1 <= T <= 65536, 1 <= E <= 1024, 1 <= top_k <= min(E, 16).
 * Errors: MOET_EINVAL on any limit, NULL or misaligned pointer, bad score_fn.
 */
moet_status moet_route(const float *logits, int32_t T, int32_t E, int32_t top_k, int32_t score_fn,
               int32_t renormalize, float route_scale,
               int32_t *topk_ids, float *topk_w, int32_t *expert_offsets, int32_t *sorted_pairs,
               void *stream);

/* 2-bit planes of a stack of matrices (device pointers; layout above).
 * codebook: uint8 [n_mat] codebook id of each matrix (0, 1 or 2, as
 * moet_requant writes it; larger values read as 2), or NULL: every matrix
 * uses codebook 0. */
typedef struct {
    const uint32_t *codes;
    const uint8_t *scales;
    const float *scale2;
    const uint8_t *codebook;
} moet_w2;

/* FP4 delta planes of a stack of matrices (device pointers; layout above). */
typedef struct {
    const uint8_t *codes;
    const uint8_t *scales;
    const float *scale2;
} moet_fp4;

/*
 * One MoE layer.  w13: stack of 2E matrices [I][H] (expert e: gate = 2e,
 * up = 2e+1); w2: stack of E matrices [H][I].  has_shared != 0 adds one
 * always-on shared expert (shared13: 2 matrices [I][H], shared2: 1 matrix
 * [H][I]) with weight 1 and no delta.  n_slots > 0 enables the delta cache:
 * slot_of_expert int32 [E] (device; -1 = not resident), d13: stack of
 * 2*n_slots matrices [I][H] (slot s: gate 2s, up 2s+1), d2: n_slots matrices
 * [H][I].  swiglu_limit > 0 clamps gate <= L and |up| <= L before SwiGLU.
 * Expert cache (README, "When the model doesn't fit at all — the GPU as an
 * expert cache"): base_slot_of_expert == NULL means w13/w2 hold every expert
 * as above.  Otherwise base_slot_of_expert int32 [E] (device) places expert e
 * at cache slot base_slot_of_expert[e] of w13 (2*n_base_slots matrices) and
 * w2 (n_base_slots matrices); a slot outside [0, n_base_slots) marks the
 * expert missing: its routings contribute nothing and are counted.
 * NVFP4 shared expert (README, "How it fits": only the routed experts go to
 * 2 bits, the rest keeps the checkpoint's precision): has_shared != 0 and
 * shared_fp4 != 0 take the shared expert from shared13_fp4 (gate = matrix 0,
 * up = matrix 1, [I][H]) and shared2_fp4 ([H][I]) in the FP4 layout
 * (moet_pack_nvfp4 builds them from a modelopt export); shared13 / shared2
 * are then unused.
 */
typedef struct {
    int32_t H, I, E;
    moet_w2 w13, w2;
    int32_t has_shared;
    moet_w2 shared13, shared2;
    int32_t n_slots;
    const int32_t *slot_of_expert;
    moet_fp4 d13, d2;
    float swiglu_limit;
    const int32_t *base_slot_of_expert;
    int32_t n_base_slots;
    int32_t shared_fp4;
    moet_fp4 shared13_fp4, shared2_fp4;
} moet_layer;

/* Workspace bytes moet_moe_forward needs for T tokens and top_k. */
size_t moet_moe_workspace_bytes(const moet_layer *L, int32_t T, int32_t top_k);

/*
 * moet_moe_forward - the routed-expert layer forward.
 * (README "Frontier MoE on consumer Blackwell (SM120)", section "How it fits
 * — 2-bit experts at FP4 quality".)
 *
 * x bf16 [T][H]; topk_ids/topk_w/expert_offsets/sorted_pairs as produced by
 * moet_route; gate_flags uint8 [T] (device, may be NULL = none flagged).
 * miss_count int32 (device, may be NULL): set to the number of (token,
 * expert) routings whose expert is missing from the expert cache (0 without
 * a cache); the call writes it, the caller need not clear it.
 * For every pair (t, e): u = W13_e x_t (+ D13_slot x_t when gate_flags[t] and
 * slot_of_expert[e] >= 0), h = bf16(silu(u_gate) * u_up), y = W2_e h
 * (+ D2_slot h); out bf16 [T][H] = bf16(sum_j topk_w[t][j] * y_(t,j) +
 * y_shared(t)).  Accumulation is fp32; h and out are rounded to nearest-even.
 * Decode-sized batches (T*top_k <= 1024) run the GEMV kernels; larger
 * batches run the MFMA grouped-GEMM kernels when I % 128 == 0 and
 * H % 256 == 0 (the FP4 delta and an NVFP4 shared expert then run as an FP4
 * MFMA pass: the 2-bit gate/up kernel stores the fp32 pre-activations of a
 * delta expert's rows, the FP4 kernel adds D13 x_t, each product scaled by
 * its own scale2, before SwiGLU, and the FP4 down kernel adds D2 h to y),
 * else the GEMV kernels, which take at most T*top_k work entries, plus T
 * with a shared expert, up to 65535 (MOET_EUNSUPPORTED beyond).
 * workspace: at least moet_moe_workspace_bytes(L, T, top_k) bytes of device
 * memory, 256-byte aligned; its contents need no initialisation.
 * Expert ids outside [0, E) and slots outside [0, n_slots) contribute
 * nothing (the kernels skip them instead of reading out of bounds).
 * Errors: MOET_EINVAL on shapes (H, I % 128; 1 <= E <= 1024;
 * 1 <= top_k <= min(E, 16); 1 <= T <= 65536), NULL or misaligned pointers, a
 * delta cache with NULL members; MOET_EWORKSPACE if the workspace is short.
 */
moet_status moet_moe_forward(const moet_layer *L, const uint16_t *x, int32_t T, int32_t top_k,
                     const int32_t *topk_ids, const float *topk_w,
                     const int32_t *expert_offsets, const int32_t *sorted_pairs,
                     const uint8_t *gate_flags, uint16_t *out, int32_t *miss_count,
                     void *workspace, size_t workspace_bytes, void *stream);

/*
 * moet_moe_forward_noalloc - moet_moe_forward for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, hosts that
 * forbid allocation.  It allocates nothing and takes no workspace: the h and
 * y rows the kernels pass between launches live in a static device array of
 * the library, MOET_NOALLOC_SCRATCH_BYTES (16 MiB) per GPU, held from the
 * library's first use on that GPU until the process ends.  Arguments, results
 * and errors are those of moet_moe_forward (same kernels, bitwise the same
 * output), except that a batch whose moet_moe_workspace_bytes exceeds
 * MOET_NOALLOC_SCRATCH_BYTES returns MOET_EWORKSPACE before any HIP call
 * (16 MiB holds decode steps up to T * (top_k + 1) = 500 at H = 7168,
 * I = 2048).  Every call on one GPU shares that GPU's array, which keeps the
 * last call's contents: calls that overlap on one GPU (other streams or
 * threads) race and must be ordered by the caller.  The first call on each
 * device looks up the array's device address (hipGetSymbolAddress).
 */
#define MOET_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
moet_status moet_moe_forward_noalloc(const moet_layer *L, const uint16_t *x, int32_t T, int32_t top_k,
                             const int32_t *topk_ids, const float *topk_w,
                             const int32_t *expert_offsets, const int32_t *sorted_pairs,
                             const uint8_t *gate_flags, uint16_t *out, int32_t *miss_count,
                             void *stream);

/*
 * moet_delta_forward - standalone FP4 delta GEMM/GEMV accumulate.
 * (README "Frontier MoE on consumer Blackwell (SM120)", section "How it fits".)
 *
 * D: stack of n_slots FP4 matrices [N][K] (FP4 layout); act bf16 [R][K];
 * row_slot int32 [R] (device).  For every r with 0 <= row_slot[r] < n_slots:
 * acc[r][n] += sum_k D_{row_slot[r]}[n][k] * act[r][k] (fp32 accumulation,
 * one fp32 add into acc per element); other rows are left unchanged.
 * Errors: MOET_EINVAL for n_slots < 1, N % 64, K % 128, R < 0, NULL or
 * misaligned pointers.
 */
moet_status moet_delta_forward(const moet_fp4 *D, int32_t n_slots, int32_t N, int32_t K,
                       const uint16_t *act, const int32_t *row_slot, int32_t R, float *acc,
                       void *stream);

/*
 * moet_confidence_gate - flags the tokens whose next-token distribution is not
 * confident, so that moet_moe_forward adds the FP4 delta for them.
 * (README "Frontier MoE on consumer Blackwell (SM120)", section "How it fits
 * — 2-bit experts at FP4 quality": the confidence gate re-runs low-confidence
 * steps at FP4; its benchmark runs use tau = 0.60.)
 *
 * logits fp32 [T][V] (device; finite, or -inf for masked entries, with a
 * finite maximum per row).  confidence(t) = max_v softmax(logits[t])_v =
 * 1 / sum_v exp(l_v - l_max), computed in float64; gate_flags uint8 [T]
 * (device) = 1 where confidence < tau, else 0; confidence_out fp32 [T]
 * (device, may be NULL) receives the confidence rounded to fp32.
 * workspace: at least moet_gate_workspace_bytes(T, V) bytes of device memory,
 * 16-byte aligned, owned by the caller and free again when the stream reaches
 * the end of the call (may be NULL when that size is 0, i.e. when every row
 * runs in one workgroup).  Few rows are cut into chunks spread over the chip;
 * the chunk partials go through the workspace and are combined in a fixed
 * order, so the result is bitwise repeatable.
 * Errors: MOET_EINVAL for T outside [1, 65535], V < 1, tau not finite, NULL
 * or misaligned pointers (logits 16-byte aligned); MOET_EWORKSPACE if the
 * workspace is missing or short.
 */
size_t moet_gate_workspace_bytes(int32_t T, int32_t V);
moet_status moet_confidence_gate(const float *logits, int32_t T, int32_t V, float tau, uint8_t *gate_flags,
                         float *confidence_out, void *workspace, size_t workspace_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MOET_H */
