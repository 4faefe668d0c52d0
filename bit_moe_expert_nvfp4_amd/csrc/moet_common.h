// Shared device helpers and launch utilities of libmoet (gfx950 only).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moet.h"

namespace moet {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kTile = 64;          // rows per storage tile (one wave, one row per lane)
constexpr int kGroupK = 128;       // k per scale group (4 two-bit blocks, 8 FP4 blocks)

// ---------------------------------------------------------------------------
// Scalars
// ---------------------------------------------------------------------------

// bf16 bits -> float (exact)
__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// float -> bf16 bits, round to nearest even (inputs are finite)
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f)
{
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

// e4m3fn byte `B` of a packed word -> float.  gfx950's fp8 conversion reads the
// OCP E4M3 encoding (bias 7, max 448), which is exactly the block-scale format.
template <int B>
__device__ __forceinline__ float e4m3_byte(uint32_t word) { return __builtin_amdgcn_cvt_f32_fp8(word, B); }

// e4m3fn value * 2^9 as an exact integer for codes 0x00..0x7E
__device__ __forceinline__ int e4m3_x512(int t)
{
    int e = (t >> 3) & 15, m = t & 7;
    return e == 0 ? m : ((8 + m) << (e - 1));
}

__device__ __forceinline__ float silu_f32(float z) { return z / (1.0f + expf(-z)); }

// ---------------------------------------------------------------------------
// 2-bit decode.  Nibble j of a code word holds element j in bits 2-3 and
// element j + 8 in bits 0-1, each as (s, m) with m the lower bit.  Masking
// one bit pair per nibble and or-ing 0b0010 into the rest gives an FP4 (e2m1)
// nibble s|m|1|0 = +-1 (m = 0) or +-4 (m = 1) (codebook 0), so one and-or
// turns eight codes into eight e2m1 values, and the hardware FP4 -> bf16
// conversion then makes one bf16 pair per instruction.
// ---------------------------------------------------------------------------
constexpr uint32_t kW2Mask = 0xCCCCCCCCu;   // bits 2-3 of every nibble
constexpr uint32_t kW2Or = 0x22222222u;     // e2m1 exponent low bit

// The other codebooks of the layout differ only in the or-constant: with
// 0b0001 the e2m1 nibble s|m|0|1 is +-1/2 (m = 0) or +-3 (m = 1); with 0 it is
// s|m|0|0 = +-0 or +-2.  Codebook id (0, 1, 2; larger reads as 2) -> or-constant.
__device__ __forceinline__ uint32_t w2_or_of(uint32_t cb) { return cb == 0 ? kW2Or : cb == 1 ? 0x11111111u : 0u; }
// codebook id of matrix m of a stack (0 when the stack carries no ids)
__device__ __forceinline__ uint32_t w2_codebook(const moet_w2 &W, int m) { return W.codebook ? W.codebook[m] : 0u; }

// v_and_or_b32 with the mask in an SGPR and the or-constant in a VGPR (gfx9 VOP3
// takes no literal operands, and the compiler would otherwise emit and + or).
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t smask, uint32_t vbase)
{
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "s"(smask), "v"(vbase));
    return r;
}

// the same with a per-lane mask
__device__ __forceinline__ uint32_t and_or_v(uint32_t x, uint32_t vmask, uint32_t vbase)
{
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "v"(vmask), "v"(vbase));
    return r;
}

// FP4 (e2m1) byte `B` of a word -> two bf16 (low nibble first), exact
template <int B>
__device__ __forceinline__ uint32_t fp4_pair(uint32_t w)
{
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, B));
}

// e2m1 image of elements 0..7 (lo) or 8..15 (hi) of a 2-bit code word
__device__ __forceinline__ uint32_t w2_fp4_lo(uint32_t w, uint32_t smask, uint32_t vbase) { return and_or(w, smask, vbase); }
__device__ __forceinline__ uint32_t w2_fp4_hi(uint32_t w, uint32_t smask, uint32_t vbase) { return and_or(w << 2, smask, vbase); }

// Wave-uniform read-only data (activations) is read through the constant
// address space so that uniform addresses become scalar loads into SGPRs.
typedef const uint32_t __attribute__((address_space(4))) cu32;
__device__ __forceinline__ const cu32 *as_const(const void *p) { return (const cu32 *)(uintptr_t)p; }

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c)
{
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}

// ---------------------------------------------------------------------------
// Storage layout indices (see include/moet.h)
// ---------------------------------------------------------------------------
// uint4 index of the 64-k chunk c of row (tile, r) in a 2-bit matrix with K cols
__device__ __forceinline__ size_t w2_chunk_idx(int tile, int c, int r, int K) { return ((size_t)tile * (K / 64) + c) * 64 + r; }
// uint32 index of the scale group g (4 bytes) of row (tile, r)
__device__ __forceinline__ size_t w2_scale_idx(int tile, int g, int r, int K) { return ((size_t)tile * (K / 128) + g) * 64 + r; }
// uint4 index of the 32-k chunk c of row (tile, r) in an FP4 matrix
__device__ __forceinline__ size_t fp4_chunk_idx(int tile, int c, int r, int K) { return ((size_t)tile * (K / 32) + c) * 64 + r; }
// uint2 index of the scale group g (8 bytes) of row (tile, r) in an FP4 matrix
__device__ __forceinline__ size_t fp4_scale_idx(int tile, int g, int r, int K) { return ((size_t)tile * (K / 128) + g) * 64 + r; }

// bit positions of element e (0..15) of a 2-bit word: nibble e%8, upper bit
// pair for e < 8, lower pair for e >= 8 (m below s)
__device__ __forceinline__ int mbit(int e) { return 4 * (e & 7) + ((e & 8) ? 0 : 2); }
__device__ __forceinline__ int sbit(int e) { return mbit(e) + 1; }

// writes the two code words and the scale byte of block b (k = 32b .. 32b+31)
// of row n of matrix mat in the tiled 2-bit layout
__device__ __forceinline__ void store_w2_block(uint32_t *wcodes, uint8_t *wscales, size_t mat, int N, int K, int n,
                                               int b, const uint32_t out[2], int tau)
{
    const int tile = n / 64, r = n % 64;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        const int q = 2 * b + half;  // 16-k word index along the row
        const size_t widx = (((size_t)tile * (K / 64) + q / 4) * 64 + r) * 4 + (q % 4);
        wcodes[mat * (size_t)N * (K / 16) + widx] = out[half];
    }
    const size_t sidx = (((size_t)tile * (K / 128) + b / 4) * 64 + r) * 4 + (b % 4);
    wscales[mat * (size_t)N * (K / 32) + sidx] = (uint8_t)tau;
}

}  // namespace moet

// ---------------------------------------------------------------------------
// Host-side error plumbing shared by the entry points
// ---------------------------------------------------------------------------
namespace moet {
void set_error(const char *fmt, ...);
int fail(int status, const char *fmt, ...);
int check_launch(const char *what);
bool aligned16(const void *p);
bool timing_events(hipEvent_t *start, hipEvent_t *stop);  // the caller's timing events, if set

// moet_moe_forward in two halves: argument checks (host only), then the workspace checks and launches
int check_forward(const moet_layer *L, const uint16_t *x, int32_t T, int32_t top_k, const int32_t *topk_ids,
                  const float *topk_w, const int32_t *expert_offsets, const int32_t *sorted_pairs,
                  const uint8_t *gate_flags, const uint16_t *out, const int32_t *miss_count);
size_t forward_workspace_bytes(const moet_layer *L, int32_t T, int32_t top_k);
int dispatch_forward(const moet_layer *L, const uint16_t *x, int32_t T, int32_t top_k, const int32_t *topk_ids,
                     const float *topk_w, const int32_t *expert_offsets, const int32_t *sorted_pairs,
                     const uint8_t *gate_flags, uint16_t *out, int32_t *miss_count, void *workspace,
                     size_t workspace_bytes, hipStream_t stream);
}  // namespace moet
