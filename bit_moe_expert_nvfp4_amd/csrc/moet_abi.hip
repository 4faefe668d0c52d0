// extern "C" entry points of libmoet: argument validation on the host, then
// dispatch to the kernels.  Every check happens before any HIP call, so a
// rejected call never touches the GPU.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "moet_common.h"
#include "moet_instrument.h"

namespace moet {

static thread_local char g_err[512];
static thread_local hipEvent_t g_ev_start = nullptr, g_ev_stop = nullptr;

// The timing events for the next timed launch, or false when none are set.
// The launch hands them to hipExtLaunchKernel, which stamps them from the
// kernel's own dispatch (no separate marker packets in the stream).
bool timing_events(hipEvent_t *start, hipEvent_t *stop)
{
    *start = g_ev_start;
    *stop = g_ev_stop;
    return g_ev_start != nullptr;
}

void set_error(const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
}

int fail(int status, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return status;
}

int check_launch(const char *what)
{
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(MOET_EHIP, "%s: %s", what, hipGetErrorString(e));
    return MOET_OK;
}

bool aligned16(const void *p) { return p != nullptr && (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int launch_requant(const uint8_t *, const uint8_t *, const float *, int64_t, int, int, uint32_t *, uint8_t *, float *,
                   uint8_t *, const int32_t *, int64_t, uint8_t *, uint8_t *, float *, int, int, hipStream_t);
int launch_remap_mxfp4(const uint8_t *, const uint8_t *, int64_t, int, int, int, uint32_t *, uint8_t *, float *,
                       hipStream_t);
int launch_pack_nvfp4(const uint8_t *, const uint8_t *, const float *, int64_t, int, int, uint8_t *, uint8_t *, float *,
                      hipStream_t);
int launch_requant_fp8(const uint8_t *, const float *, int64_t, int, int, int, uint32_t *, uint8_t *, float *,
                       hipStream_t);
int launch_route(const float *, int, int, int, int, int, float, int32_t *, float *, int32_t *, int32_t *, hipStream_t);
size_t decode_workspace_bytes(int T, int k, int H, int I);
int launch_decode(const moet_layer *, const uint16_t *, int, int, const int32_t *, const float *, const int32_t *,
                  const int32_t *, const uint8_t *, uint16_t *, int32_t *, void *, hipStream_t);
int launch_delta(const moet_fp4 *, int, int, int, const uint16_t *, const int32_t *, int, float *, hipStream_t);
int launch_gate(const float *, int, int, float, uint8_t *, float *, void *, hipStream_t);
size_t gate_workspace_bytes(int T, int V);
size_t prefill_workspace_bytes(int T, int k, int H, int I, int E);
int launch_prefill(const moet_layer *, const uint16_t *, int, int, const int32_t *, const float *, const int32_t *,
                   const int32_t *, const uint8_t *, uint16_t *, int32_t *, void *, hipStream_t);

static bool w2_ok(const moet_w2 &w)
{
    return aligned16(w.codes) && aligned16(w.scales) && aligned16(w.scale2) && (!w.codebook || aligned16(w.codebook));
}
static bool fp4_ok(const moet_fp4 &w) { return aligned16(w.codes) && aligned16(w.scales) && aligned16(w.scale2); }

static int check_layer(const moet_layer *L)
{
    if (!L) return fail(MOET_EINVAL, "layer is NULL");
    if (L->H <= 0 || L->I <= 0 || L->H % 128 || L->I % 128)
        return fail(MOET_EINVAL, "H (%d) and I (%d) must be positive multiples of 128", L->H, L->I);
    if (L->E < 1 || L->E > 1024) return fail(MOET_EINVAL, "E (%d) must be in [1, 1024]", L->E);
    if ((!L->base_slot_of_expert || L->n_base_slots > 0) && (!w2_ok(L->w13) || !w2_ok(L->w2)))
        return fail(MOET_EINVAL, "w13 / w2 pointers must be non-NULL and 16-byte aligned");
    if (L->has_shared && !L->shared_fp4 && (!w2_ok(L->shared13) || !w2_ok(L->shared2)))
        return fail(MOET_EINVAL, "shared expert pointers must be non-NULL and 16-byte aligned");
    if (L->has_shared && L->shared_fp4 && (!fp4_ok(L->shared13_fp4) || !fp4_ok(L->shared2_fp4)))
        return fail(MOET_EINVAL, "NVFP4 shared expert pointers must be non-NULL and 16-byte aligned");
    if (L->n_slots < 0) return fail(MOET_EINVAL, "n_slots (%d) must be >= 0", L->n_slots);
    if (L->base_slot_of_expert && (!aligned16(L->base_slot_of_expert) || L->n_base_slots < 0))
        return fail(MOET_EINVAL, "expert cache: base_slot_of_expert must be 16-byte aligned and n_base_slots >= 0");
    if (L->n_slots > 0 && (!aligned16(L->slot_of_expert) || !fp4_ok(L->d13) || !fp4_ok(L->d2)))
        return fail(MOET_EINVAL, "delta cache pointers must be non-NULL and 16-byte aligned");
    if (!(L->swiglu_limit >= 0.f)) return fail(MOET_EINVAL, "swiglu_limit must be >= 0");
    return MOET_OK;
}

constexpr int kDecodeMaxPairs = 1024;

static bool use_decode(int T, int k) { return (int64_t)T * k <= kDecodeMaxPairs; }

// Checks of moet_moe_forward's arguments other than the workspace (host only, no HIP call).
int check_forward(const moet_layer *L, const uint16_t *x, int32_t T, int32_t top_k, const int32_t *topk_ids,
                  const float *topk_w, const int32_t *expert_offsets, const int32_t *sorted_pairs,
                  const uint8_t *gate_flags, const uint16_t *out, const int32_t *miss_count)
{
    int rc = check_layer(L);
    if (rc != MOET_OK) return rc;
    if (T < 1 || T > 65536) return fail(MOET_EINVAL, "T (%d) must be in [1, 65536]", T);
    if (top_k < 1 || top_k > L->E || top_k > 16) return fail(MOET_EINVAL, "top_k (%d) must be in [1, min(E, 16)]", top_k);
    if (!aligned16(x) || !aligned16(topk_ids) || !aligned16(topk_w) || !aligned16(expert_offsets) ||
        !aligned16(sorted_pairs) || !aligned16(out))
        return fail(MOET_EINVAL, "pointers must be non-NULL and 16-byte aligned");
    if (gate_flags && !aligned16(gate_flags)) return fail(MOET_EINVAL, "gate_flags must be 16-byte aligned");
    if (miss_count && (reinterpret_cast<uintptr_t>(miss_count) & 3u)) return fail(MOET_EINVAL, "miss_count must be 4-byte aligned");
    return MOET_OK;
}

size_t forward_workspace_bytes(const moet_layer *L, int32_t T, int32_t top_k)
{
    if (!L || T < 1 || top_k < 1 || L->H <= 0 || L->I <= 0 || L->E < 1) return 0;
    if (use_decode(T, top_k)) return decode_workspace_bytes(T, top_k, L->H, L->I);
    return prefill_workspace_bytes(T, top_k, L->H, L->I, L->E);
}

// The workspace checks, then the decode (GEMV) or prefill (grouped-GEMM) launches.
int dispatch_forward(const moet_layer *L, const uint16_t *x, int32_t T, int32_t top_k, const int32_t *topk_ids,
                     const float *topk_w, const int32_t *expert_offsets, const int32_t *sorted_pairs,
                     const uint8_t *gate_flags, uint16_t *out, int32_t *miss_count, void *workspace,
                     size_t workspace_bytes, hipStream_t stream)
{
    const size_t need = forward_workspace_bytes(L, T, top_k);
    if (!workspace || workspace_bytes < need)
        return fail(MOET_EWORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace_bytes);
    if (reinterpret_cast<uintptr_t>(workspace) & 255u) return fail(MOET_EINVAL, "workspace must be 256-byte aligned");
    if (use_decode(T, top_k))
        return launch_decode(L, x, T, top_k, topk_ids, topk_w, expert_offsets, sorted_pairs, gate_flags, out, miss_count,
                             workspace, stream);
    return launch_prefill(L, x, T, top_k, topk_ids, topk_w, expert_offsets, sorted_pairs, gate_flags, out, miss_count,
                          workspace, stream);
}

}  // namespace moet

using namespace moet;

extern "C" {

const char *moet_status_str(moet_status s)
{
    switch (s) {
    case MOET_OK: return "MOET_OK";
    case MOET_EINVAL: return "MOET_EINVAL";
    case MOET_EUNSUPPORTED: return "MOET_EUNSUPPORTED";
    case MOET_EWORKSPACE: return "MOET_EWORKSPACE";
    case MOET_EHIP: return "MOET_EHIP";
    default: return "MOET_UNKNOWN";
    }
}

const char *moet_last_error(void) { return g_err; }

int moet_abi_version(void) { return 6; }

// shape checks shared by the load-time conversions (`allowed`: the flags the entry point takes)
static int check_stack(int64_t n_mat, int64_t N, int64_t K, uint32_t flags,
                       uint32_t allowed = MOET_BALANCE_ZERO_SIGNS)
{
    if (n_mat < 1) return fail(MOET_EINVAL, "n_mat (%lld) must be >= 1", (long long)n_mat);
    if (N < 64 || N % 64 || N > (1 << 24)) return fail(MOET_EINVAL, "N (%lld) must be a positive multiple of 64", (long long)N);
    if (K < 128 || K % 128 || K > (1 << 24)) return fail(MOET_EINVAL, "K (%lld) must be a positive multiple of 128", (long long)K);
    if ((unsigned long long)n_mat * N * (K / 32) >= (1ull << 40)) return fail(MOET_EINVAL, "stack too large");
    if ((unsigned long long)n_mat * N * (K / 32) / 256 >= (1ull << 31)) return fail(MOET_EINVAL, "stack too large for one launch");
    if (flags & ~allowed) return fail(MOET_EINVAL, "unknown flags 0x%x", flags);
    return MOET_OK;
}

moet_status moet_requant(const uint8_t *fp4_codes, const uint8_t *fp4_scales, const float *fp4_scale2, int64_t n_mat,
                 int64_t N, int64_t K, uint32_t *w2_codes, uint8_t *w2_scales, float *w2_scale2,
                 uint8_t *w2_codebook, const int32_t *delta_sel, int64_t n_sel, uint8_t *d_codes,
                 uint8_t *d_scales, float *d_scale2, uint32_t flags, void *stream)
{
    g_err[0] = 0;
    int rc = check_stack(n_mat, N, K, flags, MOET_BALANCE_ZERO_SIGNS | MOET_PICK_CODEBOOK);
    if (rc != MOET_OK) return (moet_status)(rc);
    const bool pick = (flags & MOET_PICK_CODEBOOK) != 0;
    if (pick && !aligned16(w2_codebook))
        return (moet_status)(fail(MOET_EINVAL, "MOET_PICK_CODEBOOK needs a non-NULL, 16-byte aligned w2_codebook"));
    if (w2_codebook && !aligned16(w2_codebook))
        return (moet_status)(fail(MOET_EINVAL, "w2_codebook must be 16-byte aligned"));
    if (!aligned16(fp4_codes) || !aligned16(fp4_scales) || !aligned16(fp4_scale2) || !aligned16(w2_codes) ||
        !aligned16(w2_scales) || !aligned16(w2_scale2))
        return (moet_status)(fail(MOET_EINVAL, "pointers must be non-NULL and 16-byte aligned"));
    if (n_sel < 0 || n_sel > n_mat)
        return (moet_status)(fail(MOET_EINVAL, "n_sel (%lld) must be in [0, n_mat]", (long long)n_sel));
    if (n_sel > 0 && (!aligned16(delta_sel) || !aligned16(d_codes) || !aligned16(d_scales) || !aligned16(d_scale2)))
        return (moet_status)(fail(MOET_EINVAL, "delta pointers must be non-NULL and 16-byte aligned when n_sel > 0"));
    return (moet_status)launch_requant(fp4_codes, fp4_scales, fp4_scale2, n_mat, (int)N, (int)K, w2_codes, w2_scales, w2_scale2,
                                       w2_codebook, delta_sel, n_sel, d_codes, d_scales, d_scale2,
                                       (int)(flags & MOET_BALANCE_ZERO_SIGNS), (int)pick, (hipStream_t)stream);
}

moet_status moet_pack_nvfp4(const uint8_t *fp4_codes, const uint8_t *fp4_scales, const float *fp4_scale2, int64_t n_mat,
                    int64_t N, int64_t K, uint8_t *d_codes, uint8_t *d_scales, float *d_scale2, void *stream)
{
    g_err[0] = 0;
    int rc = check_stack(n_mat, N, K, 0);
    if (rc != MOET_OK) return (moet_status)(rc);
    if (!aligned16(fp4_codes) || !aligned16(fp4_scales) || !aligned16(fp4_scale2) || !aligned16(d_codes) ||
        !aligned16(d_scales) || !aligned16(d_scale2))
        return (moet_status)(fail(MOET_EINVAL, "pointers must be non-NULL and 16-byte aligned"));
    return (moet_status)launch_pack_nvfp4(fp4_codes, fp4_scales, fp4_scale2, n_mat, (int)N, (int)K, d_codes, d_scales, d_scale2,
                                          (hipStream_t)stream);
}

moet_status moet_remap_mxfp4(const uint8_t *mx_codes, const uint8_t *mx_scales, int64_t n_mat, int64_t N, int64_t K,
                     uint32_t *w2_codes, uint8_t *w2_scales, float *w2_scale2, uint32_t flags, void *stream)
{
    g_err[0] = 0;
    int rc = check_stack(n_mat, N, K, flags);
    if (rc != MOET_OK) return (moet_status)(rc);
    if (!aligned16(mx_codes) || !aligned16(mx_scales) || !aligned16(w2_codes) || !aligned16(w2_scales) ||
        !aligned16(w2_scale2))
        return (moet_status)(fail(MOET_EINVAL, "pointers must be non-NULL and 16-byte aligned"));
    return (moet_status)launch_remap_mxfp4(mx_codes, mx_scales, n_mat, (int)N, (int)K, (int)(flags & MOET_BALANCE_ZERO_SIGNS),
                                           w2_codes, w2_scales, w2_scale2, (hipStream_t)stream);
}

moet_status moet_requant_fp8(const uint8_t *fp8_w, const float *fp8_scales, int64_t n_mat, int64_t N, int64_t K,
                     uint32_t *w2_codes, uint8_t *w2_scales, float *w2_scale2, uint32_t flags, void *stream)
{
    g_err[0] = 0;
    int rc = check_stack(n_mat, N, K, flags);
    if (rc != MOET_OK) return (moet_status)(rc);
    if (!aligned16(fp8_w) || !aligned16(fp8_scales) || !aligned16(w2_codes) || !aligned16(w2_scales) ||
        !aligned16(w2_scale2))
        return (moet_status)(fail(MOET_EINVAL, "pointers must be non-NULL and 16-byte aligned"));
    return (moet_status)launch_requant_fp8(fp8_w, fp8_scales, n_mat, (int)N, (int)K, (int)(flags & MOET_BALANCE_ZERO_SIGNS),
                                           w2_codes, w2_scales, w2_scale2, (hipStream_t)stream);
}

moet_status moet_route(const float *logits, int32_t T, int32_t E, int32_t top_k, int32_t score_fn, int32_t renormalize,
               float route_scale, int32_t *topk_ids, float *topk_w, int32_t *expert_offsets, int32_t *sorted_pairs,
               void *stream)
{
    g_err[0] = 0;
    if (T < 1 || T > 65536) return (moet_status)(fail(MOET_EINVAL, "T (%d) must be in [1, 65536]", T));
    if (E < 1 || E > 1024) return (moet_status)(fail(MOET_EINVAL, "E (%d) must be in [1, 1024]", E));
    if (top_k < 1 || top_k > E || top_k > 16)
        return (moet_status)(fail(MOET_EINVAL, "top_k (%d) must be in [1, min(E, 16)]", top_k));
    if (score_fn != MOET_SOFTMAX && score_fn != MOET_SIGMOID)
        return (moet_status)(fail(MOET_EINVAL, "unknown score_fn %d", score_fn));
    if (!(route_scale == route_scale)) return (moet_status)(fail(MOET_EINVAL, "route_scale is NaN"));
    if (!aligned16(logits) || !aligned16(topk_ids) || !aligned16(topk_w) || !aligned16(expert_offsets) ||
        !aligned16(sorted_pairs))
        return (moet_status)(fail(MOET_EINVAL, "pointers must be non-NULL and 16-byte aligned"));
    return (moet_status)launch_route(logits, T, E, top_k, score_fn, renormalize, route_scale, topk_ids, topk_w, expert_offsets,
                                     sorted_pairs, (hipStream_t)stream);
}

size_t moet_moe_workspace_bytes(const moet_layer *L, int32_t T, int32_t top_k)
{
    return forward_workspace_bytes(L, T, top_k);
}

moet_status moet_moe_forward(const moet_layer *L, const uint16_t *x, int32_t T, int32_t top_k, const int32_t *topk_ids,
                     const float *topk_w, const int32_t *expert_offsets, const int32_t *sorted_pairs,
                     const uint8_t *gate_flags, uint16_t *out, int32_t *miss_count, void *workspace,
                     size_t workspace_bytes, void *stream)
{
    g_err[0] = 0;
    int rc = check_forward(L, x, T, top_k, topk_ids, topk_w, expert_offsets, sorted_pairs, gate_flags, out, miss_count);
    if (rc != MOET_OK) return (moet_status)(rc);
    return (moet_status)dispatch_forward(L, x, T, top_k, topk_ids, topk_w, expert_offsets, sorted_pairs, gate_flags, out,
                                         miss_count, workspace, workspace_bytes, (hipStream_t)stream);
}

moet_status moet_set_timing_events(void *start, void *stop)
{
    g_err[0] = 0;
    if ((start == nullptr) != (stop == nullptr))
        return (moet_status)(fail(MOET_EINVAL, "set both timing events or neither"));
    g_ev_start = (hipEvent_t)start;
    g_ev_stop = (hipEvent_t)stop;
    return (moet_status)(MOET_OK);
}

moet_status moet_delta_forward(const moet_fp4 *D, int32_t n_slots, int32_t N, int32_t K, const uint16_t *act,
                       const int32_t *row_slot, int32_t R, float *acc, void *stream)
{
    g_err[0] = 0;
    if (!D) return (moet_status)(fail(MOET_EINVAL, "D is NULL"));
    if (n_slots < 1) return (moet_status)(fail(MOET_EINVAL, "n_slots (%d) must be >= 1", n_slots));
    if (N < 64 || N % 64) return (moet_status)(fail(MOET_EINVAL, "N (%d) must be a positive multiple of 64", N));
    if (K < 128 || K % 128) return (moet_status)(fail(MOET_EINVAL, "K (%d) must be a positive multiple of 128", K));
    if (R < 0 || R > 65535) return (moet_status)(fail(MOET_EINVAL, "R (%d) must be in [0, 65535]", R));
    if (R == 0) return (moet_status)(MOET_OK);
    if (!aligned16(D->codes) || !aligned16(D->scales) || !aligned16(D->scale2) || !aligned16(act) ||
        !aligned16(row_slot) || !aligned16(acc))
        return (moet_status)(fail(MOET_EINVAL, "pointers must be non-NULL and 16-byte aligned"));
    return (moet_status)launch_delta(D, n_slots, N, K, act, row_slot, R, acc, (hipStream_t)stream);
}

size_t moet_gate_workspace_bytes(int32_t T, int32_t V)
{
    if (T < 1 || T > 65535 || V < 1) return 0;
    return gate_workspace_bytes(T, V);
}

moet_status moet_confidence_gate(const float *logits, int32_t T, int32_t V, float tau, uint8_t *gate_flags,
                         float *confidence_out, void *workspace, size_t workspace_bytes, void *stream)
{
    g_err[0] = 0;
    if (T < 1 || T > 65535) return (moet_status)(fail(MOET_EINVAL, "T (%d) must be in [1, 65535]", T));
    if (V < 1) return (moet_status)(fail(MOET_EINVAL, "V (%d) must be >= 1", V));
    if (!(tau == tau) || tau > 3.4e38f || tau < -3.4e38f) return (moet_status)(fail(MOET_EINVAL, "tau must be finite"));
    if (!aligned16(logits) || !gate_flags)
        return (moet_status)(fail(MOET_EINVAL, "logits (16-byte aligned) and gate_flags must be non-NULL"));
    if (confidence_out && (reinterpret_cast<uintptr_t>(confidence_out) & 3u))
        return (moet_status)(fail(MOET_EINVAL, "confidence_out must be 4-byte aligned"));
    const size_t need = gate_workspace_bytes(T, V);
    if (need && (!workspace || workspace_bytes < need))
        return (moet_status)(fail(MOET_EWORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace_bytes));
    if (need && !aligned16(workspace)) return (moet_status)(fail(MOET_EINVAL, "workspace must be 16-byte aligned"));
    return (moet_status)launch_gate(logits, T, V, tau, gate_flags, confidence_out, workspace, (hipStream_t)stream);
}

}  // extern "C"
