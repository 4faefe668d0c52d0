// Prefill-sized MoE layer forward (placeholder: runs the GEMV kernels).
#include "moet_common.h"

namespace moet {

size_t decode_workspace_bytes(int T, int k, int H, int I);
int launch_decode(const moet_layer *, const uint16_t *, int, int, const int32_t *, const float *, const int32_t *,
                  const int32_t *, const uint8_t *, uint16_t *, void *, hipStream_t);

size_t prefill_workspace_bytes(int T, int k, int H, int I, int E) { (void)E; return decode_workspace_bytes(T, k, H, I); }

int launch_prefill(const moet_layer *L, const uint16_t *x, int T, int k, const int32_t *ids, const float *w,
                   const int32_t *offsets, const int32_t *sorted, const uint8_t *gate, uint16_t *out, void *ws,
                   hipStream_t stream)
{
    if ((int64_t)T * k + 1 > 65535) return fail(MOET_EUNSUPPORTED, "T*top_k too large for this build");
    return launch_decode(L, x, T, k, ids, w, offsets, sorted, gate, out, ws, stream);
}

}  // namespace moet
