"""Expert FFN, routed combine and FP4 GEMM (oracle; test infrastructure only).

Sources: README "Frontier MoE on consumer Blackwell (SM120)", section
"How it fits — 2-bit experts at FP4 quality" (the 2-bit MoE GEMM runs the
experts from the 2-bit planes; an FP4 delta GEMM adds a residual for experts
in the delta cache, and the confidence gate decides which steps use it);
airanks.app "kacper-daftcode/vLLM-Moet", section "Quality vs native" (a
checkpoint may carry a SwiGLU clamp).

Readings (fixed rounding points, so that the kernels' fp32 accumulation can be
compared tightly):
  u_g = W_g x, u_u = W_u x (+ D_g x, D_u x for a flagged token on a resident
  expert), optional clamp u_g <= L, -L <= u_u <= L when L > 0,
  h = bf16_rne(silu(u_g) * u_u), silu(z) = z / (1 + e^-z);
  y = W_d h (+ D_d h), not rounded;
  out_t = bf16_rne(sum_j w_tj * y_(t,j) + y_shared(t)); the shared expert uses
  the same FFN with weight 1 and no delta.
All real arithmetic is float64 on exactly dequantised weights.

Expert cache (README, section "When the model doesn't fit at all — the GPU
as an expert cache"): when only some experts' base weights are on the GPU, a
routing to a missing expert contributes nothing to its token's output (its
weight is not redistributed) and is counted; once the missing experts are
fetched, the same step reproduces the fully resident output exactly.
"""
from __future__ import annotations

from typing import Callable, Optional, Sequence

import numpy as np

from .formats import bf16_bits_to_f64, bf16_rne_bits


def silu(z: np.ndarray) -> np.ndarray:
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def expert_hidden(x: np.ndarray, Wg: np.ndarray, Wu: np.ndarray, swiglu_limit: float = 0.0,
                  Dg: Optional[np.ndarray] = None, Du: Optional[np.ndarray] = None) -> np.ndarray:
    """h (float64 values of bf16) for token rows x [M, H]; W* [I, H]."""
    ug = x @ Wg.T
    uu = x @ Wu.T
    if Dg is not None:
        ug = ug + x @ Dg.T
        uu = uu + x @ Du.T
    if swiglu_limit > 0:
        ug = np.minimum(ug, swiglu_limit)
        uu = np.clip(uu, -swiglu_limit, swiglu_limit)
    return bf16_bits_to_f64(bf16_rne_bits(silu(ug) * uu))


def expert_out(h: np.ndarray, Wd: np.ndarray, Dd: Optional[np.ndarray] = None) -> np.ndarray:
    """y = W_d h (+ D_d h), float64, [M, H]; Wd [H, I]."""
    y = h @ Wd.T
    if Dd is not None:
        y = y + h @ Dd.T
    return y


WeightFn = Callable[[int], Sequence[np.ndarray]]


def moe_forward(x_bits: np.ndarray, topk_ids: np.ndarray, topk_w: np.ndarray,
                expert_weights: WeightFn, shared_weights: Optional[Sequence[np.ndarray]] = None,
                gate_flags: Optional[np.ndarray] = None, slot_of_expert: Optional[np.ndarray] = None,
                delta_weights: Optional[WeightFn] = None, swiglu_limit: float = 0.0,
                tokens: Optional[Sequence[int]] = None,
                resident: Optional[np.ndarray] = None) -> np.ndarray:
    """Layer output as bf16 bit patterns [len(tokens), H].

    x_bits: bf16 bits [T, H]; expert_weights(e) -> (Wg, Wu, Wd) float64;
    delta_weights(slot) -> (Dg, Du, Dd) float64; a pair (t, e) takes the delta
    iff gate_flags[t] != 0 and slot_of_expert[e] >= 0.  ``tokens`` restricts
    the computation to a subset of rows (each output row depends only on its
    own token).  ``resident`` (bool [E], None = all): pairs whose expert is not
    resident contribute nothing.
    """
    x = bf16_bits_to_f64(x_bits)
    T, H = x.shape
    ids = np.asarray(topk_ids, dtype=np.int64)
    w = np.asarray(topk_w, dtype=np.float64)
    if tokens is None:
        tokens = range(T)
    tokens = list(tokens)
    acc = np.zeros((len(tokens), H), dtype=np.float64)
    # group the requested (token, slot) pairs by expert so each expert is dequantised once
    by_expert = {}
    for ti, t in enumerate(tokens):
        for j in range(ids.shape[1]):
            by_expert.setdefault(int(ids[t, j]), []).append((ti, t, j))
    for e, lst in sorted(by_expert.items()):
        if resident is not None and not resident[e]:
            continue
        Wg, Wu, Wd = expert_weights(e)
        for ti, t, j in lst:
            use_delta = (gate_flags is not None and slot_of_expert is not None and delta_weights is not None
                         and gate_flags[t] != 0 and slot_of_expert[e] >= 0)
            if use_delta:
                Dg, Du, Dd = delta_weights(int(slot_of_expert[e]))
            else:
                Dg = Du = Dd = None
            h = expert_hidden(x[t:t + 1], Wg, Wu, swiglu_limit, Dg, Du)
            y = expert_out(h, Wd, Dd)
            acc[ti] += w[t, j] * y[0]
    if shared_weights is not None:
        Wg, Wu, Wd = shared_weights
        h = expert_hidden(x[tokens], Wg, Wu, swiglu_limit)
        acc += expert_out(h, Wd)
    return bf16_rne_bits(acc)


def miss_count(topk_ids: np.ndarray, resident: np.ndarray) -> int:
    """Number of (token, expert) routings whose expert is not resident."""
    ids = np.asarray(topk_ids, dtype=np.int64).reshape(-1)
    return int(np.count_nonzero(~np.asarray(resident, dtype=bool)[ids]))


def fp4_gemm_accumulate(acc: np.ndarray, act_bits: np.ndarray, row_slot: np.ndarray,
                        delta_of_slot: Callable[[int], np.ndarray]) -> np.ndarray:
    """acc[r, :] + D_{row_slot[r]} @ act[r, :] for row_slot[r] >= 0, float64 (rows with a
    negative slot are left unchanged)."""
    out = np.asarray(acc, dtype=np.float64).copy()
    a = bf16_bits_to_f64(act_bits)
    for r, s in enumerate(np.asarray(row_slot)):
        if s >= 0:
            out[r] += delta_of_slot(int(s)) @ a[r]
    return out
