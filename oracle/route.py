"""Router top-k, routing weights and token permutation (oracle; test infrastructure only).

Sources: README "Frontier MoE on consumer Blackwell (SM120)", section
"How it fits — 2-bit experts at FP4 quality" (routed experts are selected per
token and their outputs combined) and section "When the model doesn't fit at
all — the GPU as an expert cache" (a descriptor step groups the step's
token->expert routings per expert before the expert GEMMs).

Readings (the pages name neither the score function nor the tie order):
  * selection is on the raw fp32 logits, largest first, equal logits -> lower
    expert id first (softmax and sigmoid are monotonic, so this is exact);
  * softmax weights: exp(l_j - l_max) / sum over the selected experts when
    renormalising (equal to softmax over all experts then renormalised), else
    softmax over all E evaluated at the selected ids;
  * sigmoid weights: sigma(l_j), divided by their sum over the selected experts
    when renormalising;
  * every weight is then multiplied by route_scale;
  * pair id p = t*k + j; sorted_pairs lists all pairs ordered by
    (expert, p) ascending; expert_offsets[e] = number of pairs with expert < e,
    expert_offsets[E] = T*k.
"""
from __future__ import annotations

import numpy as np

SOFTMAX = 0
SIGMOID = 1


def topk_ids(logits: np.ndarray, k: int) -> np.ndarray:
    """ids [T, k] int32: per row the k largest logits, ties -> lower id."""
    lg = np.asarray(logits, dtype=np.float32)
    T, E = lg.shape
    ids = np.arange(E)
    out = np.empty((T, k), dtype=np.int32)
    for t in range(T):
        order = np.lexsort((ids, -lg[t].astype(np.float64)))   # primary: -logit, then id
        out[t] = order[:k]
    return out


def topk_weights(logits: np.ndarray, ids: np.ndarray, fn: int, renormalize: bool,
                 route_scale: float = 1.0) -> np.ndarray:
    """Routing weights [T, k] in float64."""
    lg = np.asarray(logits, dtype=np.float32).astype(np.float64)
    sel = np.take_along_axis(lg, np.asarray(ids, dtype=np.int64), axis=1)
    if fn == SOFTMAX:
        if renormalize:
            z = np.exp(sel - sel.max(axis=1, keepdims=True))
            w = z / z.sum(axis=1, keepdims=True)
        else:
            mx = lg.max(axis=1, keepdims=True)
            w = np.exp(sel - mx) / np.exp(lg - mx).sum(axis=1, keepdims=True)
    elif fn == SIGMOID:
        s = 1.0 / (1.0 + np.exp(-sel))
        w = s / s.sum(axis=1, keepdims=True) if renormalize else s
    else:
        raise ValueError("unknown score function")
    return w * float(np.float32(route_scale))


def permute(ids: np.ndarray, E: int):
    """(expert_offsets int32 [E+1], sorted_pairs int32 [T*k])."""
    flat = np.asarray(ids, dtype=np.int64).reshape(-1)
    counts = np.bincount(flat, minlength=E)
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    order = np.argsort(flat, kind="stable")
    return offsets.astype(np.int32), order.astype(np.int32)


def route(logits: np.ndarray, k: int, fn: int, renormalize: bool = True, route_scale: float = 1.0):
    """Full routing step: (ids, weights f64, offsets, sorted_pairs)."""
    ids = topk_ids(logits, k)
    w = topk_weights(logits, ids, fn, renormalize, route_scale)
    offs, pairs = permute(ids, np.asarray(logits).shape[1])
    return ids, w, offs, pairs
