"""Confidence gate (oracle; test infrastructure only).

Source: README "Frontier MoE on consumer Blackwell (SM120)", section "How it
fits — 2-bit experts at FP4 quality" (a confidence gate re-runs the
low-confidence steps with the FP4 delta; the benchmark table runs it at
tau = 0.60).

Reading (the pages name the threshold but not the statistic): a token is low
confidence when the largest probability of its next-token distribution,
softmax(logits)[argmax] = 1 / sum_v exp(l_v - l_max), is below tau; such a
token is flagged so that its experts take the FP4 delta.  The decision is made
in float64 from float32 logits (l_v - l_max is exact in float64); logits may be
-inf (masked) but each row needs a finite maximum.
"""
from __future__ import annotations

import numpy as np


def confidence(logits: np.ndarray) -> np.ndarray:
    """Largest next-token probability per row, float64 [T], from float32 logits [T, V]."""
    l = np.asarray(logits, dtype=np.float32).astype(np.float64)
    m = l.max(axis=1, keepdims=True)
    s = np.exp(l - m).sum(axis=1)
    return 1.0 / s


def gate_flags(logits: np.ndarray, tau: float) -> np.ndarray:
    """uint8 [T]: 1 where the largest next-token probability is below tau."""
    return (confidence(logits) < float(np.float32(tau))).astype(np.uint8)
