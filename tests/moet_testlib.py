"""Shared helpers for the parity tests: run the oracle on the same seeded
inputs the HIP path consumes and compare.  Nothing here computes the method
itself; it only moves bytes between torch and the oracle."""
from __future__ import annotations

import numpy as np
import torch

from oracle import formats as OF
from oracle import layout as OL
from oracle import requant as OR
from oracle import route as ORT
from oracle import ffn as OFF


def np_(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


class OracleMatrix:
    """Oracle requant (and optional delta) of one NVFP4 matrix, plus its packed layout."""

    def __init__(self, codes: np.ndarray, scales: np.ndarray, scale_2: float, with_delta: bool = False):
        self.codes, self.scales, self.scale_2 = codes, scales, float(scale_2)
        self.c2, self.tau, self.s2 = OR.requant(codes, scales, scale_2)
        self.N, self.K = self.c2.shape
        self.dc = self.ds = self.d2 = None
        if with_delta:
            self.dc, self.ds, self.d2 = OR.delta(codes, scales, scale_2, self.c2, self.tau)

    def packed_codes(self):
        return OL.pack_2bit_codes(self.c2)

    def packed_scales(self):
        return OL.pack_2bit_scales(self.tau)

    def packed_delta(self):
        return OL.pack_fp4_codes(self.dc), OL.pack_fp4_scales(self.ds)

    def w2bit(self):
        return OR.dequant_2bit(self.c2, self.tau, self.s2)

    def wdelta(self):
        return OR.dequant_fp4_codes(self.dc, self.ds, self.d2)


class OracleLayer:
    """Lazily requantises the experts the oracle needs, straight from the NVFP4 bytes."""

    def __init__(self, src, slot_of_expert=None, shared_nvfp4=False):
        self.src = src
        self.cfg = src.cfg
        self.soe = None if slot_of_expert is None else np_(slot_of_expert)
        self.shared_nvfp4 = shared_nvfp4
        self._cache = {}

    def _mat(self, stack, i, with_delta):
        key = (id(stack), i, with_delta)
        if key not in self._cache:
            c, s, s2 = stack
            self._cache[key] = OracleMatrix(np_(c[i]), np_(s[i]), float(s2[i]), with_delta)
        return self._cache[key]

    def resident(self, e):
        return self.soe is not None and self.soe[e] >= 0

    def expert(self, e):
        d = self.resident(e)
        g = self._mat(self.src.w13, 2 * e, d)
        u = self._mat(self.src.w13, 2 * e + 1, d)
        dn = self._mat(self.src.w2, e, d)
        return g, u, dn

    def expert_weights(self, e):
        g, u, dn = self.expert(e)
        return g.w2bit(), u.w2bit(), dn.w2bit()

    def delta_weights_of_slot(self, slot):
        e = int(np.nonzero(self.soe == slot)[0][0])
        g, u, dn = self.expert(e)
        return g.wdelta(), u.wdelta(), dn.wdelta()

    def shared_weights(self):
        if self.src.shared13 is None:
            return None
        if self.shared_nvfp4:      # the shared expert keeps its NVFP4 values
            dq = lambda st, i: OF.nvfp4_decode(np_(st[0][i]), np_(st[1][i]), float(st[2][i]))
            return dq(self.src.shared13, 0), dq(self.src.shared13, 1), dq(self.src.shared2, 0)
        g = self._mat(self.src.shared13, 0, False)
        u = self._mat(self.src.shared13, 1, False)
        dn = self._mat(self.src.shared2, 0, False)
        return g.w2bit(), u.w2bit(), dn.w2bit()

    def forward(self, x_bits, ids, w, gate_flags=None, tokens=None, resident=None):
        return OFF.moe_forward(x_bits, ids, w, self.expert_weights, self.shared_weights(),
                               gate_flags=gate_flags, slot_of_expert=self.soe,
                               delta_weights=self.delta_weights_of_slot if self.soe is not None else None,
                               swiglu_limit=self.cfg.swiglu_limit, tokens=tokens, resident=resident)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return np_(t.contiguous().view(torch.int16)).astype(np.uint16)


def rel_l2(gpu_bits: np.ndarray, ref_bits: np.ndarray) -> float:
    a = OF.bf16_bits_to_f64(gpu_bits)
    b = OF.bf16_bits_to_f64(ref_bits)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def oracle_route(logits: torch.Tensor, k: int, fn: int, renorm: bool = True, scale: float = 1.0):
    return ORT.route(np_(logits), k, fn, renorm, scale)


#: floating-point bar of the method (relative L2 error of the layer output)
REL_L2_BAR = 2e-3
