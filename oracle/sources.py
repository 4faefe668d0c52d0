"""Other source formats of the expert weights (oracle; test infrastructure only).

README "Frontier MoE on consumer Blackwell (SM120)", section "How it fits —
2-bit experts at FP4 quality": besides modelopt NVFP4, two more checkpoint
flavours load into the same sign-symmetric 2-bit planes.  FP4 experts have
their codes remapped; FP8 block-quantised experts are requantised at load in
float64 like the NVFP4 ones.  The pages name the flavours only; the readings
taken here:

MXFP4 codes remap (``remap_mxfp4``)
  * source: OCP microscaling FP4, e2m1 codes (two per byte, even k in the low
    nibble) and one e8m0 scale byte E per 32 weights along K, value
    e2m1 * 2^(E - 127); E = 0xFF (NaN) is rejected;
  * the 2-bit codebook {-4,-1,1,4} is a subset of the e2m1 grid (codes 2 and
    6), so a remap sends every e2m1 code to the nearest of those four values
    in units of the block scale: magnitudes 0, 0.5, 1, 1.5, 2 -> 1 and
    3, 4, 6 -> 4 (the midpoint 2.5 is not on the grid, so there are no ties);
    the sign is the code's sign bit (zeros included) or, when asked for,
    alternating over a block's zeros as in the NVFP4 requant;
  * the block scales carry over: with Emax the largest E over the blocks that
    hold a non-zero code, the tensor scale is S = 2^(Emax - 8 - 127) and the
    block's e4m3 scale is 2^(E - Emax + 8), exact for E >= Emax - 17; a
    block further down, or one with no non-zero code, gets scale 0.  A tensor
    with no non-zero code gets S = 1 and scale 0 everywhere.

FP8 block-quant requant (``requant_fp8``): exact statement in
``oracle/c/requant_ref.c`` (e4m3fn weights with one fp32 scale per 128 x 128
block; power-of-two tensor scale; the block scale minimising the float64 L2
error over all e4m3 codes, evaluated in a fixed order).
"""
from __future__ import annotations

import numpy as np

from .formats import e2m1_value, e4m3fn_value, unpack_nibbles
from .requant import BLOCK, _get, _ptr


def e8m0_value(byte) -> np.ndarray:
    """Value of an e8m0 scale byte: 2^(E - 127), NaN for 0xFF."""
    b = np.asarray(byte, dtype=np.int64)
    return np.where(b == 255, np.nan, np.exp2(b.astype(np.float64) - 127.0))


def mxfp4_decode(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """x[n, k] = e2m1(code) * 2^(E[n, k//32] - 127), exact in float64."""
    v = e2m1_value(unpack_nibbles(codes))
    return v * np.repeat(e8m0_value(scales), 32, axis=1)


def _e4m3_code_pow2(d: np.ndarray) -> np.ndarray:
    """e4m3fn code of 2^d for -9 <= d <= 8 (normal: exponent field d + 7,
    mantissa 0; subnormal: mantissa 2^(d + 9))."""
    d = np.asarray(d, dtype=np.int64)
    return np.where(d >= -6, (d + 7) << 3, np.left_shift(1, np.clip(d + 9, 0, 2))).astype(np.uint8)


def remap_mxfp4(codes: np.ndarray, scales: np.ndarray, balance_zero_signs: bool = False):
    """MXFP4 [N, K] -> (codes2 uint8 [N, K], tau uint8 [N, K/32], scale2_out float32)."""
    nib = unpack_nibbles(codes)
    N, K = nib.shape
    E = np.asarray(scales, dtype=np.int64)
    assert E.shape == (N, K // 32)
    if (E == 255).any():
        raise ValueError("MXFP4 block scale is NaN (0xFF)")
    mag = nib & 7
    live = (mag.reshape(N, K // 32, 32) != 0).any(axis=2)
    if live.any():
        emax = int(E[live].max())
        s2 = np.float32(np.ldexp(1.0, emax - 8 - 127))
        d = E - (emax - 8)
        tau = np.where(live & (d >= -9), _e4m3_code_pow2(d), 0).astype(np.uint8)
    else:
        s2 = np.float32(1.0)
        tau = np.zeros((N, K // 32), dtype=np.uint8)
    m = (mag >= 5).astype(np.uint8)                 # |e2m1| in {3, 4, 6}
    s = ((nib >> 3) & 1).astype(np.uint8)
    if balance_zero_signs:
        s = _balance(s, mag == 0, 32)
    return (s << 1) | m, tau, s2


def _balance(sign: np.ndarray, zero: np.ndarray, block: int) -> np.ndarray:
    """Signs of the zeros of each block replaced by 0, 1, 0, 1, ... in k order."""
    N, K = zero.shape
    z = zero.reshape(N, K // block, block)
    rank = np.cumsum(z, axis=2) - 1                 # index of each zero among its block's zeros
    out = np.where(z, rank & 1, sign.reshape(N, K // block, block))
    return out.reshape(N, K).astype(np.uint8)


def fp8_block_decode(w: np.ndarray, bscale: np.ndarray) -> np.ndarray:
    """x[n, k] = e4m3fn(w[n, k]) * bscale[n // 128, k // 128], exact in float64."""
    w = np.asarray(w, dtype=np.uint8)
    N, K = w.shape
    s = np.asarray(bscale, dtype=np.float32).astype(np.float64)
    full = np.repeat(np.repeat(s, 128, axis=0)[:N], 128, axis=1)
    return e4m3fn_value(w) * full


def requant_fp8(w: np.ndarray, bscale: np.ndarray, block: int = BLOCK, balance_zero_signs: bool = False):
    """FP8 block-quant [N, K] -> (codes2 uint8 [N, K], tau uint8 [N, K/block], scale2_out float32)."""
    w = np.ascontiguousarray(w, dtype=np.uint8)
    N, K = w.shape
    bscale = np.ascontiguousarray(bscale, dtype=np.float32)
    assert K % 128 == 0 and K % block == 0 and bscale.shape == ((N + 127) // 128, K // 128)
    codes2 = np.empty((N, K), dtype=np.uint8)
    tau = np.empty((N, K // block), dtype=np.uint8)
    s2 = np.zeros(1, dtype=np.float32)
    rc = _get().oracle_requant_fp8(_ptr(w), _ptr(bscale), N, K, block, int(bool(balance_zero_signs)),
                                   _ptr(codes2), _ptr(tau), _ptr(s2))
    if rc != 0:
        raise ValueError("FP8 weight is NaN or a block scale is negative or not finite")
    return codes2, tau, s2[0]
