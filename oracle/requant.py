"""NVFP4 -> 2-bit requantisation and FP4 delta (oracle; test infrastructure only).

Thin ctypes wrapper around ``oracle/c/requant_ref.c`` (exact int64 search) plus
float64 dequantisation of its results.  See the C file for the sources and
the readings taken where the pages leave the method open.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

from .formats import e2m1_value, e4m3fn_value

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "c", "requant_ref.c")
_LIB = os.path.join(_HERE, "c", "liboracle_requant.so")
_lib = None

#: block length of the 2-bit per-block scale along K (reading: 32, which gives
#: 2.25 bits per weight)
BLOCK = 32
#: 2-bit code -> level of the sign-symmetric codebook {-4,-1,1,4} (codebook 0, the default)
LEVELS = np.array([1.0, 4.0, -1.0, -4.0])
#: the per-tensor codebooks a tensor may pick (code -> level; code 0/1 = +lo/+hi, 2/3 = -lo/-hi) and
#: the power of two between their tensor scale and the source scale_2 (README "How it fits": nearly
#: every tensor picks {-4,-1,1,4}; the candidates are the other sign-symmetric four-level codebooks
#: with FP4 levels {1/2, 3} and {0, 2})
CODEBOOK_LEVELS = (LEVELS, np.array([0.5, 3.0, -0.5, -3.0]), np.array([0.0, 2.0, -0.0, -2.0]))
CODEBOOK_SCALE2 = (2.0, 2.0, 4.0)


def build_oracle_lib(force: bool = False) -> str:
    """Compile the C oracle with gcc (OpenMP over rows)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-shared", "-fPIC", "-o", tmp, _SRC])
        os.replace(tmp, _LIB)
    return _LIB


def _get():
    global _lib
    if _lib is None:
        build_oracle_lib()
        lib = ctypes.CDLL(_LIB)
        p = ctypes.c_void_p
        i64 = ctypes.c_int64
        lib.oracle_requant.argtypes = [p, p, i64, i64, i64, ctypes.c_int, ctypes.c_int, p, p, p]
        lib.oracle_requant.restype = ctypes.c_int
        lib.oracle_requant_fp8.argtypes = [p, p, i64, i64, i64, ctypes.c_int, p, p, p]
        lib.oracle_requant_fp8.restype = ctypes.c_int
        lib.oracle_delta.argtypes = [p, p, i64, i64, i64, ctypes.c_int, p, p, p, p]
        lib.oracle_delta.restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def requant(codes: np.ndarray, scales: np.ndarray, scale_2: float, block: int = BLOCK,
            return_err: bool = False, balance_zero_signs: bool = False, codebook: int = 0):
    """Requantise one NVFP4 matrix [N, K] (codes uint8 [N, K/2], scales uint8 [N, K/16]) with
    codebook `codebook` (0: {-4,-1,1,4}; 1: {-3,-1/2,1/2,3}; 2: {-2,-0,+0,2}).

    balance_zero_signs: zeros of a block take alternating signs (+, -, +, ...)
    in k order instead of their own sign bit.
    Returns (codes2 uint8 [N, K] in 0..3, tau uint8 [N, K/block], scale2_out float32[, err int64]).
    """
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    N, Kh = codes.shape
    K = Kh * 2
    assert scales.shape == (N, K // 16) and K % block == 0
    codes2 = np.empty((N, K), dtype=np.uint8)
    tau = np.empty((N, K // block), dtype=np.uint8)
    err = np.empty((N, K // block), dtype=np.int64) if return_err else None
    rc = _get().oracle_requant(_ptr(codes), _ptr(scales), N, K, block, int(bool(balance_zero_signs)),
                               int(codebook), _ptr(codes2), _ptr(tau), _ptr(err) if err is not None else None)
    if rc != 0:
        raise ValueError("NVFP4 block scale is negative or NaN, or unknown codebook")
    s2 = np.float32(CODEBOOK_SCALE2[codebook]) * np.float32(scale_2)
    return (codes2, tau, s2, err) if return_err else (codes2, tau, s2)


def pick_codebook(codes: np.ndarray, scales: np.ndarray, scale_2: float, block: int = BLOCK,
                  balance_zero_signs: bool = False):
    """Per-tensor codebook pick: the codebook whose requantisation has the smallest exact total L2
    error over the whole matrix (block errors summed as Python integers), ties to the lower index.
    Returns (codebook, codes2, tau, scale2_out, total errors of every codebook)."""
    best = None
    totals = []
    for cb in range(len(CODEBOOK_LEVELS)):
        c2, tau, s2, err = requant(codes, scales, scale_2, block, True, balance_zero_signs, cb)
        tot = sum(int(e) for e in err.reshape(-1))
        totals.append(tot)
        if best is None or tot < best[0]:
            best = (tot, cb, c2, tau, s2)
    return best[1], best[2], best[3], best[4], totals


def delta(codes: np.ndarray, scales: np.ndarray, scale_2: float, codes2: np.ndarray,
          tau: np.ndarray, block: int = BLOCK, codebook: int = 0):
    """FP4 re-encoding of W_nvfp4 - W_2bit (W_2bit in codebook `codebook`).  Returns (dcodes uint8
    [N, K] 4-bit codes, dscales uint8 [N, K/16], dscale2 float32 = scale_2)."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    codes2 = np.ascontiguousarray(codes2, dtype=np.uint8)
    tau = np.ascontiguousarray(tau, dtype=np.uint8)
    N, Kh = codes.shape
    K = Kh * 2
    dcodes = np.empty((N, K), dtype=np.uint8)
    dscales = np.empty((N, K // 16), dtype=np.uint8)
    rc = _get().oracle_delta(_ptr(codes), _ptr(scales), N, K, block, int(codebook), _ptr(codes2), _ptr(tau),
                             _ptr(dcodes), _ptr(dscales))
    if rc != 0:
        raise ValueError("NVFP4 block scale is negative or NaN")
    return dcodes, dscales, np.float32(scale_2)


def dequant_2bit(codes2: np.ndarray, tau: np.ndarray, scale2_out: float, block: int = BLOCK,
                 codebook: int = 0) -> np.ndarray:
    """W_2bit[n,k] = level(code) * e4m3(tau[n, k//block]) * scale2_out, exact in float64."""
    c = np.asarray(codes2)
    N, K = c.shape
    lv = np.take(CODEBOOK_LEVELS[codebook], c).reshape(N, K // block, block)
    s = e4m3fn_value(np.asarray(tau, dtype=np.uint8)) * np.float64(np.float32(scale2_out))   # exact
    lv *= s[:, :, None]
    return lv.reshape(N, K)


def dequant_fp4_codes(dcodes: np.ndarray, dscales: np.ndarray, dscale2: float) -> np.ndarray:
    """Decode FP4 codes given one code per element ([N, K] 4-bit) and block-16 scales."""
    v = e2m1_value(np.asarray(dcodes, dtype=np.int64))
    s = np.repeat(e4m3fn_value(np.asarray(dscales, dtype=np.uint8)), 16, axis=1)
    return v * s * np.float64(np.float32(dscale2))


def pack_nibbles(dcodes: np.ndarray) -> np.ndarray:
    """[N, K] 4-bit codes -> uint8 [N, K/2] with the even k in the low nibble."""
    d = np.asarray(dcodes, dtype=np.uint8)
    return (d[:, 0::2] & 15) | ((d[:, 1::2] & 15) << 4)
