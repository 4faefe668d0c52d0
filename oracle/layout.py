"""Packing of the oracle's plain arrays into the library's storage layout
(oracle; test infrastructure only).

The layout is the library's own choice (the pages fix none of it); it is
written out here from its definition so the HIP requantiser's output can be
compared byte for byte.  Every matrix [N][K] (N % 64 == 0, K % 128 == 0) is
stored in row tiles of 64 rows:

2-bit codes, uint32 words:
    word((n, k)) = ((n//64 * K/64 + k//64) * 64 + n%64) * 4 + (k%64)//16
  inside a word, element e = k%16 with code c = (s<<1)|m is stored as
    e < 8:  m at bit 4e + 2,      s at bit 4e + 3
    e >= 8: m at bit 4(e-8),      s at bit 4(e-8) + 1
  i.e. the word's nibble j holds element j in its upper two bits and element
  j + 8 in its lower two bits.
2-bit block scales (one e4m3 byte per 32 along K):
    byte((n, b)) = ((n//64 * K/128 + b//4) * 64 + n%64) * 4 + b%4
FP4 delta codes (two per byte, even k in the low nibble):
    byte((n, k)) = ((n//64 * K/32 + k//32) * 64 + n%64) * 16 + (k%32)//2
FP4 delta block scales (one e4m3 byte per 16 along K):
    byte((n, b)) = ((n//64 * K/128 + b//8) * 64 + n%64) * 8 + b%8
"""
from __future__ import annotations

import numpy as np

TILE = 64


def _check(N, K):
    if N % TILE or K % 128:
        raise ValueError(f"layout needs N % 64 == 0 and K % 128 == 0, got N={N} K={K}")


def _bit_positions():
    pm = np.zeros(16, dtype=np.int64)
    ps = np.zeros(16, dtype=np.int64)
    for e in range(16):
        nibble = e % 8
        low_half = e >= 8
        pm[e] = 4 * nibble + (0 if low_half else 2)
        ps[e] = pm[e] + 1
    return pm, ps


def pack_2bit_codes(codes2: np.ndarray) -> np.ndarray:
    """codes2 uint8 [N, K] (values 0..3) -> uint32 [N*K/16] in the tiled layout."""
    c = np.asarray(codes2, dtype=np.uint32)
    N, K = c.shape
    _check(N, K)
    pm, ps = _bit_positions()
    c = c.reshape(N // TILE, TILE, K // 64, 4, 16)          # [tile, r, chunk, word, e]
    c = np.ascontiguousarray(np.moveaxis(c, -1, 0))          # [e, tile, r, chunk, word]
    words = np.zeros(c.shape[1:], dtype=np.uint32)
    for e in range(16):
        words |= (c[e] & 1) << np.uint32(pm[e])
        words |= ((c[e] >> 1) & 1) << np.uint32(ps[e])
    words = words.transpose(0, 2, 1, 3)      # [tile, chunk, r, word]
    return np.ascontiguousarray(words).reshape(-1)


def unpack_2bit_codes(words: np.ndarray, N: int, K: int) -> np.ndarray:
    _check(N, K)
    pm, ps = _bit_positions()
    w = np.asarray(words, dtype=np.uint64).reshape(N // TILE, K // 64, TILE, 4)
    w = w.transpose(0, 2, 1, 3)[..., None]   # [tile, r, chunk, word, 1]
    m = (w >> pm.astype(np.uint64)) & 1
    s = (w >> ps.astype(np.uint64)) & 1
    return ((s << 1) | m).reshape(N, K).astype(np.uint8)


def pack_2bit_scales(tau: np.ndarray) -> np.ndarray:
    """tau uint8 [N, K/32] -> uint8 [N*K/32] in the tiled layout."""
    t = np.asarray(tau, dtype=np.uint8)
    N, nb = t.shape
    _check(N, nb * 32)
    t = t.reshape(N // TILE, TILE, nb // 4, 4).transpose(0, 2, 1, 3)
    return np.ascontiguousarray(t).reshape(-1)


def pack_fp4_codes(dcodes: np.ndarray) -> np.ndarray:
    """dcodes [N, K] 4-bit codes -> uint8 [N*K/2] in the tiled layout."""
    d = np.asarray(dcodes, dtype=np.uint8)
    N, K = d.shape
    _check(N, K)
    b = (d[:, 0::2] & 15) | ((d[:, 1::2] & 15) << 4)        # [N, K/2]
    b = b.reshape(N // TILE, TILE, K // 32, 16).transpose(0, 2, 1, 3)
    return np.ascontiguousarray(b).reshape(-1)


def pack_fp4_scales(dscales: np.ndarray) -> np.ndarray:
    """dscales uint8 [N, K/16] -> uint8 [N*K/16] in the tiled layout."""
    s = np.asarray(dscales, dtype=np.uint8)
    N, nb = s.shape
    _check(N, nb * 16)
    s = s.reshape(N // TILE, TILE, nb // 8, 8).transpose(0, 2, 1, 3)
    return np.ascontiguousarray(s).reshape(-1)


def unpack_fp4_codes(b: np.ndarray, N: int, K: int) -> np.ndarray:
    _check(N, K)
    x = np.asarray(b, dtype=np.uint8).reshape(N // TILE, K // 32, TILE, 16).transpose(0, 2, 1, 3)
    x = x.reshape(N, K // 2)
    out = np.empty((N, K), dtype=np.uint8)
    out[:, 0::2] = x & 15
    out[:, 1::2] = x >> 4
    return out


def unpack_fp4_scales(s: np.ndarray, N: int, K: int) -> np.ndarray:
    _check(N, K)
    x = np.asarray(s, dtype=np.uint8).reshape(N // TILE, K // 128, TILE, 8).transpose(0, 2, 1, 3)
    return x.reshape(N, K // 16)


def unpack_2bit_scales(s: np.ndarray, N: int, K: int) -> np.ndarray:
    _check(N, K)
    x = np.asarray(s, dtype=np.uint8).reshape(N // TILE, K // 128, TILE, 4).transpose(0, 2, 1, 3)
    return x.reshape(N, K // 32)
