"""Number formats: e2m1, e4m3fn, bf16 and NVFP4 decode (oracle; test infrastructure only).

Source: README "Frontier MoE on consumer Blackwell (SM120)", section
"GLM-5.2 (753B) — the headline model": the experts arrive as modelopt NVFP4,
i.e. 4-bit e2m1 values, one e4m3 scale per 16 consecutive weights along the
reduction axis, and one fp32 per-tensor scale (``scale_2``).  The pages do not
spell the bit layouts out; the readings taken are:

* e2m1: sign-magnitude 4-bit float, bit 3 = sign, 2 exponent bits (bias 1),
  1 mantissa bit; magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6.  -0 exists.
* e4m3: the "FN" variant (bias 7, no infinities, 0x7F/0xFF are NaN, largest
  finite 448, subnormals m/8 * 2^-6).
* two e2m1 codes per byte, the even element in the low nibble.
* bf16: IEEE binary32 with the low 16 bits cut, rounded to nearest-even
  directly from the float64 value (no float32 intermediate rounding).
"""
from __future__ import annotations

import numpy as np


def e2m1_value(code) -> np.ndarray:
    """Value of a 4-bit e2m1 code (array-friendly), float64."""
    c = np.asarray(code, dtype=np.int64)
    sign = np.where((c >> 3) & 1, -1.0, 1.0)
    e = (c >> 1) & 3
    m = c & 1
    mag = np.where(e == 0, m * 0.5, (1.0 + m / 2.0) * np.exp2(e - 1.0))
    return sign * mag


def e4m3fn_value(byte) -> np.ndarray:
    """Value of an 8-bit e4m3fn code, float64 (NaN for 0x7F / 0xFF)."""
    b = np.asarray(byte, dtype=np.int64)
    sign = np.where((b >> 7) & 1, -1.0, 1.0)
    e = (b >> 3) & 15
    m = b & 7
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


# Integer forms used by the exact requantisation: 2*|e2m1| and e4m3 * 2^9 are
# integers for every finite code.
E2M1_MAG2 = np.array([0, 1, 2, 3, 4, 6, 8, 12], dtype=np.int64)          # 2*|value| of codes 0..7
E4M3_X512 = np.array([int(round(float(e4m3fn_value(t)) * 512)) for t in range(127)], dtype=np.int64)


def bf16_rne_bits(x) -> np.ndarray:
    """Round float64 values to bf16 (nearest, ties to even); returns uint16 bit patterns.

    The rounding is done on the float64 value itself: the quantum of x's binade
    (8 significant bits, subnormal quantum 2^-133) is found exactly with frexp,
    x / quantum is rounded half-to-even with rint (exact in float64), and the
    already-representable result is converted to float32 without further
    rounding.  Overflow to infinity is not expected for this layer's values.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros(x.shape, dtype=np.float64)
    nz = (x != 0) & np.isfinite(x)
    xs = x[nz]
    _, ex = np.frexp(xs)                      # xs = f * 2^ex, 0.5 <= |f| < 1
    binade = np.maximum(ex - 1, -126)         # floor(log2|x|), clamped at bf16's min normal
    quantum = np.exp2(binade - 7.0)
    out[nz] = np.rint(xs / quantum) * quantum
    out[~nz] = x[~nz]
    f32 = out.astype(np.float32)              # exact: out has <= 8 significant bits
    bits = f32.view(np.uint32) >> 16
    # keep the sign of zero from x
    bits = np.where(out == 0, np.where(np.signbit(x), 0x8000, 0), bits)
    return bits.astype(np.uint16)


def bf16_bits_to_f64(bits) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint32) << 16
    return b.astype(np.uint32).view(np.float32).astype(np.float64)


def nvfp4_decode(codes: np.ndarray, scales: np.ndarray, scale_2: float) -> np.ndarray:
    """Dequantise one NVFP4 matrix exactly: x[n,k] = e2m1(code) * e4m3(S[n, k//16]) * scale_2.

    codes: uint8 [N, K/2] (even k in the low nibble), scales: uint8 [N, K/16].
    The product has at most 2+4+24 significant bits, so float64 holds it exactly.
    """
    codes = np.asarray(codes, dtype=np.uint8)
    N, Kh = codes.shape
    nib = np.empty((N, Kh * 2), dtype=np.int64)
    nib[:, 0::2] = codes & 0xF
    nib[:, 1::2] = codes >> 4
    s = e4m3fn_value(np.asarray(scales, dtype=np.uint8))
    s_full = np.repeat(s, 16, axis=1)
    return e2m1_value(nib) * s_full * np.float64(np.float32(scale_2))


def unpack_nibbles(codes: np.ndarray) -> np.ndarray:
    """uint8 [N, K/2] -> int64 [N, K] of 4-bit codes (even k from the low nibble)."""
    codes = np.asarray(codes, dtype=np.uint8)
    N, Kh = codes.shape
    nib = np.empty((N, Kh * 2), dtype=np.int64)
    nib[:, 0::2] = codes & 0xF
    nib[:, 1::2] = codes >> 4
    return nib
