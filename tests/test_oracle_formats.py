"""Pins for the oracle's number formats (CPU only).

e2m1 is checked against the magnitudes the OCP microscaling spec lists, e4m3fn
against torch's own float8_e4m3fn conversion (an independent library routine),
bf16 rounding against torch's float32->bfloat16 cast and hand-made edge cases.
"""
import numpy as np
import pytest
import torch

from oracle import formats as F


def test_e2m1_table():
    mags = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    for c in range(16):
        v = float(F.e2m1_value(c))
        want = mags[c & 7] * (-1.0 if c & 8 else 1.0)
        assert v == want
        assert np.signbit(v) == bool(c & 8)       # -0 exists for code 8


def test_e2m1_mag2_integers():
    assert list(F.E2M1_MAG2) == [int(2 * abs(F.e2m1_value(c))) for c in range(8)]


def test_e4m3fn_all_codes_against_torch():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    mine = F.e4m3fn_value(np.arange(256))
    nan = np.isnan(ref)
    assert (np.isnan(mine) == nan).all()
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    assert (mine[~nan] == ref[~nan]).all()
    assert float(F.e4m3fn_value(0x7E)) == 448.0
    assert float(F.e4m3fn_value(0x01)) == 2.0 ** -9


def test_e4m3_x512_is_integer_and_monotonic():
    v = F.E4M3_X512
    assert len(v) == 127 and v[0] == 0 and v[1] == 1 and v[-1] == 448 * 512
    assert (np.diff(v) > 0).all()


def test_bf16_rne_matches_torch_on_float32_inputs():
    rng = np.random.default_rng(1)
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32),
        (rng.standard_normal(2000) * 1e-39).astype(np.float32),     # float32 subnormals
        (rng.standard_normal(2000) * 1e30).astype(np.float32),
        np.array([0.0, -0.0, 1.0, -1.0, 3.0e38], dtype=np.float32),
    ])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().astype(np.uint16)
    mine = F.bf16_rne_bits(x.astype(np.float64))
    assert (mine == ref).all()


def test_bf16_ties_and_no_double_rounding():
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7 -> even (1.0)
    assert F.bf16_rne_bits(1.0 + 2.0 ** -8) == 0x3F80
    # 1 + 3*2^-8 is a tie between 1+2^-7 and 1+2^-6 -> even (1 + 2^-6)
    assert F.bf16_rne_bits(1.0 + 3 * 2.0 ** -8) == 0x3F82
    # just above the tie: float64 keeps the extra bit, a float32 detour would drop it
    x = 1.0 + 2.0 ** -8 + 2.0 ** -30
    assert float(np.float32(x)) == 1.0 + 2.0 ** -8
    assert F.bf16_rne_bits(x) == 0x3F81
    # signed zero and bf16 subnormals
    assert F.bf16_rne_bits(-0.0) == 0x8000
    assert F.bf16_rne_bits(2.0 ** -133) == 0x0001
    assert F.bf16_rne_bits(-(2.0 ** -135)) == 0x8000
    assert F.bf16_bits_to_f64(0x3F81) == 1.0 + 2.0 ** -7


def test_nvfp4_decode_hand_example():
    # one row, K = 32: codes 0..15 then 15..0; scales 1.0 (0x38) and 0.375 (0x1C... e=3,m=4 -> 1.5*2^-4)
    nibbles = list(range(16)) + list(range(15, -1, -1))
    packed = np.array([[nibbles[2 * i] | (nibbles[2 * i + 1] << 4) for i in range(16)]], dtype=np.uint8)
    scales = np.array([[0x38, 0x1C]], dtype=np.uint8)
    x = F.nvfp4_decode(packed, scales, 0.5)
    mags = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    s1 = 1.5 * 2.0 ** -4
    for k in range(32):
        c = nibbles[k]
        v = mags[c & 7] * (-1 if c & 8 else 1) * (1.0 if k < 16 else s1) * 0.5
        assert x[0, k] == v
    # a zero block scale gives zeros
    assert (F.nvfp4_decode(packed, np.zeros((1, 2), np.uint8), 3.0) == 0).all()


def test_unpack_nibbles_order():
    packed = np.array([[0x21, 0x43]], dtype=np.uint8)
    assert F.unpack_nibbles(packed).tolist() == [[1, 2, 3, 4]]
