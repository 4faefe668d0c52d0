"""Pins for the oracle's other source formats and the zero-sign balancing (CPU only).

Reference points, none of them the oracle's own formula retyped:
  * exact rational arithmetic (fractions.Fraction) over every e4m3 block scale
    and every codebook level, on the dequantised float64 source values;
  * the e2m1 / e8m0 / e4m3 value tables, enumerated;
  * invariants any correct implementation keeps (power-of-two rescaling, sign
    flips, blocks that are already 2-bit, all-zero inputs);
  * the exact integer NVFP4 requant on tensors that both it and the FP8 path
    can hold.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

from bit_moe_expert_nvfp4_amd import synth
from oracle import formats as F
from oracle import requant as R
from oracle import sources as S

LEVELS = [Fraction(1), Fraction(4), Fraction(-1), Fraction(-4)]


def _pack(nib):
    nib = np.asarray(nib, dtype=np.int64)
    return (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)


# ---------------------------------------------------------------------------
# zero-sign balancing (NVFP4 requant)
# ---------------------------------------------------------------------------

def test_balance_hand_block():
    """A block whose zeros (all +0) sit at k = 0, 3, 7, 20: balanced signs +, -, +, -."""
    nib = np.full((64, 128), 2, dtype=np.int64)          # every weight 1.0 ...
    nib[0, [0, 3, 7, 20]] = 0                              # ... but four +0
    nib[0, 5] = 8 | 2                                      # one -1.0
    packed = _pack(nib)
    scales = np.full((64, 8), 0x38, dtype=np.uint8)        # e4m3 1.0
    c_keep, t_keep, _ = R.requant(packed, scales, 1.0)
    c_bal, t_bal, _ = R.requant(packed, scales, 1.0, balance_zero_signs=True)
    assert (t_keep == t_bal).all()
    assert [int(c_keep[0, k]) >> 1 for k in (0, 3, 7, 20)] == [0, 0, 0, 0]
    assert [int(c_bal[0, k]) >> 1 for k in (0, 3, 7, 20)] == [0, 1, 0, 1]
    nz = nib[0] & 7 != 0
    assert (c_keep[0, nz] == c_bal[0, nz]).all()
    assert int(c_bal[0, 5]) >> 1 == 1                      # a real sign stays


def test_balance_all_plus_zero_export_removes_the_bias():
    """An export that writes zeros as +0 puts every zero at +a (a bias of one level per
    zero); balancing leaves at most one unpaired +a per block and changes nothing else."""
    W = torch.randn((128, 512), generator=synth._gen("cpu", 3, "bal"), dtype=torch.float32) * 0.02
    W[torch.rand(W.shape, generator=synth._gen("cpu", 4, "bal")) < 0.2] = 0.0
    codes, scales, s2 = synth.nvfp4_export(W, plus_zeros=True)
    codes, scales = codes.numpy(), scales.numpy()
    nib = F.unpack_nibbles(codes)
    zero = (nib & 7) == 0
    assert zero.sum() > 1000 and not (nib[zero] & 8).any()
    c_keep, t_keep, s2o = R.requant(codes, scales, float(s2))
    c_bal, t_bal, _ = R.requant(codes, scales, float(s2), balance_zero_signs=True)
    assert (t_keep == t_bal).all()
    assert (c_keep[~zero] == c_bal[~zero]).all()
    w_keep = R.dequant_2bit(c_keep, t_keep, s2o)
    w_bal = R.dequant_2bit(c_bal, t_bal, s2o)
    a = np.repeat(F.e4m3fn_value(t_keep), 32, axis=1) * np.float64(s2o)
    live = zero & (a > 0)
    assert np.allclose(w_keep[live] / a[live], 1.0)        # unbalanced: every zero at +a
    per_block = np.where(zero, w_bal / np.where(a > 0, a, 1.0), 0.0).reshape(128, 16, 32).sum(axis=2)
    nzeros = zero.reshape(128, 16, 32).sum(axis=2)
    assert (np.abs(per_block - (nzeros % 2)) < 1e-12)[t_keep.reshape(128, 16) > 0].all()


def test_balance_ignores_source_sign_of_zeros():
    rng = np.random.default_rng(5)
    nib = rng.integers(0, 16, size=(64, 256))
    nib[rng.random(nib.shape) < 0.3] = 0
    flipped = nib.copy()
    z = (nib & 7) == 0
    flipped[z] = np.where(rng.random(int(z.sum())) < 0.5, 8, 0)
    scales = rng.integers(0x20, 0x50, size=(64, 16)).astype(np.uint8)
    a = R.requant(_pack(nib), scales, 0.5, balance_zero_signs=True)
    b = R.requant(_pack(flipped), scales, 0.5, balance_zero_signs=True)
    assert (a[0] == b[0]).all() and (a[1] == b[1]).all()


# ---------------------------------------------------------------------------
# MXFP4 codes remap
# ---------------------------------------------------------------------------

def test_e8m0_values():
    assert S.e8m0_value(127) == 1.0 and S.e8m0_value(0) == 2.0 ** -127 and S.e8m0_value(254) == 2.0 ** 127
    assert np.isnan(S.e8m0_value(255))


def test_remap_code_table_all_sixteen_codes():
    """Every e2m1 code goes to the nearest of -4, -1, 1, 4 (in block-scale units)."""
    nib = np.tile(np.arange(16), 8)[None, :].repeat(64, axis=0)
    scales = np.full((64, 4), 127, dtype=np.uint8)
    c2, tau, s2 = S.remap_mxfp4(_pack(nib), scales)
    for code in range(16):
        v = Fraction(float(F.e2m1_value(code)))
        errs = [(v - lv) ** 2 for lv in LEVELS]
        got = int(c2[0, code])
        assert errs[got] == min(errs), (code, got)
        assert got >> 1 == code >> 3                      # sign from the code, zeros too
    assert s2 == np.float32(2.0 ** -8) and (tau == 0x78).all()


def test_remap_scales_carry_over_exactly():
    rng = np.random.default_rng(7)
    nib = rng.integers(0, 16, size=(64, 256))
    E = rng.integers(110, 131, size=(64, 8)).astype(np.uint8)
    E[0, 0] = 140
    c2, tau, s2 = S.remap_mxfp4(_pack(nib), E)
    emax = 140
    assert s2 == np.float32(2.0 ** (emax - 8 - 127))
    x = S.mxfp4_decode(_pack(nib), E)
    w2 = R.dequant_2bit(c2, tau, s2)
    blk_scale = F.e4m3fn_value(tau) * np.float64(s2)
    live = (E.astype(np.int64) >= emax - 17)
    assert (blk_scale[live] == np.exp2(E[live].astype(np.float64) - 127)).all()
    assert (tau[~live] == 0).all() and (~live).any()
    # every element of a carried block is the nearest codebook value to the source value
    xs = x.reshape(64, 8, 32)[live]
    ws = w2.reshape(64, 8, 32)[live]
    bs = np.exp2(E[live].astype(np.float64) - 127)[:, None]
    cand = np.stack([lv * bs for lv in (1.0, 4.0, -1.0, -4.0)], axis=-1)
    d = (xs[..., None] - cand) ** 2
    assert (np.take_along_axis(d, np.argmin(np.abs(ws[..., None] - cand), axis=-1)[..., None], -1)[..., 0]
            == d.min(axis=-1)).all()


def test_remap_flush_edge_and_zero_blocks():
    nib = np.full((64, 128), 3, dtype=np.int64)           # 1.5 everywhere
    nib[1, 32:64] = 0                                     # row 1 block 1: no non-zero code
    E = np.full((64, 4), 100, dtype=np.uint8)
    E[0, 0] = 150                                         # Emax
    E[0, 1] = 150 - 17                                    # lowest carried exponent: e4m3 2^-9
    E[0, 2] = 150 - 18                                    # flushed
    E[1, 1] = 200                                         # ignored: that block holds only zeros
    c2, tau, s2 = S.remap_mxfp4(_pack(nib), E)
    assert s2 == np.float32(2.0 ** (150 - 8 - 127))
    assert tau[0, 0] == 0x78 and tau[0, 1] == 0x01 and tau[0, 2] == 0 and tau[1, 1] == 0
    z = np.zeros((64, 64), dtype=np.uint8)
    c2, tau, s2 = S.remap_mxfp4(z, np.full((64, 4), 127, dtype=np.uint8))
    assert s2 == 1.0 and (tau == 0).all()
    with pytest.raises(ValueError):
        S.remap_mxfp4(z, np.full((64, 4), 255, dtype=np.uint8))


def test_remap_exponent_shift_and_sign_flip():
    codes, E = synth.mxfp4_export(torch.randn((64, 256), generator=synth._gen("cpu", 9, "mx")) * 0.02)
    codes, E = codes.numpy(), E.numpy()
    c2, tau, s2 = S.remap_mxfp4(codes, E)
    c2j, tauj, s2j = S.remap_mxfp4(codes, E + np.uint8(5))
    assert (c2 == c2j).all() and (tau == tauj).all() and s2j == s2 * np.float32(32.0)
    c2f, tauf, _ = S.remap_mxfp4(codes ^ np.uint8(0x88), E)
    assert (c2f == (c2 ^ 2)).all() and (tauf == tau).all()


# ---------------------------------------------------------------------------
# FP8 block-quant requant
# ---------------------------------------------------------------------------

def _fp8_codes_of(values):
    """e4m3fn codes of values that are exactly representable (checked)."""
    t = torch.tensor(np.asarray(values, dtype=np.float32)).to(torch.float8_e4m3fn)
    back = t.to(torch.float32).numpy()
    assert (back == np.asarray(values, dtype=np.float32)).all()
    return t.view(torch.uint8).numpy()


def test_fp8_tensor_scale_rule():
    rng = np.random.default_rng(11)
    w = rng.integers(0, 0x7F, size=(128, 256)).astype(np.uint8)
    bs = rng.uniform(0.001, 0.01, size=(1, 2)).astype(np.float32)
    _, _, s2 = S.requant_fp8(w, bs)
    amax = np.abs(S.fp8_block_decode(w, bs)).max()
    assert np.log2(s2) == int(np.log2(s2))
    assert 1792.0 * float(s2) >= amax > 896.0 * float(s2)
    z = np.zeros((64, 128), dtype=np.uint8)
    c2, tau, s2 = S.requant_fp8(z, np.ones((1, 1), np.float32))
    assert s2 == 1.0 and (tau == 0).all()


def test_fp8_block_search_against_exact_rationals():
    """Tiny blocks (B = 4): the chosen scale reaches the exact minimum of the L2 error
    over every e4m3 scale and every codebook level per element (brute force in
    Fraction arithmetic), and each element takes its nearest level."""
    rng = np.random.default_rng(13)
    w = rng.integers(0, 0x7F, size=(2, 128)).astype(np.uint8) | (rng.integers(0, 2, size=(2, 128)) << 7).astype(np.uint8)
    w[0, :4] = 0                                           # an all-zero block
    bs = np.array([[0.0123]], dtype=np.float32)
    c2, tau, s2 = S.requant_fp8(w, bs, block=4)
    x = S.fp8_block_decode(w, bs)
    grid = [Fraction(float(F.e4m3fn_value(t))) * Fraction(float(s2)) for t in range(127)]
    for n in range(2):
        for b in range(32):
            vals = [Fraction(float(v)) for v in x[n, 4 * b:4 * b + 4]]
            errs = [sum(min((v - lv * a) ** 2 for lv in LEVELS) for v in vals) for a in grid]
            best = min(errs)
            t = int(tau[n, b])
            assert errs[t] == best or float(errs[t] - best) <= 1e-15 * float(best), (n, b, t)
            assert t == min(i for i in range(127) if errs[i] == errs[t])
            a = grid[t]
            for i, v in enumerate(vals):
                e = [(v - lv * a) ** 2 for lv in LEVELS]
                assert e[int(c2[n, 4 * b + i])] == min(e)
    assert tau[0, 0] == 0


def test_fp8_block_already_two_bit_returns_itself():
    S2 = 0.25                                             # set by the 448 below: 1792 * 0.25 = 448
    w = np.zeros((64, 128), dtype=np.uint8)
    vals = np.array([0.125, -0.5, 0.5, -0.125] * 8, dtype=np.float32)
    w[0, :32] = _fp8_codes_of(vals)
    w[1, 0] = _fp8_codes_of([448.0])[0]
    c2, tau, s2 = S.requant_fp8(w, np.ones((1, 1), np.float32))
    assert s2 == np.float32(S2)
    assert float(F.e4m3fn_value(tau[0, 0])) * S2 == 0.125
    assert (R.dequant_2bit(c2, tau, s2)[0, :32] == vals).all()


def test_fp8_scale_rescale_and_sign_flip():
    w, bs = synth.fp8_block_export(torch.randn((192, 256), generator=synth._gen("cpu", 2, "fp8")) * 0.02)
    w, bs = w.numpy(), bs.numpy()
    c2, tau, s2 = S.requant_fp8(w, bs)
    c2j, tauj, s2j = S.requant_fp8(w, bs * np.float32(8.0))
    assert (c2 == c2j).all() and (tau == tauj).all() and s2j == s2 * np.float32(8.0)
    c2f, tauf, _ = S.requant_fp8(w ^ np.uint8(0x80), bs)
    assert (c2f == (c2 ^ 2)).all() and (tauf == tau).all()
    with pytest.raises(ValueError):
        S.requant_fp8(np.full((64, 128), 0x7F, np.uint8), np.ones((1, 1), np.float32))
    with pytest.raises(ValueError):
        S.requant_fp8(w, -bs)


def test_fp8_agrees_with_exact_integer_nvfp4_requant():
    """NVFP4 tensors with power-of-two block scales and scale_2 are also FP8 block-quant
    tensors (e2m1 times a power of two is an e4m3 value).  Both paths must give the
    same dequantised 2-bit weights: the NVFP4 one decides in exact integers."""
    rng = np.random.default_rng(17)
    N, K = 128, 256
    nib = rng.integers(0, 16, size=(N, K))
    pow2 = rng.integers(5, 10, size=(N, K // 16))          # e4m3 2^(e-7), mantissa 0
    scales = (pow2 << 3).astype(np.uint8)
    scale_2 = 2.0 ** -4
    x = F.nvfp4_decode(_pack(nib), scales, scale_2)
    fp8 = _fp8_codes_of(x / 2.0 ** -4)                     # block scale 2^-4 everywhere
    c2n, tn, s2n = R.requant(_pack(nib), scales, scale_2)
    c2f, tf, s2f = S.requant_fp8(fp8, np.full((1, 2), 2.0 ** -4, np.float32))
    wn = R.dequant_2bit(c2n, tn, s2n)
    wf = R.dequant_2bit(c2f, tf, s2f)
    assert (wn == wf).all()
