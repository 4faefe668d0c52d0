"""Pins for the oracle's per-tensor codebook pick (CPU only).

Reading (README "Frontier MoE on consumer Blackwell (SM120)", section "How
it fits - 2-bit experts at FP4 quality": a per-tensor pick in which nearly
every tensor picks the sign-symmetric {-4,-1,1,4}): a tensor picks, by the
smallest exact total L2 error (ties to the lower index), one of three
sign-symmetric four-level codebooks with FP4 levels: 0: {1, 4}, 1: {1/2, 3},
2: {0, 2} (magnitudes times the block scale), with tensor scales 2, 2 and 4
times the source scale_2.

Reference points: joint brute force over every block scale code and every
code vector in exact rationals, for every codebook; the pick re-derived from
brute-force block minima; tensors that one codebook represents exactly pick
it with zero error; sign-flip and power-of-two invariances; the all-zero tie;
synthetic N(0, 0.02) tensors pick {-4,-1,1,4}.
"""
import itertools
from fractions import Fraction

import numpy as np
import pytest

from oracle import formats as F
from oracle import requant as R

LEVELS = [[Fraction(1), Fraction(4), Fraction(-1), Fraction(-4)],
          [Fraction(1, 2), Fraction(3), Fraction(-1, 2), Fraction(-3)],
          [Fraction(0), Fraction(2), Fraction(0), Fraction(-2)]]
SCALE2 = [2, 2, 4]
GRID = [Fraction(float(F.e4m3fn_value(t))) for t in range(127)]


def _random_nvfp4(rng, N, K, scale_lo=0x28, scale_hi=0x48):
    nib = rng.integers(0, 16, size=(N, K))
    packed = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    scales = rng.integers(scale_lo, scale_hi, size=(N, K // 16)).astype(np.uint8)
    return packed, scales


def _brute_block(vals, cb, scale_2):
    """Joint enumeration of scale code x code vector for one block: (min error, smallest minimising
    scale code)."""
    s2 = Fraction(float(np.float32(SCALE2[cb]) * np.float32(scale_2)))
    best = None
    for t in range(127):
        a = GRID[t] * s2
        for cv in itertools.product(range(4), repeat=len(vals)):
            e = sum((v - LEVELS[cb][c] * a) ** 2 for v, c in zip(vals, cv))
            if best is None or e < best[0]:
                best = (e, t)
    return best


@pytest.mark.parametrize("cb", [0, 1, 2])
def test_bruteforce_tiny_blocks_every_codebook(cb):
    """Blocks of 3 elements: every scale code x every code vector (127 * 4^3) in exact rationals;
    the oracle reaches the minimum error with the smallest minimising scale code, and its codes
    reproduce that error."""
    B = 3
    rng = np.random.default_rng(300 + cb)
    codes, scales = _random_nvfp4(rng, 1, 48)
    scale_2 = 0.0173
    c2, tau, s2, err = R.requant(codes, scales, scale_2, block=B, return_err=True, codebook=cb)
    assert s2 == np.float32(SCALE2[cb]) * np.float32(scale_2)
    vals = F.nvfp4_decode(codes, scales, scale_2)[0]
    for b in range(0, 48 // B, 4):      # every 4th block keeps the test quick
        v = [Fraction(float(x)) for x in vals[b * B:(b + 1) * B]]
        e_min, t_min = _brute_block(v, cb, scale_2)
        assert int(tau[0, b]) == t_min, (cb, b)
        a = GRID[int(tau[0, b])] * Fraction(float(s2))
        e_codes = sum((vv - LEVELS[cb][int(c)] * a) ** 2 for vv, c in zip(v, c2[0, b * B:(b + 1) * B]))
        assert e_codes == e_min
        # the integer error the oracle reports is the same quantity in units of 2^-10 scale_2
        unit = Fraction(float(np.float32(scale_2))) / 1024
        assert Fraction(int(err[0, b])) * unit * unit == e_min


def test_pick_equals_bruteforce_tensor_minimum():
    """The pick is the codebook with the smallest total of brute-force block minima (ties lower)."""
    B = 3
    rng = np.random.default_rng(311)
    for trial in range(6):
        codes, scales = _random_nvfp4(rng, 1, 48)
        scale_2 = float(rng.uniform(0.01, 0.05))
        vals = F.nvfp4_decode(codes, scales, scale_2)[0]
        totals = []
        for cb in range(3):
            tot = Fraction(0)
            for b in range(len(vals) // B):
                tot += _brute_block([Fraction(float(x)) for x in vals[b * B:(b + 1) * B]], cb, scale_2)[0]
            totals.append(tot)
        want = min(range(3), key=lambda c: (totals[c], c))
        got, _, _, _, tot_int = R.pick_codebook(codes, scales, scale_2, block=B)
        assert got == want, (trial, totals)
        unit = Fraction(float(np.float32(scale_2))) / 1024
        assert [Fraction(t) * unit * unit for t in tot_int] == totals


def _block_from_magnitudes(mags, signs, scale_code):
    """One NVFP4 row of 32 weights (two block-16 scales equal to scale_code) from e2m1 magnitude
    codes and sign bits."""
    nib = (np.asarray(mags) & 7) | (np.asarray(signs) << 3)
    packed = (nib[0::2] | (nib[1::2] << 4)).astype(np.uint8)[None, :]
    scales = np.full((1, 2), scale_code, dtype=np.uint8)
    return packed, scales


@pytest.mark.parametrize("cb,mag_codes", [
    (0, (2, 6)),     # e2m1 1 and 4
    (1, (1, 5)),     # e2m1 1/2 and 3
    (2, (0, 4)),     # e2m1 0 and 2
])
def test_tensor_on_a_codebook_picks_it_with_zero_error(cb, mag_codes):
    rng = np.random.default_rng(320 + cb)
    rows_c, rows_s = [], []
    for r in range(64):
        mags = rng.choice(mag_codes, size=32)
        signs = rng.integers(0, 2, size=32)
        c, s = _block_from_magnitudes(mags, signs, 0x38 + (r % 8))   # block-16 scales 1.0 .. 1.875
        rows_c.append(c)
        rows_s.append(s)
    codes, scales = np.concatenate(rows_c), np.concatenate(rows_s)
    scale_2 = 0.0625
    got, c2, tau, s2, totals = R.pick_codebook(codes, scales, scale_2)
    assert got == cb and totals[cb] == 0
    assert all(t > 0 for i, t in enumerate(totals) if i != cb)
    W = R.dequant_2bit(c2, tau, s2, codebook=cb)
    assert (W == F.nvfp4_decode(codes, scales, scale_2)).all()


def test_all_zero_tensor_ties_to_the_default():
    codes = np.zeros((64, 64), dtype=np.uint8)
    scales = np.full((64, 8), 0x38, dtype=np.uint8)
    got, _, tau, _, totals = R.pick_codebook(codes, scales, 0.5)
    assert got == 0 and totals == [0, 0, 0] and (tau == 0).all()


def test_pick_invariant_to_sign_flip_and_power_of_two_scale():
    rng = np.random.default_rng(330)
    codes, scales = _random_nvfp4(rng, 64, 128)
    cb, c2, tau, s2, tot = R.pick_codebook(codes, scales, 0.02)
    flipped = codes ^ 0x88
    cbf, c2f, tauf, s2f, totf = R.pick_codebook(flipped, scales, 0.02)
    assert cbf == cb and (tauf == tau).all() and totf == tot
    nz = F.nvfp4_decode(codes, scales, 0.02) != 0
    assert ((c2f ^ 2)[nz] == c2[nz]).all()
    cb4, c24, tau4, s24, tot4 = R.pick_codebook(codes, scales, 0.08)
    assert cb4 == cb and (c24 == c2).all() and (tau4 == tau).all() and s24 == 4 * s2


def test_delta_of_a_picked_codebook():
    """The FP4 delta of a tensor on codebook 1 or 2 restores it within the delta's rounding bound,
    and is zero where the 2-bit planes are exact."""
    rng = np.random.default_rng(340)
    codes, scales = _random_nvfp4(rng, 64, 128)
    Y = F.nvfp4_decode(codes, scales, 0.03)
    for cb in (1, 2):
        c2, tau, s2 = R.requant(codes, scales, 0.03, codebook=cb)
        dc, ds, d2 = R.delta(codes, scales, 0.03, c2, tau, codebook=cb)
        W = R.dequant_2bit(c2, tau, s2, codebook=cb)
        D = R.dequant_fp4_codes(dc, ds, d2)
        resid = np.abs(W + D - Y)
        # nearest e2m1: half the largest e2m1 gap (2) times the block-16 scale
        bound = np.repeat(F.e4m3fn_value(ds), 16, axis=1) * float(d2) * 1.0
        assert (resid <= bound + 1e-300).all()
    exact_c, exact_s = _block_from_magnitudes(rng.choice((1, 5), size=32), rng.integers(0, 2, size=32), 0x38)
    c2, tau, s2 = R.requant(exact_c, exact_s, 0.25, codebook=1)
    dc, ds, _ = R.delta(exact_c, exact_s, 0.25, c2, tau, codebook=1)
    assert (dc == 0).all() and (ds == 0).all()


def test_synthetic_tensors_pick_the_sign_symmetric_default():
    """N(0, 0.02) weights exported to NVFP4 pick {-4,-1,1,4}, with the other codebooks clearly worse
    (the page reports nearly every real tensor picks it)."""
    from bit_moe_expert_nvfp4_amd import synth
    st = synth.make_nvfp4_stack(6, 128, 512, 3, "pick")
    c, s, z = (t.numpy() for t in st)
    for m in range(6):
        cb, _, _, _, tot = R.pick_codebook(c[m], s[m], float(z[m]))
        assert cb == 0 and tot[1] > 1.05 * tot[0] and tot[2] > 1.3 * tot[0]
