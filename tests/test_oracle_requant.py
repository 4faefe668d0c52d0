"""Pins for the oracle's NVFP4 -> 2-bit requantisation and FP4 delta (CPU only).

The reference point is brute force in exact rational arithmetic on the
dequantised float64 values (fractions.Fraction), enumerating every finite
e4m3 block scale and every codebook level per element, plus invariants that
hold for any correct implementation.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import formats as F
from oracle import requant as R
from oracle import layout as L

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _random_nvfp4(rng, N, K, zero_frac=0.1, scale_lo=0x20, scale_hi=0x50):
    nib = rng.integers(0, 16, size=(N, K))
    mask = rng.random((N, K)) < zero_frac
    nib[mask] = rng.choice([0, 8], size=int(mask.sum()))
    packed = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    scales = rng.integers(scale_lo, scale_hi, size=(N, K // 16)).astype(np.uint8)
    return packed, scales


def _exact_block_search(vals, sign_bits, scale2_out):
    """Brute force: returns (set of minimising scale codes, per-code total error list)."""
    grid = [Fraction(float(F.e4m3fn_value(t))) for t in range(127)]
    levels = [Fraction(1), Fraction(4), Fraction(-1), Fraction(-4)]
    s2 = Fraction(float(scale2_out))
    errs = []
    for t in range(127):
        tot = Fraction(0)
        for v in vals:
            tot += min((v - lv * grid[t] * s2) ** 2 for lv in levels)
        errs.append(tot)
    best = min(errs)
    return [t for t in range(127) if errs[t] == best], errs


def _check_block(codes_row, scales_row, scale_2, k0, B, codes2, tau, s2out):
    vals_f = F.nvfp4_decode(codes_row[None, :], scales_row[None, :], scale_2)[0, k0:k0 + B]
    vals = [Fraction(float(v)) for v in vals_f]
    nib = F.unpack_nibbles(codes_row[None, :])[0, k0:k0 + B]
    argmins, errs = _exact_block_search(vals, nib >> 3, s2out)
    t = int(tau)
    assert t == min(argmins), (t, argmins)
    a = Fraction(float(F.e4m3fn_value(t))) * Fraction(float(s2out))
    levels = [Fraction(1), Fraction(4), Fraction(-1), Fraction(-4)]
    for i, v in enumerate(vals):
        c = int(codes2[i])
        e = [(v - lv * a) ** 2 for lv in levels]
        assert e[c] == min(e), (i, v, c)
        if v == 0:
            # zero: magnitude 1, sign from the NVFP4 sign bit (also for -0)
            assert c & 1 == 0 and (c >> 1) == (nib[i] >> 3)
        else:
            # equal-error choices only arise between magnitudes 1 and 4: magnitude 1 wins
            tied = [cc for cc in range(4) if e[cc] == e[c]]
            if len(tied) > 1:
                assert c & 1 == 0
            if a > 0:
                assert (c >> 1) == (1 if v < 0 else 0)
    return errs[t]


def test_codebook_golden():
    g = json.load(open(os.path.join(GOLDEN, "codebook.json")))
    assert sorted(R.LEVELS.tolist()) == sorted(float(x) for x in g["levels"])


def test_bruteforce_tiny_blocks_joint_enumeration():
    """Blocks of B = 4 elements: enumerate every scale code and every code vector jointly
    (127 * 4^4) in exact rationals and compare the minimum with the oracle's choice."""
    import itertools
    B = 4
    rng = np.random.default_rng(104)
    codes, scales = _random_nvfp4(rng, 1, 16)
    scale_2 = 0.0371
    c2, tau, s2 = R.requant(codes, scales, scale_2, block=B)
    levels = [1, 4, -1, -4]
    vals = F.nvfp4_decode(codes, scales, scale_2)
    for b in range(16 // B):
        v = [Fraction(float(x)) for x in vals[0, b * B:(b + 1) * B]]
        best = None
        for t in range(127):
            a = Fraction(float(F.e4m3fn_value(t))) * Fraction(float(s2))
            for cv in itertools.product(range(4), repeat=B):
                e = sum((v[i] - levels[cv[i]] * a) ** 2 for i in range(B))
                if best is None or e < best[0]:
                    best = (e, t)
        got_t = int(tau[0, b])
        got_a = Fraction(float(F.e4m3fn_value(got_t))) * Fraction(float(s2))
        got_e = sum((v[i] - levels[c2[0, b * B + i]] * got_a) ** 2 for i in range(B))
        assert got_e == best[0]
        assert got_t == best[1]          # first minimiser in increasing scale order


def test_bruteforce_full_blocks_exact():
    rng = np.random.default_rng(7)
    codes, scales = _random_nvfp4(rng, 3, 64)
    scale_2 = 1.0 / 3.0
    c2, tau, s2, err = R.requant(codes, scales, scale_2, return_err=True)
    assert s2 == np.float32(2.0) * np.float32(scale_2)
    for n in range(3):
        for b in range(2):
            e = _check_block(codes[n], scales[n], scale_2, 32 * b, 32, c2[n, 32 * b:32 * b + 32],
                             tau[n, b], s2)
            # the oracle's integer error is the same quantity in units of (2^-10 * scale_2)^2
            u = Fraction(float(np.float32(scale_2))) / 1024
            assert Fraction(int(err[n, b])) * u * u == e


def test_representable_block_returns_itself():
    # scale 1.0 (0x38) on both halves; e2m1 0.5 and 2.0 give |Y| in {a, 4a} with
    # a on the grid at e4m3 0.25 (0x28) for scale2_out = 2*scale_2
    rng = np.random.default_rng(3)
    mags = rng.choice([1, 4], size=32)            # e2m1 codes: 1 -> 0.5, 4 -> 2.0
    signs = rng.integers(0, 2, size=32)
    nib = mags | (signs << 3)
    packed = (nib[0::2] | (nib[1::2] << 4)).astype(np.uint8)[None, :]
    scales = np.array([[0x38, 0x38]], dtype=np.uint8)
    c2, tau, s2, err = R.requant(packed, scales, 0.75, return_err=True)
    assert tau[0, 0] == 0x28 and err[0, 0] == 0
    assert ((c2[0] & 1) == (mags == 4)).all() and ((c2[0] >> 1) == signs).all()
    w2 = R.dequant_2bit(c2, tau, s2)
    assert (w2 == F.nvfp4_decode(packed, scales, 0.75)).all()
    # and the delta of a representable block is exactly zero with a zero scale and +0 codes
    dc, ds, d2 = R.delta(packed, scales, 0.75, c2, tau)
    assert (dc == 0).all() and (ds == 0).all()


def test_all_zero_block_and_zero_signs():
    nib = np.array([0] * 16 + [8] * 16)              # +0 then -0
    packed = (nib[0::2] | (nib[1::2] << 4)).astype(np.uint8)[None, :]
    scales = np.array([[0x40, 0x40]], dtype=np.uint8)
    c2, tau, s2 = R.requant(packed, scales, 1.0)
    assert tau[0, 0] == 0
    assert (c2[0, :16] == 0).all() and (c2[0, 16:] == 2).all()   # +1 / -1 by the sign bit


def test_zero_sign_rule_in_a_live_block():
    rng = np.random.default_rng(11)
    codes, scales = _random_nvfp4(rng, 4, 128, zero_frac=0.3)
    c2, tau, s2 = R.requant(codes, scales, 0.01)
    nib = F.unpack_nibbles(codes)
    z = (nib & 7) == 0
    assert z.any()
    assert ((c2[z] & 1) == 0).all()
    assert ((c2[z] >> 1) == (nib[z] >> 3)).all()


def test_element_tie_goes_to_magnitude_one():
    # a block found by random search in which element 7 lies exactly at 2.5a for
    # the chosen scale (both magnitudes give the same error; magnitude 1 must win)
    packed = np.array([[1, 211, 53, 64, 233, 62, 169, 1, 152, 194, 144, 245, 148, 96, 74, 174]],
                      dtype=np.uint8)
    scales = np.array([[66, 64]], dtype=np.uint8)
    c2, tau, s2 = R.requant(packed, scales, 1.0)
    _check_block(packed[0], scales[0], 1.0, 0, 32, c2[0], tau[0, 0], s2)
    a = F.e4m3fn_value(tau[0, 0]) * float(s2)
    y = abs(F.nvfp4_decode(packed, scales, 1.0)[0, 7])
    assert 2 * y == 5 * a
    assert c2[0, 7] & 1 == 0


def test_sign_flip_and_power_of_two_invariance():
    rng = np.random.default_rng(5)
    codes, scales = _random_nvfp4(rng, 8, 256)
    c2, tau, s2 = R.requant(codes, scales, 0.02)
    flipped = codes ^ 0x88
    c2f, tauf, s2f = R.requant(flipped, scales, 0.02)
    assert (tauf == tau).all() and ((c2f ^ 2) == c2).all()
    for j in (-3, 5):
        c2j, tauj, s2j = R.requant(codes, scales, 0.02 * 2.0 ** j)
        assert (c2j == c2).all() and (tauj == tau).all()
        assert s2j == np.float32(s2 * np.float32(2.0 ** j))


def test_largest_nvfp4_block_stays_in_range():
    nib = np.full(32, 7)                               # e2m1 6.0
    packed = (nib[0::2] | (nib[1::2] << 4)).astype(np.uint8)[None, :]
    scales = np.array([[0x7E, 0x7E]], dtype=np.uint8)  # 448
    c2, tau, s2 = R.requant(packed, scales, 1.0)
    w2 = R.dequant_2bit(c2, tau, s2)
    assert tau[0, 0] <= 0x7E
    assert np.allclose(w2, 6 * 448, rtol=0.1)


def test_requant_improves_on_absmax_scale():
    """On synthetic N(0, 0.02) NVFP4 the L2-optimal block scale beats the plain
    absmax/4 scale (sanity of the objective, not a tight pin)."""
    import torch
    from bit_moe_expert_nvfp4_amd import synth
    c, s, s2 = synth.make_nvfp4_stack(1, 64, 512, seed=1, tag="req")
    c, s, s2 = c[0].numpy(), s[0].numpy(), float(s2[0])
    x = F.nvfp4_decode(c, s, s2)
    c2, tau, s2o = R.requant(c, s, s2)
    w = R.dequant_2bit(c2, tau, s2o)
    rel = np.linalg.norm(w - x) / np.linalg.norm(x)
    blk = np.abs(x).reshape(64, -1, 32).max(-1, keepdims=True) / 4
    q = np.sign(x).reshape(64, -1, 32) * np.where(np.abs(x).reshape(64, -1, 32) > 2.5 * blk, 4 * blk, blk)
    rel_absmax = np.linalg.norm(q.reshape(64, -1) - x) / np.linalg.norm(x)
    assert rel < rel_absmax
    assert 0.2 < rel < 0.45


def _fp4_nearest_bruteforce(v, S):
    """nearest e2m1 code for value v at block scale S (exact), ties to the even code."""
    cands = []
    for c in range(16):
        val = Fraction(float(F.e2m1_value(c))) * S
        cands.append((abs(v - val), c))
    best = min(d for d, _ in cands)
    return [c for d, c in cands if d == best]


def test_delta_bruteforce_and_bound():
    rng = np.random.default_rng(21)
    codes, scales = _random_nvfp4(rng, 2, 128)
    scale_2 = 0.125
    c2, tau, s2 = R.requant(codes, scales, scale_2)
    dc, ds, d2 = R.delta(codes, scales, scale_2, c2, tau)
    assert d2 == np.float32(scale_2)
    wn = F.nvfp4_decode(codes, scales, scale_2)
    w2 = R.dequant_2bit(c2, tau, s2)
    dq = R.dequant_fp4_codes(dc, ds, d2)
    grid = [Fraction(float(F.e4m3fn_value(t))) for t in range(127)]
    for n in range(2):
        for g in range(128 // 16):
            sl = slice(16 * g, 16 * g + 16)
            D = [Fraction(float(a)) - Fraction(float(b)) for a, b in zip(wn[n, sl], w2[n, sl])]
            target = max(abs(d) for d in D) / (6 * Fraction(float(d2)))
            dist = [abs(target - x) for x in grid]
            best = min(dist)
            tied = [t for t in range(127) if dist[t] == best]
            want_t = tied[0] if len(tied) == 1 else [t for t in tied if t % 2 == 0][0]
            assert ds[n, g] == want_t
            S = grid[want_t] * Fraction(float(d2))
            for i, d in enumerate(D):
                c = int(dc[n, 16 * g + i])
                if S == 0 or d == 0:
                    assert c == 0
                    continue
                ok = _fp4_nearest_bruteforce(d, S)
                if len(ok) > 1:
                    ok = [x for x in ok if (x & 1) == 0 and (x >> 3) == (1 if d < 0 else 0)] or ok
                assert (c & 7) in [x & 7 for x in ok]
                assert (c >> 3) == (1 if d < 0 else 0)       # rounding to zero keeps D's sign
            # elementwise bound: |W_2bit + Q(D) - W_nvfp4| <= half the local e2m1 gap * S
            for i, d in enumerate(D):
                q = Fraction(float(dq[n, 16 * g + i]))
                mag = abs(d) / S if S else 0
                if S and mag <= 6:
                    gap = Fraction(1, 2) if mag <= 2 else (Fraction(1) if mag <= 4 else Fraction(2))
                    assert abs(q - d) <= gap / 2 * S


def test_delta_reconstruction_closer_than_2bit():
    rng = np.random.default_rng(8)
    codes, scales = _random_nvfp4(rng, 64, 256)
    c2, tau, s2 = R.requant(codes, scales, 0.05)
    dc, ds, d2 = R.delta(codes, scales, 0.05, c2, tau)
    wn = F.nvfp4_decode(codes, scales, 0.05)
    w2 = R.dequant_2bit(c2, tau, s2)
    wd = w2 + R.dequant_fp4_codes(dc, ds, d2)
    assert np.linalg.norm(wd - wn) < 0.2 * np.linalg.norm(w2 - wn)


def test_layout_roundtrip_and_density():
    rng = np.random.default_rng(9)
    N, K = 128, 256
    c2 = rng.integers(0, 4, size=(N, K)).astype(np.uint8)
    tau = rng.integers(0, 127, size=(N, K // 32)).astype(np.uint8)
    words = L.pack_2bit_codes(c2)
    sc = L.pack_2bit_scales(tau)
    assert words.dtype == np.uint32 and words.size == N * K // 16
    assert (L.unpack_2bit_codes(words, N, K) == c2).all()
    assert (L.unpack_2bit_scales(sc, N, K) == tau).all()
    # 2.25 bits per weight: K/4 code bytes + K/32 scale bytes per row
    assert (words.nbytes + sc.nbytes) * 8 / (N * K) == 2.25
    dc = rng.integers(0, 16, size=(N, K)).astype(np.uint8)
    ds = rng.integers(0, 127, size=(N, K // 16)).astype(np.uint8)
    assert (L.unpack_fp4_codes(L.pack_fp4_codes(dc), N, K) == dc).all()
    assert (L.unpack_fp4_scales(L.pack_fp4_scales(ds), N, K) == ds).all()


def test_layout_bit_positions_hand_example():
    # nibble j of a word holds element j in bits 2..3 and element j + 8 in bits 0..1
    # (m in the lower bit of each pair).  A code 1 (m=1, s=0) at k=0 of row 0 sets
    # bit 2 of word 0; code 2 (s=1) at k=1 sets bit 7; code 3 at k=10 (nibble 2,
    # lower pair) sets bits 8 and 9; code 1 at k=15 sets bit 28.
    N, K = 64, 128
    c2 = np.zeros((N, K), dtype=np.uint8)
    c2[0, 0] = 1
    w = L.pack_2bit_codes(c2)
    assert w[0] == 1 << 2 and (w[1:] == 0).all()
    c2[0, 0] = 0
    c2[0, 1] = 2
    assert L.pack_2bit_codes(c2)[0] == 1 << 7
    c2[0, 1] = 0
    c2[0, 10] = 3
    assert L.pack_2bit_codes(c2)[0] == (1 << 8) | (1 << 9)
    c2[0, 10] = 0
    c2[0, 15] = 1
    assert L.pack_2bit_codes(c2)[0] == 1 << 28
    # k = 16 starts the next word of the same 64-k chunk
    c2[0, 15] = 0
    c2[0, 16] = 2
    w = L.pack_2bit_codes(c2)
    assert w[1] == 1 << 3 and np.count_nonzero(w) == 1
    # row 1, k = 64 lives in chunk 1: word index (1*64 + 1)*4
    c2[0, 16] = 0
    c2[1, 64] = 1
    w = L.pack_2bit_codes(c2)
    assert w[(1 * 64 + 1) * 4] == 1 << 2 and np.count_nonzero(w) == 1
