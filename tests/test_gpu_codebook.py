"""GPU parity of the per-tensor codebook pick (moet_requant with MOET_PICK_CODEBOOK) and of the
forward over a layer whose matrices use different codebooks.

The pick (README "Frontier MoE on consumer Blackwell (SM120)", section "How it fits - 2-bit experts
at FP4 quality": a per-tensor pick, nearly always {-4,-1,1,4}) chooses among the three
sign-symmetric four-level codebooks of the 2-bit layout by the smallest exact total L2 error, ties to
the lower id.  Its id, codes, block scales, scale2 and FP4 delta are integer/byte results: they must
match the oracle bit for bit.  Synthetic N(0, 0.02) tensors all pick codebook 0, so the inputs here
move a fraction of each chosen matrix's e2m1 magnitudes onto two values (synth.skew_magnitudes),
which makes codebook 1 or 2 the better fit; every test asserts that the oracle's picks cover the
codebooks it is meant to exercise.  The forward is compared element by element with the oracle's
forward on the oracle's picks, as the other forward parity tests do.
"""
import zlib

import numpy as np
import pytest
import torch

from bit_moe_expert_nvfp4_amd import moet, synth
from moet_testlib import (C1_MAGS, C2_MAGS, OracleLayer, OracleMatrix, assert_elementwise, bf16_bits,
                          check_out_rows, check_pair_rows, mixed_codebook_layer, np_, oracle_route, rel_l2,
                          REL_L2_BAR, alarm_rel_l2)

pytestmark = pytest.mark.gpu
DEV = "cuda"



def _print_case(name):
    print(f"[case] {name}", flush=True)


def _u32(t):
    return np_(t).view(np.uint32)


def _check_planes(w, d, codes, scales, s2, sel, pick=True):
    """Every matrix's codebook id, codes, scales, scale2 (and the delta of the matrices in sel) against
    the oracle, bit for bit.  Returns the oracle's picks."""
    picks = []
    for m in range(codes.shape[0]):
        o = OracleMatrix(codes[m], scales[m], float(s2[m]), with_delta=m in sel, pick=pick)
        picks.append(o.cb)
        if pick:
            assert int(np_(w.codebook)[m]) == o.cb, f"codebook of matrix {m}: oracle totals {o.totals}"
        assert (_u32(w.codes[m]) == o.packed_codes()).all(), f"codes of matrix {m} (codebook {o.cb})"
        assert (np_(w.scales[m]) == o.packed_scales()).all(), f"scales of matrix {m} (codebook {o.cb})"
        assert np_(w.scale2)[m] == o.s2, f"scale2 of matrix {m}"
        if m in sel:
            slot = sel.index(m)
            pc, ps = o.packed_delta()
            assert (np_(d.codes[slot]) == pc).all(), f"delta codes of matrix {m} (codebook {o.cb})"
            assert (np_(d.scales[slot]) == ps).all(), f"delta scales of matrix {m}"
            assert np_(d.scale2)[slot] == np.float32(s2[m])
    return picks


def _skewed_stack(n, N, K, seed, c1, c2, frac1=0.9, frac2=0.95):
    c, s, z = synth.make_nvfp4_stack(n, N, K, seed, "codebook")
    c = synth.skew_magnitudes(c, c1, C1_MAGS, frac1, seed, "c1")
    c = synth.skew_magnitudes(c, c2, C2_MAGS, frac2, seed, "c2")
    return c, s, z


def test_pick_requant_and_delta_bitexact():
    """Seven matrices [128][512]: synthetic (codebook 0), skewed towards codebook 1 and 2, two near the
    0/1 boundary, exactly on codebook 1, all zero (a three-way tie -> 0); with the delta of five."""
    _print_case("codebook pick n=7 N=128 K=512")
    N, K = 128, 512
    c, s, z = _skewed_stack(7, N, K, 21, c1=[1], c2=[2])
    # near the codebook 0 / 1 boundary: totals of codebook 1 within 0.13 % of codebook 0's, either side
    c = synth.skew_magnitudes(c, [3], C1_MAGS, 0.75, 21, "near")
    c = synth.skew_magnitudes(c, [4], C1_MAGS, 0.76, 21, "near")
    c = synth.skew_magnitudes(c, [5], C1_MAGS, 1.0, 21, "exact")      # every weight on {1/2, 3}
    c[6] = 0
    codes, scales, s2 = np_(c), np_(s), np_(z)
    sel = [1, 2, 5, 6, 0]
    w, d = moet.requant(c.to(DEV), s.to(DEV), z.to(DEV), torch.tensor(sel, dtype=torch.int32, device=DEV),
                        pick_codebook=True)
    torch.cuda.synchronize()
    picks = _check_planes(w, d, codes, scales, s2, sel)
    print(f"picks={picks}", flush=True)
    assert picks[0] == 0 and picks[1] == 1 and picks[2] == 2 and picks[5] == 1 and picks[6] == 0
    assert picks[3] == 0 and picks[4] == 1, "the boundary pair should straddle the 0/1 boundary"


def test_without_pick_writes_codebook_zero():
    """flags without MOET_PICK_CODEBOOK and a w2_codebook array: every id 0, planes as codebook 0."""
    _print_case("requant without pick, codebook array given")
    N, K = 64, 256
    c, s, z = _skewed_stack(3, N, K, 22, c1=[1], c2=[2])
    cd, sd, zd = c.to(DEV), s.to(DEV), z.to(DEV)
    w = moet._new_w2(3, N, K, DEV)
    cb = torch.full((3,), 7, dtype=torch.uint8, device=DEV)
    rc = moet.lib().moet_requant(moet._ptr(cd), moet._ptr(sd), moet._ptr(zd), 3, N, K, moet._ptr(w.codes),
                                 moet._ptr(w.scales), moet._ptr(w.scale2), moet._ptr(cb), None, 0, None, None,
                                 None, 0, moet._stream())
    assert rc == 0, moet.lib().moet_last_error()
    torch.cuda.synchronize()
    assert (np_(cb) == 0).all()
    _check_planes(w, None, np_(c), np_(s), np_(z), [], pick=False)


def test_pick_full_size_matrices():
    """Gate/up-shaped matrices [2048][7168] (the benchmark's): synthetic, skewed to codebook 1, skewed
    to codebook 2 -- picks, codes, scales and scale2 over every element."""
    _print_case("codebook pick full size n=3 N=2048 K=7168")
    c, s, z = _skewed_stack(3, 2048, 7168, 23, c1=[1], c2=[2])
    w = moet.requant(c.to(DEV), s.to(DEV), z.to(DEV), pick_codebook=True)
    torch.cuda.synchronize()
    picks = _check_planes(w, None, np_(c), np_(s), np_(z), [])
    assert picks == [0, 1, 2]


# ---------------------------------------------------------------------------
# forward over a mixed-codebook layer
# ---------------------------------------------------------------------------
def _small_cfg(**kw):
    base = dict(name="mixed", T=4, H=256, I=128, E=8, k=2, score=synth.SIGMOID)
    base.update(kw)
    return synth.LayerConfig(**base)


@pytest.mark.parametrize("case", [
    # decode GEMV path (per-lane codebook of gate / up rows)
    dict(T=5, E=8, k=2, H=512, I=256, shared=True, n_resident=3, n_flagged=2),
    dict(T=3, E=8, k=4, H=7168, I=512, shared=True),
    # MFMA grouped GEMM: 2-bit tiles with the generic dequant, FP4 delta pass on compacted rows
    dict(T=300, E=16, k=8, H=512, I=256, shared=True, n_resident=6, n_flagged=120),
    dict(T=700, E=8, k=2, H=512, I=256, shared=True),
])
def test_forward_mixed_codebooks(case):
    cfg = _small_cfg(**case)
    _print_case(f"forward mixed codebooks {case}")
    seed = zlib.crc32(str(sorted(case.items())).encode()) & 0xFFFF
    src = mixed_codebook_layer(synth.make_layer(cfg, seed=seed), seed)
    soe = synth.slot_of_expert(cfg, seed) if cfg.n_resident else None
    layer = moet.layer_from_nvfp4(src, soe, swiglu_limit=cfg.swiglu_limit, pick_codebook=True)
    ol = OracleLayer(src, soe, pick_codebook=True)
    # the layer carries the oracle's picks, and the picks cover every codebook
    want13 = [ol._mat(src.w13, m, False).cb for m in range(2 * cfg.E)]
    want2 = [ol._mat(src.w2, m, False).cb for m in range(cfg.E)]
    assert list(np_(layer.w13.codebook)) == want13
    assert list(np_(layer.w2.codebook)) == want2
    assert set(want13) == {0, 1, 2} and set(want2) == {0, 1, 2}, (want13, want2)
    if cfg.shared:
        assert int(np_(layer.shared13.codebook)[0]) == ol._mat(src.shared13, 0, False).cb == 2
        assert int(np_(layer.shared2.codebook)[0]) == ol._mat(src.shared2, 0, False).cb == 1
    x = synth.make_activations(cfg.T, cfg.H, seed)
    lg = synth.make_logits(cfg, seed)
    flags = synth.gate_flags(cfg, seed) if cfg.n_flagged else None
    ids, w, offs, pairs = moet.route(lg.to(DEV), cfg.k, cfg.score, cfg.renormalize)
    ws = moet.alloc_workspace(layer, cfg.T, cfg.k, DEV)
    out = moet.moe_forward(layer, x.to(DEV), ids, w, offs, pairs, flags.to(DEV) if flags is not None else None,
                           workspace=ws)
    torch.cuda.synchronize()
    o_ids, o_w, _, o_pairs = oracle_route(lg, cfg.k, cfg.score, cfg.renormalize)
    assert (np_(ids) == o_ids).all()
    fl = np_(flags) if flags is not None else None
    ref = ol.forward(bf16_bits(x), o_ids, o_w, gate_flags=fl)
    got = bf16_bits(out)
    rows = check_pair_rows(ws, ol, bf16_bits(x), o_ids, o_pairs, cfg.H, cfg.I, gate_flags=fl)
    assert_elementwise(rows.h, rows.y, check_out_rows(got, ref, range(cfg.T), o_w, rows))
    err = rel_l2(got, ref)
    print(f"rel_l2={err:.3e}", flush=True)
    assert err <= REL_L2_BAR
    assert err <= alarm_rel_l2(cfg.H)


def test_pick_with_balanced_zero_signs():
    """Both load flags at once (MOET_PICK_CODEBOOK | MOET_BALANCE_ZERO_SIGNS) on a +0-only export
    (every zero written as +0), skewed so that each codebook is picked: ids, codes, scales and scale2
    equal the oracle's pick with balanced zeros."""
    from oracle import layout as OL
    from oracle import requant as OR
    _print_case("codebook pick + balanced zero signs n=4 N=128 K=256")
    c, s, z = synth.make_nvfp4_stack(4, 128, 256, 24, "balanced", plus_zeros=True)
    c = synth.skew_magnitudes(c, [1], C1_MAGS, 0.9, 24, "c1")
    c = synth.skew_magnitudes(c, [2, 3], C2_MAGS, 0.95, 24, "c2")
    w = moet.requant(c.to(DEV), s.to(DEV), z.to(DEV), balance_zero_signs=True, pick_codebook=True)
    torch.cuda.synchronize()
    picks = []
    for m in range(4):
        cb, c2, tau, s2, _ = OR.pick_codebook(np_(c)[m], np_(s)[m], float(z[m]), balance_zero_signs=True)
        picks.append(cb)
        assert int(np_(w.codebook)[m]) == cb
        assert (_u32(w.codes[m]) == OL.pack_2bit_codes(c2)).all(), f"codes of matrix {m}"
        assert (np_(w.scales[m]) == OL.pack_2bit_scales(tau)).all(), f"scales of matrix {m}"
        assert np_(w.scale2)[m] == s2
    assert set(picks) == {0, 1, 2}, picks
