"""GPU parity of the load-time conversions from the other checkpoint flavours
(MXFP4 codes remap, FP8 block-quant requant) and of the zero-sign balancing,
against the oracle: codes, block scales and tensor scales bit for bit, then a
layer forward on converted weights against the oracle forward of the same
dequantised weights.

Inputs span several 64-row tiles, a ragged last 128-row FP8 scale block
(N = 192), every e4m3 / e8m0 pattern class (flushed, subnormal and all-zero
blocks, -0 and +0 zeros) and both zero-sign modes.
"""
import numpy as np
import pytest
import torch

from bit_moe_expert_nvfp4_amd import moet, synth
from oracle import ffn as OFF
from oracle import layout as OL
from oracle import requant as OR
from oracle import sources as OS
from moet_testlib import REL_L2_BAR, bf16_bits, np_, oracle_route, rel_l2

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _print_case(name):
    print(f"[case] {name}", flush=True)


def _check_planes(w, m, c2, tau, s2, what):
    assert (np_(w.codes[m]).view(np.uint32) == OL.pack_2bit_codes(c2)).all(), f"{what}: codes of matrix {m}"
    assert (np_(w.scales[m]) == OL.pack_2bit_scales(tau)).all(), f"{what}: scales of matrix {m}"
    assert np_(w.scale2)[m] == np.float32(s2), f"{what}: scale2 of matrix {m}"


@pytest.mark.parametrize("balance", [False, True])
def test_requant_zero_sign_balance_bitexact(balance):
    _print_case(f"requant +0 export balance={balance} n=3 N=128 K=512")
    codes, scales, s2 = synth.make_nvfp4_stack(3, 128, 512, 21, "plus0", plus_zeros=True)
    codes, scales, s2 = np_(codes), np_(scales), np_(s2)
    codes[1, :, :40] &= 0x0F                        # sparse rows: many zeros per block
    sel = [1, 2]
    w, d = moet.requant(torch.from_numpy(codes).to(DEV), torch.from_numpy(scales).to(DEV),
                        torch.from_numpy(s2).to(DEV), torch.tensor(sel, dtype=torch.int32, device=DEV),
                        balance_zero_signs=balance)
    torch.cuda.synchronize()
    for m in range(3):
        c2, tau, so = OR.requant(codes[m], scales[m], float(s2[m]), balance_zero_signs=balance)
        _check_planes(w, m, c2, tau, so, "requant")
        if m in sel:
            dc, ds, _ = OR.delta(codes[m], scales[m], float(s2[m]), c2, tau)
            slot = sel.index(m)
            assert (np_(d.codes[slot]) == OL.pack_fp4_codes(dc)).all(), f"delta codes of matrix {m}"
            assert (np_(d.scales[slot]) == OL.pack_fp4_scales(ds)).all(), f"delta scales of matrix {m}"


def _mx_random(rng, n, N, K):
    codes = rng.integers(0, 256, size=(n, N, K // 2), dtype=np.uint8)
    E = rng.integers(100, 140, size=(n, N, K // 32), dtype=np.uint8)
    codes[:, ::5, :16] = 0                          # +0 blocks (no non-zero code)
    codes[:, 2::9, 16:32] = 0x88                    # -0 blocks
    codes[:, 1::3, 32:48] &= 0x99                   # mostly 0 / 0.5 / -0 codes
    E[:, 4::7, :] = 121                             # near the flush edge (Emax 150 below)
    E[:, 6::7, :] = 133
    E[0, 0, 0] = 150
    E[1, 3, 1] = 254                                # largest exponent
    E[1, 3, 2] = 0                                  # smallest: flushed
    E[2, :, :] = rng.integers(0, 9, size=(N, K // 32))   # tiny exponents: subnormal tensor scale
    E[2, 0, 0] = 8
    return codes, E


@pytest.mark.parametrize("balance", [False, True])
def test_remap_mxfp4_bitexact(balance):
    _print_case(f"remap mxfp4 balance={balance}")
    rng = np.random.default_rng(31)
    cases = [("random n=3 N=128 K=512", *_mx_random(rng, 3, 128, 512))]
    c, e = synth.make_mxfp4_stack(2, 192, 384, 7, "mx")
    cases.append(("synthetic n=2 N=192 K=384", np_(c), np_(e)))
    z = np.zeros((1, 64, 64), dtype=np.uint8)
    cases.append(("all zero N=64 K=128", z, np.full((1, 64, 4), 127, dtype=np.uint8)))
    for name, codes, E in cases:
        _print_case(f"remap mxfp4 {name}")
        w = moet.remap_mxfp4(torch.from_numpy(codes).to(DEV), torch.from_numpy(E).to(DEV), balance_zero_signs=balance)
        torch.cuda.synchronize()
        for m in range(codes.shape[0]):
            c2, tau, s2 = OS.remap_mxfp4(codes[m], E[m], balance_zero_signs=balance)
            _check_planes(w, m, c2, tau, s2, name)


def _fp8_random(rng, n, N, K):
    w = rng.integers(0, 256, size=(n, N, K), dtype=np.uint8)
    w[(w & 0x7F) == 0x7F] = 0x7E                    # no NaN codes
    w[:, ::7, :32] = 0                              # +0 blocks
    w[:, 3::11, 32:64] = 0x80                       # -0 blocks
    w[:, 1::4, 64:96] &= 0x87                       # subnormal weights
    nb = (N + 127) // 128
    bs = np.exp2(rng.uniform(-12, -2, size=(n, nb, K // 128))).astype(np.float32)
    bs[0, 0, 0] = 0.0                               # a zero block scale
    bs[1] *= np.float32(2.0 ** -120)                # tiny: tensor scale near the float32 floor
    return w, bs


@pytest.mark.parametrize("balance", [False, True])
def test_requant_fp8_bitexact(balance):
    _print_case(f"requant fp8 balance={balance}")
    rng = np.random.default_rng(41)
    cases = [("random n=3 N=192 K=384", *_fp8_random(rng, 3, 192, 384))]
    wq, bs = synth.make_fp8_stack(2, 320, 512, 5, "fp8")
    cases.append(("synthetic n=2 N=320 K=512", np_(wq), np_(bs)))
    cases.append(("all zero N=64 K=128", np.zeros((1, 64, 128), np.uint8), np.ones((1, 1, 1), np.float32)))
    for name, wq, bs in cases:
        _print_case(f"requant fp8 {name}")
        w = moet.requant_fp8(torch.from_numpy(wq).to(DEV), torch.from_numpy(bs).to(DEV), balance_zero_signs=balance)
        torch.cuda.synchronize()
        for m in range(wq.shape[0]):
            c2, tau, s2 = OS.requant_fp8(wq[m], bs[m], balance_zero_signs=balance)
            _check_planes(w, m, c2, tau, s2, name)


@pytest.mark.parametrize("fmt", ["mxfp4", "fp8"])
def test_forward_on_converted_weights(fmt):
    """A small layer loaded from the other flavours runs through the same forward;
    the oracle's forward uses its own conversion of the same source bytes."""
    H, I, E, T, k = 512, 256, 8, 5, 2
    _print_case(f"forward on {fmt} weights H={H} I={I} E={E} T={T}")
    if fmt == "mxfp4":
        c13, e13 = synth.make_mxfp4_stack(2 * E, I, H, 3, "mx13")
        c2_, e2_ = synth.make_mxfp4_stack(E, H, I, 3, "mx2")
        w13 = moet.remap_mxfp4(c13.to(DEV), e13.to(DEV))
        w2 = moet.remap_mxfp4(c2_.to(DEV), e2_.to(DEV))
        conv13 = lambda m: OS.remap_mxfp4(np_(c13[m]), np_(e13[m]))
        conv2 = lambda m: OS.remap_mxfp4(np_(c2_[m]), np_(e2_[m]))
    else:
        q13, b13 = synth.make_fp8_stack(2 * E, I, H, 3, "f13")
        q2, b2 = synth.make_fp8_stack(E, H, I, 3, "f2")
        w13 = moet.requant_fp8(q13.to(DEV), b13.to(DEV))
        w2 = moet.requant_fp8(q2.to(DEV), b2.to(DEV))
        conv13 = lambda m: OS.requant_fp8(np_(q13[m]), np_(b13[m]))
        conv2 = lambda m: OS.requant_fp8(np_(q2[m]), np_(b2[m]))
    layer = moet.Layer(H, I, E, w13, w2)
    x = synth.make_activations(T, H, 8)
    lg = torch.randn((T, E), generator=torch.Generator().manual_seed(4))
    ids, w, offs, pairs = moet.route(lg.to(DEV), k, moet.SOFTMAX, True)
    out = moet.moe_forward(layer, x.to(DEV), ids, w, offs, pairs)
    torch.cuda.synchronize()
    o_ids, o_w, _, _ = oracle_route(lg, k, moet.SOFTMAX, True)
    dq = lambda conv, m: OR.dequant_2bit(*conv(m))
    ref = OFF.moe_forward(bf16_bits(x), o_ids, o_w, lambda e: (dq(conv13, 2 * e), dq(conv13, 2 * e + 1), dq(conv2, e)))
    err = rel_l2(bf16_bits(out), ref)
    print(f"rel_l2={err:.3e}", flush=True)
    assert err <= REL_L2_BAR
    assert err <= 3e-4


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp4", "fp8"])
def test_full_size_conversions_sampled(fmt):
    """The load-time conversions at the benchmark's size (16 gate/up matrices [2048][7168]),
    two sampled matrices compared with the oracle byte for byte."""
    n, N, K = 16, 2048, 7168
    _print_case(f"full-size {fmt} conversion n={n} N={N} K={K}")
    if fmt == "nvfp4":
        src = synth.make_nvfp4_stack(n, N, K, 0, "conv_nvfp4", device=DEV)
        w = moet.requant(*src)
        conv = lambda m: OR.requant(np_(src[0][m]), np_(src[1][m]), float(np_(src[2])[m]))
    elif fmt == "mxfp4":
        src = synth.make_mxfp4_stack(n, N, K, 0, "conv_mxfp4", device=DEV)
        w = moet.remap_mxfp4(*src)
        conv = lambda m: OS.remap_mxfp4(np_(src[0][m]), np_(src[1][m]))
    else:
        src = synth.make_fp8_stack(n, N, K, 0, "conv_fp8", device=DEV)
        w = moet.requant_fp8(*src)
        conv = lambda m: OS.requant_fp8(np_(src[0][m]), np_(src[1][m]))
    torch.cuda.synchronize()
    for m in (3, n - 1):
        c2, tau, s2 = conv(m)
        _check_planes(w, m, c2, tau, s2, f"{fmt} full size")
