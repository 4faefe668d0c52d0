"""Pins for the oracle's routing, permutation and expert FFN (CPU only).

Routing is checked against a pure-Python sort with the stated key, against
scipy's softmax / expit, and on ties and k = E.  The FFN is checked against
an independent block-wise formulation (sum of level*x per block, then the
block scale, then the tensor scale), against linearity in the delta, and
against a dense all-experts formulation of the combine.
"""
import numpy as np
import pytest
import scipy.special as sp

from oracle import formats as F
from oracle import requant as R
from oracle import route as RT
from oracle import ffn as FF


def test_topk_matches_python_sort_with_ties():
    rng = np.random.default_rng(0)
    T, E, k = 16, 12, 4
    lg = rng.integers(-3, 3, size=(T, E)).astype(np.float32)     # many equal logits
    ids = RT.topk_ids(lg, k)
    for t in range(T):
        want = sorted(range(E), key=lambda e: (-float(lg[t, e]), e))[:k]
        assert ids[t].tolist() == want


def test_topk_k_equals_E_and_distinct():
    rng = np.random.default_rng(1)
    lg = rng.standard_normal((5, 8)).astype(np.float32)
    ids = RT.topk_ids(lg, 8)
    assert all(sorted(r) == list(range(8)) for r in ids.tolist())


def test_weights_against_scipy():
    rng = np.random.default_rng(2)
    lg = rng.standard_normal((6, 32)).astype(np.float32)
    ids = RT.topk_ids(lg, 8)
    lg64 = lg.astype(np.float64)
    full = sp.softmax(lg64, axis=1)
    sel = np.take_along_axis(full, ids.astype(np.int64), 1)
    w = RT.topk_weights(lg, ids, RT.SOFTMAX, True)
    assert np.allclose(w, sel / sel.sum(1, keepdims=True), rtol=1e-13, atol=0)
    assert np.allclose(w.sum(1), 1.0, atol=1e-12)
    w2 = RT.topk_weights(lg, ids, RT.SOFTMAX, False)
    assert np.allclose(w2, sel, rtol=1e-13)
    sg = sp.expit(np.take_along_axis(lg64, ids.astype(np.int64), 1))
    w3 = RT.topk_weights(lg, ids, RT.SIGMOID, True, route_scale=2.5)
    assert np.allclose(w3, 2.5 * sg / sg.sum(1, keepdims=True), rtol=1e-13)
    w4 = RT.topk_weights(lg, ids, RT.SIGMOID, False)
    assert np.allclose(w4, sg, rtol=1e-13)


def test_permutation_against_bruteforce():
    rng = np.random.default_rng(3)
    T, E, k = 37, 10, 3
    lg = rng.standard_normal((T, E)).astype(np.float32)
    ids = RT.topk_ids(lg, k)
    offs, pairs = RT.permute(ids, E)
    allp = [(int(ids[p // k, p % k]), p) for p in range(T * k)]
    want = [p for _, p in sorted(allp)]
    assert pairs.tolist() == want
    for e in range(E):
        assert offs[e] == sum(1 for x, _ in allp if x < e)
    assert offs[E] == T * k
    # an expert nobody picked has an empty range
    empty = [e for e in range(E) if offs[e] == offs[e + 1]]
    for e in empty:
        assert e not in ids


def _tiny_matrix(rng, N, K):
    nib = rng.integers(0, 16, size=(N, K))
    packed = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    scales = rng.integers(0x28, 0x40, size=(N, K // 16)).astype(np.uint8)
    return packed, scales


def test_2bit_gemm_equals_blockwise_formulation():
    """dense matmul on dequantised 2-bit weights == sum over blocks of
    (sum level*x) * block scale, times the tensor scale (1e-12 relative)."""
    rng = np.random.default_rng(4)
    N, K = 16, 256
    c, s = _tiny_matrix(rng, N, K)
    c2, tau, s2 = R.requant(c, s, 0.013)
    W = R.dequant_2bit(c2, tau, s2)
    x = F.bf16_bits_to_f64(F.bf16_rne_bits(rng.standard_normal((3, K))))
    dense = x @ W.T
    lv = R.LEVELS[c2.astype(np.int64)]                       # [N, K]
    blk = np.zeros_like(dense)
    for b in range(K // 32):
        part = x[:, 32 * b:32 * b + 32] @ lv[:, 32 * b:32 * b + 32].T
        blk += part * F.e4m3fn_value(tau[:, b])[None, :]
    blk *= float(s2)
    assert np.allclose(dense, blk, rtol=1e-12, atol=1e-300)


def test_delta_linearity_and_fp4_gemm():
    rng = np.random.default_rng(5)
    I, H = 8, 128
    mats = [_tiny_matrix(rng, I, H) for _ in range(2)]
    ws, ds = [], []
    for c, s in mats:
        c2, tau, s2 = R.requant(c, s, 0.02)
        ws.append(R.dequant_2bit(c2, tau, s2))
        dc, dsc, d2 = R.delta(c, s, 0.02, c2, tau)
        ds.append(R.dequant_fp4_codes(dc, dsc, d2))
    x = F.bf16_bits_to_f64(F.bf16_rne_bits(rng.standard_normal((2, H))))
    h1 = FF.expert_hidden(x, ws[0], ws[1], 0.0, ds[0], ds[1])
    h2 = FF.expert_hidden(x, ws[0] + ds[0], ws[1] + ds[1], 0.0)
    # bf16 rounding of equal-up-to-1e-16 pre-activations agrees except on exact ties
    assert np.mean(h1 == h2) > 0.99
    acc = rng.standard_normal((2, I))
    out = FF.fp4_gemm_accumulate(acc, F.bf16_rne_bits(x), np.array([0, -1]), lambda s: ds[s])
    assert np.allclose(out[0], acc[0] + ds[0] @ x[0], rtol=1e-13)
    assert (out[1] == acc[1]).all()


def test_silu_closed_forms():
    assert FF.silu(0.0) == 0.0
    assert FF.silu(50.0) == pytest.approx(50.0, rel=1e-15)
    assert FF.silu(-800.0) == 0.0
    assert FF.silu(1.0) == pytest.approx(1.0 / (1.0 + np.exp(-1.0)), rel=1e-15)


def _tiny_layer(rng, E, H, I):
    experts = []
    for e in range(E):
        mats = []
        for (N, K) in ((I, H), (I, H), (H, I)):
            c, s = _tiny_matrix(rng, N, K)
            c2, tau, s2 = R.requant(c, s, 0.01 * (1 + e))
            mats.append(R.dequant_2bit(c2, tau, s2))
        experts.append(mats)
    return experts


def test_moe_forward_single_expert_and_shared():
    rng = np.random.default_rng(6)
    E, H, I = 3, 128, 64
    ex = _tiny_layer(rng, E, H, I)
    xb = F.bf16_rne_bits(rng.standard_normal((2, H)))
    x = F.bf16_bits_to_f64(xb)
    ids = np.array([[2], [0]])
    w = np.ones((2, 1))
    out = FF.moe_forward(xb, ids, w, lambda e: ex[e], shared_weights=ex[1])
    for t in range(2):
        e = ids[t, 0]
        y = FF.expert_out(FF.expert_hidden(x[t:t + 1], ex[e][0], ex[e][1]), ex[e][2])
        ysh = FF.expert_out(FF.expert_hidden(x[t:t + 1], ex[1][0], ex[1][1]), ex[1][2])
        assert (out[t] == F.bf16_rne_bits(y[0] + ysh[0])).all()


def test_moe_forward_equals_dense_formulation():
    """Dense form: every expert on every token, combined with a [T, E] weight matrix
    that is zero off the routed set (summed in expert order, not slot order)."""
    rng = np.random.default_rng(7)
    E, H, I, T, k = 5, 128, 64, 6, 2
    ex = _tiny_layer(rng, E, H, I)
    xb = F.bf16_rne_bits(rng.standard_normal((T, H)))
    x = F.bf16_bits_to_f64(xb)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    ids, w, offs, pairs = RT.route(lg, k, RT.SIGMOID)
    out = FF.moe_forward(xb, ids, w, lambda e: ex[e])
    Wd = np.zeros((T, E))
    for t in range(T):
        for j in range(k):
            Wd[t, ids[t, j]] = w[t, j]
    acc = np.zeros((T, H))
    for e in range(E):
        y = FF.expert_out(FF.expert_hidden(x, ex[e][0], ex[e][1]), ex[e][2])
        acc += Wd[:, e:e + 1] * y
    ref = F.bf16_rne_bits(acc)
    assert (out == ref).all()
    # token subset gives the same rows
    sub = FF.moe_forward(xb, ids, w, lambda e: ex[e], tokens=[4, 1])
    assert (sub == out[[4, 1]]).all()


def test_swiglu_clamp():
    rng = np.random.default_rng(8)
    ex = _tiny_layer(rng, 1, 128, 64)[0]
    x = F.bf16_bits_to_f64(F.bf16_rne_bits(4 * rng.standard_normal((1, 128))))
    L = 0.05
    h = FF.expert_hidden(x, ex[0], ex[1], L)
    ug = np.minimum(x @ ex[0].T, L)
    uu = np.clip(x @ ex[1].T, -L, L)
    assert (h == F.bf16_bits_to_f64(F.bf16_rne_bits(ug / (1 + np.exp(-ug)) * uu))).all()
    # silu on (-inf, L] is bounded by max(0.2785, silu(L)) in magnitude
    assert np.abs(h).max() <= max(0.2785, L / (1 + np.exp(-L))) * L * 1.01


def test_moe_forward_expert_cache_mask():
    """Missing experts contribute nothing and are counted (README, "When the model doesn't fit at all
    — the GPU as an expert cache"): checked against the dense form with the missing experts' combine
    weights set to zero, against a loop count of missed routings, and at the two ends (all resident ==
    no mask bit for bit; nothing resident == only the shared expert)."""
    rng = np.random.default_rng(11)
    E, H, I, T, k = 6, 128, 64, 7, 3
    ex = _tiny_layer(rng, E, H, I)
    sh = _tiny_layer(rng, 1, H, I)[0]
    xb = F.bf16_rne_bits(rng.standard_normal((T, H)))
    x = F.bf16_bits_to_f64(xb)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    ids, w, _, _ = RT.route(lg, k, RT.SOFTMAX)
    resident = np.array([True, False, True, True, False, True])
    out = FF.moe_forward(xb, ids, w, lambda e: ex[e], shared_weights=sh, resident=resident)
    Wt = np.zeros((T, E))
    for t in range(T):
        for j in range(k):
            if resident[ids[t, j]]:
                Wt[t, ids[t, j]] = w[t, j]
    dense = np.zeros((T, H))
    for e in range(E):
        dense += Wt[:, e:e + 1] * FF.expert_out(FF.expert_hidden(x, ex[e][0], ex[e][1]), ex[e][2])
    dense += FF.expert_out(FF.expert_hidden(x, sh[0], sh[1]), sh[2])
    assert (out == F.bf16_rne_bits(dense)).all()
    misses = sum(1 for t in range(T) for j in range(k) if not resident[ids[t, j]])
    assert FF.miss_count(ids, resident) == misses > 0
    full = FF.moe_forward(xb, ids, w, lambda e: ex[e], shared_weights=sh)
    assert (FF.moe_forward(xb, ids, w, lambda e: ex[e], shared_weights=sh, resident=np.ones(E, bool)) == full).all()
    none = FF.moe_forward(xb, ids, w, lambda e: ex[e], shared_weights=sh, resident=np.zeros(E, bool))
    shared_only = F.bf16_rne_bits(FF.expert_out(FF.expert_hidden(x, sh[0], sh[1]), sh[2]))
    assert (none == shared_only).all()
    assert FF.miss_count(ids, np.zeros(E, bool)) == T * k
