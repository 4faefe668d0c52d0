"""GPU parity of the prefill grouped GEMM over every M-tile shape it instantiates.

The 2-bit prefill kernels cut an expert's run of pairs into tiles of up to 160
rows and issue MFMAs per 16-row block, with one code path per block count
(1..10); the FP4 delta kernels take up to 128 flagged rows per tile, one path
per block count 1..8.  Here top-1 routing is built so that the experts' row
counts hit every block count and the ragged cases around each 16-row boundary
(r = 16 b - 1, 16 b, 16 b + 1), plus runs of several tiles and an empty
expert; the delta case flags chosen numbers of each expert's tokens (all, some,
none).  Every h and y row and every output element is compared with the
oracle, as in the other forward parity tests.
"""
import numpy as np
import pytest
import torch

from bit_moe_expert_nvfp4_amd import moet, synth
from moet_testlib import (OracleLayer, REL_L2_BAR, alarm_rel_l2, assert_elementwise, bf16_bits, check_out_rows,
                          check_pair_rows, np_, oracle_route, rel_l2)

pytestmark = pytest.mark.gpu
DEV = "cuda"

# rows per expert: every 16-row block count 1..10 with r = 16 b - 1, 16 b, 16 b + 1 around the
# boundaries, two- and three-tile runs (161, 320, 481) and an empty expert
COUNTS = [1, 15, 16, 17, 31, 32, 33, 47, 49, 63, 64, 65, 79, 81, 95, 97, 111, 113, 127, 128, 129,
          143, 145, 159, 160, 161, 320, 481, 0, 2, 7, 100]


def _routing(counts, seed):
    """fp32 logits [T, E] whose top-1 expert of token t is e(t), with expert e taking counts[e]
    tokens in a shuffled order; returns (logits, e(t))."""
    rng = np.random.default_rng(seed)
    owner = np.concatenate([np.full(c, e, dtype=np.int64) for e, c in enumerate(counts)])
    rng.shuffle(owner)
    T, E = owner.size, len(counts)
    lg = rng.standard_normal((T, E)).astype(np.float32) * 0.5
    lg[np.arange(T), owner] = 4.0 + rng.random(T).astype(np.float32)
    return torch.from_numpy(lg), owner


def _run(counts, seed, flag_share=None):
    T, E = sum(counts), len(counts)
    assert T > 1024   # the grouped-GEMM path
    delta = flag_share is not None
    cfg = synth.LayerConfig(name="blocks", T=T, H=256, I=128, E=E, k=1, score=synth.SIGMOID,
                            n_resident=E if delta else 0, n_flagged=0)
    src = synth.make_layer(cfg, seed=seed)
    soe = torch.arange(E, dtype=torch.int32) if delta else None   # every expert holds its own delta slot
    layer = moet.layer_from_nvfp4(src, soe)
    x = synth.make_activations(T, cfg.H, seed)
    lg, owner = _routing(counts, seed)
    flags = None
    if delta:
        # expert e flags the first flag_share[e] of its tokens (in token order)
        f = np.zeros(T, dtype=np.uint8)
        for e, share in enumerate(flag_share):
            toks = np.nonzero(owner == e)[0]
            f[toks[: int(share)]] = 1
        flags = torch.from_numpy(f)
    ids, w, offs, pairs = moet.route(lg.to(DEV), 1, cfg.score, cfg.renormalize)
    assert (np_(offs)[1:] - np_(offs)[:-1] == np.asarray(counts)).all(), "routing does not give the planned counts"
    ws = moet.alloc_workspace(layer, T, 1, DEV)
    out = moet.moe_forward(layer, x.to(DEV), ids, w, offs, pairs, flags.to(DEV) if flags is not None else None,
                           workspace=ws)
    torch.cuda.synchronize()
    o_ids, o_w, _, o_pairs = oracle_route(lg, 1, cfg.score, cfg.renormalize)
    assert (np_(ids) == o_ids).all()
    ol = OracleLayer(src, soe)
    fl = np_(flags) if flags is not None else None
    ref = ol.forward(bf16_bits(x), o_ids, o_w, gate_flags=fl)
    got = bf16_bits(out)
    rows = check_pair_rows(ws, ol, bf16_bits(x), o_ids, o_pairs, cfg.H, cfg.I, gate_flags=fl)
    assert_elementwise(rows.h, rows.y, check_out_rows(got, ref, range(T), o_w, rows))
    err = rel_l2(got, ref)
    print(f"rel_l2={err:.3e}", flush=True)
    assert err <= REL_L2_BAR
    assert err <= alarm_rel_l2(cfg.H)


def test_prefill_every_block_count():
    print(f"[case] prefill row counts {COUNTS}", flush=True)
    _run(COUNTS, seed=31)


def test_prefill_delta_every_block_count():
    # flagged rows per delta expert: FP4 block counts 1..8 with ragged tails, a tile of 128, two tiles
    # (129, 160, 200), all of a run, part of a run, none
    share = [1, 15, 16, 17, 31, 32, 33, 40, 49, 63, 64, 65, 79, 81, 95, 97, 111, 113, 127, 128, 129,
             0, 145, 100, 160, 20, 200, 481, 0, 2, 7, 50]
    share = [min(s, c) for s, c in zip(share, COUNTS)]
    print(f"[case] prefill delta flagged rows {share}", flush=True)
    _run(COUNTS, seed=32, flag_share=share)
