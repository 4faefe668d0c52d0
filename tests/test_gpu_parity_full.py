"""GPU parity at the full layer sizes, in the launch configuration the
benchmark times (moet_route + moet_moe_forward on whole synthetic layers
generated on the GPU).

* Routing of all tokens is compared bit for bit.
* Decode shapes (3 and 24 tokens): every token's output is compared with the
  oracle element by element, and every h and y row of the step.
* The 4096-token prefill chunk: 64 tokens are compared (chosen so that their
  experts overlap, which bounds the oracle's work, and so that every expert
  whose rows span two 160-row M-tiles is among them), and every h and y row
  of every expert those tokens touch (about 120 experts, 15k pairs).
* The requantised planes of every expert the oracle touched are compared byte
  for byte, and the forward is checked for bitwise determinism.
The oracle recomputes everything from the NVFP4 bytes (its own requantisation
of each touched expert)."""
import dataclasses
import time

import numpy as np
import pytest
import torch

from bit_moe_expert_nvfp4_amd import moet, synth
from moet_testlib import (OracleLayer, REL_L2_BAR, assert_elementwise, bf16_bits, check_out_rows, check_pair_rows,
                          mixed_codebook_layer, np_, oracle_route, rel_l2)

pytestmark = pytest.mark.gpu
DEV = "cuda"
SEED = 11
PREFILL_TILE = 160          # rows per M-tile of the grouped-GEMM kernels


def _u32(t):
    return np_(t).view(np.uint32)


def _variant(cfg_name, variant):
    """The benchmark's other full-size workloads: the prefill chunk with a gated FP4 delta,
    the decode layer with an NVFP4 shared expert, one GPU's share of a TP4 layer; and the decode
    layer with a delta cache whose matrices pick different codebooks."""
    cfg = synth.CONFIGS[cfg_name]
    if variant == "prefill_delta":
        cfg = dataclasses.replace(cfg, name="prefill_delta", n_resident=32, n_flagged=2048)
    elif variant == "tp4_shard":
        cfg = dataclasses.replace(cfg, name=f"{cfg.name}_tp4_shard", I=cfg.I // 4)
    return cfg


def _choose_tokens(ids: np.ndarray, n_tok: int, flags=None, soe=None):
    """n_tok tokens whose experts overlap as much as possible (greedy: each step adds the token that
    brings the fewest new experts), seeded with one token of every expert spanning two M-tiles and,
    with a delta cache, 16 gate-flagged tokens routed to resident experts."""
    T, k = ids.shape
    sets = [set(r) for r in ids.tolist()]
    counts = np.bincount(ids.reshape(-1), minlength=int(ids.max()) + 1)
    chosen, union = [], set()

    def take(t):
        chosen.append(t)
        union.update(sets[t])
    for e in np.nonzero(counts > PREFILL_TILE)[0]:
        t = int(np.nonzero((ids == e).any(1))[0][0])
        if t not in chosen:
            take(t)
    if flags is not None and soe is not None:
        cand = [t for t in range(T) if flags[t] and any(soe[e] >= 0 for e in sets[t]) and t not in chosen]
        for t in cand[:16]:
            take(t)
    taken = set(chosen)
    while len(chosen) < n_tok:
        best = min((len(sets[t] - union), t) for t in range(T) if t not in taken)[1]
        take(best)
        taken.add(best)
    return sorted(chosen), union, counts


@pytest.mark.timeout(900)
@pytest.mark.parametrize("cfg_name,variant", [("decode_mtp", None), ("decode_mtp_delta", None), ("batched_decode", None),
                                              ("prefill", None), ("prefill", "prefill_delta"),
                                              ("decode_mtp", "nvfp4_shared"), ("decode_mtp", "tp4_shard"),
                                              ("decode_mtp_delta", "mixed_codebooks")])
def test_full_size_forward(cfg_name, variant):
    cfg = _variant(cfg_name, variant)
    shared_nvfp4 = variant == "nvfp4_shared"
    pick = variant == "mixed_codebooks"
    print(f"[case] full-size config {cfg.name} T={cfg.T} E={cfg.E} I={cfg.I} variant={variant}", flush=True)
    t0 = time.time()
    src = synth.make_layer(cfg, seed=SEED, device=DEV)
    if pick:
        src = mixed_codebook_layer(src, SEED)
    soe = synth.slot_of_expert(cfg, SEED) if cfg.n_resident else None
    layer = moet.layer_from_nvfp4(src, soe, shared_nvfp4=shared_nvfp4, pick_codebook=pick)
    x = synth.make_activations(cfg.T, cfg.H, SEED, device=DEV)
    lg = synth.make_logits(cfg, SEED, device=DEV)
    flags = synth.gate_flags(cfg, SEED).to(DEV) if cfg.n_flagged else None
    ids, w, offs, pairs = moet.route(lg, cfg.k, cfg.score, cfg.renormalize)
    ws = moet.alloc_workspace(layer, cfg.T, cfg.k, DEV)
    out = moet.moe_forward(layer, x, ids, w, offs, pairs, flags, workspace=ws)
    out2 = moet.moe_forward(layer, x, ids, w, offs, pairs, flags)
    torch.cuda.synchronize()
    assert (bf16_bits(out) == bf16_bits(out2)).all(), "forward is not bitwise deterministic"

    o_ids, o_w, o_offs, o_pairs = oracle_route(lg, cfg.k, cfg.score, cfg.renormalize)
    assert (np_(ids) == o_ids).all()
    assert (np_(offs) == o_offs).all()
    assert (np_(pairs) == o_pairs).all()
    assert np.allclose(np_(w), o_w, rtol=2e-6, atol=1e-7)

    fl = np_(flags) if flags is not None else None
    soe_np = np_(soe) if soe is not None else None
    if cfg.T <= 64:
        toks = list(range(cfg.T))
        experts = None
    else:
        toks, experts, counts = _choose_tokens(o_ids, 64, fl, soe_np)
        two_tile = [int(e) for e in np.nonzero(counts > PREFILL_TILE)[0]]
        assert len(toks) == 64 and len(experts) >= 32
        assert set(two_tile) <= experts
        print(f"{len(toks)} tokens over {len(experts)} experts; experts spanning two M-tiles: {two_tile}", flush=True)
    ol = OracleLayer(src, soe, shared_nvfp4=shared_nvfp4, pick_codebook=pick)
    ol.prefetch(set(o_ids[toks].reshape(-1).tolist()))
    ref = ol.forward(bf16_bits(x), o_ids, o_w, gate_flags=fl, tokens=toks)
    print(f"oracle outputs done ({time.time() - t0:.0f} s)", flush=True)
    got = bf16_bits(out)[toks]
    err = rel_l2(got, ref)
    print(f"tokens={toks if len(toks) <= 24 else len(toks)} rel_l2={err:.3e}", flush=True)
    assert err <= REL_L2_BAR
    # At K = 7168 the fp32 accumulation order differs from the float64 oracle by
    # ~1e-6 relative, which flips the bf16 rounding of a few h and out elements by
    # one ulp (2^-8); that alone gives rel-L2 of a few 1e-4.  Anything near the
    # bar would be an arithmetic error, so alarm at half of it.
    assert err <= 1e-3

    # h and y of every pair of the touched experts (all pairs of the step at decode sizes) and every
    # compared output element
    ol.prefetch(experts if experts is not None else set(o_ids.reshape(-1).tolist()))
    rows = check_pair_rows(ws, ol, bf16_bits(x), o_ids, o_pairs, cfg.H, cfg.I, gate_flags=fl, experts=experts,
                           out_tokens=toks)
    print(f"oracle rows done ({time.time() - t0:.0f} s)", flush=True)
    assert_elementwise(rows.h, rows.y, check_out_rows(got, ref, toks, o_w, rows))

    # every matrix the oracle requantised matches the GPU planes byte for byte (host copies of the
    # stacks, compared on a thread pool)
    host = {}

    def h(t):
        if id(t) not in host:
            host[id(t)] = np_(t)
        return host[id(t)]
    jobs = []
    for (sid, i, with_delta), om in list(ol._cache.items()):
        if sid == id(src.w13):
            planes, dpl, dslot = layer.w13, layer.d13, None
            if with_delta:
                dslot = 2 * int(soe_np[i // 2]) + (i % 2)
        elif sid == id(src.w2):
            planes, dpl, dslot = layer.w2, layer.d2, None
            if with_delta:
                dslot = int(soe_np[i])
        elif sid == id(src.shared13):
            planes, dpl, dslot = layer.shared13, None, None
        else:
            planes, dpl, dslot = layer.shared2, None, None
        if planes is None:      # NVFP4 shared expert: no 2-bit planes (the oracle decodes NVFP4 itself)
            continue
        jobs.append((om, h(planes.codes)[i].view(np.uint32), h(planes.scales)[i],
                     None if dslot is None else (h(dpl.codes)[dslot], h(dpl.scales)[dslot])))

    if pick:     # the oracle's picks: every codebook among the touched matrices, and the layer's ids equal them
        cbs = {}
        for (sid, i, _), om in ol._cache.items():
            stack = {id(src.w13): layer.w13, id(src.w2): layer.w2, id(src.shared13): layer.shared13,
                     id(src.shared2): layer.shared2}[sid]
            assert int(h(stack.codebook)[i]) == om.cb, f"codebook of matrix {i}"
            cbs[om.cb] = cbs.get(om.cb, 0) + 1
        print(f"codebooks of the touched matrices: {cbs}", flush=True)
        assert set(cbs) == {0, 1, 2}

    def same(job):
        om, codes, scales, delta = job
        ok = (codes == om.packed_codes()).all() and (scales == om.packed_scales()).all()
        if delta is not None:
            pc, ps = om.packed_delta()
            ok = ok and (delta[0] == pc).all() and (delta[1] == ps).all()
        return bool(ok)
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(8) as ex:
        results = list(ex.map(same, jobs))
    print(f"requant planes checked: {len(jobs)} matrices ({time.time() - t0:.0f} s)", flush=True)
    assert jobs and all(results), f"{results.count(False)} matrices differ"
