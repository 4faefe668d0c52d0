"""moet_moe_forward_noalloc (the layer forward with the library's static
scratch, for callers that cannot allocate) against moet_moe_forward with a
caller workspace: the same kernels, so the outputs must agree bit for bit.
Each case runs two calls in a row, the second on a smaller batch, so the
second reads a scratch array that still holds the first call's rows.  A batch
whose workspace exceeds the static scratch is rejected on the host."""
import numpy as np
import pytest
import torch

from bit_moe_expert_nvfp4_amd import moet, synth
from moet_testlib import bf16_bits, np_

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _case(cfg, seed, T):
    x = synth.make_activations(T, cfg.H, seed, device=DEV)
    lg = torch.randn((T, cfg.E), generator=torch.Generator().manual_seed(seed)).to(DEV)
    ids, w, offs, pairs = moet.route(lg, cfg.k, cfg.score, cfg.renormalize)
    flags = None
    if cfg.n_resident:
        flags = (torch.arange(T) % 2 == 0).to(torch.uint8).to(DEV)
    return x, ids, w, offs, pairs, flags


@pytest.mark.parametrize("shape", [
    dict(H=512, I=256, E=16, k=4, shared=True, n_resident=6, T=(24, 5)),            # GEMV kernels
    dict(H=512, I=256, E=16, k=8, shared=False, n_resident=0, T=(300, 100)),        # grouped GEMM, then GEMV
    dict(H=7168, I=2048, E=256, k=8, shared=True, n_resident=32, T=(3, 1)),         # the MTP decode layer
])
def test_noalloc_matches_workspace_forward(shape):
    T1, T2 = shape["T"]
    cfg = synth.LayerConfig("noalloc", T=T1, H=shape["H"], I=shape["I"], E=shape["E"], k=shape["k"],
                            score=synth.SIGMOID, shared=shape["shared"], n_resident=shape["n_resident"])
    print(f"[case] noalloc {shape}", flush=True)
    src = synth.make_layer(cfg, seed=5, device=DEV)
    soe = synth.slot_of_expert(cfg, 5) if cfg.n_resident else None
    layer = moet.layer_from_nvfp4(src, soe)
    for T, seed in ((T1, 1), (T2, 2)):
        assert moet.moe_workspace_bytes(layer, T, cfg.k) <= moet.NOALLOC_SCRATCH_BYTES
        x, ids, w, offs, pairs, flags = _case(cfg, seed, T)
        ref = moet.moe_forward(layer, x, ids, w, offs, pairs, flags)
        out = torch.full((T, cfg.H), float("nan"), dtype=torch.bfloat16, device=DEV)
        miss = torch.full((1,), -1, dtype=torch.int32, device=DEV)
        moet.moe_forward_noalloc(layer, x, ids, w, offs, pairs, out, flags, miss)
        torch.cuda.synchronize()
        assert (bf16_bits(out) == bf16_bits(ref)).all(), f"T={T}: noalloc output differs"
        assert int(miss.item()) == 0
        print(f"T={T}: {T * cfg.H} outputs bit-identical", flush=True)


def test_noalloc_rejects_batches_beyond_the_scratch():
    cfg = synth.LayerConfig("noalloc_big", T=4096, H=7168, I=2048, E=8, k=8, score=synth.SIGMOID)
    z = moet.W2Planes(torch.zeros(16, dtype=torch.int32, device=DEV), torch.zeros(16, dtype=torch.uint8, device=DEV),
                      torch.zeros(16, device=DEV), 1, 1)
    layer = moet.Layer(cfg.H, cfg.I, cfg.E, z, z)
    T, k = 64, 8
    assert moet.moe_workspace_bytes(layer, T, k) > moet.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((T, cfg.H), dtype=torch.bfloat16, device=DEV)
    ids = torch.zeros((T, k), dtype=torch.int32, device=DEV)
    w = torch.zeros((T, k), dtype=torch.float32, device=DEV)
    offs = torch.zeros((cfg.E + 1,), dtype=torch.int32, device=DEV)
    pairs = torch.zeros((T * k,), dtype=torch.int32, device=DEV)
    out = torch.zeros((T, cfg.H), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(moet.MoetError) as ei:
        moet.moe_forward_noalloc(layer, x, ids, w, offs, pairs, out)
    assert ei.value.status == moet.MOET_EWORKSPACE and "static scratch" in str(ei.value)
