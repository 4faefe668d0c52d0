"""C ABI checks that need no GPU: the library loads, exports every function
the headers under include/ declare, and rejects bad arguments on the host
before any HIP call."""
import ctypes
import glob
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    names = set()
    for h in sorted(glob.glob(os.path.join(ROOT, "include", "*.h"))):
        txt = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(moet_[a-z_0-9]+)\s*\(", txt))
    return sorted(names)


@pytest.fixture(scope="module")
def L():
    from bit_moe_expert_nvfp4_amd import moet
    if not os.path.exists(moet.LIB_PATH):
        from bit_moe_expert_nvfp4_amd import build
        build.build()
    return moet.lib()


def test_exports_every_declared_symbol(L):
    names = _declared_functions()
    assert {"moet_requant", "moet_route", "moet_moe_forward", "moet_delta_forward",
            "moet_set_timing_events"} <= set(names)
    for n in names:
        assert hasattr(L, n), n


def test_status_strings(L):
    assert L.moet_status_str(0) == b"MOET_OK"
    assert L.moet_status_str(3) == b"MOET_EWORKSPACE"
    assert L.moet_abi_version() >= 1


def test_requant_rejects_bad_shapes(L):
    buf = ctypes.c_void_p(16)      # never dereferenced: checks fail first
    # codes, scales, scale2, n_mat, N, K, w2 codes/scales/scale2/codebook, sel, n_sel, d x3, flags, stream
    args = [buf, buf, buf, 1, 64, 128, buf, buf, buf, None, None, 0, None, None, None, 0, None]
    for i, bad in [(4, 63), (5, 96), (3, 0), (11, -1), (11, 2), (15, 4), (15, 0x80000000),
                   (15, 2),                           # the codebook pick needs w2_codebook
                   (9, ctypes.c_void_p(8))]:          # misaligned w2_codebook
        a = list(args)
        a[i] = bad
        assert L.moet_requant(*a) == 1, (i, bad)
    a = list(args)
    a[0] = ctypes.c_void_p(8)      # misaligned
    assert L.moet_requant(*a) == 1
    assert b"aligned" in L.moet_last_error()
    a = list(args)
    a[15] = 2
    a[9] = ctypes.c_void_p(8)
    assert L.moet_requant(*a) == 1
    assert b"w2_codebook" in L.moet_last_error()


def test_source_conversions_reject_bad_args(L):
    buf = ctypes.c_void_p(16)      # never dereferenced: checks fail first
    for fn in (L.moet_remap_mxfp4, L.moet_requant_fp8):
        args = [buf, buf, 1, 64, 128, buf, buf, buf, 0, None]
        for i, bad in [(3, 63), (4, 96), (2, 0), (8, 2), (8, 4), (8, 0x80000000)]:   # no codebook pick here
            a = list(args)
            a[i] = bad
            assert fn(*a) == 1, (fn, i, bad)
        a = list(args)
        a[5] = ctypes.c_void_p(8)  # misaligned
        assert fn(*a) == 1
        assert b"aligned" in L.moet_last_error()


def test_pack_nvfp4_rejects_bad_args(L):
    buf = ctypes.c_void_p(16)      # never dereferenced: checks fail first
    args = [buf, buf, buf, 1, 64, 128, buf, buf, buf, None]
    for i, bad in [(4, 63), (5, 96), (3, 0), (0, None), (7, ctypes.c_void_p(8))]:
        a = list(args)
        a[i] = bad
        assert L.moet_pack_nvfp4(*a) == 1, (i, bad)


def test_route_rejects_bad_args(L):
    b = ctypes.c_void_p(16)
    f = ctypes.c_float(1.0)
    assert L.moet_route(b, 0, 8, 2, 0, 1, f, b, b, b, b, None) == 1
    assert L.moet_route(b, 4, 2000, 2, 0, 1, f, b, b, b, b, None) == 1
    assert L.moet_route(b, 4, 8, 9, 0, 1, f, b, b, b, b, None) == 1
    assert L.moet_route(b, 4, 32, 17, 0, 1, f, b, b, b, b, None) == 1
    assert L.moet_route(b, 4, 8, 2, 7, 1, f, b, b, b, b, None) == 1
    assert L.moet_route(None, 4, 8, 2, 0, 1, f, b, b, b, b, None) == 1


def _layer(H=256, I=128, E=8):
    from bit_moe_expert_nvfp4_amd import moet
    z = moet.W2(16, 16, 16)
    return moet.LayerC(H, I, E, z, z, 0, moet.W2(None, None, None), moet.W2(None, None, None), 0, None,
                       moet.FP4(None, None, None), moet.FP4(None, None, None), 0.0, None, 0)


def test_forward_rejects_bad_args_and_short_workspace(L):
    from bit_moe_expert_nvfp4_amd import moet
    b = ctypes.c_void_p(256)
    lay = _layer()
    need = L.moet_moe_workspace_bytes(ctypes.byref(lay), 4, 2)
    assert need > 0
    assert L.moet_moe_workspace_bytes(ctypes.byref(lay), 8, 2) >= need
    # short workspace
    assert L.moet_moe_forward(ctypes.byref(lay), b, 4, 2, b, b, b, b, None, b, None, b, need - 1, None) == 3
    # bad shapes
    for H, I, E in [(200, 128, 8), (256, 64, 8), (256, 128, 0), (256, 128, 2000)]:
        bad = _layer(H, I, E)
        assert L.moet_moe_forward(ctypes.byref(bad), b, 4, 2, b, b, b, b, None, b, None, b, 1 << 30, None) == 1
    assert L.moet_moe_forward(ctypes.byref(lay), b, 4, 9, b, b, b, b, None, b, None, b, 1 << 30, None) == 1
    assert L.moet_moe_forward(ctypes.byref(lay), b, 0, 2, b, b, b, b, None, b, None, b, 1 << 30, None) == 1
    # delta cache with missing pointers
    lay.n_slots = 2
    assert L.moet_moe_forward(ctypes.byref(lay), b, 4, 2, b, b, b, b, None, b, None, b, 1 << 30, None) == 1
    # shared expert with missing pointers
    lay2 = _layer()
    lay2.has_shared = 1
    assert L.moet_moe_forward(ctypes.byref(lay2), b, 4, 2, b, b, b, b, None, b, None, b, 1 << 30, None) == 1
    # NVFP4 shared expert with missing FP4 planes (the 2-bit shared planes are then not needed)
    lay4 = _layer()
    lay4.has_shared = 1
    lay4.shared_fp4 = 1
    lay4.shared13_fp4 = moet.FP4(16, 16, 16)
    assert L.moet_moe_forward(ctypes.byref(lay4), b, 4, 2, b, b, b, b, None, b, None, b, 1 << 30, None) == 1
    assert b"NVFP4 shared" in L.moet_last_error()
    # misaligned miss counter; expert cache with a bad map or slot count
    assert L.moet_moe_forward(ctypes.byref(lay), b, 4, 2, b, b, b, b, None, b, ctypes.c_void_p(258), b, 1 << 30,
                              None) == 1
    lay3 = _layer()
    lay3.base_slot_of_expert = ctypes.c_void_p(264)
    assert L.moet_moe_forward(ctypes.byref(lay3), b, 4, 2, b, b, b, b, None, b, None, b, 1 << 30, None) == 1
    lay3.base_slot_of_expert = b
    lay3.n_base_slots = -1
    assert L.moet_moe_forward(ctypes.byref(lay3), b, 4, 2, b, b, b, b, None, b, None, b, 1 << 30, None) == 1
    # unaligned workspace
    assert L.moet_moe_forward(ctypes.byref(lay), b, 4, 2, b, b, b, b, None, b, None, ctypes.c_void_p(272), 1 << 30,
                              None) == 1


def test_delta_forward_rejects_bad_args(L):
    from bit_moe_expert_nvfp4_amd import moet
    b = ctypes.c_void_p(16)
    D = moet.FP4(16, 16, 16)
    assert L.moet_delta_forward(ctypes.byref(D), 1, 65, 128, b, b, 1, b, None) == 1
    assert L.moet_delta_forward(ctypes.byref(D), 1, 64, 100, b, b, 1, b, None) == 1
    assert L.moet_delta_forward(ctypes.byref(D), 0, 64, 128, b, b, 1, b, None) == 1
    assert L.moet_delta_forward(ctypes.byref(D), 1, 64, 128, b, b, -1, b, None) == 1
    assert L.moet_delta_forward(None, 1, 64, 128, b, b, 1, b, None) == 1
    # R == 0 is a no-op that touches nothing
    assert L.moet_delta_forward(ctypes.byref(D), 1, 64, 128, b, b, 0, b, None) == 0


def test_confidence_gate_rejects_bad_args(L):
    b = ctypes.c_void_p(256)
    f = ctypes.c_float(0.6)
    # T = 1024 rows run one workgroup each: no workspace needed
    assert L.moet_confidence_gate(b, 0, 10, f, b, None, None, 0, None) == 1
    assert L.moet_confidence_gate(b, 70000, 10, f, b, None, None, 0, None) == 1
    assert L.moet_confidence_gate(b, 2, 0, f, b, None, None, 0, None) == 1
    assert L.moet_confidence_gate(b, 2, 10, ctypes.c_float(float("nan")), b, None, None, 0, None) == 1
    assert L.moet_confidence_gate(None, 2, 10, f, b, None, None, 0, None) == 1
    assert L.moet_confidence_gate(ctypes.c_void_p(260), 2, 10, f, b, None, None, 0, None) == 1
    assert L.moet_confidence_gate(b, 2, 10, f, None, None, None, 0, None) == 1
    assert L.moet_confidence_gate(b, 2, 10, f, b, ctypes.c_void_p(258), None, 0, None) == 1
    # split rows need the workspace: missing or short -> MOET_EWORKSPACE, misaligned -> MOET_EINVAL
    need = L.moet_gate_workspace_bytes(3, 151552)
    assert L.moet_confidence_gate(b, 3, 151552, f, b, None, None, 0, None) == 3
    assert L.moet_confidence_gate(b, 3, 151552, f, b, None, b, need - 1, None) == 3
    assert L.moet_confidence_gate(b, 3, 151552, f, b, None, ctypes.c_void_p(264), need, None) == 1


def test_gate_workspace_bytes(L):
    """Chunking of the confidence gate: rows of at least 2048 logits per chunk, about 1024 chunk
    workgroups over all rows; one 16-byte partial per chunk."""
    ws = L.moet_gate_workspace_bytes
    assert ws(3, 151552) == 3 * 74 * 16          # 74 chunks of 2048
    assert ws(24, 151552) == 24 * 43 * 16        # 43 chunks of 3528
    assert ws(1, 4) == 0 and ws(5, 1001) == 0    # one chunk: the one-workgroup-per-row kernel
    assert ws(1024, 151552) == 0 and ws(4096, 151552) == 0
    assert ws(1, 4097) == 3 * 16                  # 3 chunks of 1368 (the last 1361)
    assert ws(0, 10) == 0 and ws(2, 0) == 0
    assert ws(1, 2**31 - 1) == 1024 * 16          # no int overflow at the largest V

def test_gemv_fallback_grid_bound(L):
    """Large batches whose H is not a multiple of 256 run the GEMV kernels, one grid row per routed pair
    plus one per token of the shared expert; past 65535 rows the call is MOET_EUNSUPPORTED (host check,
    no launch)."""
    from bit_moe_expert_nvfp4_amd import moet
    b = ctypes.c_void_p(256)
    z = moet.W2(16, 16, 16)
    lay = moet.LayerC(384, 128, 8, z, z, 1, z, z, 0, None, moet.FP4(None, None, None), moet.FP4(None, None, None),
                      0.0, None, 0)
    T = 65535 // 3 + 1                     # T * 2 + T = 65538 rows with the shared expert
    assert L.moet_moe_forward(ctypes.byref(lay), b, T, 2, b, b, b, b, None, b, None, b, 1 << 40, None) == 2
    assert b"65535" in L.moet_last_error()
    lay.has_shared = 0
    assert L.moet_moe_forward(ctypes.byref(lay), b, 32768, 2, b, b, b, b, None, b, None, b, 1 << 40, None) == 2


def test_moe_forward_binding_checks_shapes():
    """The binding compares every tensor with the layer before calling the library: a narrower x, an out
    of the wrong shape, int64 offsets or routing arrays of the wrong length raise ValueError (the kernels
    would index them with the layer's H and the batch's T, top_k)."""
    import torch
    from bit_moe_expert_nvfp4_amd import moet
    z = moet.W2Planes(torch.zeros(1, dtype=torch.int32), torch.zeros(1, dtype=torch.uint8), torch.zeros(1), 1, 1)
    layer = moet.Layer(256, 128, 8, z, z)
    T, k = 4, 2
    good = dict(x=torch.zeros(T, 256, dtype=torch.bfloat16), topk_ids=torch.zeros(T, k, dtype=torch.int32),
                topk_w=torch.zeros(T, k), expert_offsets=torch.zeros(9, dtype=torch.int32),
                sorted_pairs=torch.zeros(T * k, dtype=torch.int32))
    bad = [dict(x=torch.zeros(T, 128, dtype=torch.bfloat16)),
           dict(x=torch.zeros(T, 256, dtype=torch.float32)),
           dict(topk_ids=torch.zeros(T, k, dtype=torch.int64)),
           dict(topk_ids=torch.zeros(T + 1, k, dtype=torch.int32)),
           dict(topk_w=torch.zeros(T, k + 1)),
           dict(expert_offsets=torch.zeros(9, dtype=torch.int64)),
           dict(expert_offsets=torch.zeros(8, dtype=torch.int32)),
           dict(sorted_pairs=torch.zeros(T * k - 1, dtype=torch.int32)),
           dict(gate_flags=torch.zeros(T + 1, dtype=torch.uint8)),
           dict(out=torch.zeros(T, 128, dtype=torch.bfloat16)),
           dict(out=torch.zeros(T, 256, dtype=torch.float32)),
           dict(miss_count=torch.zeros(1, dtype=torch.int64))]
    for b in bad:
        args = dict(good, **b)
        with pytest.raises(ValueError):
            moet.moe_forward(layer, **args)
    # right shapes on CPU tensors: rejected as not on the GPU, before any library call
    with pytest.raises(TypeError):
        moet.moe_forward(layer, **good)
    # per-matrix codebook ids: one uint8 per matrix of the stack
    import dataclasses
    for cb in (torch.zeros(2, dtype=torch.uint8), torch.zeros(1, dtype=torch.int32)):
        zc = dataclasses.replace(z, codebook=cb)
        with pytest.raises(ValueError):
            moet.moe_forward(moet.Layer(256, 128, 8, zc, z), **good)


def test_probes_reject_bad_args(L):
    """The measurement references validate on the host (no GPU needed for the rejections)."""
    buf = ctypes.c_void_p(16)      # never dereferenced: checks fail first
    for args in [(None, 16, buf, None), (buf, 0, buf, None), (buf, 24, buf, None), (buf, 16, None, None),
                 (ctypes.c_void_p(8), 16, buf, None)]:
        assert L.moet_probe_read(*args) == 1, args
    for args in [(7, 1, buf, None), (0, 0, buf, None), (1, -3, buf, None), (0, 1, None, None)]:
        assert L.moet_probe_peak(*args) == 1, args


def test_probe_bindings_reject_host_tensors():
    import torch
    from bit_moe_expert_nvfp4_amd import moet
    sink = torch.zeros(moet.PROBE_SINK_WORDS, dtype=torch.int32)
    with pytest.raises(TypeError):
        moet.probe_read(torch.zeros(1024, dtype=torch.int32), sink)
    with pytest.raises(TypeError):
        moet.probe_peak(moet.PROBE_MFMA_BF16, 4, sink)
    with pytest.raises(ValueError):
        moet.probe_peak(moet.PROBE_DOT2_BF16, 4, torch.zeros(16, dtype=torch.int32))


def test_conversion_bindings_check_shapes():
    """Mismatched scale or scale2 shapes raise ValueError before any device check or library call (the
    kernels would index the scales with the dimensions of the codes)."""
    import torch
    from bit_moe_expert_nvfp4_amd import moet
    c = torch.zeros(2, 64, 64, dtype=torch.uint8)
    for s, z in [(torch.zeros(2, 64, 7, dtype=torch.uint8), torch.zeros(2)),
                 (torch.zeros(2, 64, 8, dtype=torch.uint8), torch.zeros(3)),
                 (torch.zeros(1, 64, 8, dtype=torch.uint8), torch.zeros(2))]:
        with pytest.raises(ValueError):
            moet.requant(c, s, z)
        with pytest.raises(ValueError):
            moet.pack_nvfp4(c, s, z)
    with pytest.raises(ValueError):
        moet.remap_mxfp4(c, torch.zeros(2, 64, 8, dtype=torch.uint8))     # MXFP4 scales are per 32
    with pytest.raises(ValueError):
        moet.requant(torch.zeros(64, 64, dtype=torch.uint8), torch.zeros(64, 8, dtype=torch.uint8), torch.zeros(1))
    with pytest.raises(ValueError):
        moet.route(torch.zeros(4, 8, 2), 2)
    with pytest.raises(TypeError):      # right shapes, host tensors
        moet.requant(c, torch.zeros(2, 64, 8, dtype=torch.uint8), torch.zeros(2))


def test_delta_and_gate_bindings_check_shapes():
    import torch
    from bit_moe_expert_nvfp4_amd import moet
    D = moet.FP4Planes(torch.zeros(1, 64 * 128 // 2, dtype=torch.uint8), torch.zeros(1, 64 * 128 // 16, dtype=torch.uint8),
                       torch.zeros(1), 64, 128)
    R = 3
    good = dict(act=torch.zeros(R, 128, dtype=torch.bfloat16), row_slot=torch.zeros(R, dtype=torch.int32),
                acc=torch.zeros(R, 64))
    for b in [dict(act=torch.zeros(R, 256, dtype=torch.bfloat16)), dict(row_slot=torch.zeros(R + 1, dtype=torch.int32)),
              dict(acc=torch.zeros(R, 128)), dict(acc=torch.zeros(R, 64, dtype=torch.float64))]:
        with pytest.raises(ValueError):
            moet.delta_forward(D, **dict(good, **b))
    with pytest.raises(TypeError):
        moet.delta_forward(D, **good)
    lg = torch.zeros(4, 100)
    with pytest.raises(ValueError):
        moet.confidence_gate(lg, flags=torch.zeros(5, dtype=torch.uint8))
    with pytest.raises(ValueError):
        moet.confidence_gate(lg, confidence=torch.zeros(3))
    with pytest.raises(ValueError):
        moet.confidence_gate(torch.zeros(100))
