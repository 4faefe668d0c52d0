"""Python binding of libmoet (ctypes; argument marshalling only).

Every computation runs in the HIP kernels behind the C ABI declared in
``include/moet.h``; this module only checks dtypes/shapes of torch tensors,
allocates outputs with torch, and passes device pointers and the current
stream.  The library must be built (``bit_moe_expert_nvfp4_amd.build``); there
is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Sequence

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoet.so")

MOET_OK, MOET_EINVAL, MOET_EUNSUPPORTED, MOET_EWORKSPACE, MOET_EHIP = range(5)
SOFTMAX, SIGMOID = 0, 1
BALANCE_ZERO_SIGNS = 1
PICK_CODEBOOK = 2
ABI_VERSION = 6        # the moet.h this binding mirrors

_vp = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64


class W2(ctypes.Structure):
    _fields_ = [("codes", _vp), ("scales", _vp), ("scale2", _vp), ("codebook", _vp)]


class FP4(ctypes.Structure):
    _fields_ = [("codes", _vp), ("scales", _vp), ("scale2", _vp)]


class LayerC(ctypes.Structure):
    _fields_ = [("H", _i32), ("I", _i32), ("E", _i32), ("w13", W2), ("w2", W2), ("has_shared", _i32),
                ("shared13", W2), ("shared2", W2), ("n_slots", _i32), ("slot_of_expert", _vp),
                ("d13", FP4), ("d2", FP4), ("swiglu_limit", ctypes.c_float),
                ("base_slot_of_expert", _vp), ("n_base_slots", _i32),
                ("shared_fp4", _i32), ("shared13_fp4", FP4), ("shared2_fp4", FP4)]


_lib = None


class MoetError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


def lib():
    """Load libmoet.so (raises if it was not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with bit_moe_expert_nvfp4_amd.build.build()")
        L = ctypes.CDLL(LIB_PATH)
        L.moet_status_str.argtypes = [ctypes.c_int]
        L.moet_status_str.restype = ctypes.c_char_p
        L.moet_last_error.argtypes = []
        L.moet_last_error.restype = ctypes.c_char_p
        L.moet_abi_version.restype = ctypes.c_int
        if L.moet_abi_version() != ABI_VERSION:
            raise RuntimeError(f"{LIB_PATH} has ABI version {L.moet_abi_version()}, this binding needs "
                               f"{ABI_VERSION}: rebuild it")
        L.moet_requant.argtypes = [_vp, _vp, _vp, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _i64, _vp, _vp, _vp,
                                   ctypes.c_uint32, _vp]
        L.moet_requant.restype = ctypes.c_int
        L.moet_pack_nvfp4.argtypes = [_vp, _vp, _vp, _i64, _i64, _i64, _vp, _vp, _vp, _vp]
        L.moet_pack_nvfp4.restype = ctypes.c_int
        L.moet_remap_mxfp4.argtypes = [_vp, _vp, _i64, _i64, _i64, _vp, _vp, _vp, ctypes.c_uint32, _vp]
        L.moet_remap_mxfp4.restype = ctypes.c_int
        L.moet_requant_fp8.argtypes = [_vp, _vp, _i64, _i64, _i64, _vp, _vp, _vp, ctypes.c_uint32, _vp]
        L.moet_requant_fp8.restype = ctypes.c_int
        L.moet_route.argtypes = [_vp, _i32, _i32, _i32, _i32, _i32, ctypes.c_float, _vp, _vp, _vp, _vp, _vp]
        L.moet_route.restype = ctypes.c_int
        L.moet_moe_workspace_bytes.argtypes = [ctypes.POINTER(LayerC), _i32, _i32]
        L.moet_moe_workspace_bytes.restype = ctypes.c_size_t
        L.moet_moe_forward.argtypes = [ctypes.POINTER(LayerC), _vp, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                       _vp, ctypes.c_size_t, _vp]
        L.moet_moe_forward.restype = ctypes.c_int
        L.moet_moe_forward_noalloc.argtypes = [ctypes.POINTER(LayerC), _vp, _i32, _i32, _vp, _vp, _vp, _vp, _vp,
                                               _vp, _vp, _vp]
        L.moet_moe_forward_noalloc.restype = ctypes.c_int
        L.moet_delta_forward.argtypes = [ctypes.POINTER(FP4), _i32, _i32, _i32, _vp, _vp, _i32, _vp, _vp]
        L.moet_delta_forward.restype = ctypes.c_int
        L.moet_confidence_gate.argtypes = [_vp, _i32, _i32, ctypes.c_float, _vp, _vp, _vp, ctypes.c_size_t, _vp]
        L.moet_gate_workspace_bytes.argtypes = [_i32, _i32]
        L.moet_gate_workspace_bytes.restype = ctypes.c_size_t
        L.moet_confidence_gate.restype = ctypes.c_int
        L.moet_set_timing_events.argtypes = [_vp, _vp]
        L.moet_set_timing_events.restype = ctypes.c_int
        L.moet_probe_read.argtypes = [_vp, ctypes.c_size_t, _vp, _vp]
        L.moet_probe_read.restype = ctypes.c_int
        L.moet_probe_peak.argtypes = [ctypes.c_int, _i32, _vp, _vp]
        L.moet_probe_peak.restype = ctypes.c_int
        _lib = L
    return _lib


def _check(rc: int) -> None:
    if rc != MOET_OK:
        L = lib()
        raise MoetError(rc, f"{L.moet_status_str(rc).decode()}: {L.moet_last_error().decode()}")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _need(t: torch.Tensor, dtype, name: str):
    if t.dtype != dtype or not t.is_cuda or not t.is_contiguous():
        raise TypeError(f"{name} must be a contiguous CUDA tensor of dtype {dtype}, got {t.dtype} on {t.device}")


def _need_shape(t: torch.Tensor, dtype, shape, name: str, device_check: bool = True):
    """ValueError unless t has this dtype and shape, then (device_check) the device/contiguity check of _need."""
    if not isinstance(t, torch.Tensor) or t.dtype != dtype or tuple(t.shape) != tuple(shape):
        got = (t.dtype, tuple(t.shape)) if isinstance(t, torch.Tensor) else type(t).__name__
        raise ValueError(f"{name} must be {dtype} of shape {tuple(shape)}, got {got}")
    if device_check:
        _need(t, dtype, name)


# ---------------------------------------------------------------------------
# moet_requant
# ---------------------------------------------------------------------------
@dataclass
class W2Planes:
    """2-bit planes of a stack of n_mat matrices [N][K] (library layout)."""
    codes: torch.Tensor    # uint32 -> stored as int32 [n_mat, N*K/16]
    scales: torch.Tensor   # uint8 [n_mat, N*K/32]
    scale2: torch.Tensor   # float32 [n_mat]
    N: int
    K: int
    codebook: Optional[torch.Tensor] = None   # uint8 [n_mat] codebook ids (None: codebook 0 everywhere)

    def c(self) -> W2:
        return W2(self.codes.data_ptr(), self.scales.data_ptr(), self.scale2.data_ptr(),
                  self.codebook.data_ptr() if self.codebook is not None else None)


@dataclass
class FP4Planes:
    """FP4 delta planes of a stack of n matrices [N][K] (library layout)."""
    codes: torch.Tensor    # uint8 [n, N*K/2]
    scales: torch.Tensor   # uint8 [n, N*K/16]
    scale2: torch.Tensor   # float32 [n]
    N: int
    K: int

    def c(self) -> FP4:
        return FP4(self.codes.data_ptr(), self.scales.data_ptr(), self.scale2.data_ptr())


def _new_w2(n: int, N: int, K: int, dev) -> W2Planes:
    return W2Planes(torch.empty((n, N * K // 16), dtype=torch.int32, device=dev),
                    torch.empty((n, N * K // 32), dtype=torch.uint8, device=dev),
                    torch.empty((n,), dtype=torch.float32, device=dev), N, K)


def _nvfp4_stack_dims(codes, scales, scale2, scale_group=16):
    """(n, N, K) of a stack of [N][K] matrices (codes uint8 [n, N, K/2], block scales uint8
    [n, N, K/scale_group], optional scale2 f32 [n]); ValueError on any mismatch (the kernels index the
    scales with the dimensions taken from the codes)."""
    if codes.dim() != 3:
        raise ValueError(f"codes must be [n, N, K/2], got {tuple(codes.shape)}")
    n, N, Kh = (int(v) for v in codes.shape)
    K = 2 * Kh
    if tuple(scales.shape) != (n, N, K // scale_group) or K % scale_group:
        raise ValueError(f"scales must be [{n}, {N}, {K // scale_group}], got {tuple(scales.shape)}")
    if scale2 is not None and tuple(scale2.shape) != (n,):
        raise ValueError(f"scale2 must be [{n}], got {tuple(scale2.shape)}")
    return n, N, K


def requant(codes: torch.Tensor, scales: torch.Tensor, scale2: torch.Tensor,
            delta_sel: Optional[torch.Tensor] = None, balance_zero_signs: bool = False,
            pick_codebook: bool = False):
    """NVFP4 stack (codes uint8 [n, N, K/2], scales uint8 [n, N, K/16], scale2 f32 [n]) ->
    W2Planes (and FP4Planes of the matrices listed in delta_sel, int32).  pick_codebook: each
    matrix picks its codebook (W2Planes.codebook holds the ids); otherwise codebook 0."""
    n, N, K = _nvfp4_stack_dims(codes, scales, scale2)
    _need(codes, torch.uint8, "codes")
    _need(scales, torch.uint8, "scales")
    _need(scale2, torch.float32, "scale2")
    dev = codes.device
    w = _new_w2(n, N, K, dev)
    if pick_codebook:
        w.codebook = torch.empty((n,), dtype=torch.uint8, device=dev)
    d = None
    n_sel = 0
    if delta_sel is not None:
        _need(delta_sel, torch.int32, "delta_sel")
        n_sel = int(delta_sel.numel())
        d = FP4Planes(torch.empty((n_sel, N * K // 2), dtype=torch.uint8, device=dev),
                      torch.empty((n_sel, N * K // 16), dtype=torch.uint8, device=dev),
                      torch.empty((n_sel,), dtype=torch.float32, device=dev), N, K)
    _check(lib().moet_requant(_ptr(codes), _ptr(scales), _ptr(scale2), n, N, K,
                              _ptr(w.codes), _ptr(w.scales), _ptr(w.scale2), _ptr(w.codebook),
                              _ptr(delta_sel) if n_sel else None, n_sel,
                              _ptr(d.codes) if d else None, _ptr(d.scales) if d else None,
                              _ptr(d.scale2) if d else None,
                              (BALANCE_ZERO_SIGNS if balance_zero_signs else 0)
                              | (PICK_CODEBOOK if pick_codebook else 0), _stream()))
    return (w, d) if delta_sel is not None else w


def pack_nvfp4(codes: torch.Tensor, scales: torch.Tensor, scale2: torch.Tensor) -> FP4Planes:
    """NVFP4 stack (codes uint8 [n, N, K/2], scales uint8 [n, N, K/16], scale2 f32 [n]) in the FP4
    layout, values unchanged (the form of an NVFP4 shared expert)."""
    n, N, K = _nvfp4_stack_dims(codes, scales, scale2)
    _need(codes, torch.uint8, "codes")
    _need(scales, torch.uint8, "scales")
    _need(scale2, torch.float32, "scale2")
    dev = codes.device
    d = FP4Planes(torch.empty((n, N * K // 2), dtype=torch.uint8, device=dev),
                  torch.empty((n, N * K // 16), dtype=torch.uint8, device=dev),
                  torch.empty((n,), dtype=torch.float32, device=dev), N, K)
    _check(lib().moet_pack_nvfp4(_ptr(codes), _ptr(scales), _ptr(scale2), n, N, K, _ptr(d.codes), _ptr(d.scales),
                                 _ptr(d.scale2), _stream()))
    return d


def remap_mxfp4(codes: torch.Tensor, scales: torch.Tensor, balance_zero_signs: bool = False) -> W2Planes:
    """MXFP4 stack (codes uint8 [n, N, K/2], e8m0 scales uint8 [n, N, K/32]) -> W2Planes."""
    n, N, K = _nvfp4_stack_dims(codes, scales, None, scale_group=32)
    _need(codes, torch.uint8, "codes")
    _need(scales, torch.uint8, "scales")
    w = _new_w2(n, N, K, codes.device)
    _check(lib().moet_remap_mxfp4(_ptr(codes), _ptr(scales), n, N, K, _ptr(w.codes), _ptr(w.scales),
                                  _ptr(w.scale2), BALANCE_ZERO_SIGNS if balance_zero_signs else 0, _stream()))
    return w


def requant_fp8(weights: torch.Tensor, block_scales: torch.Tensor, balance_zero_signs: bool = False) -> W2Planes:
    """FP8 block-quant stack (e4m3fn bytes uint8 [n, N, K], fp32 scales [n, ceil(N/128), K/128]) -> W2Planes."""
    if weights.dim() != 3:
        raise ValueError(f"weights must be [n, N, K], got {tuple(weights.shape)}")
    n, N, K = (int(v) for v in weights.shape)
    if tuple(block_scales.shape) != (n, (N + 127) // 128, K // 128):
        raise ValueError(f"block_scales must be [{n}, {(N + 127) // 128}, {K // 128}], got {tuple(block_scales.shape)}")
    _need(weights, torch.uint8, "weights")
    _need(block_scales, torch.float32, "block_scales")
    w = _new_w2(n, N, K, weights.device)
    _check(lib().moet_requant_fp8(_ptr(weights), _ptr(block_scales), n, N, K, _ptr(w.codes), _ptr(w.scales),
                                  _ptr(w.scale2), BALANCE_ZERO_SIGNS if balance_zero_signs else 0, _stream()))
    return w


# ---------------------------------------------------------------------------
# moet_route
# ---------------------------------------------------------------------------
def route(logits: torch.Tensor, top_k: int, score_fn: int = SIGMOID, renormalize: bool = True,
          route_scale: float = 1.0, out=None):
    """Returns (topk_ids int32 [T,k], topk_w f32 [T,k], expert_offsets int32 [E+1], sorted_pairs int32 [T*k])."""
    if logits.dim() != 2:
        raise ValueError(f"logits must be [T, E], got {tuple(logits.shape)}")
    _need(logits, torch.float32, "logits")
    T, E = (int(v) for v in logits.shape)
    dev = logits.device
    if out is None:
        out = (torch.empty((T, top_k), dtype=torch.int32, device=dev),
               torch.empty((T, top_k), dtype=torch.float32, device=dev),
               torch.empty((E + 1,), dtype=torch.int32, device=dev),
               torch.empty((T * top_k,), dtype=torch.int32, device=dev))
    else:
        for t, dt, shape, name in zip(out, (torch.int32, torch.float32, torch.int32, torch.int32),
                                      ((T, top_k), (T, top_k), (E + 1,), (T * top_k,)),
                                      ("topk_ids", "topk_w", "expert_offsets", "sorted_pairs")):
            _need_shape(t, dt, shape, name)
    ids, w, offs, pairs = out
    _check(lib().moet_route(_ptr(logits), T, E, top_k, score_fn, int(bool(renormalize)), float(route_scale),
                            _ptr(ids), _ptr(w), _ptr(offs), _ptr(pairs), _stream()))
    return ids, w, offs, pairs


# ---------------------------------------------------------------------------
# moet_moe_forward
# ---------------------------------------------------------------------------
@dataclass
class Layer:
    """A MoE layer in library form: w13 = 2E matrices [I][H] (gate 2e, up 2e+1), w2 = E
    matrices [H][I]; optional shared expert; optional FP4 delta cache."""
    H: int
    I: int
    E: int
    w13: W2Planes
    w2: W2Planes
    shared13: Optional[W2Planes] = None
    shared2: Optional[W2Planes] = None
    slot_of_expert: Optional[torch.Tensor] = None   # int32 [E]
    d13: Optional[FP4Planes] = None                 # 2*n_slots matrices [I][H]
    d2: Optional[FP4Planes] = None                  # n_slots matrices [H][I]
    swiglu_limit: float = 0.0
    # expert cache: w13/w2 hold only the experts with base_slot_of_expert[e] >= 0 (int32 [E]), at that slot
    base_slot_of_expert: Optional[torch.Tensor] = None
    # NVFP4 shared expert (instead of shared13 / shared2): gate + up [I][H] and down [H][I] in the FP4 layout
    shared13_fp4: Optional[FP4Planes] = None
    shared2_fp4: Optional[FP4Planes] = None

    def c(self) -> LayerC:
        z = W2(None, None, None)
        zf = FP4(None, None, None)
        n_slots = 0 if self.d2 is None else int(self.d2.scale2.numel())
        sh4 = self.shared13_fp4 is not None
        return LayerC(self.H, self.I, self.E, self.w13.c(), self.w2.c(),
                      1 if (self.shared13 is not None or sh4) else 0,
                      self.shared13.c() if self.shared13 is not None else z,
                      self.shared2.c() if self.shared2 is not None else z,
                      n_slots, self.slot_of_expert.data_ptr() if n_slots else None,
                      self.d13.c() if n_slots else zf, self.d2.c() if n_slots else zf,
                      float(self.swiglu_limit),
                      self.base_slot_of_expert.data_ptr() if self.base_slot_of_expert is not None else None,
                      int(self.w2.scale2.numel()) if self.base_slot_of_expert is not None else 0,
                      1 if sh4 else 0, self.shared13_fp4.c() if sh4 else zf,
                      self.shared2_fp4.c() if sh4 else zf)


def expert_cache(layer: Layer, slot_of_expert) -> Layer:
    """A copy of ``layer`` whose w13/w2 stacks hold only the experts with slot_of_expert[e] >= 0 (int [E],
    host array or tensor), each at its slot; the others are missing from the cache (their routings
    contribute nothing and are counted by moe_forward's miss_count).  Shared expert and delta cache are
    kept as they are."""
    import dataclasses
    soe = torch.as_tensor(slot_of_expert, dtype=torch.int64).cpu()
    if soe.numel() != layer.E:
        raise ValueError(f"slot_of_expert has {soe.numel()} entries, the layer {layer.E} experts")
    n = int(soe.max().item()) + 1 if bool((soe >= 0).any()) else 1
    order = torch.zeros(n, dtype=torch.int64)      # slot -> expert (an unused slot repeats expert 0)
    res = torch.nonzero(soe >= 0).flatten()
    order[soe[res]] = res
    dev = layer.w2.codes.device
    idx13 = torch.stack([2 * order, 2 * order + 1], 1).reshape(-1).to(dev)
    idx2 = order.to(dev)

    def pick(pl: W2Planes, idx) -> W2Planes:
        return W2Planes(pl.codes[idx].contiguous(), pl.scales[idx].contiguous(), pl.scale2[idx].contiguous(),
                        pl.N, pl.K, pl.codebook[idx].contiguous() if pl.codebook is not None else None)
    return dataclasses.replace(layer, w13=pick(layer.w13, idx13), w2=pick(layer.w2, idx2),
                               base_slot_of_expert=soe.to(torch.int32).to(dev))


def moe_workspace_bytes(layer: Layer, T: int, top_k: int) -> int:
    Lc = layer.c()
    return int(lib().moet_moe_workspace_bytes(ctypes.byref(Lc), T, top_k))


def alloc_workspace(layer: Layer, T: int, top_k: int, device="cuda") -> torch.Tensor:
    n = moe_workspace_bytes(layer, T, top_k)
    return torch.empty((max(n, 256),), dtype=torch.uint8, device=device)


def _check_forward_args(layer: Layer, x, topk_ids, topk_w, expert_offsets, sorted_pairs, gate_flags, out,
                        workspace, miss_count):
    """Shapes and dtypes of moe_forward's tensors against the layer (the kernels index x, out and the
    routing arrays with the layer's H and the batch's T, top_k, so a mismatch would read or write out of
    bounds): ValueError on a mismatch, TypeError for a tensor that is not a contiguous CUDA tensor."""
    if not isinstance(x, torch.Tensor) or x.dim() != 2 or x.shape[1] != layer.H or x.shape[0] < 1:
        raise ValueError(f"x must be [T, {layer.H}] (the layer's H), got {tuple(getattr(x, 'shape', ()))}")
    T = int(x.shape[0])
    if not isinstance(topk_ids, torch.Tensor) or topk_ids.dim() != 2 or topk_ids.shape[0] != T:
        raise ValueError(f"topk_ids must be int32 [{T}, top_k], got {tuple(getattr(topk_ids, 'shape', ()))}")
    k = int(topk_ids.shape[1])
    spec = [(x, torch.bfloat16, (T, layer.H), "x"), (topk_ids, torch.int32, (T, k), "topk_ids"),
            (topk_w, torch.float32, (T, k), "topk_w"), (expert_offsets, torch.int32, (layer.E + 1,), "expert_offsets"),
            (sorted_pairs, torch.int32, (T * k,), "sorted_pairs")]
    if gate_flags is not None:
        spec.append((gate_flags, torch.uint8, (T,), "gate_flags"))
    if out is not None:
        spec.append((out, torch.bfloat16, (T, layer.H), "out"))
    if miss_count is not None:
        spec.append((miss_count, torch.int32, (1,), "miss_count"))
    if workspace is not None:
        spec.append((workspace, torch.uint8, (workspace.numel(),), "workspace"))
    for name in ("w13", "w2", "shared13", "shared2"):     # per-matrix codebook ids: one per matrix of the stack
        pl = getattr(layer, name)
        if pl is not None and pl.codebook is not None:
            spec.append((pl.codebook, torch.uint8, (pl.scale2.numel(),), f"{name}.codebook"))
    for t, dt, shape, name in spec:        # every shape first, so a mismatch is reported as such
        _need_shape(t, dt, shape, name, device_check=False)
    for t, dt, _, name in spec:
        _need(t, dt, name)
    return T, k


def moe_forward(layer: Layer, x: torch.Tensor, topk_ids, topk_w, expert_offsets, sorted_pairs,
                gate_flags: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                workspace: Optional[torch.Tensor] = None, miss_count: Optional[torch.Tensor] = None) -> torch.Tensor:
    T, k = _check_forward_args(layer, x, topk_ids, topk_w, expert_offsets, sorted_pairs, gate_flags, out,
                               workspace, miss_count)
    H = layer.H
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
    if workspace is None:
        workspace = alloc_workspace(layer, T, k, x.device)
    Lc = layer.c()
    _check(lib().moet_moe_forward(ctypes.byref(Lc), _ptr(x), T, k, _ptr(topk_ids), _ptr(topk_w),
                                  _ptr(expert_offsets), _ptr(sorted_pairs), _ptr(gate_flags), _ptr(out),
                                  _ptr(miss_count), _ptr(workspace), workspace.numel(), _stream()))
    return out


#: bytes of the static scratch of moe_forward_noalloc (MOET_NOALLOC_SCRATCH_BYTES in include/moet.h)
NOALLOC_SCRATCH_BYTES = 16 << 20


def moe_forward_noalloc(layer: Layer, x: torch.Tensor, topk_ids, topk_w, expert_offsets, sorted_pairs,
                        out: torch.Tensor, gate_flags: Optional[torch.Tensor] = None,
                        miss_count: Optional[torch.Tensor] = None) -> torch.Tensor:
    """moet_moe_forward_noalloc: the layer forward with the library's static scratch instead of a
    workspace; the caller passes every input and the output (nothing is allocated)."""
    T, k = _check_forward_args(layer, x, topk_ids, topk_w, expert_offsets, sorted_pairs, gate_flags, out,
                               None, miss_count)
    Lc = layer.c()
    _check(lib().moet_moe_forward_noalloc(ctypes.byref(Lc), _ptr(x), T, k, _ptr(topk_ids), _ptr(topk_w),
                                          _ptr(expert_offsets), _ptr(sorted_pairs), _ptr(gate_flags), _ptr(out),
                                          _ptr(miss_count), _stream()))
    return out


# ---------------------------------------------------------------------------
# moet_delta_forward
# ---------------------------------------------------------------------------
def delta_forward(D: FP4Planes, act: torch.Tensor, row_slot: torch.Tensor, acc: torch.Tensor) -> torch.Tensor:
    """acc[r] += D[row_slot[r]] @ act[r] (in place) for rows with a valid slot."""
    if not isinstance(act, torch.Tensor) or act.dim() != 2 or act.shape[1] != D.K:
        raise ValueError(f"act must be [R, {D.K}] (the planes' K), got {tuple(getattr(act, 'shape', ()))}")
    R, K = (int(v) for v in act.shape)
    for t, dt, shape, name in ((act, torch.bfloat16, (R, K), "act"), (row_slot, torch.int32, (R,), "row_slot"),
                               (acc, torch.float32, (R, D.N), "acc")):
        _need_shape(t, dt, shape, name, device_check=False)
    _need(act, torch.bfloat16, "act")
    _need(row_slot, torch.int32, "row_slot")
    _need(acc, torch.float32, "acc")
    Dc = D.c()
    _check(lib().moet_delta_forward(ctypes.byref(Dc), int(D.scale2.numel()), D.N, K, _ptr(act), _ptr(row_slot), R,
                                    _ptr(acc), _stream()))
    return acc


def gate_workspace_bytes(T: int, V: int) -> int:
    """moet_gate_workspace_bytes: device bytes the confidence gate needs for T rows of V logits."""
    return int(lib().moet_gate_workspace_bytes(int(T), int(V)))


def confidence_gate(logits: torch.Tensor, tau: float = 0.60, flags: Optional[torch.Tensor] = None,
                    confidence: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
    """moet_confidence_gate: uint8 [T] flags (1 = largest next-token probability below tau) from fp32
    logits [T, V]; optionally the confidence itself into an fp32 [T] tensor.  The workspace (uint8,
    gate_workspace_bytes(T, V) bytes) is allocated per call unless given.  Returns the flags."""
    if not isinstance(logits, torch.Tensor) or logits.dim() != 2:
        raise ValueError(f"logits must be [T, V], got {tuple(getattr(logits, 'shape', ()))}")
    T, V = (int(v) for v in logits.shape)
    if flags is not None:
        _need_shape(flags, torch.uint8, (T,), "flags", device_check=False)
    if confidence is not None:
        _need_shape(confidence, torch.float32, (T,), "confidence", device_check=False)
    _need(logits, torch.float32, "logits")
    if flags is None:
        flags = torch.empty((T,), dtype=torch.uint8, device=logits.device)
    _need(flags, torch.uint8, "flags")
    if confidence is not None:
        _need(confidence, torch.float32, "confidence")
    need = gate_workspace_bytes(T, V)
    if workspace is None and need:
        workspace = torch.empty((need,), dtype=torch.uint8, device=logits.device)
    nbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().moet_confidence_gate(_ptr(logits), T, V, float(tau), _ptr(flags), _ptr(confidence),
                                      _ptr(workspace), nbytes, _stream()))
    return flags


def set_timing_events(start: Optional[torch.cuda.Event], stop: Optional[torch.cuda.Event]) -> None:
    """Time the first expert kernel of the following moe_forward calls with these (recorded
    at least once, so that torch has created them) torch events; None, None disables."""
    if start is None:
        _check(lib().moet_set_timing_events(None, None))
    else:
        _check(lib().moet_set_timing_events(ctypes.c_void_p(start.cuda_event), ctypes.c_void_p(stop.cuda_event)))


PROBE_SINK_WORDS = 8192


def probe_read(buf: torch.Tensor, sink: torch.Tensor) -> None:
    """Measurement reference (moet_probe_read): read every byte of the contiguous device tensor `buf`
    once with the weight kernels' access shape; `sink` is an int32 device tensor of PROBE_SINK_WORDS."""
    if not buf.is_contiguous() or sink.dtype != torch.int32 or sink.numel() < PROBE_SINK_WORDS:
        raise ValueError("probe_read needs a contiguous buffer and an int32 sink of PROBE_SINK_WORDS words")
    if not buf.is_cuda or not sink.is_cuda or not sink.is_contiguous():
        raise TypeError("probe_read needs device tensors")
    _check(lib().moet_probe_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink), _stream()))


PROBE_MFMA_BF16, PROBE_DOT2_BF16 = 0, 1
PROBE_PEAK_WAVES = 4096   # waves of one moet_probe_peak launch


def probe_peak(kind: int, iters: int, sink: torch.Tensor) -> None:
    """Measurement reference (moet_probe_peak): a tight loop of bf16 MFMAs (PROBE_MFMA_BF16: 4 x 32,768
    flops per round per wave) or dot2 instructions (PROBE_DOT2_BF16: 8 per round per wave) over
    PROBE_PEAK_WAVES waves; `sink` is an int32 device tensor of PROBE_SINK_WORDS."""
    if sink.dtype != torch.int32 or sink.numel() < PROBE_SINK_WORDS:
        raise ValueError("probe_peak needs an int32 sink of PROBE_SINK_WORDS words")
    if not sink.is_cuda or not sink.is_contiguous():
        raise TypeError("probe_peak needs a contiguous device sink")
    _check(lib().moet_probe_peak(int(kind), int(iters), _ptr(sink), _stream()))


# ---------------------------------------------------------------------------
# Building a layer from NVFP4 sources
# ---------------------------------------------------------------------------
def layer_from_nvfp4(src, slot_of_expert: Optional[torch.Tensor] = None, swiglu_limit: float = 0.0,
                     device="cuda", shared_nvfp4: bool = False, pick_codebook: bool = False) -> Layer:
    """Requantise an NVFP4 layer (synth.NVFP4Layer-like: w13/w2/shared13/shared2 tuples of
    (codes, scales, scale2)) on the GPU and build the library layer; experts with
    slot_of_expert >= 0 also get their FP4 delta.  shared_nvfp4 keeps the shared expert
    in NVFP4 instead of requantising it.  pick_codebook: every matrix picks its codebook."""
    cfg = src.cfg
    pk = dict(pick_codebook=pick_codebook)

    def dev(t):
        return t.to(device, non_blocking=True).contiguous()

    w13_src = tuple(dev(t) for t in src.w13)
    w2_src = tuple(dev(t) for t in src.w2)
    d13 = d2 = None
    if slot_of_expert is not None and int((slot_of_expert >= 0).sum()) > 0:
        soe = slot_of_expert.to(torch.int64)
        n_slots = int(soe.max()) + 1
        res = torch.full((n_slots,), -1, dtype=torch.int64)
        for e in range(cfg.E):
            if soe[e] >= 0:
                res[soe[e]] = e
        sel13 = torch.stack([2 * res, 2 * res + 1], dim=1).reshape(-1).to(torch.int32).to(device)
        sel2 = res.to(torch.int32).to(device)
        w13, d13 = requant(*w13_src, delta_sel=sel13, **pk)
        w2, d2 = requant(*w2_src, delta_sel=sel2, **pk)
        slot_dev = slot_of_expert.to(torch.int32).to(device)
    else:
        w13 = requant(*w13_src, **pk)
        w2 = requant(*w2_src, **pk)
        slot_dev = None
    sh13 = sh2 = f13 = f2 = None
    if src.shared13 is not None and shared_nvfp4:
        f13 = pack_nvfp4(*(dev(t) for t in src.shared13))
        f2 = pack_nvfp4(*(dev(t) for t in src.shared2))
    elif src.shared13 is not None:
        sh13 = requant(*(dev(t) for t in src.shared13), **pk)
        sh2 = requant(*(dev(t) for t in src.shared2), **pk)
    return Layer(cfg.H, cfg.I, cfg.E, w13, w2, sh13, sh2, slot_dev, d13, d2, swiglu_limit,
                 shared13_fp4=f13, shared2_fp4=f2)
