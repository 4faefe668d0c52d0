"""Seeded synthetic inputs shaped like the pages' models.

This module only *produces inputs*: synthetic NVFP4 checkpoints, activations,
router logits, delta-cache residency and gate flags.  It holds none of the
layer's own arithmetic (no requantisation, routing or FFN), so both the HIP
path and the CPU oracle may consume what it makes.

Synthetic checkpoint recipe: W ~ N(0, 0.02^2) in fp32 per matrix [N][K], then
a modelopt-style NVFP4 export: scale_2 = amax(|W|) / (6*448); per 16 weights
along K the e4m3 block scale is amax16 / (6*scale_2) cast to e4m3fn
(nearest-even, via torch's float8 cast); each weight is the nearest e2m1
magnitude to W / (S*scale_2) (ties to the smaller magnitude) with W's sign.
Two codes per byte, the even k in the low nibble.

Shapes follow the pages (README "Frontier MoE on consumer Blackwell
(SM120)", sections "Kimi-K2.7-Code (1T MoE) on 4x RTX PRO 6000" and
"How it fits"): hidden 7168, expert intermediate 2048, 256 or 384 routed
experts, top-8, MTP decode with 1 + 2 tokens per step.
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass, field
from typing import Optional

import torch

SOFTMAX = 0
SIGMOID = 1


@dataclass(frozen=True)
class LayerConfig:
    name: str
    T: int
    H: int
    I: int
    E: int
    k: int
    score: int
    renormalize: bool = True
    shared: bool = False
    n_resident: int = 0          # experts with an FP4 delta in the cache
    n_flagged: int = 0           # tokens flagged by the confidence gate
    logits: str = "normal"       # "normal" or "zipf"
    zipf_s: float = 1.1
    swiglu_limit: float = 0.0
    notes: str = ""


CONFIGS = {
    "tiny": LayerConfig("tiny", T=4, H=256, I=128, E=8, k=2, score=SOFTMAX,
                   notes="parity config"),
    "decode_mtp": LayerConfig("decode_mtp", T=3, H=7168, I=2048, E=256, k=8, score=SIGMOID, shared=True,
                   notes="single-stream MTP decode, 1 + 2 tokens, 2-bit base only"),
    "decode_mtp_delta": LayerConfig("decode_mtp_delta", T=3, H=7168, I=2048, E=256, k=8, score=SIGMOID, shared=True,
                   n_resident=32, n_flagged=2, notes="decode + FP4 delta for 32 experts, 2 of 3 tokens gated"),
    "batched_decode": LayerConfig("batched_decode", T=24, H=7168, I=2048, E=384, k=8, score=SIGMOID,
                   n_resident=64, n_flagged=12, logits="zipf",
                   notes="8 streams x 3 tokens, Zipf(1.1) expert popularity"),
    "prefill": LayerConfig("prefill", T=4096, H=7168, I=2048, E=256, k=8, score=SIGMOID,
                   notes="prefill chunk, MFMA grouped GEMM"),
}


def _seed(*parts) -> int:
    h = hashlib.sha256(("/".join(str(p) for p in parts)).encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def _gen(device, *parts) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(_seed(*parts))
    return g


_E2M1_MIDPOINTS = (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0)


def nvfp4_export(W: torch.Tensor, plus_zeros: bool = False):
    """modelopt-style NVFP4 export of one fp32 matrix [N, K] (synthetic checkpoint maker).

    plus_zeros: write every zero code as +0, as an export from integer weights does.
    Returns (codes uint8 [N, K/2], scales uint8 [N, K/16], scale_2 float32 0-dim)."""
    N, K = W.shape
    amax = W.abs().amax().clamp_min(1e-30)
    scale_2 = (amax / (6.0 * 448.0)).to(torch.float32)
    blk = W.view(N, K // 16, 16)
    bmax = blk.abs().amax(dim=-1)
    s = (bmax / (6.0 * scale_2)).clamp(max=448.0).to(torch.float8_e4m3fn)
    denom = (s.to(torch.float32) * scale_2).unsqueeze(-1)
    r = torch.where(denom > 0, blk / torch.where(denom > 0, denom, torch.ones_like(denom)),
                    torch.zeros_like(blk))
    bounds = torch.tensor(_E2M1_MIDPOINTS, dtype=torch.float32, device=W.device)
    mag = torch.bucketize(r.abs().contiguous(), bounds, right=False).to(torch.uint8)
    neg = (blk < 0) & (mag > 0) if plus_zeros else (blk < 0)
    code = mag | (neg.to(torch.uint8) << 3)
    code = code.view(N, K)
    packed = (code[:, 0::2] & 15) | ((code[:, 1::2] & 15) << 4)
    return packed.contiguous(), s.view(torch.uint8).contiguous(), scale_2


def make_nvfp4_stack(n_mat: int, N: int, K: int, seed: int, tag: str, device="cpu", std: float = 0.02,
                     plus_zeros: bool = False):
    """A stack of n_mat NVFP4 matrices [N, K]; matrix i is seeded by (seed, tag, i)."""
    codes = torch.empty((n_mat, N, K // 2), dtype=torch.uint8, device=device)
    scales = torch.empty((n_mat, N, K // 16), dtype=torch.uint8, device=device)
    s2 = torch.empty((n_mat,), dtype=torch.float32, device=device)
    for i in range(n_mat):
        g = _gen(device, seed, tag, i)
        W = torch.randn((N, K), generator=g, device=device, dtype=torch.float32) * std
        c, s, sc2 = nvfp4_export(W, plus_zeros=plus_zeros)
        codes[i], scales[i], s2[i] = c, s, sc2
        del W
    return codes, scales, s2


# e2m1 magnitude of each 3-bit magnitude code
_E2M1_MAGS = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)


def skew_magnitudes(codes: torch.Tensor, mats, targets, frac: float, seed: int, tag: str) -> torch.Tensor:
    """A copy of an NVFP4 code stack [n, N, K/2] in which, in the matrices `mats`, a random fraction
    `frac` of the codes take the nearer (by e2m1 value, ties to the first) of the two magnitude codes
    `targets`, sign kept: weights concentrated on two magnitudes, the shape of a tensor that another
    sign-symmetric four-level codebook than {-4,-1,1,4} fits better."""
    out = codes.clone()
    dev = out.device
    lut = torch.tensor([min(targets, key=lambda t: (abs(_E2M1_MAGS[t] - _E2M1_MAGS[m]), targets.index(t)))
                        for m in range(8)], dtype=torch.uint8, device=dev)
    for i in mats:
        g = _gen(dev, seed, tag, "skew", i)        # the stream depends on the device, as for the weights
        c = out[i]
        nib = torch.stack([c & 15, c >> 4], dim=-1)                       # [N, K/2, 2]
        pick = torch.rand(nib.shape, generator=g, device=dev) < frac
        moved = (nib & 8) | lut[(nib & 7).long()]
        nib = torch.where(pick, moved, nib)
        out[i] = nib[..., 0] | (nib[..., 1] << 4)
    return out


def mxfp4_export(W: torch.Tensor):
    """OCP microscaling FP4 export of one fp32 matrix [N, K]: per 32 weights along K
    the e8m0 scale is 2^(floor(log2(amax32)) - 2) (2 = the largest e2m1 exponent),
    E = 127 for an all-zero block; each weight is the nearest e2m1 magnitude to
    W / scale (ties to the smaller magnitude, saturating at 6) with W's sign.
    Returns (codes uint8 [N, K/2], scales uint8 [N, K/32])."""
    N, K = W.shape
    blk = W.view(N, K // 32, 32)
    bmax = blk.abs().amax(dim=-1)
    _, ex = torch.frexp(bmax)                       # bmax = f * 2^ex, 0.5 <= f < 1
    E = torch.where(bmax > 0, ex - 1 - 2 + 127, torch.full_like(ex, 127)).clamp(0, 254)
    scale = torch.exp2((E - 127).to(torch.float64)).to(torch.float32).unsqueeze(-1)
    r = blk / scale
    bounds = torch.tensor(_E2M1_MIDPOINTS, dtype=torch.float32, device=W.device)
    mag = torch.bucketize(r.abs().contiguous(), bounds, right=False).to(torch.uint8)
    code = (mag | ((blk < 0).to(torch.uint8) << 3)).view(N, K)
    packed = (code[:, 0::2] & 15) | ((code[:, 1::2] & 15) << 4)
    return packed.contiguous(), E.to(torch.uint8).contiguous()


def fp8_block_export(W: torch.Tensor):
    """FP8 block-quant export of one fp32 matrix [N, K]: one fp32 scale per
    128 x 128 block, amax / 448 (1 for an all-zero block); weight = e4m3fn
    nearest-even cast of W / scale (torch's float8 cast).
    Returns (w uint8 [N, K], bscale float32 [ceil(N/128), K/128])."""
    N, K = W.shape
    Np = (N + 127) // 128 * 128
    Wp = torch.zeros((Np, K), dtype=torch.float32, device=W.device)
    Wp[:N] = W
    blk = Wp.view(Np // 128, 128, K // 128, 128)
    bmax = blk.abs().amax(dim=(1, 3))
    s = torch.where(bmax > 0, bmax / 448.0, torch.ones_like(bmax))
    q = (blk / s[:, None, :, None]).clamp(-448.0, 448.0).to(torch.float8_e4m3fn)
    return q.view(torch.uint8).reshape(Np, K)[:N].contiguous(), s.contiguous()


def make_mxfp4_stack(n_mat: int, N: int, K: int, seed: int, tag: str, std: float = 0.02, device="cpu"):
    """A stack of n_mat MXFP4 matrices [N, K] (codes [n_mat, N, K/2], e8m0 scales [n_mat, N, K/32])."""
    codes = torch.empty((n_mat, N, K // 2), dtype=torch.uint8, device=device)
    scales = torch.empty((n_mat, N, K // 32), dtype=torch.uint8, device=device)
    for i in range(n_mat):
        W = torch.randn((N, K), generator=_gen(device, seed, tag, i), device=device, dtype=torch.float32) * std
        codes[i], scales[i] = mxfp4_export(W)
    return codes, scales


def make_fp8_stack(n_mat: int, N: int, K: int, seed: int, tag: str, std: float = 0.02, device="cpu"):
    """A stack of n_mat FP8 block-quant matrices [N, K] (weights [n_mat, N, K], scales
    [n_mat, ceil(N/128), K/128])."""
    w = torch.empty((n_mat, N, K), dtype=torch.uint8, device=device)
    s = torch.empty((n_mat, (N + 127) // 128, K // 128), dtype=torch.float32, device=device)
    for i in range(n_mat):
        W = torch.randn((N, K), generator=_gen(device, seed, tag, i), device=device, dtype=torch.float32) * std
        w[i], s[i] = fp8_block_export(W)
    return w, s


@dataclass
class NVFP4Layer:
    """NVFP4 source weights of one MoE layer.

    w13: gate/up as a stack of 2E matrices [I, H] (expert e: gate = 2e, up = 2e+1);
    w2: down as a stack of E matrices [H, I]; shared13 / shared2 likewise for one
    shared expert (or None)."""
    cfg: LayerConfig
    w13: tuple
    w2: tuple
    shared13: Optional[tuple] = None
    shared2: Optional[tuple] = None


def make_layer(cfg: LayerConfig, seed: int = 0, device="cpu", layer_index: int = 0) -> NVFP4Layer:
    w13 = make_nvfp4_stack(2 * cfg.E, cfg.I, cfg.H, seed, f"{cfg.name}/L{layer_index}/w13", device)
    w2 = make_nvfp4_stack(cfg.E, cfg.H, cfg.I, seed, f"{cfg.name}/L{layer_index}/w2", device)
    sh13 = sh2 = None
    if cfg.shared:
        sh13 = make_nvfp4_stack(2, cfg.I, cfg.H, seed, f"{cfg.name}/L{layer_index}/shared13", device)
        sh2 = make_nvfp4_stack(1, cfg.H, cfg.I, seed, f"{cfg.name}/L{layer_index}/shared2", device)
    return NVFP4Layer(cfg, w13, w2, sh13, sh2)


def make_activations(T: int, H: int, seed: int, tag: str = "x", device="cpu") -> torch.Tensor:
    """bf16 [T, H] ~ N(0, 1) (cast with round-to-nearest-even)."""
    g = _gen(device, seed, tag, T, H)
    return torch.randn((T, H), generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)


def make_logits(cfg: LayerConfig, seed: int, tag: str = "logits", device="cpu") -> torch.Tensor:
    """fp32 router logits [T, E]: N(0,1), or Zipf-Gumbel (l = -s*ln(rank(e)) + Gumbel(0,1)
    with rank a seeded permutation of 1..E, which makes top-k a Plackett-Luce draw from Zipf(s))."""
    g = _gen(device, seed, tag, cfg.name)
    if cfg.logits == "normal":
        return torch.randn((cfg.T, cfg.E), generator=g, device=device, dtype=torch.float32)
    rank = expert_ranks(cfg, seed).to(device).to(torch.float32)
    u = torch.rand((cfg.T, cfg.E), generator=g, device=device, dtype=torch.float32).clamp(1e-12, 1 - 1e-7)
    gumbel = -torch.log(-torch.log(u))
    return (-cfg.zipf_s * torch.log(rank)).unsqueeze(0) + gumbel


def expert_ranks(cfg: LayerConfig, seed: int) -> torch.Tensor:
    """Popularity rank (1 = hottest) of each expert, a seeded permutation of 1..E."""
    g = _gen("cpu", seed, "rank", cfg.name)
    return torch.randperm(cfg.E, generator=g) + 1


def slot_of_expert(cfg: LayerConfig, seed: int) -> torch.Tensor:
    """int32 [E]: delta-cache slot of each expert, -1 when not resident.  Zipf layers keep
    the hottest experts resident; the others pick a seeded subset."""
    out = torch.full((cfg.E,), -1, dtype=torch.int32)
    if cfg.n_resident == 0:
        return out
    if cfg.logits == "zipf":
        rank = expert_ranks(cfg, seed)
        res = torch.argsort(rank)[: cfg.n_resident]
    else:
        g = _gen("cpu", seed, "resident", cfg.name)
        res = torch.randperm(cfg.E, generator=g)[: cfg.n_resident]
    res = torch.sort(res).values
    out[res] = torch.arange(cfg.n_resident, dtype=torch.int32)
    return out


def gate_flags(cfg: LayerConfig, seed: int, tag: str = "gate") -> torch.Tensor:
    """uint8 [T]: 1 for the tokens the confidence gate flags (a seeded subset)."""
    g = _gen("cpu", seed, tag, cfg.name)
    f = torch.zeros((cfg.T,), dtype=torch.uint8)
    if cfg.n_flagged:
        f[torch.randperm(cfg.T, generator=g)[: cfg.n_flagged]] = 1
    return f
