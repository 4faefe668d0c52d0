"""Shared helpers for the parity tests: run the oracle on the same seeded
inputs the HIP path consumes and compare.  Nothing here computes the method
itself; it only moves bytes between torch and the oracle."""
from __future__ import annotations

import numpy as np
import torch

from oracle import formats as OF
from oracle import layout as OL
from oracle import requant as OR
from oracle import route as ORT
from oracle import ffn as OFF


def np_(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


class OracleMatrix:
    """Oracle requant (and optional delta) of one NVFP4 matrix, plus its packed layout.  pick: the
    matrix picks its codebook (else codebook 0)."""

    def __init__(self, codes: np.ndarray, scales: np.ndarray, scale_2: float, with_delta: bool = False,
                 pick: bool = False):
        self.codes, self.scales, self.scale_2 = codes, scales, float(scale_2)
        if pick:
            self.cb, self.c2, self.tau, self.s2, self.totals = OR.pick_codebook(codes, scales, scale_2)
        else:
            self.cb = 0
            self.c2, self.tau, self.s2 = OR.requant(codes, scales, scale_2)
        self.N, self.K = self.c2.shape
        self.dc = self.ds = self.d2 = None
        if with_delta:
            self.dc, self.ds, self.d2 = OR.delta(codes, scales, scale_2, self.c2, self.tau, codebook=self.cb)

    def packed_codes(self):
        return OL.pack_2bit_codes(self.c2)

    def packed_scales(self):
        return OL.pack_2bit_scales(self.tau)

    def packed_delta(self):
        return OL.pack_fp4_codes(self.dc), OL.pack_fp4_scales(self.ds)

    def w2bit(self):
        return OR.dequant_2bit(self.c2, self.tau, self.s2, codebook=self.cb)

    def wdelta(self):
        return OR.dequant_fp4_codes(self.dc, self.ds, self.d2)


#: e2m1 magnitude codes of 1/2 and 3 (codebook 1's levels) and of 0 and 2 (codebook 2's)
C1_MAGS = (1, 5)
C2_MAGS = (0, 4)


def mixed_codebook_layer(src, seed):
    """The synthetic layer `src` with some matrices moved towards codebook 1 or 2
    (synth.skew_magnitudes): expert e's gate for e % 3 == 1, its up for e % 3 == 2, both (gate 1,
    up 2) for e % 4 == 3; its down to 1 for odd e and to 2 for e % 6 == 0; the shared expert's gate
    to 2 and its down to 1."""
    from bit_moe_expert_nvfp4_amd import synth
    E = src.cfg.E
    g1 = [2 * e for e in range(E) if e % 3 == 1 or e % 4 == 3]
    u2 = [2 * e + 1 for e in range(E) if e % 3 == 2 or e % 4 == 3]
    c13 = synth.skew_magnitudes(src.w13[0], g1, C1_MAGS, 0.9, seed, "w13c1")
    c13 = synth.skew_magnitudes(c13, u2, C2_MAGS, 0.95, seed, "w13c2")
    d1 = [e for e in range(E) if e % 2 == 1]
    d2 = [e for e in range(E) if e % 6 == 0]
    c2 = synth.skew_magnitudes(src.w2[0], d1, C1_MAGS, 0.9, seed, "w2c1")
    c2 = synth.skew_magnitudes(c2, d2, C2_MAGS, 0.95, seed, "w2c2")
    sh13, sh2 = src.shared13, src.shared2
    if sh13 is not None:
        sh13 = (synth.skew_magnitudes(sh13[0], [0], C2_MAGS, 0.95, seed, "sh13"),) + tuple(sh13[1:])
        sh2 = (synth.skew_magnitudes(sh2[0], [0], C1_MAGS, 0.9, seed, "sh2"),) + tuple(sh2[1:])
    return synth.NVFP4Layer(src.cfg, (c13,) + tuple(src.w13[1:]), (c2,) + tuple(src.w2[1:]), sh13, sh2)


class ExpertPrefetch:
    """Calls fn(e) for the experts of `order` on a thread pool, up to `window` experts ahead of the
    caller, who then asks for them in that order (the oracle's C requantisation and numpy's large
    array operations run without the interpreter lock).  An expert asked for out of order is computed
    on the spot."""

    def __init__(self, fn, order, window=8, workers=8):
        from concurrent.futures import ThreadPoolExecutor
        self.fn = fn
        self.order = list(order)
        self.ex = ThreadPoolExecutor(workers)
        self.fut = {}
        self.next = 0
        self.window = window
        self._fill()

    def _fill(self):
        while self.next < len(self.order) and len(self.fut) < self.window:
            e = self.order[self.next]
            self.fut[e] = self.ex.submit(self.fn, e)
            self.next += 1

    def __call__(self, e):
        f = self.fut.pop(e, None)
        r = f.result() if f is not None else self.fn(e)
        self._fill()
        return r

    def close(self):
        self.ex.shutdown(wait=True)


class OracleLayer:
    """Lazily requantises the experts the oracle needs, straight from the NVFP4 bytes."""

    def __init__(self, src, slot_of_expert=None, shared_nvfp4=False, pick_codebook=False):
        self.src = src
        self.cfg = src.cfg
        self.soe = None if slot_of_expert is None else np_(slot_of_expert)
        self.shared_nvfp4 = shared_nvfp4
        self.pick = pick_codebook
        self._cache = {}
        self._prefetch = None
        # host copies of the NVFP4 stacks, made once (threads then slice them without the GPU)
        self._host = {}

    def prefetch(self, experts):
        """Compute expert_weights for these experts (ascending order) ahead of their use."""
        if self._prefetch is not None:
            self._prefetch.close()
        self._host_stack(self.src.w13)       # one host copy of each stack before the threads start
        self._host_stack(self.src.w2)
        self._prefetch = ExpertPrefetch(self._expert_weights, sorted(int(e) for e in experts))

    def _host_stack(self, stack):
        key = id(stack)
        if key not in self._host:
            self._host[key] = tuple(np_(t) if isinstance(t, torch.Tensor) else t for t in stack)
        return self._host[key]

    def _mat(self, stack, i, with_delta):
        key = (id(stack), i, with_delta)
        if key not in self._cache:
            c, s, s2 = self._host_stack(stack)
            self._cache[key] = OracleMatrix(c[i], s[i], float(s2[i]), with_delta, pick=self.pick)
        return self._cache[key]

    def resident(self, e):
        return self.soe is not None and self.soe[e] >= 0

    def expert(self, e):
        d = self.resident(e)
        g = self._mat(self.src.w13, 2 * e, d)
        u = self._mat(self.src.w13, 2 * e + 1, d)
        dn = self._mat(self.src.w2, e, d)
        return g, u, dn

    def _expert_weights(self, e):
        g, u, dn = self.expert(e)
        return g.w2bit(), u.w2bit(), dn.w2bit()

    def expert_weights(self, e):
        if self._prefetch is not None:
            return self._prefetch(e)
        return self._expert_weights(e)

    def delta_weights_of_slot(self, slot):
        e = int(np.nonzero(self.soe == slot)[0][0])
        g, u, dn = self.expert(e)
        return g.wdelta(), u.wdelta(), dn.wdelta()

    def shared_weights(self):
        if self.src.shared13 is None:
            return None
        if self.shared_nvfp4:      # the shared expert keeps its NVFP4 values
            dq = lambda st, i: OF.nvfp4_decode(np_(st[0][i]), np_(st[1][i]), float(st[2][i]))
            return dq(self.src.shared13, 0), dq(self.src.shared13, 1), dq(self.src.shared2, 0)
        g = self._mat(self.src.shared13, 0, False)
        u = self._mat(self.src.shared13, 1, False)
        dn = self._mat(self.src.shared2, 0, False)
        return g.w2bit(), u.w2bit(), dn.w2bit()

    def forward(self, x_bits, ids, w, gate_flags=None, tokens=None, resident=None):
        return OFF.moe_forward(x_bits, ids, w, self.expert_weights, self.shared_weights(),
                               gate_flags=gate_flags, slot_of_expert=self.soe,
                               delta_weights=self.delta_weights_of_slot if self.soe is not None else None,
                               swiglu_limit=self.cfg.swiglu_limit, tokens=tokens, resident=resident)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return np_(t.contiguous().view(torch.int16)).astype(np.uint16)


def rel_l2(gpu_bits: np.ndarray, ref_bits: np.ndarray) -> float:
    a = OF.bf16_bits_to_f64(gpu_bits)
    b = OF.bf16_bits_to_f64(ref_bits)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def oracle_route(logits: torch.Tensor, k: int, fn: int, renorm: bool = True, scale: float = 1.0):
    return ORT.route(np_(logits), k, fn, renorm, scale)


#: floating-point bar of the method (relative L2 error of the layer output)
REL_L2_BAR = 2e-3


# ---------------------------------------------------------------------------
# Element-wise comparison of the layer's intermediate rows (h, y) and output.
# The forward's workspace holds, after a call, h = bf16(silu(g) * u) rows and
# fp32 y rows: h by pair id on the GEMV path, by sorted position on the MFMA
# grouped-GEMM path (the shared expert at row T*k + t on both); y by pair id.
# ---------------------------------------------------------------------------
def _al256(b: int) -> int:
    return (b + 255) & ~255


def workspace_views(ws: torch.Tensor, T: int, k: int, H: int, I: int):
    """(h bits uint16 [T*k + T, I], y fp32 [T*k + T, H]) views of a forward's workspace."""
    rows = T * k + T
    hb = ws[:rows * I * 2].view(torch.int16).view(rows, I)
    off = _al256(rows * I * 2)
    y = ws[off:off + rows * H * 4].view(torch.float32).view(rows, H)
    return hb, y


def partitioned_order(ids: np.ndarray, sorted_pairs: np.ndarray, offsets: np.ndarray, soe, gate_flags, resident=None):
    """The pair order of the grouped-GEMM path with a gated delta: each expert's run of sorted pairs,
    with the pairs of gate-flagged tokens first when the expert takes the delta (it holds a delta
    slot no lower expert holds, and its 2-bit planes are resident); both parts keep their order.
    Returns (order, flagged count per expert)."""
    T, k = ids.shape
    E = len(offsets) - 1
    order = np.asarray(sorted_pairs, dtype=np.int64).copy()
    nflag = np.zeros(E, dtype=np.int64)
    seen = set()
    for e in range(E):
        run = order[offsets[e]:offsets[e + 1]].copy()
        ds = int(soe[e]) if soe is not None else -1
        takes = ds >= 0 and ds not in seen and (resident is None or resident[e])
        if ds >= 0:
            seen.add(ds)
        if not takes:
            continue
        fl = np.asarray(gate_flags)[run // k] != 0
        order[offsets[e]:offsets[e + 1]] = np.concatenate([run[fl], run[~fl]])
        nflag[e] = int(fl.sum())
    return order, nflag


def mfma_path(T: int, k: int, H: int) -> bool:
    """Whether moet_moe_forward runs the grouped-GEMM kernels for this batch (else the GEMV kernels)."""
    return T * k > 1024 and H % 256 == 0


def ulp_bf16(v: np.ndarray) -> np.ndarray:
    """Spacing of bf16 values at |v| (subnormal spacing below 2^-126)."""
    a = np.abs(np.asarray(v, dtype=np.float64))
    _, ex = np.frexp(np.where(a > 0, a, 1.0))
    return np.exp2(np.maximum(ex - 1, -126) - 7.0)


class ElementCheck:
    """Accumulates element-wise differences between GPU and oracle rows.

    h (bf16): an element passes when it equals the oracle's, or is its bf16
    neighbour of the same sign (the fp32 sum landed on the other side of a
    rounding boundary), or differs by at most 2^-14 of its row's rms (sign
    flips of values near zero after cancellation).  The number of non-equal
    elements is reported.
    y, out: |gpu - oracle| <= bound, an element-wise bound given by the caller
    (the propagated h differences plus the fp32 accumulation error).
    """

    def __init__(self, name: str):
        self.name = name
        self.n = 0
        self.n_diff = 0
        self.bad = []
        self.worst = 0.0     # largest |gpu - oracle| / bound

    def h_rows(self, gpu_bits: np.ndarray, ref_bits: np.ndarray, tag=""):
        g = np.asarray(gpu_bits, dtype=np.uint16).astype(np.int64)
        r = np.asarray(ref_bits, dtype=np.uint16).astype(np.int64)
        a, b = OF.bf16_bits_to_f64(g), OF.bf16_bits_to_f64(r)
        rms = np.sqrt(np.mean(b * b, axis=-1, keepdims=True))
        diff = g != r
        adjacent = ((g & 0x8000) == (r & 0x8000)) & (np.abs(g - r) == 1)
        tiny = np.abs(a - b) <= 2.0 ** -14 * rms
        bad = diff & ~adjacent & ~tiny
        self.n += g.size
        self.n_diff += int(diff.sum())
        if bad.any():
            idx = np.argwhere(bad)[:5]
            self.bad += [(tag, tuple(i), float(a[tuple(i)]), float(b[tuple(i)])) for i in idx]
        return self

    def f_rows(self, gpu: np.ndarray, ref: np.ndarray, bound: np.ndarray, tag=""):
        a = np.asarray(gpu, dtype=np.float64)
        b = np.asarray(ref, dtype=np.float64)
        err = np.abs(a - b)
        bad = err > bound
        self.n += a.size
        self.n_diff += int((a != b).sum())
        if a.size:
            self.worst = max(self.worst, float(np.max(err / np.maximum(bound, 1e-300))))
        if bad.any():
            idx = np.argwhere(bad)[:5]
            self.bad += [(tag, tuple(i), float(a[tuple(i)]), float(b[tuple(i)]), float(bound[tuple(i)]))
                         for i in idx]
        return self

    def report(self) -> str:
        frac = self.n_diff / max(self.n, 1)
        return (f"{self.name}: {self.n} elements, {self.n_diff} not identical ({frac:.2e}), "
                f"worst |d|/bound {self.worst:.2e}, {len(self.bad)} outside the bound")


#: fp32 accumulation error allowed, as a fraction of the sum of |terms| (a 2048-long K loop in
#: steps of 16 rounds about 130 times: 130 * 2^-24 = 7.7e-6, well inside 2^-14 = 6.1e-5)
ACC_REL = 2.0 ** -14
#: error of the combine's fp32 sum (k + 1 terms, routing weights rounded to fp32), relative to sum |w y|
COMBINE_REL = 2.0 ** -16
#: non-identical h elements allowed (one-ulp neighbours), as a fraction of the compared elements
H_DIFF_FRAC = 2e-3


def alarm_rel_l2(H: int) -> float:
    """Tighter-than-bar rel-L2 alarm: h rounding flips grow with the reduction length, so the alarm
    scales with H, capped at half the bar."""
    return min(3e-4 * max(1.0, H / 512), 0.5 * REL_L2_BAR)


def oracle_pair_rows(ol: "OracleLayer", x_bits: np.ndarray, ids: np.ndarray, gate_flags=None, experts=None,
                     resident=None, with_shared=True):
    """Yield (pair ids or None for shared, tokens, h bits [n, I], y float64 [n, H], |W_d| (+ |D_d|) [H, I])
    from the oracle, expert by expert (only experts in ``experts`` when given; missing experts of an
    expert cache are skipped, their rows are never written)."""
    x = OF.bf16_bits_to_f64(x_bits)
    T, k = ids.shape
    L = ol.cfg.swiglu_limit
    by_e = {}
    for p in range(T * k):
        by_e.setdefault(int(ids[p // k, p % k]), []).append(p)
    for e in sorted(by_e):
        if experts is not None and e not in experts:
            continue
        if resident is not None and not resident[e]:
            continue
        Wg, Wu, Wd = ol.expert_weights(e)
        pairs = np.array(by_e[e], dtype=np.int64)
        toks = pairs // k
        flag = np.zeros(len(pairs), dtype=bool)
        if gate_flags is not None and ol.soe is not None and ol.soe[e] >= 0:
            flag = np.asarray(gate_flags)[toks] != 0
        for sel, use_d in ((~flag, False), (flag, True)):
            if not sel.any():
                continue
            if use_d:
                Dg, Du, Dd = ol.delta_weights_of_slot(int(ol.soe[e]))
            else:
                Dg = Du = Dd = None
            h = OFF.expert_hidden(x[toks[sel]], Wg, Wu, L, Dg, Du)
            y = OFF.expert_out(h, Wd, Dd)
            absw = np.abs(Wd) if Dd is None else np.abs(Wd) + np.abs(Dd)
            yield pairs[sel], toks[sel], OF.bf16_rne_bits(h), y, absw
    sh = ol.shared_weights() if with_shared else None
    if sh is not None:
        h = OFF.expert_hidden(x, sh[0], sh[1], L)
        yield None, np.arange(T), OF.bf16_rne_bits(h), OFF.expert_out(h, sh[2]), np.abs(sh[2])


class PairRows:
    """Result of check_pair_rows: the h / y checks and, per pair (and per token for the shared
    expert), the element-wise bound on y that carries over to the layer output."""

    def __init__(self):
        self.h = ElementCheck("h")
        self.y = ElementCheck("y")
        self.ybound = {}       # pair id -> bound on |y_gpu - y_oracle| + COMBINE_REL |y_oracle|
        self.ybound_sh = {}    # token -> the same for the shared expert's y


def check_pair_rows(ws: torch.Tensor, ol: "OracleLayer", x_bits, ids, sorted_pairs, H, I, gate_flags=None,
                    experts=None, resident=None, with_shared=True, out_tokens=None) -> PairRows:
    """Compare the workspace's h and y rows with the oracle's, element by element.

    h: each element equal to the oracle's or its bf16 neighbour (ElementCheck.h_rows).
    y: |y_gpu - y_oracle| <= |W_d| |h_gpu - h_oracle| + ACC_REL |W_d| |h_oracle| per element: the h
    elements that landed one ulp away carry through the down projection, plus the fp32 accumulation
    error.  The bounds of the pairs of ``out_tokens`` are kept for check_out_rows."""
    T, k = ids.shape
    hb, y = workspace_views(ws, T, k, H, I)
    hb = np_(hb).astype(np.uint16)
    y = np_(y)
    if mfma_path(T, k, H):
        # h rows follow the pair order of the grouped GEMM: sorted, or with a gated delta the partitioned
        # order, which the workspace also holds (compared here as index data, bit for bit)
        rows_of = np.asarray(sorted_pairs, dtype=np.int64)
        if gate_flags is not None and ol.soe is not None and (ol.soe >= 0).any():
            E = len(ol.soe)
            offsets = np.concatenate([[0], np.cumsum(np.bincount(ids.reshape(-1), minlength=E))])
            exp_order, exp_nflag = partitioned_order(ids, sorted_pairs, offsets, ol.soe, gate_flags, resident)
            P = T * k
            off = _al256((P + T) * I * 2) + _al256((P + T) * H * 4)
            got = np_(ws[off:off + P * 4].view(torch.int32))
            off2 = off + _al256(P * 4)
            got_nf = np_(ws[off2:off2 + E * 4].view(torch.int32))
            assert (got == exp_order).all(), "partitioned pair order differs"
            assert (got_nf == exp_nflag).all(), "flagged counts differ"
            rows_of = exp_order
        row_of_pair = np.empty(T * k, dtype=np.int64)
        row_of_pair[rows_of] = np.arange(T * k)
    else:
        row_of_pair = np.arange(T * k)
    keep = set(range(T)) if out_tokens is None else set(int(t) for t in out_tokens)
    res = PairRows()
    for pairs, toks, h_ref, y_ref, absw in oracle_pair_rows(ol, x_bits, ids, gate_flags, experts, resident,
                                                           with_shared):
        if pairs is None:
            hr = yr = T * k + toks
            tag = "shared"
        else:
            hr = row_of_pair[pairs]
            yr = pairs
            tag = f"expert {int(ids[pairs[0] // k, pairs[0] % k])}"
        hg = hb[hr]
        res.h.h_rows(hg, h_ref, tag)
        dh = np.abs(OF.bf16_bits_to_f64(hg) - OF.bf16_bits_to_f64(h_ref))
        bound = dh @ absw.T + ACC_REL * (np.abs(OF.bf16_bits_to_f64(h_ref)) @ absw.T)
        res.y.f_rows(y[yr], y_ref, bound, tag)
        carry = bound + COMBINE_REL * np.abs(y_ref)
        for i, t in enumerate(toks):
            if int(t) in keep:
                if pairs is None:
                    res.ybound_sh[int(t)] = carry[i]
                else:
                    res.ybound[int(pairs[i])] = carry[i]
    return res


def check_out_rows(gpu_bits: np.ndarray, ref_bits: np.ndarray, tokens=None, topk_w=None, rows: PairRows = None,
                   resident=None, ids=None) -> ElementCheck:
    """Layer output against the oracle's.  With the per-pair y bounds of check_pair_rows the bound is
    sum_j |w_j| bound_y(t, j) + bound_y_shared(t) + 1.5 bf16 ulps of the oracle value (each side rounds
    once, by at most half an ulp of its own binade, and the GPU value may sit one binade up); without
    them (a test that has no rows) it is 2^-7 of the row's rms plus 1.5 ulps, which still rejects any
    wrong column or row (errors of the order of the rms)."""
    a = OF.bf16_bits_to_f64(gpu_bits)
    b = OF.bf16_bits_to_f64(ref_bits)
    if rows is None:
        rms = np.sqrt(np.mean(b * b, axis=-1, keepdims=True))
        bound = 2.0 ** -7 * rms + 1.5 * ulp_bf16(b)
    else:
        k = topk_w.shape[1]
        bound = 1.5 * np.array(ulp_bf16(b), dtype=np.float64)
        for i, t in enumerate(tokens):
            for j in range(k):
                p = int(t) * k + j
                if resident is not None and not resident[int(ids[t, j])]:
                    continue
                bound[i] += abs(float(topk_w[t, j])) * rows.ybound[p]
            if int(t) in rows.ybound_sh:
                bound[i] += rows.ybound_sh[int(t)]
    return ElementCheck("out").f_rows(a, b, bound)


def assert_elementwise(*checks: ElementCheck, h_frac: float = H_DIFF_FRAC):
    for c in checks:
        print(c.report(), flush=True)
    for c in checks:
        assert not c.bad, f"{c.name}: elements outside the bound, e.g. {c.bad[:3]}"
        if c.name == "h":
            assert c.n_diff <= h_frac * c.n + 8, f"h: {c.n_diff} of {c.n} elements differ"
