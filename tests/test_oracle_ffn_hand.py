"""Pins of the oracle's expert FFN and FP4 GEMM against hand-derived values.

``tests/golden/ffn_hand.json`` holds tiny experts whose outputs were worked out
by hand (closed forms of silu at ln 3 and at large arguments, exact binary
fractions, bf16 ties); each entry states its derivation.  The oracle must
reproduce every value bit for bit.  The last test plants the plausible
mistakes one by one in a copy of the oracle's SwiGLU step (roles of gate and
up swapped, clamp applied after silu, one-sided clamp, no clamp, a float32
step before the bf16 rounding, truncation or round-half-away instead of
ties-to-even, the delta added after the clamp) and checks that the golden
cases reject each of them.

Sources: README "Frontier MoE on consumer Blackwell (SM120)", section "How it
fits - 2-bit experts at FP4 quality"; airanks.app "kacper-daftcode/vLLM-Moet",
section "Quality vs native" (SwiGLU clamp).
"""
import json
import os

import numpy as np
import pytest

from oracle import ffn as FF
from oracle import formats as F

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "ffn_hand.json")


def _f(s) -> float:
    s = str(s)
    return float.fromhex(s) if s.lower().lstrip("-").startswith("0x1.") or "p" in s.lower() else float(s)


def _mat(rows):
    return np.array([[_f(v) for v in r] for r in rows], dtype=np.float64)


def _bits(v) -> int:
    return int(str(v), 16) if isinstance(v, str) else int(v)


def _load():
    with open(GOLDEN) as fh:
        return json.load(fh)


def _hidden_case(c, fn):
    Dg = _mat(c["Dg"]) if "Dg" in c else None
    Du = _mat(c["Du"]) if "Du" in c else None
    h = fn(_mat(c["x"]), _mat(c["Wg"]), _mat(c["Wu"]), _f(c["L"]), Dg, Du)
    return F.bf16_rne_bits(h)[0].tolist() == [_bits(b) for b in c["h_bits"]]


def _moe_case(c):
    ex = [(_mat(e["Wg"]), _mat(e["Wu"]), _mat(e["Wd"])) for e in c["experts"]]
    sh = c.get("shared")
    shared = (_mat(sh["Wg"]), _mat(sh["Wu"]), _mat(sh["Wd"])) if sh else None
    kw = {}
    if "deltas" in c:
        dl = [(_mat(d["Dg"]), _mat(d["Du"]), _mat(d["Dd"])) for d in c["deltas"]]
        kw = dict(gate_flags=np.array(c["gate_flags"]), slot_of_expert=np.array(c["slot_of_expert"]),
                  delta_weights=lambda s: dl[s])
    xb = np.array([[_bits(b) for b in r] for r in c["x_bits"]], dtype=np.uint16)
    out = FF.moe_forward(xb, np.array(c["topk_ids"]), _mat(c["topk_w"]), lambda e: ex[e], shared, **kw)
    return out.tolist() == [[_bits(b) for b in r] for r in c["out_bits"]]


def _golden_all_pass(fn=None) -> bool:
    """True when every hand case holds (fn: SwiGLU step to use, default the oracle's)."""
    g = _load()
    fn = fn or FF.expert_hidden
    ok = all(_hidden_case(c, fn) for c in g["expert_hidden"])
    return ok and all(_moe_case(c) for c in g["moe_forward"])


@pytest.mark.parametrize("name", [c["name"] for c in _load()["expert_hidden"]])
def test_expert_hidden_hand_values(name):
    c = next(c for c in _load()["expert_hidden"] if c["name"] == name)
    assert _hidden_case(c, FF.expert_hidden), c["derivation"]


@pytest.mark.parametrize("name", [c["name"] for c in _load()["expert_out"]])
def test_expert_out_hand_values(name):
    c = next(c for c in _load()["expert_out"] if c["name"] == name)
    y = FF.expert_out(_mat(c["h"]), _mat(c["Wd"]), _mat(c["Dd"]) if "Dd" in c else None)
    assert y[0].tolist() == [_f(v) for v in c["y"]], c["derivation"]


@pytest.mark.parametrize("name", [c["name"] for c in _load()["moe_forward"]])
def test_moe_forward_hand_values(name):
    c = next(c for c in _load()["moe_forward"] if c["name"] == name)
    assert _moe_case(c), c["derivation"]


def test_fp4_gemm_hand_values():
    for c in _load()["fp4_gemm_accumulate"]:
        slots = [F.nvfp4_decode(np.array(s["codes"], dtype=np.uint8), np.array(s["scales"], dtype=np.uint8),
                                _f(s["scale_2"])) for s in c["slots"]]
        act = F.bf16_rne_bits(_mat(c["act"]))
        out = FF.fp4_gemm_accumulate(_mat(c["acc"]), act, np.array(c["row_slot"]), lambda s: slots[s])
        assert out.tolist() == _mat(c["out"]).tolist(), c["derivation"]


# --- planted mistakes (copies of the SwiGLU step with one error each) -------------------------------

def _mutant(kind):
    def fn(x, Wg, Wu, L=0.0, Dg=None, Du=None):
        ug, uu = x @ Wg.T, x @ Wu.T
        if Dg is not None and kind != "delta_after_clamp":
            ug, uu = ug + x @ Dg.T, uu + x @ Du.T
        if kind == "swap_roles":
            ug, uu = uu, ug
        if L > 0 and kind not in ("no_clamp", "clamp_after_silu"):
            ug = np.minimum(ug, L) if kind != "two_sided_gate" else np.clip(ug, -L, L)
            uu = np.clip(uu, -L, L) if kind != "up_upper_only" else np.minimum(uu, L)
        if Dg is not None and kind == "delta_after_clamp":
            ug, uu = ug + x @ Dg.T, uu + x @ Du.T
        s = FF.silu(ug)
        if L > 0 and kind == "clamp_after_silu":
            s, uu = np.minimum(s, L), np.clip(uu, -L, L)
        v = s * uu
        if kind == "float32_step":
            v = v.astype(np.float32).astype(np.float64)
        if kind in ("truncate", "half_away"):
            b = F.bf16_rne_bits(v)
            lo = F.bf16_bits_to_f64(b)
            q = np.abs(v - lo)
            step = np.abs(F.bf16_bits_to_f64(b + 1) - lo)
            if kind == "truncate":            # toward zero
                over = np.abs(lo) > np.abs(v)
                lo = np.where(over, F.bf16_bits_to_f64(b - 1), lo)
            else:                             # ties away from zero
                tie = (q * 2 == step) & (np.abs(lo) < np.abs(v))
                lo = np.where(tie, F.bf16_bits_to_f64(b + 1), lo)
            return lo
        return F.bf16_bits_to_f64(F.bf16_rne_bits(v))
    return fn


@pytest.mark.parametrize("kind", ["swap_roles", "clamp_after_silu", "no_clamp", "two_sided_gate", "up_upper_only",
                                  "float32_step", "truncate", "half_away", "delta_after_clamp"])
def test_golden_cases_reject_planted_mistakes(kind, monkeypatch):
    assert _golden_all_pass()                      # the oracle itself passes
    monkeypatch.setattr(FF, "expert_hidden", _mutant(kind))
    assert not _golden_all_pass(_mutant(kind)), f"the hand cases do not catch a SwiGLU step with '{kind}'"


def test_unmutated_copy_passes():
    """The mutant harness without a mutation is the oracle's step (so the rejections above are the mutations)."""
    assert _golden_all_pass(_mutant("none"))
