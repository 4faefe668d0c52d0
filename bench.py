#!/usr/bin/env python3
"""Benchmark: the routed-expert MoE layer forward at decode on one MI355X.

One step = moet_route + moet_moe_forward (gate/up + SwiGLU kernel, down +
combine kernel) for one synthetic layer shaped like the pages' decode case:
3 tokens (1 + 2 MTP drafts), hidden 7168, expert intermediate 2048, 256
routed experts top-8 (sigmoid, renormalised) plus one shared expert, 2-bit
planes.  Inputs are resident in HBM before timing.  Steps rotate over a pool
of layers (so no expert stays in the 256 MB last-level cache between uses)
and over 8 input sets (so the routed experts change every step).

Printed value: effective HBM GB/s = algorithmic bytes of the step (2-bit
planes of every distinct expert it routes to, shared expert, activations,
logits, output; computed per step from that step's routing) / step time.
The roofline object covers the dominant kernel (gate/up), timed by HIP
events recorded on its stream around each launch inside the timed region.
The CPU baseline times the float64 oracle on a bounded sample (one token's
experts) on the host cores.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, AMD published peak
W2_BYTES_PER_WEIGHT = 2.25 / 8.0
FP4_BYTES_PER_WEIGHT = 4.5 / 8.0
MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak, AMD published


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="decode_mtp", help="synthetic decode layer (a key of synth.CONFIGS)")
    ap.add_argument("--layers", type=int, default=4, help="layers in the rotating pool")
    ap.add_argument("--inputs", type=int, default=8, help="input sets in the rotation")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="skip the HIP-graph replay measurement")
    ap.add_argument("--no-cold", action="store_true", help="skip the cold-cache steps (1 GiB read between steps)")
    ap.add_argument("--no-prefill", action="store_true", help="skip the prefill-chunk (T=4096) measurement")
    ap.add_argument("--prefill-steps", type=int, default=20)
    ap.add_argument("--no-extra", action="store_true", help="skip the delta-cache and batched decode legs")
    ap.add_argument("--extra-steps", type=int, default=100)
    ap.add_argument("--seed", type=int, default=1234)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB read + 1 GiB write elementwise kernel (HBM counter calibration)")
    ap.add_argument("--summarize-counters", metavar="CSV",
                    help="print per-kernel means of a rocprofv3 counter_collection.csv and exit (no GPU use)")
    return ap.parse_args()


COPY_BYTES = 1 << 30


def calibrate_copy(reps=10):
    """A plain elementwise kernel of known traffic: reads COPY_BYTES, writes COPY_BYTES per launch."""
    import torch
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        torch.mul(src, 2.0, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "torch.mul fp32", "read_bytes": COPY_BYTES, "write_bytes": COPY_BYTES,
                      "launches": reps}), flush=True)


def achievable_refs(dev, reps=10):
    """Measured achievable rates of this device, for the fractions beside the published peaks: a
    streaming read of 1 GiB (moet_probe_read: 16-byte loads, grid-stride, the weight kernels' access
    shape), a 1 GiB device copy (torch copy_: 1 GiB read + 1 GiB written) and a bf16 GEMM
    8192 x 8192 x 8192 (torch.matmul, hipBLASLt); the median of `reps` launches of each, HIP events
    around every launch."""
    import numpy as np
    import torch
    from bit_moe_expert_nvfp4_amd import moet

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for a, b in evs:
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        return float(np.median([a.elapsed_time(b) for a, b in evs])) / 1e3

    buf = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(buf)
    sink = torch.empty((moet.PROBE_SINK_WORDS,), dtype=torch.int32, device=dev)
    rd = timed(lambda: moet.probe_read(buf, sink))
    cp = timed(lambda: dst.copy_(buf))
    del buf, dst
    M = 8192
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    a = torch.randn((M, M), generator=g, device=dev).to(torch.bfloat16)
    b = torch.randn((M, M), generator=g, device=dev).to(torch.bfloat16).contiguous()
    mm = timed(lambda: torch.matmul(a, b))
    del a, b
    torch.cuda.empty_cache()
    it_m, it_v = 4096, 8192
    t_m = timed(lambda: moet.probe_peak(moet.PROBE_MFMA_BF16, it_m, sink))
    t_v = timed(lambda: moet.probe_peak(moet.PROBE_DOT2_BF16, it_v, sink))
    w = moet.PROBE_PEAK_WAVES
    return {"read_GBps": round(COPY_BYTES / rd / 1e9, 1), "copy_GBps": round(2 * COPY_BYTES / cp / 1e9, 1),
            "bf16_gemm_TFLOPs": round(2.0 * M ** 3 / mm / 1e12, 1),
            "mfma_bf16_loop_TFLOPs": round(w * 4 * it_m * 32768 / t_m / 1e12, 1),
            "dot2_loop_Twave_inst_per_s": round(w * 8 * it_v / t_v / 1e12, 4),
            "method": f"median of {reps} launches each: moet_probe_read over 1 GiB (read rate); torch copy_ "
                      f"1 GiB -> 1 GiB (read + write bytes / time); torch.matmul bf16 {M}^3 (2 M^3 / time); "
                      f"moet_probe_peak tight loops of v_mfma_f32_32x32x16_bf16 and v_dot2_f32_bf16 "
                      f"(independent chains, no memory traffic, {w} waves)"}


def summarize_counters(path):
    """Mean counter value per dispatch, per kernel name, of a rocprofv3 --pmc CSV."""
    import csv
    acc = {}
    with open(path, newline="") as f:
        for row in csv.DictReader(f):
            key = (row["Kernel_Name"], row["Counter_Name"])
            a = acc.setdefault(key, [0, 0.0])
            a[0] += 1
            a[1] += float(row["Counter_Value"])
    for (name, ctr), (n, tot) in sorted(acc.items(), key=lambda kv: -kv[1][1]):
        print(f"{ctr:12s} dispatches {n:6d} mean {tot / n:14.1f}  {name[:110]}")


def counted_traffic(profile="fc1_decode_kernel_hbm_counters_T3_H7168_I2048_E256.md",
                    sources=("moe_decode.hip", "moet_common.h")):
    """HBM bytes per launch of a kernel from a committed counter summary under profiles/, if that summary
    was taken on the current kernel source (else None)."""
    import hashlib
    path = os.path.join(ROOT, "profiles", profile)
    src = os.path.join(ROOT, "bit_moe_expert_nvfp4_amd", "csrc")
    try:
        h = hashlib.sha256()
        for name in sources:
            with open(os.path.join(src, name), "rb") as f:
                h.update(f.read())
        fields = {}
        with open(path) as f:
            for line in f:
                if ":" in line and line.startswith("- "):
                    k, v = line[2:].split(":", 1)
                    fields[k.strip()] = v.strip().strip("`")
        if fields.get("kernel source sha256") != h.hexdigest():
            return None
        return float(fields["HBM bytes per launch"])
    except (OSError, KeyError, ValueError):
        return None


def step_bytes(cfg, ids_np, flags_np, soe_np, resident=None, shared_nvfp4=False):
    """Algorithmic bytes of one decode step and of its gate/up kernel launch (with an expert cache, only
    the resident experts' planes are read; an NVFP4 shared expert reads its FP4 planes)."""
    w13 = 2 * cfg.I * cfg.H * W2_BYTES_PER_WEIGHT
    w2 = cfg.H * cfg.I * W2_BYTES_PER_WEIGHT
    d13 = 2 * cfg.I * cfg.H * FP4_BYTES_PER_WEIGHT
    d2 = cfg.H * cfg.I * FP4_BYTES_PER_WEIGHT
    experts = set(int(e) for e in ids_np.reshape(-1) if resident is None or resident[int(e)])
    n = len(experts) + (1 if cfg.shared and not shared_nvfp4 else 0)
    delta_experts = set()
    if flags_np is not None and soe_np is not None:
        for t in range(cfg.T):
            if flags_np[t]:
                for e in ids_np[t]:
                    if soe_np[int(e)] >= 0 and (resident is None or resident[int(e)]):
                        delta_experts.add(int(e))
    nd = len(delta_experts)
    if cfg.shared and shared_nvfp4:
        nd += 1                       # the shared expert's FP4 planes
    io = 2 * cfg.T * cfg.H * 2 + 4 * cfg.T * cfg.E
    total = n * (w13 + w2) + nd * (d13 + d2) + io
    fc1 = n * w13 + nd * d13 + 2 * cfg.T * cfg.H + 2 * (cfg.T * cfg.k + cfg.T) * cfg.I
    return total, fc1, n, nd


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def _median_time(fn, runs=3):
    ts = []
    for _ in range(runs):
        t0 = time.perf_counter()
        fn()
        ts.append(time.perf_counter() - t0)
    return float(sorted(ts)[len(ts) // 2]), ts


def cpu_baseline(cfg, src, x, lg, seed, cfg_prefill=None, x_prefill=None, lg_prefill=None, runs=3):
    """Time the float64 oracle on the host cores (median of `runs` runs of each bounded sample):
    the decode step (route + the layer output of every token), the load-time requant of two matrices
    (scaled to a layer), and a prefill sample (route of the whole chunk, the expert FFN of every pair
    routed to two experts; scaled to the chunk)."""
    import numpy as np
    from oracle import formats as OF
    from oracle import requant as OR
    from oracle import route as ORT
    from oracle import ffn as OFF

    def npy(t):
        return t.detach().cpu().numpy()

    lg_np = npy(lg)
    ids, w, _, _ = ORT.route(lg_np, cfg.k, cfg.score, cfg.renormalize)
    experts = sorted(set(int(e) for e in ids.reshape(-1)))
    # load-time part (not timed): the oracle's own requantisation of the touched experts
    planes = {}

    def rq(stack, i):
        c, s, s2 = stack
        return OR.requant(npy(c[i]), npy(s[i]), float(s2[i]))
    for e in experts:
        planes[e] = (rq(src.w13, 2 * e), rq(src.w13, 2 * e + 1), rq(src.w2, e))
    shared = (rq(src.shared13, 0), rq(src.shared13, 1), rq(src.shared2, 0)) if cfg.shared else None
    xb = OF.bf16_rne_bits(npy(x.float()).astype(np.float64))

    def dq(p):
        return OR.dequant_2bit(*p)

    def decode_step():
        ids2, w2, _, _ = ORT.route(lg_np, cfg.k, cfg.score, cfg.renormalize)
        OFF.moe_forward(xb, ids2, w2, lambda e: tuple(dq(p) for p in planes[e]),
                        tuple(dq(p) for p in shared) if shared else None)
    dt, dts = _median_time(decode_step, runs)
    n = len(experts) + (1 if cfg.shared else 0)
    nbytes = n * 3 * cfg.I * cfg.H * W2_BYTES_PER_WEIGHT + 2 * cfg.T * cfg.H * 2 + 4 * cfg.T * cfg.E
    omp = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or len(os.sched_getaffinity(0))
    res = {"value": nbytes / dt / 1e9, "unit": "GB/s", "cores": _blas_threads(), "kind": "oracle",
           "cpu_model": _cpu_model(), "runs": runs, "run_seconds": [round(t, 3) for t in dts],
           "sample": f"one full decode step of input set 0, median of {runs} runs: routing and the layer "
                     f"output of all {cfg.T} tokens ({n} distinct experts incl. shared, {nbytes / 1e6:.1f} MB "
                     f"of 2-bit planes, dequantised and applied in float64 numpy from the oracle's own "
                     f"requantised planes), {dt:.2f} s"}

    # load-time requant: two gate/up matrices of the layer, scaled to the layer's matrices
    c13, s13, z13 = (npy(t[:2]) for t in src.w13)
    rq_t, _ = _median_time(lambda: [OR.requant(c13[i], s13[i], float(z13[i])) for i in range(2)], runs)
    n_mat = 3 * cfg.E + (3 if cfg.shared else 0)
    res["requant"] = {"s_per_matrix": round(rq_t / 2, 3), "scaled_s_per_layer": round(rq_t / 2 * n_mat, 1),
                      "threads": omp,
                      "sample": f"oracle requant (C, exact 127-code scan, OpenMP over rows) of gate/up matrices "
                                f"0 and 1 [{cfg.I}][{cfg.H}] of the layer, median of {runs} runs; scaled by "
                                f"{n_mat} / 2 to the layer's {n_mat} equal-size matrices"}

    if cfg_prefill is not None:
        cp = cfg_prefill
        lgp = npy(lg_prefill)
        xpb = OF.bf16_rne_bits(npy(x_prefill.float()).astype(np.float64))
        xpv = OF.bf16_bits_to_f64(xpb)
        route_t, _ = _median_time(lambda: ORT.route(lgp, cp.k, cp.score, cp.renormalize), runs)
        pids, _, offs, pairs = ORT.route(lgp, cp.k, cp.score, cp.renormalize)
        rng = np.random.default_rng(seed)
        sample_e = sorted(int(e) for e in rng.choice(cp.E, size=2, replace=False))
        sp = {e: (rq(src.w13, 2 * e), rq(src.w13, 2 * e + 1), rq(src.w2, e)) for e in sample_e}
        toks = {e: pairs[offs[e]:offs[e + 1]] // cp.k for e in sample_e}
        n_pairs = sum(len(v) for v in toks.values())

        def deq():
            return {e: tuple(dq(p) for p in sp[e]) for e in sample_e}
        deq_t, _ = _median_time(deq, runs)
        W = deq()

        def ffn():
            for e in sample_e:
                Wg, Wu, Wd = W[e]
                OFF.expert_out(OFF.expert_hidden(xpv[toks[e]], Wg, Wu, cp.swiglu_limit), Wd)
        ffn_t, _ = _median_time(ffn, runs)
        chunk_s = route_t + deq_t / 2 * cp.E + ffn_t / max(n_pairs, 1) * cp.T * cp.k
        res["prefill"] = {"value": round(cp.T / chunk_s, 2), "unit": "tokens/s",
                          "scaled_s_per_chunk": round(chunk_s, 1),
                          "sample": f"prefill chunk T={cp.T} (the GPU leg's logits and activations): oracle route "
                                    f"of all {cp.T} tokens ({route_t:.2f} s), dequantisation of experts "
                                    f"{sample_e} ({deq_t:.2f} s) and their expert FFN over all {n_pairs} routed "
                                    f"pairs ({ffn_t:.2f} s), medians of {runs} runs; chunk time = route + "
                                    f"dequant x {cp.E}/2 experts + FFN x {cp.T * cp.k}/{n_pairs} pairs (the "
                                    f"weighted combine, {cp.T}x{cp.k}x{cp.H} multiply-adds, is left out)"}
    return res


def _blas_threads():
    """Threads the oracle's numpy BLAS uses on this host."""
    try:
        from threadpoolctl import threadpool_info
        n = [d.get("num_threads", 0) for d in threadpool_info() if d.get("user_api") == "blas"]
        if n:
            return int(max(n))
    except Exception:
        pass
    return len(os.sched_getaffinity(0))


def decode_leg(cfg_name, steps, warmup, seed, dev, n_layers=2, n_inputs=8, cache_fraction=None, tp=1,
               shared_nvfp4=False):
    """Route + forward of another decode configuration (FP4 delta cache, batched streams, one GPU's
    share of a tensor-parallel layer), timed like the main step over its own pool of layers and input sets."""
    import dataclasses
    import numpy as np
    import torch
    from bit_moe_expert_nvfp4_amd import moet, synth

    cfg = synth.CONFIGS[cfg_name]
    if tp > 1:                         # rows I/tp of gate/up and columns I/tp of down per GPU
        cfg = dataclasses.replace(cfg, name=f"{cfg.name}_tp{tp}_shard", I=cfg.I // tp)
    soe = synth.slot_of_expert(cfg, seed) if cfg.n_resident else None
    layers = []
    resident = None
    if cache_fraction is not None:     # expert cache holding a seeded fraction of the experts
        g = torch.Generator().manual_seed(seed)
        perm = torch.randperm(cfg.E, generator=g)
        n_res = int(round(cache_fraction * cfg.E))
        base_soe = torch.full((cfg.E,), -1, dtype=torch.int64)
        base_soe[perm[:n_res]] = torch.arange(n_res)
        resident = (base_soe >= 0).numpy()
    for li in range(n_layers):
        src = synth.make_layer(cfg, seed=seed, device=dev, layer_index=li)
        lay = moet.layer_from_nvfp4(src, soe, shared_nvfp4=shared_nvfp4)
        del src
        if resident is not None:
            lay = moet.expert_cache(lay, base_soe)
        layers.append(lay)
        torch.cuda.empty_cache()
    miss = torch.zeros((1,), dtype=torch.int32, device=dev)
    xs = [synth.make_activations(cfg.T, cfg.H, seed, tag=f"x{i}", device=dev) for i in range(n_inputs)]
    lgs = [synth.make_logits(cfg, seed, tag=f"logits{i}", device=dev) for i in range(n_inputs)]
    flags = synth.gate_flags(cfg, seed).to(dev) if cfg.n_flagged else None
    ro = [(torch.empty((cfg.T, cfg.k), dtype=torch.int32, device=dev),
           torch.empty((cfg.T, cfg.k), dtype=torch.float32, device=dev),
           torch.empty((cfg.E + 1,), dtype=torch.int32, device=dev),
           torch.empty((cfg.T * cfg.k,), dtype=torch.int32, device=dev)) for _ in range(n_inputs)]
    out = torch.empty((cfg.T, cfg.H), dtype=torch.bfloat16, device=dev)
    ws = moet.alloc_workspace(layers[0], cfg.T, cfg.k, dev)

    def step(i):
        j = i % n_inputs
        ids, w, offs, pairs = moet.route(lgs[j], cfg.k, cfg.score, cfg.renormalize, out=ro[j])
        moet.moe_forward(layers[i % n_layers], xs[j], ids, w, offs, pairs, flags, out=out, workspace=ws,
                         miss_count=miss if resident is not None else None)

    for i in range(warmup):
        step(i)
    for j in range(n_inputs):          # every input set's routing, whatever the warm-up count
        moet.route(lgs[j], cfg.k, cfg.score, cfg.renormalize, out=ro[j])
    torch.cuda.synchronize()
    flags_np = flags.cpu().numpy() if flags is not None else None
    soe_np = soe.numpy() if soe is not None else None
    per_input = [step_bytes(cfg, ro[j][0].cpu().numpy(), flags_np, soe_np, resident, shared_nvfp4)
                 for j in range(n_inputs)]
    misses = [int((~resident[ro[j][0].cpu().numpy().reshape(-1)]).sum()) if resident is not None else 0
              for j in range(n_inputs)]
    if resident is not None and warmup > 0:   # the on-device counter of the last warm-up step
        assert int(miss.item()) == misses[(warmup - 1) % n_inputs], "miss counter disagrees with the routing"
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in ev:
        a.record()
        b.record()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for i in range(steps):          # timed with nothing recorded between the launches
        step(warmup + i)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    for i in range(steps):          # the same steps again, timing the gate/up launches
        moet.set_timing_events(*ev[i])
        step(warmup + i)
    torch.cuda.synchronize()
    moet.set_timing_events(None, None)
    sel = [per_input[(warmup + i) % n_inputs] for i in range(steps)]
    nbytes = float(np.mean([b[0] for b in sel]))
    fc1_bytes = float(np.mean([b[1] for b in sel]))
    fc1_ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    cache_txt = (f", expert cache holding {int(resident.sum())} of {cfg.E} experts (seeded choice)"
                 if resident is not None else "")
    res = {
        "workload": f"{cfg.name}: T={cfg.T} H={cfg.H} I={cfg.I} E={cfg.E} top{cfg.k} sigmoid+renorm"
                    f"{' (Zipf-skewed logits)' if cfg.logits == 'zipf' else ''}"
                    f"{(' + NVFP4 shared expert' if shared_nvfp4 else ' + shared expert') if cfg.shared else ''}"
                    f"{f' + FP4 delta ({cfg.n_resident} resident, {cfg.n_flagged} of {cfg.T} tokens flagged)' if cfg.n_resident else ''}"
                    f"{cache_txt}, {n_layers}-layer pool, {n_inputs} input sets",
        "us_per_layer": round(ms * 1e3, 2),
        "GBps": round(nbytes / (ms / 1e3) / 1e9, 1),
        "pct_hbm_peak": round(100.0 * nbytes / (ms / 1e3) / 1e9 / HBM_PEAK_GBS, 1),
        "tokens_per_s": round(cfg.T / (ms / 1e3), 1),
        "algorithmic_bytes_per_step": round(nbytes),
        "mean_experts_per_step": round(float(np.mean([b[2] for b in sel])), 2),
        "mean_delta_experts_per_step": round(float(np.mean([b[3] for b in sel])), 2),
        "fc1_avg_launch_us": round(fc1_ms * 1e3, 2),
        "fc1_GBps": round(fc1_bytes / (fc1_ms / 1e3) / 1e9, 1),
    }
    if resident is not None:
        res["mean_missed_routings_per_step"] = round(float(np.mean([misses[(warmup + i) % n_inputs]
                                                                    for i in range(steps)])), 2)
    del layers, ws
    torch.cuda.empty_cache()
    return res


def gate_leg(seed, dev, steps=200, V=151552):
    """moet_confidence_gate on next-token logits of one decode step (T=3) and of 8 batched streams (T=24)."""
    import torch
    from bit_moe_expert_nvfp4_amd import moet
    res = {}
    for T in (3, 24):
        g = torch.Generator(device=dev)
        g.manual_seed(seed + T)
        lg = torch.randn((T, V), generator=g, device=dev) * torch.linspace(0.5, 14.0, T, device=dev).unsqueeze(1)
        flags = torch.empty((T,), dtype=torch.uint8, device=dev)
        ws = torch.empty((max(1, moet.gate_workspace_bytes(T, V)),), dtype=torch.uint8, device=dev)
        for _ in range(10):
            moet.confidence_gate(lg, 0.60, flags=flags, workspace=ws)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            moet.confidence_gate(lg, 0.60, flags=flags, workspace=ws)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / steps * 1e3
        res[f"T{T}"] = {"workload": f"T={T} rows of V={V} fp32 next-token logits, tau=0.60",
                        "us": round(us, 2), "GBps": round(T * V * 4 / (us * 1e-6) / 1e9, 1),
                        "flagged": int(flags.sum().item())}
    return res


def conversion_leg(seed, dev, n_mat=16, N=2048, K=7168, steps=5):
    """Load-time conversions into 2-bit planes of a stack of gate/up-shaped matrices
    [2048][7168] (8 experts): NVFP4 requant, MXFP4 codes remap, FP8 block-quant requant."""
    import torch
    from bit_moe_expert_nvfp4_amd import moet, synth
    nv = synth.make_nvfp4_stack(n_mat, N, K, seed, "conv_nvfp4", device=dev)
    mx = synth.make_mxfp4_stack(n_mat, N, K, seed, "conv_mxfp4", device=dev)
    f8 = synth.make_fp8_stack(n_mat, N, K, seed, "conv_fp8", device=dev)
    out_bytes = n_mat * (N * K // 4 + N * K // 32)
    legs = (("nvfp4_requant", lambda: moet.requant(*nv), n_mat * (N * K // 2 + N * K // 16)),
            ("nvfp4_requant_codebook_pick", lambda: moet.requant(*nv, pick_codebook=True),
             n_mat * (N * K // 2 + N * K // 16)),
            ("mxfp4_remap", lambda: moet.remap_mxfp4(*mx), n_mat * (N * K // 2 + N * K // 32)),
            ("fp8_requant", lambda: moet.requant_fp8(*f8), n_mat * (N * K + 4 * ((N + 127) // 128) * (K // 128))))
    res = {}
    for name, fn, src_bytes in legs:
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        res[name] = {"workload": f"{n_mat} matrices [{N}][{K}]", "ms": round(ms, 3),
                     "ms_per_matrix": round(ms / n_mat, 4),
                     "GBps_source_plus_planes": round((src_bytes + out_bytes) / (ms * 1e-3) / 1e9, 1)}
    del nv, mx, f8
    torch.cuda.empty_cache()
    return res


def prefill_leg(layer, cfg5, steps, seed, dev, flags=None, soe=None):
    """Time route + forward of a prefill chunk (MFMA grouped GEMM path) on one pool layer; with
    gate flags and a delta cache, flagged rows of resident experts also run the FP4 pass."""
    import numpy as np
    import torch
    from bit_moe_expert_nvfp4_amd import moet, synth

    import dataclasses
    T, k = cfg5.T, cfg5.k
    # activations and router logits of the plain chunk in every leg, so that a leg with the delta
    # routes exactly the same pairs and differs from the plain one only by the delta's work
    base = dataclasses.replace(cfg5, name=synth.CONFIGS["prefill"].name)
    x = synth.make_activations(T, cfg5.H, seed, tag="prefill_x", device=dev)
    lg = synth.make_logits(base, seed, tag="prefill_logits", device=dev)
    ws = moet.alloc_workspace(layer, T, k, dev)
    out = torch.empty((T, cfg5.H), dtype=torch.bfloat16, device=dev)
    ro = (torch.empty((T, k), dtype=torch.int32, device=dev), torch.empty((T, k), dtype=torch.float32, device=dev),
          torch.empty((cfg5.E + 1,), dtype=torch.int32, device=dev), torch.empty((T * k,), dtype=torch.int32, device=dev))

    def step():
        ids, w, offs, pairs = moet.route(lg, k, cfg5.score, cfg5.renormalize, out=ro)
        moet.moe_forward(layer, x, ids, w, offs, pairs, flags, out=out, workspace=ws)

    for _ in range(3):
        step()
    torch.cuda.synchronize()
    delta_pairs = 0
    if flags is not None:
        ids_np = ro[0].cpu().numpy()
        fl_np = flags.cpu().numpy().astype(bool)
        soe_np = soe.cpu().numpy()
        delta_pairs = int((fl_np[:, None] & (soe_np[ids_np] >= 0)).sum())
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in ev:
        a.record()
        b.record()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for i in range(steps):          # timed with nothing recorded between the launches
        step()
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    for i in range(steps):          # the same steps again, timing the gate/up launches
        moet.set_timing_events(*ev[i])
        step()
    torch.cuda.synchronize()
    moet.set_timing_events(None, None)
    fc1_ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    P = T * k
    fl_fc1 = 2.0 * P * 2 * cfg5.I * cfg5.H
    fl = fl_fc1 + 2.0 * P * cfg5.H * cfg5.I
    peak = MFMA_BF16_PEAK_TFLOPS
    extra = ""
    if flags is not None:
        extra = (f", FP4 delta for {int(flags.sum().item())} gate-flagged tokens on {int((soe >= 0).sum().item())} "
                 f"delta-cache experts ({delta_pairs} flagged pairs; their FP4 pass is counted in the flops)")
        fl_fc1 += 2.0 * delta_pairs * 2 * cfg5.I * cfg5.H
        fl += 2.0 * delta_pairs * 3 * cfg5.I * cfg5.H
    return {
        "workload": f"prefill chunk: T={T} H={cfg5.H} I={cfg5.I} E={cfg5.E} top{k} sigmoid+renorm, "
                    f"N(0,1) logits, no shared expert, 2-bit planes -> bf16 MFMA grouped GEMM{extra}",
        "us_per_layer": round(ms * 1e3, 1),
        "tokens_per_s": round(T / (ms / 1e3), 1),
        "useful_tflops": round(fl / (ms / 1e3) / 1e12, 1),
        "mfma_frac": round(fl / (ms / 1e3) / 1e12 / peak, 4),
        "roofline": {"kernel": "fc1_prefill_kernel (gate/up grouped GEMM + SwiGLU)", "bound": "mfma",
                     "achieved": round(fl_fc1 / (fc1_ms / 1e3) / 1e12, 1), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(fl_fc1 / (fc1_ms / 1e3) / 1e12 / peak, 4),
                     # counters were taken on the chunk without gated tokens
                     "traffic": None if flags is not None else counted_traffic(
                         "prefill_kernels_mfma_hbm_counters_T4096_H7168_I2048_E256.md",
                         ("moe_prefill.hip", "moet_common.h")),
                     "avg_launch_us": round(fc1_ms * 1e3, 1), "algorithmic_flop_per_launch": fl_fc1},
    }


def main():
    args = parse()
    if args.summarize_counters:
        summarize_counters(args.summarize_counters)
        return
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the layer is not sharded across GPUs.",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch
    from bit_moe_expert_nvfp4_amd import moet, synth

    dev = "cuda"
    cfg = synth.CONFIGS[args.config]
    torch.cuda.set_device(0)
    print(f"[bench] building {args.layers} synthetic layers of '{cfg.name}' on the GPU", file=sys.stderr, flush=True)
    layers, srcs = [], []
    soe = synth.slot_of_expert(cfg, args.seed) if cfg.n_resident else None
    rq_ms = []
    for li in range(args.layers):
        src = synth.make_layer(cfg, seed=args.seed, device=dev, layer_index=li)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        layer = moet.layer_from_nvfp4(src, soe)
        e1.record()
        torch.cuda.synchronize()
        rq_ms.append(e0.elapsed_time(e1))
        layers.append(layer)
        if li == 0 and not args.no_cpu_baseline:
            srcs.append(src)
        else:
            del src
        torch.cuda.empty_cache()
        print(f"[bench] layer {li} ready (requant {rq_ms[-1]:.1f} ms)", file=sys.stderr, flush=True)

    xs = [synth.make_activations(cfg.T, cfg.H, args.seed, tag=f"x{i}", device=dev) for i in range(args.inputs)]
    lgs = [synth.make_logits(cfg, args.seed, tag=f"logits{i}", device=dev) for i in range(args.inputs)]
    flags = synth.gate_flags(cfg, args.seed).to(dev) if cfg.n_flagged else None
    route_out = [(torch.empty((cfg.T, cfg.k), dtype=torch.int32, device=dev),
                  torch.empty((cfg.T, cfg.k), dtype=torch.float32, device=dev),
                  torch.empty((cfg.E + 1,), dtype=torch.int32, device=dev),
                  torch.empty((cfg.T * cfg.k,), dtype=torch.int32, device=dev)) for _ in range(args.inputs)]
    out = torch.empty((cfg.T, cfg.H), dtype=torch.bfloat16, device=dev)
    ws = moet.alloc_workspace(layers[0], cfg.T, cfg.k, dev)

    def step(i):
        j = i % args.inputs
        layer = layers[i % args.layers]
        ids, w, offs, pairs = moet.route(lgs[j], cfg.k, cfg.score, cfg.renormalize, out=route_out[j])
        moet.moe_forward(layer, xs[j], ids, w, offs, pairs, flags, out=out, workspace=ws)

    for i in range(args.warmup):
        step(i)
    for j in range(args.inputs):       # every input set's routing, whatever the warm-up count
        moet.route(lgs[j], cfg.k, cfg.score, cfg.renormalize, out=route_out[j])
    torch.cuda.synchronize()
    # algorithmic bytes of each input set's routing (deterministic per input set)
    flags_np = flags.cpu().numpy() if flags is not None else None
    soe_np = soe.numpy() if soe is not None else None
    per_input = [step_bytes(cfg, route_out[j][0].cpu().numpy(), flags_np, soe_np) for j in range(args.inputs)]

    K = args.steps
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    for a, b in ev:      # create the underlying HIP events before handing them to the library
        a.record()
        b.record()
    # The timed region: K steps and nothing else inside it (event records between
    # launches add several microseconds per step on this runtime).
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record()
    for i in range(K):
        step(args.warmup + i)
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0

    # The same K steps again, instrumented: events at the step boundaries
    # (median / percentiles) and on the stream around every gate/up launch
    # (the roofline kernel's duration).
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
    torch.cuda.synchronize()
    marks[0].record()
    for i in range(K):
        moet.set_timing_events(*ev[i])
        step(args.warmup + i)
        marks[i + 1].record()
    torch.cuda.synchronize()
    moet.set_timing_events(None, None)
    step_us = np.array([marks[i].elapsed_time(marks[i + 1]) * 1e3 for i in range(K)])
    instrumented_us = marks[0].elapsed_time(marks[K]) / K * 1e3

    # cold steps: a 1 GiB streaming read between steps evicts the caches (the 256 MB last-level cache
    # and the L2s) without leaving dirty lines to write back during the step; only the step is timed
    cold = None
    if not args.no_cold:
        scratch = torch.ones((COPY_BYTES // 4,), dtype=torch.float32, device=dev)
        sink = torch.empty((moet.PROBE_SINK_WORDS,), dtype=torch.int32, device=dev)
        nc = min(K, 50)
        ce = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(nc)]
        torch.cuda.synchronize()
        for i in range(nc):
            moet.probe_read(scratch, sink)
            ce[i][0].record()
            step(args.warmup + i)
            ce[i][1].record()
        torch.cuda.synchronize()
        cus = np.array([a.elapsed_time(b) * 1e3 for a, b in ce])
        cold = {"steps": nc, "eviction": "1 GiB streaming read between steps",
                "median_us": round(float(np.median(cus)), 2), "p10_us": round(float(np.percentile(cus, 10)), 2),
                "p90_us": round(float(np.percentile(cus, 90)), 2)}
        del scratch, sink
        torch.cuda.empty_cache()

    # the same steps replayed from HIP graphs (one graph per layer/input combination)
    graph = None
    if not args.no_graph:
        import math
        combos = args.layers * args.inputs // math.gcd(args.layers, args.inputs)
        graphs = []
        cap = torch.cuda.Stream()
        cap.wait_stream(torch.cuda.current_stream())
        for c in range(combos):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cap):
                step(c)
            graphs.append(g)
        torch.cuda.synchronize()
        for i in range(args.warmup):
            graphs[i % combos].replay()
        torch.cuda.synchronize()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record()
        for i in range(K):
            graphs[(args.warmup + i) % combos].replay()
        g1.record()
        torch.cuda.synchronize()
        gms = g0.elapsed_time(g1) / K
        gbytes = sum(per_input[(args.warmup + i) % combos % args.inputs][0] for i in range(K)) / K
        graph = {"us_per_layer": round(gms * 1e3, 2), "GBps": round(gbytes / (gms / 1e3) / 1e9, 1),
                 "pct_hbm_peak": round(100.0 * gbytes / (gms / 1e3) / 1e9 / HBM_PEAK_GBS, 1),
                 "steps_per_graph": 1}
        # one graph holding all `combos` steps back to back (a whole model's decode step is one graph
        # in a serving loop): separates the per-graph-launch cost from the per-kernel-node cost
        gm = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gm, stream=cap):
            for c in range(combos):
                step(c)
        torch.cuda.synchronize()
        reps = max(1, K // combos)
        for _ in range(2):
            gm.replay()
        torch.cuda.synchronize()
        g0.record()
        for _ in range(reps):
            gm.replay()
        g1.record()
        torch.cuda.synchronize()
        mms = g0.elapsed_time(g1) / (reps * combos)
        mbytes = sum(per_input[c % args.inputs][0] for c in range(combos)) / combos
        graph["multi_step"] = {"steps_per_graph": combos, "replays": reps, "us_per_layer": round(mms * 1e3, 2),
                               "GBps": round(mbytes / (mms / 1e3) / 1e9, 1)}
        # replayed graphs must reproduce the eager output bit for bit
        ref = out.clone()
        step(args.warmup + K - 1)
        eager_last = out.clone()
        graphs[(args.warmup + K - 1) % combos].replay()
        torch.cuda.synchronize()
        graph["replay_matches_eager"] = bool(torch.equal(out, eager_last))
        del ref

    print("[bench] measuring the achievable HBM read / copy and bf16 GEMM rates", file=sys.stderr, flush=True)
    ach = achievable_refs(dev)

    total_ms = t_start.elapsed_time(t_end)
    ms_per_step = total_ms / K
    fc1_ms = [ev[i][0].elapsed_time(ev[i][1]) for i in range(K)]
    tot_bytes = sum(per_input[(args.warmup + i) % args.inputs][0] for i in range(K))
    fc1_bytes = sum(per_input[(args.warmup + i) % args.inputs][1] for i in range(K))
    gbs = tot_bytes / (total_ms / 1e3) / 1e9
    fc1_gbs = fc1_bytes / (sum(fc1_ms) / 1e3) / 1e9
    n_experts = np.mean([p[2] for p in per_input])

    result = {
        "metric": "MoE layer decode us + effective weight HBM GB/s (% peak), 1 MI355X",
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: T={cfg.T} H={cfg.H} I={cfg.I} E={cfg.E} top{cfg.k} "
                               f"{'sigmoid' if cfg.score else 'softmax'}+renorm"
                               f"{' + shared expert' if cfg.shared else ''}"
                               f"{f' + FP4 delta ({cfg.n_resident} resident, {cfg.n_flagged} flagged)' if cfg.n_resident else ''}"
                               f", 2-bit planes, {args.layers}-layer pool, {args.inputs} input sets",
                   "T": cfg.T, "H": cfg.H, "I": cfg.I, "E": cfg.E, "top_k": cfg.k},
        "us_per_layer": round(ms_per_step * 1e3, 2),
        "pct_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 1),
        "pct_hbm_achievable_read": round(100.0 * gbs / ach["read_GBps"], 1),
        "achievable": ach,
        "tokens_per_s": round(cfg.T / (ms_per_step / 1e3), 1),
        "mean_experts_per_step": round(float(n_experts), 2),
        "algorithmic_bytes_per_step": round(tot_bytes / K),
        "requant_ms_per_layer": round(float(np.median(rq_ms)), 2),
        "instrumented_us_per_layer": round(instrumented_us, 2),
        "step_us_median": round(float(np.median(step_us)), 2),
        "step_us_p10": round(float(np.percentile(step_us, 10)), 2),
        "step_us_p90": round(float(np.percentile(step_us, 90)), 2),
        "cold": cold,
        "wall_s_timed_region": round(wall, 4),
        "graph_replay": graph,
        "roofline": {
            "kernel": "fc1_decode_kernel (gate/up GEMV + SwiGLU)",
            "bound": "hbm",
            "achieved": round(fc1_gbs, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(fc1_gbs / HBM_PEAK_GBS, 4),
            "traffic": counted_traffic(),
            "achievable_peak": ach["read_GBps"],
            "frac_achievable": round(fc1_gbs / ach["read_GBps"], 4),
            "avg_launch_us": round(1e3 * float(np.mean(fc1_ms)), 2),
            "algorithmic_bytes_per_launch": round(fc1_bytes / K),
        },
    }
    if not args.no_prefill:
        print("[bench] timing the prefill chunk", file=sys.stderr, flush=True)
        import dataclasses
        pl = dataclasses.replace(layers[0], shared13=None, shared2=None)
        result["prefill"] = prefill_leg(pl, synth.CONFIGS["prefill"], args.prefill_steps, args.seed, dev)
        # the same chunk with gate-flagged tokens on delta-cache experts, right after and with as many steps
        print("[bench] timing the prefill chunk with the FP4 delta", file=sys.stderr, flush=True)
        cfgd = dataclasses.replace(synth.CONFIGS["prefill"], name="prefill_delta", n_resident=32, n_flagged=2048)
        srcd = synth.make_layer(cfgd, seed=args.seed, device=dev)
        soed = synth.slot_of_expert(cfgd, args.seed)
        ld = moet.layer_from_nvfp4(srcd, soed)
        del srcd
        torch.cuda.empty_cache()
        result["prefill_delta"] = prefill_leg(ld, cfgd, args.prefill_steps, args.seed, dev,
                                              flags=synth.gate_flags(cfgd, args.seed).to(dev), soe=soed)
        del ld
        torch.cuda.empty_cache()
        for key in ("prefill", "prefill_delta"):
            rf = result[key]["roofline"]
            rf["achievable_peak"] = ach["mfma_bf16_loop_TFLOPs"]
            rf["frac_achievable"] = round(rf["achieved"] / ach["mfma_bf16_loop_TFLOPs"], 4)
            rf["frac_of_hipblaslt_gemm"] = round(rf["achieved"] / ach["bf16_gemm_TFLOPs"], 4)
    if not args.no_extra:
        print("[bench] timing the confidence gate", file=sys.stderr, flush=True)
        result["confidence_gate"] = gate_leg(args.seed, dev)
        print("[bench] timing the load-time conversions", file=sys.stderr, flush=True)
        result["load_conversions"] = conversion_leg(args.seed, dev)
        del layers
        torch.cuda.empty_cache()
        result["other_decode"] = {}
        for cname, key, frac, tp in (("decode_mtp_delta", "delta_cache", None, 1),
                                     ("batched_decode", "batched", None, 1),
                                     ("decode_mtp", "expert_cache_half", 0.5, 1),
                                     ("decode_mtp", "tp2_shard", None, 2),
                                     ("decode_mtp", "tp4_shard", None, 4)):
            print(f"[bench] timing decode config {key}", file=sys.stderr, flush=True)
            result["other_decode"][key] = decode_leg(cname, args.extra_steps, 10, args.seed, dev,
                                                     cache_fraction=frac, tp=tp)
        print("[bench] timing decode with an NVFP4 shared expert", file=sys.stderr, flush=True)
        result["other_decode"]["nvfp4_shared"] = decode_leg("decode_mtp", args.extra_steps, 10, args.seed, dev,
                                                            shared_nvfp4=True)
    if not args.no_cpu_baseline:
        print("[bench] timing the oracle on the host (bounded sample)", file=sys.stderr, flush=True)
        c5 = synth.CONFIGS["prefill"]
        cb = cpu_baseline(cfg, srcs[0], xs[0], lgs[0], args.seed, cfg_prefill=c5,
                          x_prefill=synth.make_activations(c5.T, c5.H, args.seed, tag="prefill_x", device=dev),
                          lg_prefill=synth.make_logits(c5, args.seed, tag="prefill_logits", device=dev))
        cb["value"] = round(cb["value"], 4)
        result["cpu_baseline"] = cb
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
