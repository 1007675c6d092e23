"""Benchmark of the MoE-layer hot path on one MI355X.

One step = one forward pass of the whole layer over one batch.  The default
workload is the largest single-GPU one, the 128-expert top-6 sigmoid model
(T=8192 tokens, d=2688, E=128, k=6, ffn 1856, weights normalised over the
6 chosen, bf16 storage, fp32 accumulation and router math):
    route -> permute (index work only) -> grouped SwiGLU on tile-packed
    weights (fc1 gathers the token rows from x by the permute's row map; fc2
    applies the routing weight as its row scale) -> combine
Inputs are seeded synthetic tensors already resident in HBM; every launch
goes through the C ABI (libmoe_mi355x.so).

Prints ONE JSON line.  `value` is layer tokens/s; the grouped-GEMM TFLOP/s
and its fraction of the bf16 MFMA peak are reported beside it.  `roofline`
describes the grouped-GEMM forward call (its fc1 and fc2 launches on one
stream), timed with HIP events around that call inside the timed region;
the timed steps record no other event (an event record is a barrier between
kernels) and the per-stage breakdown comes from a further, untimed pass.
`cpu_baseline` times the CPU oracle in float32, stage by stage, on the same
batch.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0        # MI355X dense bf16 MFMA, AMD's published figure
PEAK_FP8_TFLOPS = 5000.0         # MI355X dense fp8 MFMA, AMD's published figure
PEAK_HBM_GBS = 8000.0            # MI355X HBM3E, AMD's published figure
COLD_FLUSH_BYTES = 1 << 30        # scratch read before each cold stage (> L2 + 256 MB MALL)

# HBM bytes per grouped-GEMM forward call (fc1 + fc2 dispatches), from
# `rocprofv3 --pmc FETCH_SIZE` and `--pmc WRITE_SIZE` runs of this script,
# each counter scaled by what it reads for a 1 GiB device copy
# (--copy-calibration: FETCH_SIZE x 2.0, WRITE_SIZE x 1.0); summary in
# profiles/grouped_gemm_fwd_<workload>_hbm_bytes.md.  Valid only for the
# kernel sources the counters were taken on (sha256 over KERNEL_SOURCES):
# reported as null once they change.
KERNEL_SOURCES = ("mixture_experts_layer_05_amd/csrc/moe_grouped_fwd.hip",
                  "mixture_experts_layer_05_amd/csrc/moe_gemm_common.h",
                  "mixture_experts_layer_05_amd/csrc/moe_device.h")
KERNEL_SOURCES_FP8 = ("mixture_experts_layer_05_amd/csrc/moe_grouped_mx.hip",
                      "mixture_experts_layer_05_amd/csrc/moe_sched.h",
                      "mixture_experts_layer_05_amd/csrc/moe_gemm_common.h",
                      "mixture_experts_layer_05_amd/csrc/moe_device.h")
# (fp8: profiles/fp8_grouped_gemm_qwen3_30b_hbm_bytes.md, the quantiser + fc1 + fc2)
MEASURED_TRAFFIC = {
    # profiles/grouped_gemm_fwd_qwen3_30b_hbm_bytes.md
    "qwen3_30b": {"bytes": 1618103002,
                  "sources_sha256": "c092b99d9bd5523c6145da816aaf9d0b24e5fb96220a1024d7bf8fe392d0f769"},
    # profiles/grouped_gemm_fwd_dsv_30b_hbm_bytes.md
    "dsv_30b": {"bytes": 5522464015,
                "sources_sha256": "c092b99d9bd5523c6145da816aaf9d0b24e5fb96220a1024d7bf8fe392d0f769"},
    # profiles/grouped_gemm_fwd_skew_shared_hbm_bytes.md
    "skew_shared": {"bytes": 3649920218,
                    "sources_sha256": "c092b99d9bd5523c6145da816aaf9d0b24e5fb96220a1024d7bf8fe392d0f769"},
    "qwen3_30b:fp8": {"bytes": 966677333,
                      "sources_sha256": "b0b29d0cde5fa5331b7045cb561580f6e813dd4eb7905a37d057c41c0c94631a"},
}


def measured_traffic(workload, fp8=False):
    import hashlib
    rec = MEASURED_TRAFFIC.get(workload + (":fp8" if fp8 else ""))
    if rec is None:
        return None
    h = hashlib.sha256()
    for f in (KERNEL_SOURCES_FP8 if fp8 else KERNEL_SOURCES):
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return rec["bytes"] if h.hexdigest() == rec["sources_sha256"] else None


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="dsv_30b")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--fp8", action="store_true",
                    help="expert GEMMs in MXFP8 (E4M3, 32-value E8M0 block scales)")
    ap.add_argument("--cpu-sample-tokens", type=int, default=8192)
    ap.add_argument("--train", action="store_true",
                    help="time a training step of the layer (forward keeping what the "
                         "backward needs + the full backward) instead of the forward")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain device copy of known size (scales the HBM "
                         "byte counters FETCH_SIZE / WRITE_SIZE) and exit")
    return ap.parse_args()


COPY_CAL_BYTES = 1 << 30


def copy_calibration():
    """A plain 1 GiB device-to-device copy, five times; under `rocprofv3 --pmc`
    each dispatch should read and write COPY_CAL_BYTES."""
    import torch
    dev = torch.device("cuda", 0)
    src = torch.ones(COPY_CAL_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": COPY_CAL_BYTES, "dispatches": 5}), flush=True)


def algorithmic(cfg, fp8=False, fold_shared=False):
    """Per-call algorithmic work (what the method itself must move or do).
    With fold_shared the grouped-GEMM call also runs the shared expert (T
    more rows of ffn Fs, its weights read once, its output written)."""
    T, d, E, k, F = cfg.T, cfg.d, cfg.E, cfg.k, cfg.F
    N = T * k
    b = 2
    gemm_flop = 6.0 * N * d * F
    if fp8:
        # MX operands: a byte per value plus a scale byte per 32.  x read (bf16)
        # and its codes written by the quantiser, then read once by fc1; expert
        # weight codes read once; A's codes written and read; Y_perm written (bf16)
        q = 1.0 + 1.0 / 32
        gemm_bytes = (T * d * (b + q) + T * d * q + 3.0 * E * d * F * q + 2.0 * N * F * q
                      + N * d * b)
    else:
        # expert weights read once + token rows read once (fc1 gathers them from x)
        # + A written and read + Y_perm written
        gemm_bytes = 3.0 * E * d * F * b + T * d * b + 2.0 * N * F * b + N * d * b
    if fold_shared and cfg.Fs:
        Fs = cfg.Fs
        w = (1.0 + 1.0 / 32) if fp8 else b
        gemm_flop += 6.0 * T * d * Fs
        gemm_bytes += 3.0 * d * Fs * w + 2.0 * T * Fs * w + T * d * b
    route_bytes = T * (2 * d + 8 * k + 4) + E * d * b
    # permute without the row copy: topk_idx, topk_w read; slot_of, row_token, row_w written
    permute_bytes = T * 20 * k
    combine_bytes = T * (2 * d * (k + 1) + 4 * k)
    return dict(gemm_flop=gemm_flop, gemm_bytes=gemm_bytes, route_bytes=route_bytes,
                permute_bytes=permute_bytes, combine_bytes=combine_bytes)


def _blas_threads():
    threads = None
    try:
        from threadpoolctl import threadpool_info
        threads = max((p.get("num_threads", 1) for p in threadpool_info()), default=None)
    except Exception:
        pass
    if threads is None:
        threads = len(os.sched_getaffinity(0))
    return int(threads)


def _median_time(fn, min_total=6.0, max_reps=15, single_if_over=30.0):
    """Median wall time of repeated calls: at least 3, and as many more (up to
    `max_reps`) as fill about `min_total` seconds; one call when the first
    exceeds `single_if_over` seconds.  Returns (seconds, last result)."""
    ts, out = [], None
    t0 = time.perf_counter()
    out = fn()
    ts.append(time.perf_counter() - t0)
    if ts[0] <= single_if_over:
        reps = min(max_reps, max(3, int(min_total / max(ts[0], 1e-6))))
        for _ in range(reps - 1):
            t0 = time.perf_counter()
            out = fn()
            ts.append(time.perf_counter() - t0)
    ts.sort()
    return ts[len(ts) // 2], out


def cpu_baseline(inp, cfg, ntok):
    """The oracle as it stands, in float32 (numpy; BLAS threads = the host's
    cores), stage by stage on the first `ntok` tokens of the batch: route,
    permute, expert FFN (all experts the tokens chose), shared expert,
    combine.  Each stage is the median of 3 to 15 runs (about 6 s of work per
    stage at most); the float32 copies of the bf16 inputs are made before the
    clock starts."""
    import numpy as np
    from oracle import moe_oracle as mo
    f = inp.as_f32
    x = f("x")[:ntok]
    wr, w1, w2 = f("w_router"), f("w1"), f("w2")
    wg, ws1, ws2 = f("w_gate"), f("ws1"), f("ws2")
    p32 = np.float32
    st = {}
    st["route"], r = _median_time(lambda: mo.route(x, wr, cfg.k, cfg.score, cfg.normalize,
                                                   inp.logit_bias, wg, prec=p32))
    st["permute"], pm = _median_time(lambda: mo.permute(x, r.topk_idx, r.topk_w, cfg.E))
    st["expert_ffn"], yp = _median_time(
        lambda: mo.grouped_swiglu_fwd(pm.x_perm, w1, w2, pm.offsets, None, prec=p32))
    ysh = None
    if ws1 is not None:
        st["shared_expert"], ysh = _median_time(lambda: mo.shared_expert(x, ws1, ws2, r.gate, p32))
    st["combine"], y = _median_time(lambda: mo.unpermute_combine(yp, pm.slot_of, r.topk_w, ysh,
                                                                 prec=p32))
    assert np.isfinite(y).all()
    total = sum(st.values())
    return {"value": round(ntok / total, 1), "unit": "tokens/s", "cores": _blas_threads(),
            "kind": "oracle",
            "sample": f"first {ntok} of {cfg.T} tokens of the {cfg.name} batch, all {cfg.E} "
                      f"experts, float32 oracle forward stage by stage (median of 3-15 runs each)",
            "stage_s": {kk: round(v, 4) for kk, v in st.items()}}


def cpu_baseline_ep_share(inp, cfg):
    """The oracle (float32) on the expert-parallel share: grouped SwiGLU
    forward and the grouped-GEMM backward (dgrad + wgrad), all experts."""
    import numpy as np
    from oracle import moe_oracle as mo
    x = mw_f32(inp.x_perm)
    dy = mw_f32(inp.dy)
    w1, w2 = mw_f32(inp.w1), mw_f32(inp.w2)
    p32 = np.float32
    st = {}
    st["expert_ffn_fwd"], _ = _median_time(
        lambda: mo.grouped_swiglu_fwd(x, w1, w2, inp.offsets, None, prec=p32))
    st["expert_ffn_bwd"], g = _median_time(
        lambda: mo.grouped_swiglu_bwd(dy, x, w1, w2, inp.offsets, None, prec=p32))
    assert np.isfinite(g[0]).all()
    flop = 18.0 * cfg.N * cfg.d * cfg.F
    return {"value": round(flop / sum(st.values()) / 1e12, 4), "unit": "TFLOP/s",
            "cores": _blas_threads(), "kind": "oracle",
            "sample": f"all {cfg.N} token-slots and {cfg.E} experts of the {cfg.name} batch, "
                      "float32 oracle grouped forward + backward (median of 3-15 runs each)",
            "stage_s": {kk: round(v, 4) for kk, v in st.items()}}


def mw_f32(a):
    import moe_workloads as mw
    return mw.bf16_bits_to_f32(a) if a.dtype.name == "uint16" else a


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(expert-parallel sharding is not implemented).", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        return copy_calibration()

    import numpy as np
    import torch

    import moe_workloads as mw
    import mixture_experts_layer_05_amd as moe

    cfg = mw.get(args.workload)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    if cfg.backward:
        return bench_ep_share(args, cfg, dev)
    if args.train:
        return bench_train(args, cfg, dev)
    inp = mw.make_layer_inputs(cfg)

    def gpu(a):
        if a is None:
            return None
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    x = gpu(inp.x)
    layer = moe.MoELayer(gpu(inp.w_router), gpu(inp.w1), gpu(inp.w2), cfg.k, cfg.T, cfg.score,
                         cfg.normalize, gpu(inp.logit_bias), gpu(inp.w_gate), gpu(inp.ws1),
                         gpu(inp.ws2), fp8=args.fp8)
    stream = torch.cuda.current_stream()

    stages = ["route", "permute", "grouped_gemm", "shared", "combine"]

    def step(ev=None, gemm_ev=None):
        # the layer's forward, stage by stage (MoELayer.stages), with events
        # on the stream (all stage boundaries: ev; the grouped GEMM only: gemm_ev)
        for j, (name, fn) in enumerate(layer.stages(x)):
            if ev is not None:
                ev[j].record(stream)
            if gemm_ev is not None and name == "grouped_gemm":
                gemm_ev[0].record(stream)
            fn()
            if gemm_ev is not None and name == "grouped_gemm":
                gemm_ev[1].record(stream)
        if ev is not None:
            ev[len(stages)].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Timed steps: the only events in them bracket the grouped-GEMM stage (the
    # roofline's kernel); an event record is a barrier between kernels, so
    # the stage breakdown comes from a separate, untimed pass below.
    gev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(gemm_ev=gev[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    t_gemm_ms = sum(e[0].elapsed_time(e[1]) for e in gev) / args.steps

    nbreak = max(5, min(args.steps, 20))
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(nbreak)]
    for i in range(nbreak):
        step(evs[i])
    torch.cuda.synchronize()
    per_stage = {s: 0.0 for s in stages}
    total_ev = 0.0
    for ev in evs:
        for j, s in enumerate(stages):
            per_stage[s] += ev[j].elapsed_time(ev[j + 1])
        total_ev += ev[0].elapsed_time(ev[5])
    per_stage = {s: v / nbreak for s, v in per_stage.items()}  # ms per call

    # Cold stages: a 1 GiB scratch read (larger than L2 and the 256 MB
    # Infinity Cache) before each stage, outside its event pair; a shared
    # expert's own call (when not folded into the grouped GEMM) runs untimed.
    # A read, not a fill: a fill leaves up to 256 MB of dirty cache lines
    # whose write-back would be charged to the stage that evicts them.
    scratch = torch.ones(COLD_FLUSH_BYTES // 4, dtype=torch.float32, device=dev)
    cold_stages = ["route", "permute", "grouped_gemm", "combine"]
    ncold = 5
    cev = [[torch.cuda.Event(enable_timing=True) for _ in range(8)] for _ in range(ncold)]
    for i in range(ncold):
        j = 0
        for name, fn in layer.stages(x):
            if name in cold_stages:
                scratch.amax()
                cev[i][2 * j].record(stream)
                fn()
                cev[i][2 * j + 1].record(stream)
                j += 1
            else:
                fn()
    torch.cuda.synchronize()
    del scratch
    cold = {s: sum(e[2 * j].elapsed_time(e[2 * j + 1]) for e in cev) / ncold
            for j, s in enumerate(cold_stages)}
    ms_per_step = wall * 1e3 / args.steps
    tokens_per_s = cfg.T / (wall / args.steps)

    alg = algorithmic(cfg, args.fp8, layer.fold_shared)
    peak_mfma = PEAK_FP8_TFLOPS if args.fp8 else PEAK_BF16_TFLOPS
    t_gemm = t_gemm_ms * 1e-3
    gemm_tflops = alg["gemm_flop"] / t_gemm / 1e12
    gemm_gbs = alg["gemm_bytes"] / t_gemm / 1e9
    # the binding roof of the grouped GEMM: whichever of MFMA and HBM time is longer
    t_mfma = alg["gemm_flop"] / (peak_mfma * 1e12)
    t_hbm = alg["gemm_bytes"] / (PEAK_HBM_GBS * 1e9)
    traffic = measured_traffic(cfg.name, args.fp8)
    if t_hbm > t_mfma:
        roof = {"bound": "hbm", "achieved": round(gemm_gbs, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(gemm_gbs / PEAK_HBM_GBS, 4), "traffic": traffic}
    else:
        roof = {"bound": "mfma", "achieved": round(gemm_tflops, 1), "peak": peak_mfma,
                "unit": "TFLOP/s", "frac": round(gemm_tflops / peak_mfma, 4),
                "traffic": traffic}
    if args.fp8:
        roof["kernel"] = ("moe_quantize_mx of x + moe_grouped_swiglu_fwd_mx (persistent MXFP8 fc1 "
                          "gather+SwiGLU+A quantisation and fc2+row-scale launches)")
    else:
        roof["kernel"] = ("moe_grouped_swiglu_fwd_packed (persistent fc1 gather+SwiGLU and "
                          "fc2+row-scale launches on tile-packed weights)")
    if layer.fold_shared:
        roof["kernel"] += "; the shared expert runs in the same call as group E"
    roof["algorithmic_flop"] = alg["gemm_flop"]
    roof["algorithmic_bytes"] = alg["gemm_bytes"]
    # attainable rate on the roofline: min(MFMA peak, arithmetic intensity x HBM peak)
    attain = min(peak_mfma, alg["gemm_flop"] / alg["gemm_bytes"] * PEAK_HBM_GBS / 1e3)
    roof["attainable_tflops"] = round(attain, 1)
    roof["attainable_frac"] = round(gemm_tflops / attain, 4)
    roof["avg_launch_ms"] = round(t_gemm_ms, 4)
    roof["traffic_unit"] = "bytes per call (HBM, counter-measured)"

    def gbs(key, stage, table=None):
        t = (table or per_stage)[stage] * 1e-3
        return round(alg[key] / t / 1e9, 1) if t > 0 else None

    cold_gbs = {"route": gbs("route_bytes", "route", cold),
                "permute": gbs("permute_bytes", "permute", cold),
                "combine": gbs("combine_bytes", "combine", cold)}

    out = {
        "metric": "MoE layer tokens/sec + grouped-GEMM TFLOP/s (% bf16 MFMA peak), 1 MI355X",
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3_mx" if args.fp8 else "bf16",
        "data": "synthetic (seeded PCG64; x~N(0,1), router~N(0,1/d), experts~N(0,0.02^2))",
        "config": {"workload": f"{cfg.name}: T={cfg.T} d={cfg.d} E={cfg.E} top-{cfg.k} "
                               f"{cfg.score} ffn={cfg.F}", "T": cfg.T, "d": cfg.d, "E": cfg.E,
                   "k": cfg.k, "F": cfg.F, "Fs": cfg.Fs, "score": cfg.score,
                   "shared_expert": ("folded into the grouped GEMM" if layer.fold_shared else
                                     "own grouped call") if cfg.Fs else None,
                   "expert_gemms": ("MXFP8: E4M3 values, E8M0 scale per 32 along K, fp32 "
                                    "accumulation; routing bf16/fp32") if args.fp8 else "bf16"},
        "grouped_gemm_tflops": round(gemm_tflops, 1),
        "grouped_gemm_mfma_frac": round(gemm_tflops / peak_mfma, 4),
        "mfma_peak_tflops": peak_mfma,
        "stage_ms": {s: round(v, 4) for s, v in per_stage.items()},
        "stage_ms_note": f"from {nbreak} further steps with an event between stages (untimed)",
        "stage_gbs": {"route": gbs("route_bytes", "route"),
                      "permute": gbs("permute_bytes", "permute"),
                      "combine": gbs("combine_bytes", "combine")},
        "event_ms_per_step": round(total_ev / nbreak, 4),
        "stage_ms_cold": {s: round(v, 4) for s, v in cold.items()},
        "stage_gbs_cold": cold_gbs,
        "stage_hbm_frac_cold": {s: (round(v / PEAK_HBM_GBS, 4) if v else None)
                                for s, v in cold_gbs.items()},
        "stage_cold_note": (f"{ncold} further steps, a {COLD_FLUSH_BYTES >> 30} GiB scratch "
                            "read before each stage outside its events (L2 and Infinity Cache "
                            "evicted, no dirty lines left); algorithmic bytes / event time"),
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(inp, cfg, min(args.cpu_sample_tokens, cfg.T))
    print(json.dumps(out), flush=True)


def bench_train(args, cfg, dev):
    """One training step of the whole layer: forward in training mode (x_perm,
    G/U and unweighted expert outputs kept) + backward (combine backward,
    grouped-GEMM dgrad/wgrad, shared expert, permute + router backward)."""
    import numpy as np
    import torch

    import moe_workloads as mw
    import mixture_experts_layer_05_amd as moe

    inp = mw.make_layer_inputs(cfg)

    def gpu(a):
        if a is None:
            return None
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    x = gpu(inp.x)
    rng = np.random.default_rng(cfg.index + 500)
    dy = gpu(mw.round_to_bf16_bits(rng.standard_normal((cfg.T, cfg.d)).astype(np.float32)))
    layer = moe.MoELayer(gpu(inp.w_router), gpu(inp.w1), gpu(inp.w2), cfg.k, cfg.T, cfg.score,
                         cfg.normalize, gpu(inp.logit_bias), gpu(inp.w_gate), gpu(inp.ws1),
                         gpu(inp.ws2), train=True)
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        layer.forward(x)
        if ev is not None:
            ev[1].record(stream)
        layer.backward(dy)
        if ev is not None:
            ev[2].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    t_f = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps
    t_b = sum(e[1].elapsed_time(e[2]) for e in evs) / args.steps
    N = cfg.T * cfg.k
    flop = 18.0 * N * cfg.d * cfg.F + 18.0 * cfg.T * cfg.d * cfg.Fs
    out = {
        "metric": "MoE layer training step (fwd+bwd) tokens/s, 1 MI355X",
        "value": round(cfg.T / (wall / args.steps), 1),
        "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded PCG64, same recipe as the forward bench; dy ~ N(0,1))",
        "config": {"workload": f"{cfg.name}: T={cfg.T} d={cfg.d} E={cfg.E} top-{cfg.k} "
                               f"{cfg.score} ffn={cfg.F} shared={cfg.Fs}"},
        "fwd_ms": round(t_f, 4), "bwd_ms": round(t_b, 4),
        "expert_gemm_tflops_fwd_bwd": round(flop / ((t_f + t_b) * 1e-3) / 1e12, 1),
    }
    print(json.dumps(out), flush=True)


def bench_ep_share(args, cfg, dev):
    """One expert-parallel rank's share: grouped SwiGLU forward (saving G, U)
    plus the grouped-GEMM backward (dgrad and fp32 wgrad) per step."""
    import numpy as np
    import torch

    import moe_workloads as mw
    import mixture_experts_layer_05_amd as moe

    inp = mw.make_ep_share_inputs(cfg)

    def gpu(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    x, w1, w2, dy, off = gpu(inp.x_perm), gpu(inp.w1), gpu(inp.w2), gpu(inp.dy), gpu(inp.offsets)
    N, d, E, F = cfg.N, cfg.d, cfg.E, cfg.F
    y = torch.empty((N, d), dtype=torch.bfloat16, device=dev)
    gu = torch.empty((N, 2 * F), dtype=torch.bfloat16, device=dev)
    dx = torch.empty_like(x)
    dw1 = torch.empty((E, 2 * F, d), dtype=torch.float32, device=dev)
    dw2 = torch.empty((E, d, F), dtype=torch.float32, device=dev)
    ws_f = moe._ws(moe.fwd_workspace_size(N, F, torch.bfloat16), dev)
    ws_b = moe._ws(moe.bwd_workspace_size(N, F, torch.bfloat16, False), dev)
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        moe.grouped_swiglu_fwd(x, w1, w2, off, None, True, out=y, gu_out=gu, ws=ws_f)
        if ev is not None:
            ev[1].record(stream)
        moe.grouped_swiglu_bwd(dy, x, w1, w2, off, gu, None, False, dw1, dw2, dx_out=dx, ws=ws_b)
        if ev is not None:
            ev[2].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    t_f = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps
    t_b = sum(e[1].elapsed_time(e[2]) for e in evs) / args.steps
    flop_f = 6.0 * N * d * F
    flop_b = 12.0 * N * d * F
    out = {
        "metric": "grouped-GEMM fwd+bwd TFLOP/s on one expert-parallel share, 1 MI355X",
        "value": round((flop_f + flop_b) / (wall / args.steps) / 1e12, 1),
        "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{cfg.name}: {E} local experts, {N} token-slots, d={d} ffn={F}"},
        "fwd_ms": round(t_f, 4), "bwd_ms": round(t_b, 4),
        "fwd_tflops": round(flop_f / t_f / 1e9, 1), "bwd_tflops": round(flop_b / t_b / 1e9, 1),
    }
    # roofline of the dominant call, the backward (dgrad + fp32 wgrad): its
    # algorithmic bytes read dY, X_perm, W1, W2 and [G | U] once, write dX,
    # dW1, dW2 (fp32) once, and write and read back dH [N, 2F] and the
    # recomputed SwiGLU output [N, F] once each
    b = 2
    bytes_b = (2 * N * d * b + 3 * E * d * F * b + N * 2 * F * b + N * d * b + 3 * E * d * F * 4
               + 2 * N * 2 * F * b + 2 * N * F * b)
    t_mfma = flop_b / (PEAK_BF16_TFLOPS * 1e12)
    t_hbm = bytes_b / (PEAK_HBM_GBS * 1e9)
    tf_b = flop_b / t_b / 1e9
    gbs_b = bytes_b / t_b / 1e6
    attain = min(PEAK_BF16_TFLOPS, flop_b / bytes_b * PEAK_HBM_GBS / 1e3)
    if t_hbm > t_mfma:
        roof = {"bound": "hbm", "achieved": round(gbs_b, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(gbs_b / PEAK_HBM_GBS, 4)}
    else:
        roof = {"bound": "mfma", "achieved": round(tf_b, 1), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(tf_b / PEAK_BF16_TFLOPS, 4)}
    roof.update({"traffic": None, "kernel": "moe_grouped_swiglu_bwd (fc2 dgrad + SwiGLU backward, "
                 "fc1 dgrad, fp32 wgrad of W1 and W2)", "algorithmic_flop": flop_b,
                 "algorithmic_bytes": bytes_b, "avg_launch_ms": round(t_b, 4),
                 "attainable_tflops": round(attain, 1), "attainable_frac": round(tf_b / attain, 4)})
    out["roofline"] = roof
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_ep_share(inp, cfg)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
