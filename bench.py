"""Throughput of prefix-tree-packed tree attention + the decision epilogue on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config all|0-4[,..]] [--seed 0]

One step = one pass of the device hot path over one batch: for every forward
of the workload, the chunk's K/V cache write and the tree-attention launch
(the two launches tree_attn_forward_chunked makes, issued through its two
halves so the attention launch can be timed on its own), then the decision
epilogue for the batch. The plan (host validation, token tables, block-sparse
schedule, upload) is built once per batch before the timed region: it is
shared by every layer of a model, and its host time is reported as
plan_build_ms. Inputs are resident in HBM before timing starts.
`ms_per_step` times the K steps with nothing between their launches (an
event recorded between two launches leaves a gap of its own); the per-launch
times (attention, cache write) come from K further steps with HIP events
around each launch.

By default the four 8192-token workloads (configs 1-4) are timed one after
the other; the first (the Llama-8B-shaped forward) is the headline and the
others are reported under `configs` with the same per-launch figures.

Prints one JSON line. `value` is useful tree-attention TFLOP/s over the whole
step (useful FLOPs = 4 * head_dim * q_heads * sum over query tokens of the
keys each may see); `roofline` is the attention kernel alone, timed with HIP
events on the launch stream; `cpu_baseline` is the float64 CPU oracle on a
bounded sample of the same workload (rank 0, one GPU only). `readout` times
the readout-only last layer (MLP block at the leaf readout rows, letter
logits) on the Llama shape matching the workload's heads, against HBM
bandwidth (it streams the MLP weights once); it is not part of the step.
Every timed part first runs its own work back to back for --device-warmup-ms
of wall time (reported as `device_warmup`), then its W warm-up steps: the
device reaches its sustained clock only after about 30 ms of load, and a
timed region right after idle measures the ramp (config[1] attention ran
275 us per step over the first steps and 222 us from about 30 ms on).
`mfma_attainable` is the rate a register-only MFMA loop reaches on this device
(the shader clock under load is below the published peak's 2.4 GHz), reported
beside the published peak; `attention_ms_p10_p50_p90` spreads the timed
launches; `roofline.per_launch.algorithmic_gbps` and `kv_stream_gbps_per_forward`
give the byte rates (the bound that matters for short-block workloads).
`latency` gives the launch-latency-bound parts in microseconds: the small
144-token workload (config[0]: cache write + attention) and the decision
epilogue (config[0]'s one decision and the headline workload's batch), each
per call over calls back to back and alone (the median of single calls
between two events, which includes the events' own gaps).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_F16_TFLOPS = 2516.6   # MI355X dense f16 MFMA: 256 CU x 2.4 GHz x 4096 FLOP/clk
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "tree_attn_fwd_traffic.txt")
KERNEL_SOURCES = ["prefix_tree_packed_amd/csrc/attn_fwd.hip", "prefix_tree_packed_amd/csrc/layout.h",
                  "prefix_tree_packed_amd/build.py"]


def kernel_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(config: int, forward: int):
    """HBM bytes per launch of the attention kernel from the committed profiler
    record, or None when there is none for this workload or the kernel sources
    changed since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as fh:
            lines = [l.split() for l in fh if l.strip() and not l.startswith("#")]
    except OSError:
        return None
    rec = {l[0]: l[1:] for l in lines if len(l) == 2}
    if rec.get("kernel_sha256_16", [None])[0] != kernel_hash():
        return None
    for l in lines:
        if len(l) == 6 and l[0] == f"config{config}" and l[1] == f"forward{forward}":
            return {"fetch_bytes": int(l[3]), "write_bytes": int(l[5])}
    return None


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="all",
                    help="workload index 0-4, a comma list, or 'all' (the 8192-token workloads "
                         "1,2,3,4; the first listed of them is the headline)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--out-dtype", default="f16", choices=["f16", "f32"])
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target wall time of the headline workload's CPU-oracle sample "
                         "(the other workloads get half of it each)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--batch-invariant", action="store_true",
                    help="key tiles by position in each query's own prompt (bitwise-identical "
                         "results alone / in a batch / in a tree) instead of the union tiling")
    ap.add_argument("--rope", choices=["half", "interleaved"], default=None,
                    help="rotate Q and K at the tokens' prompt positions in the cache write "
                         "(fused rotary + cache write) before attention")
    ap.add_argument("--no-mfma-probe", action="store_true",
                    help="skip measuring the MFMA rate the device reaches (register-only loop)")
    ap.add_argument("--no-readout", action="store_true",
                    help="skip timing the readout-only last layer (MLP block and letter logits)")
    ap.add_argument("--no-latency", action="store_true",
                    help="skip timing the launch-latency-bound parts (config[0], decisions)")
    ap.add_argument("--device-warmup-ms", type=float, default=100.0,
                    help="before the W warm-up steps, run steps until this much wall time of "
                         "sustained load has passed: the device needs about 30 ms of load to "
                         "reach its sustained clock (the first steps run up to 25%% slower)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after timing, run one plain 256 MiB device copy (known bytes) so "
                         "profiler byte counters can be scaled against it")
    return ap.parse_args()


def device_warmup(fn, ms: float) -> dict:
    """Runs fn (one unit of the timed work) back to back until `ms` of wall
    time have passed, so that the timed region starts at the device's
    sustained clock rather than on its way up from idle; returns what ran."""
    import torch
    n, t0 = 0, time.perf_counter()
    batch = 1
    while (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(batch):
            fn()
        n += batch
        torch.cuda.synchronize()
        batch = min(batch * 2, 64)
    return {"ms": round((time.perf_counter() - t0) * 1e3, 1), "steps": n}


def config_list(arg: str):
    if arg == "all":
        return [1, 2, 3, 4]
    out = [int(x) for x in arg.split(",") if x.strip()]
    if not out or any(c < 0 or c > 4 for c in out):
        raise SystemExit(f"--config: expected indices 0-4 or 'all', got {arg!r}")
    return out


def bench_config(cfg: int, args, dev, stream):
    """Times one workload: for each step, every forward's cache write and
    attention launch, then the batch's decisions. Returns the measurements and
    what the rest of the report needs (workload, plans, plan infos)."""
    import torch
    import prefix_tree_packed_amd as P
    from workloads import make_config

    wl = make_config(cfg, args.seed)

    def T(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    # ---- plans (host) + device inputs -------------------------------------
    t0 = time.perf_counter()
    plans = [P.tree_attn_plan(f.tree, wl.hq, wl.hkv, wl.d, wl.scale, out_dtype=args.out_dtype,
                              batch_invariant=args.batch_invariant)
             for f in wl.forwards]
    plan_build_ms = (time.perf_counter() - t0) * 1e3
    for p in plans:
        P.tree_attn_plan_upload(p)
    infos = [p.info for p in plans]
    odt = torch.float16 if args.out_dtype == "f16" else torch.float32
    fw = []
    shared = wl.notes.get("shared_cache", False)
    cache = None
    for f, info in zip(wl.forwards, infos):
        kn, vn = f.kv_new()
        if cache is None or not shared:
            kc, vc = f.cache_before()
            cache = (T(kc), T(vc))
        fw.append(dict(q=T(f.q), kn=T(kn), vn=T(vn), kc=cache[0], vc=cache[1],
                       o=torch.empty((info["num_q_tokens"], wl.hq, wl.d), dtype=odt, device=dev)))
    d = wl.decisions
    logits, row1, row2 = T(d.logits), T(d.row1), T(d.row2)
    nl, temps = T(d.n_letters), T(d.T)
    p_avg = torch.empty((d.n_dec, d.logits.shape[1]), dtype=torch.float32, device=dev)
    p_cal = torch.empty_like(p_avg)
    torch.cuda.synchronize()

    n_fw = len(fw)
    ev_w = [[torch.cuda.Event(enable_timing=True) for _ in range(n_fw)] for _ in range(args.steps)]
    ev_a = [[torch.cuda.Event(enable_timing=True) for _ in range(n_fw)] for _ in range(args.steps)]
    ev_b = [[torch.cuda.Event(enable_timing=True) for _ in range(n_fw)] for _ in range(args.steps)]

    if args.rope:
        # the usual rotary table, theta 10000, float32 (cos, sin) per position and frequency
        max_pos = max(int(P.tree_attn_plan_export(p)["pos_id"].max()) for p in plans) + 1
        inv = 10000.0 ** (-torch.arange(0, wl.d // 2, dtype=torch.float64) * 2.0 / wl.d)
        ang = torch.arange(max_pos, dtype=torch.float64)[:, None] * inv[None, :]
        rope_tab = torch.stack([ang.cos(), ang.sin()], dim=-1).float().to(dev).contiguous()
        for x in fw:
            x["qr"] = torch.empty_like(x["q"])

    def step(i=None):
        for j, (p, x) in enumerate(zip(plans, fw)):
            if i is not None:
                ev_w[i][j].record(stream)
            if args.rope:
                P.tree_attn_rope_cache_write(p, x["q"], x["qr"], x["kn"], x["vn"], rope_tab, x["kc"],
                                             x["vc"], style=args.rope, stream=stream)
            else:
                P.tree_attn_cache_write(p, x["kn"], x["vn"], x["kc"], x["vc"], stream=stream)
            if i is not None:
                ev_a[i][j].record(stream)
            P.tree_attn_forward_cached(p, x["qr"] if args.rope else x["q"], x["kc"], x["vc"], x["o"],
                                       stream=stream)
            if i is not None:
                ev_b[i][j].record(stream)
        P.decision_readout(logits, row1, row2, nl, temps, p_avg, p_cal, stream=stream)

    dwarm = device_warmup(step, args.device_warmup_ms)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # the K timed steps, with no events between their launches (an event
    # record between launches leaves a gap of its own on the stream) ...
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(args.steps):
        step()
    end.record(stream)
    torch.cuda.synchronize()
    ms_per_step = start.elapsed_time(end) / args.steps
    # ... then K more with HIP events around each launch, for the per-launch times
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    attn_ms = [[ev_a[i][j].elapsed_time(ev_b[i][j]) for j in range(n_fw)] for i in range(args.steps)]
    attn_ms = np.array(attn_ms)                       # [steps, forwards]
    attn_ms_mean = attn_ms.mean(axis=0)               # per forward

    useful_pairs = [i["useful_pairs"] for i in infos]
    useful_flops = [4.0 * wl.d * wl.hq * u for u in useful_pairs]
    q_tokens = sum(i["num_q_tokens"] for i in infos)
    value = sum(useful_flops) / (ms_per_step * 1e-3) / 1e12
    # dominant kernel: the attention launch of the heaviest forward
    k = int(np.argmax(useful_flops))
    achieved = useful_flops[k] / (attn_ms_mean[k] * 1e-3) / 1e12
    attn_total_tflops = sum(useful_flops) / (attn_ms_mean.sum() * 1e-3) / 1e12
    # the write kernel before each attention launch (HBM-bound): K and V read
    # and written once, plus Q read and written and the table rows with --rope
    write_ms = np.array([[ev_w[i][j].elapsed_time(ev_a[i][j]) for j in range(n_fw)]
                         for i in range(args.steps)]).mean(axis=0)
    write_bytes = []
    for inf in infos:
        t = inf["num_q_tokens"]
        b = 4 * t * wl.hkv * wl.d * 2
        if args.rope:
            b += 2 * t * wl.hq * wl.d * 2 + t * (wl.d // 2) * 2 * 4
        write_bytes.append(b)
    write_gbps = sum(write_bytes) / (write_ms.sum() * 1e-3) / 1e9
    # K and V of every row-space key a forward's queries may see, read once
    kv_bytes = [2 * inf["num_kv_tokens"] * wl.hkv * wl.d * 2 for inf in infos]
    alg_bytes = [algorithmic_bytes(p, wl, args.out_dtype) for p in plans]

    # correctness guard on the timed outputs (cheap): finite everywhere
    for x in fw:
        assert torch.isfinite(x["o"].float()).all().item(), "non-finite attention output"

    traffic = [None] * n_fw
    if args.seed == 0 and args.out_dtype == "f16" and not args.batch_invariant and not args.rope:
        traffic = [measured_traffic(cfg, j) for j in range(n_fw)]
    roofline = {
        "bound": "mfma",
        "kernel": "tree_attn_fwd_kernel",
        "achieved": round(achieved, 3),
        "peak": PEAK_F16_TFLOPS,
        "unit": "TFLOP/s",
        "frac": round(achieved / PEAK_F16_TFLOPS, 4),
        "traffic": None,
        "per_launch": {"useful_flop": useful_flops[k], "avg_ms": round(float(attn_ms_mean[k]), 5),
                       "forward_index": k,
                       "algorithmic_bytes": alg_bytes[k],
                       "algorithmic_gbps": round(alg_bytes[k] / (attn_ms_mean[k] * 1e-3) / 1e9, 1)},
    }
    if traffic[k] is not None:
        roofline["traffic"] = traffic[k]["fetch_bytes"] + traffic[k]["write_bytes"]
        roofline["traffic_detail"] = dict(traffic[k], source=os.path.relpath(TRAFFIC_FILE, ROOT))
    res = {
        "value": value,
        "ms_per_step": ms_per_step,
        "packed_tokens_per_s": q_tokens / (ms_per_step * 1e-3),
        "attention_only_tflops": attn_total_tflops,
        "attention_ms_per_forward": [round(float(x), 5) for x in attn_ms_mean],
        "attention_ms_p10_p50_p90": [[round(float(np.percentile(attn_ms[:, j], q)), 5) for q in (10, 50, 90)]
                                     for j in range(n_fw)],
        "attention_tflops_per_forward": [round(fl / (t * 1e-3) / 1e12, 1)
                                         for fl, t in zip(useful_flops, attn_ms_mean)],
        "algorithmic_gbps_per_forward": [round(b / (t * 1e-3) / 1e9, 1) for b, t in zip(alg_bytes, attn_ms_mean)],
        "traffic_bytes_per_forward": [None if t is None else t["fetch_bytes"] + t["write_bytes"]
                                      for t in traffic],
        "algorithmic_bytes_per_forward": alg_bytes,
        "kv_stream_gbps_per_forward": [round(kv / (t * 1e-3) / 1e9, 1) for kv, t in zip(kv_bytes, attn_ms_mean)],
        "cache_write": {"kernel": "rope_cache_write_kernel" if args.rope else "cache_write_kernel",
                        "bound": "hbm", "us_per_forward": [round(float(x) * 1e3, 2) for x in write_ms],
                        "bytes_per_forward": write_bytes, "achieved_gbps": round(write_gbps, 1),
                        "peak_gbps": 8000.0, "frac": round(write_gbps / 8000.0, 4)},
        "plan_build_ms": round(plan_build_ms, 3),
        "device_warmup": dwarm,
        "config": {
            "workload": f"config[{cfg}] {wl.name}",
            "seed": args.seed,
            "forwards": n_fw,
            "q_tokens_per_forward": [i["num_q_tokens"] for i in infos],
            "kv_tokens_per_forward": [i["num_kv_tokens"] for i in infos],
            "q_heads": wl.hq, "kv_heads": wl.hkv, "head_dim": wl.d,
            "useful_gflop_per_step": round(sum(useful_flops) / 1e9, 3),
            "decisions": d.n_dec,
            "out_dtype": args.out_dtype,
            "key_tiling": "by prompt position" if args.batch_invariant else "union",
            "rope": args.rope,
        },
        "roofline": roofline,
    }
    return res, wl, plans, infos


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; --gpus must be 1 "
                          "(multi-GPU sharding is described in DESIGN.md, not implemented)"}))
        sys.exit(2)

    import torch

    assert torch.cuda.is_available(), "bench needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    cfgs = config_list(args.config)

    results = {}
    for c in cfgs:
        print(f"[bench] config {c}", file=sys.stderr, flush=True)
        results[c] = bench_config(c, args, dev, stream)
        if len(cfgs) > 1:     # free the workload's device buffers before the next
            torch.cuda.synchronize()
            torch.cuda.empty_cache()
    head = cfgs[0]
    res, wl, plans, infos = results[head]
    out = {
        "metric": "useful tree-attention TFLOP/s (packed tokens/s and % of f16 MFMA peak alongside)",
        "value": round(res["value"], 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(res["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "packed_tokens_per_s": round(res["packed_tokens_per_s"], 1),
        "pct_mfma_peak": round(100 * res["value"] / PEAK_F16_TFLOPS, 2),
        "attention_only_tflops": round(res["attention_only_tflops"], 3),
    }
    for key in ("attention_ms_per_forward", "attention_ms_p10_p50_p90", "attention_tflops_per_forward",
                "kv_stream_gbps_per_forward", "cache_write", "plan_build_ms", "device_warmup", "config",
                "roofline"):
        out[key] = res[key]

    if len(cfgs) > 1:
        # every timed workload: attention alone (HIP events around each launch)
        # and the whole step, useful TFLOP/s and fraction of the f16 MFMA peak
        per = {}
        for c in cfgs:
            r = results[c][0]
            a = r["attention_only_tflops"]
            per[f"config[{c}]"] = {
                "workload": r["config"]["workload"],
                "attention_tflops": round(a, 1),
                "attention_frac": round(a / PEAK_F16_TFLOPS, 4),
                "step_tflops": round(r["value"], 1),
                "ms_per_step": round(r["ms_per_step"], 5),
                "packed_tokens_per_s": round(r["packed_tokens_per_s"], 1),
                "useful_gflop_per_step": r["config"]["useful_gflop_per_step"],
                "attention_ms_per_forward": r["attention_ms_per_forward"],
                "attention_tflops_per_forward": r["attention_tflops_per_forward"],
                "algorithmic_bytes_per_forward": r["algorithmic_bytes_per_forward"],
                "algorithmic_gbps_per_forward": r["algorithmic_gbps_per_forward"],
                "traffic_bytes_per_forward": r["traffic_bytes_per_forward"],
                "cache_write_gbps": r["cache_write"]["achieved_gbps"],
                "roofline_frac_heaviest_launch": r["roofline"]["frac"],
            }
        out["configs"] = per
        flops = sum(results[c][0]["config"]["useful_gflop_per_step"] for c in cfgs)
        attn_s = sum(sum(results[c][0]["attention_ms_per_forward"]) for c in cfgs) * 1e-3
        out["configs_aggregate"] = {"attention_tflops": round(flops / attn_s / 1e3, 1),
                                    "attention_frac": round(flops / attn_s / 1e3 / PEAK_F16_TFLOPS, 4)}

    if not args.no_readout:
        out["readout"] = bench_readout(args, wl, plans, dev, stream)
    if not args.no_latency:
        out["latency"] = bench_latency(args, wl, dev, stream)
    if not args.no_mfma_probe:
        probe = mfma_attainable(dev, stream, args.device_warmup_ms)
        probe["attention_pct_of_attainable"] = round(100 * res["roofline"]["achieved"] / probe["tflops"], 2)
        out["mfma_attainable"] = probe

    if args.copy_calibration:
        src = torch.ones(64 << 20, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        out["copy_calibration_bytes"] = {"read": src.numel() * 4, "write": dst.numel() * 4}
        del src, dst
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, infos, args.cpu_seconds)
        if len(cfgs) > 1:
            for c in cfgs[1:]:
                _, wlc, _, infc = results[c]
                out["configs"][f"config[{c}]"]["cpu_baseline"] = cpu_baseline(wlc, infc, args.cpu_seconds / 2)
    print(json.dumps(out), flush=True)


def bench_latency(args, wl_head, dev, stream):
    """Microseconds per call of the launch-latency-bound parts: config[0]'s
    forward (cache write + attention, 144 tokens) and decision epilogue, and
    the headline workload's decision epilogue; back to back (K calls between
    two events) and alone (median of single calls between two events)."""
    import torch
    import prefix_tree_packed_amd as P
    from workloads import make_config

    def T(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    wl = make_config(0, args.seed)
    f = wl.forwards[0]
    p = P.tree_attn_plan(f.tree, wl.hq, wl.hkv, wl.d, wl.scale, out_dtype=args.out_dtype)
    P.tree_attn_plan_upload(p)
    kn, vn = f.kv_new()
    kc, vc = f.cache_before()
    q, kn, vn, kc, vc = (T(a) for a in (f.q, kn, vn, kc, vc))
    odt = torch.float16 if args.out_dtype == "f16" else torch.float32
    o = torch.empty((p.info["num_q_tokens"], wl.hq, wl.d), dtype=odt, device=dev)

    def decisions(d):
        args_ = [T(d.logits), T(d.row1), T(d.row2), T(d.n_letters), T(d.T)]
        pa = torch.empty((d.n_dec, d.logits.shape[1]), dtype=torch.float32, device=dev)
        pc = torch.empty_like(pa)
        return lambda: P.decision_readout(*args_, pa, pc, stream=stream)

    def forward():
        P.tree_attn_cache_write(p, kn, vn, kc, vc, stream=stream)
        P.tree_attn_forward_cached(p, q, kc, vc, o, stream=stream)

    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn, reps=200, alone_reps=50):
        device_warmup(fn, 20.0)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        b2b = e0.elapsed_time(e1) * 1e3 / reps
        ts = []
        for _ in range(alone_reps):
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e3)
        return {"us_back_to_back": round(b2b, 2), "us_alone_median": round(float(np.median(ts)), 2)}

    return {"config[0]_forward": dict(timed(forward), tokens=int(p.info["num_q_tokens"]),
                                       launches="cache write + attention"),
            "config[0]_decisions": dict(timed(decisions(wl.decisions)), decisions=int(wl.decisions.n_dec)),
            "headline_decisions": dict(timed(decisions(wl_head.decisions)),
                                       decisions=int(wl_head.decisions.n_dec))}


def mfma_attainable(dev, stream, warmup_ms):
    """The MFMA rate the device reaches on a register-only loop (4 workgroups
    of 4 waves per CU, 8 independent accumulator chains per wave)."""
    import torch
    import prefix_tree_packed_amd as P
    n_wg = 4 * torch.cuda.get_device_properties(dev).multi_processor_count
    out = torch.empty(n_wg * 256, dtype=torch.float32, device=dev)
    iters = 2000
    flops = P.tree_attn_mfma_peak_probe(n_wg, iters, out, stream=stream)
    device_warmup(lambda: P.tree_attn_mfma_peak_probe(n_wg, iters, out, stream=stream), warmup_ms)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    reps = 10
    for _ in range(reps):
        P.tree_attn_mfma_peak_probe(n_wg, iters, out, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    tflops = flops / (ms * 1e-3) / 1e12
    return {"kernel": "mfma_peak_kernel (v_mfma_f32_16x16x32_f16, register operands only)",
            "tflops": round(tflops, 1), "pct_of_published_peak": round(100 * tflops / PEAK_F16_TFLOPS, 2),
            "workgroups": n_wg, "ms": round(ms, 4)}


# Llama shapes by query heads (8B: 32 heads, 70B: 64); the tiny workload gets a
# small model of its own width
READOUT_SHAPES = {32: ("llama-8b", 4096, 14336, 128256), 64: ("llama-70b", 8192, 28672, 128256)}


def bench_readout(args, wl, plans, dev, stream):
    """The readout-only last layer (readout_mlp + letter_logits) at the last
    forward's leaf readout tokens, on the Llama shape matching the workload's
    heads, with random weights. HBM-bound: the MLP weights are read once."""
    import torch
    import prefix_tree_packed_amd as P
    name, dm, ff, vocab = READOUT_SHAPES.get(wl.hq, ("small", 256, 768, 4096))
    plan = plans[-1]
    readout = P.tree_attn_plan_export(plan)["leaf_readout_tok"]
    n, n_tok = len(readout), plan.info["num_q_tokens"]
    d = wl.decisions
    ld = int(d.logits.shape[1])
    nl = np.full(n, min(4, ld), np.int32)       # each decision's rows get its letter count
    for i in range(d.n_dec):
        for r in (int(d.row1[i]), int(d.row2[i])):
            if r < n:
                nl[r] = d.n_letters[i]
    assert ld <= 8, "the workloads use at most 8 letters"
    g = torch.Generator(device=dev)
    g.manual_seed(args.seed)
    hidden = torch.randn((n_tok, dm), device=dev, generator=g).half()
    norm_w = (1 + 0.1 * torch.randn(dm, device=dev, generator=g)).half()
    w_gate_up = (torch.randn((2 * ff, dm), device=dev, generator=g) / dm ** 0.5).half()
    w_down = (torch.randn((dm, ff), device=dev, generator=g) / ff ** 0.5).half()
    final_w = (1 + 0.1 * torch.randn(dm, device=dev, generator=g)).half()
    letters = torch.randint(0, vocab, (8,), device=dev, generator=g, dtype=torch.int32)
    lm_head = torch.zeros((vocab, dm), dtype=torch.float16, device=dev)
    lm_head[letters.long()] = (2 * torch.randn((8, dm), device=dev, generator=g) / dm ** 0.5).half()
    ids = letters[:ld].repeat(n, 1).contiguous()
    tok = torch.from_numpy(readout).to(dev)
    n_letters = torch.from_numpy(nl).to(dev)
    h_out = torch.empty((n, dm), dtype=torch.float16, device=dev)
    logits = torch.empty((n, ld), dtype=torch.float32, device=dev)
    ws = torch.empty(P.readout_mlp_workspace_size(n, dm, ff), dtype=torch.uint8, device=dev)

    def run():
        P.readout_mlp(hidden, tok, norm_w, w_gate_up, w_down, h_out, workspace=ws, stream=stream)
        P.letter_logits(h_out, final_w, lm_head, ids, n_letters, logits, stream=stream)

    device_warmup(run, args.device_warmup_ms)
    for _ in range(3):
        run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        run()
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / args.steps
    assert torch.isfinite(logits).all().item(), "non-finite letter logits"
    # algorithmic bytes: the three weight matrices once, the readout rows in and
    # out, the letters' head rows, the logits
    weight_bytes = 3 * dm * ff * 2
    nbytes = weight_bytes + n * dm * 2 * 2 + int(nl.sum()) * dm * 2 + n * ld * 4
    gbps = nbytes / (us * 1e-6) / 1e9
    del hidden, w_gate_up, w_down, lm_head
    torch.cuda.empty_cache()
    return {"kernels": "readout_norm, mlp_mfma (gate/up, down), readout_finish, letter_logits",
            "model": name, "d_model": dm, "d_ff": ff, "readout_rows": n, "letters": int(nl.sum()),
            "bound": "hbm", "us": round(us, 2), "bytes": nbytes, "achieved_gbps": round(gbps, 1),
            "peak_gbps": PEAK_HBM_GBS, "frac": round(gbps / PEAK_HBM_GBS, 4)}


def algorithmic_bytes(plan, wl, out_dtype):
    """Q read and O written once, and every K/V row some query sees read once."""
    import prefix_tree_packed_amd as P
    from prefix_tree_packed_amd.binding import key_tile_rows
    sch = P.tree_attn_plan_schedule(plan)
    seen = np.zeros(plan.info["num_kv_tokens"] + 64, dtype=bool)
    for i, (k0, n, *_rest) in enumerate(sch["key_tiles"]):
        if _rest[3] == 1:
            seen[k0:k0 + n] = True
        else:
            seen[key_tile_rows(sch, i)] = True
    ob = 2 if out_dtype == "f16" else 4
    q = plan.info["num_q_tokens"] * wl.hq * wl.d
    kv = 2 * int(seen.sum()) * wl.hkv * wl.d * 2
    return int(q * 2 + q * ob + kv)


def cpu_baseline(wl, infos, seconds):
    """The float64 oracle, as it stands, on a bounded sample of the same
    workload: query tokens of the heaviest forward in slices of 128 (spread over
    the forward) until `seconds` of wall time are spent; reported as useful
    TFLOP/s of the sampled tokens."""
    from oracle import attention as OA
    from oracle import tree as OT
    try:
        from threadpoolctl import threadpool_info
        threads = max([t.get("num_threads", 1) for t in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    useful = [i["useful_pairs"] for i in infos]
    k = int(np.argmax(useful))
    f = wl.forwards[k]
    idx = OT.build_index(f.tree)
    toks = OT.query_tokens(idx)
    vis = toks["pos_id"].astype(np.int64) + 1
    nq = len(vis)
    order = np.random.default_rng(0).permutation(nq)
    done, pairs = 0, 0
    t0 = time.perf_counter()
    while done < nq and time.perf_counter() - t0 < seconds:
        sel = np.sort(order[done:done + 128])
        OA.tree_attention(f.tree, f.q, f.k_row, f.v_row, wl.scale, sel=sel)
        pairs += int(vis[sel].sum())
        done += len(sel)
    dt = time.perf_counter() - t0
    flops = 4.0 * wl.d * wl.hq * pairs
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{done} of {nq} query tokens (random, slices of 128) of forward {k}, all "
                      f"{wl.hq} heads, float64 dense-mask oracle, {dt:.1f} s",
            "cpu": _cpu_model()}


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


if __name__ == "__main__":
    main()
