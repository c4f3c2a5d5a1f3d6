#!/usr/bin/env python3
"""Benchmark of the sparse MoE layer forward on one MI355X.

One step = one call of the whole layer (router, top-K + softmax, dispatch,
gate/up projection with SwiGLU, down projection, combine) on a resident batch.
The headline is moe_forward_packed: the expert weights packed once into MFMA
fragment order (moe_pack_up / moe_pack_down, outside the timed region, as a
deployment does at weight-load time); moe_forward on the caller's layout is
timed on the same inputs and reported under "caller_layout".  The default
workload is the Mixtral-shape prefill layer (T=8192, d=4096, f=14336, n=8,
K=2, bf16); the decode batch (T=32), the skewed-routing and the many-experts
workloads are measured in the same run.  Inputs are seeded synthetic draws
(synth/), weights random-init with the Mixtral layer's shapes.  Two weight
copies alternate between steps so repeated reads cannot be served from the
256 MB last-level cache.

Per-kernel durations come from HIP events the library records between its
stages on the launch stream (moe_forward_traced / moe_forward_packed_traced),
over the timed steps.  The CPU baseline times the fp64 oracle on a bounded
sample of each workload.

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

METRIC = "MoE-layer tokens/s at Mixtral shape; % bf16 MFMA peak (T=8192), % HBM BW (T=32)"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
STAGES = ["route", "dispatch", "up_proj", "down_proj", "combine"]


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="mixtral_prefill",
                    choices=["mixtral_prefill", "mixtral_skewed", "many_experts", "mixtral_decode"])
    ap.add_argument("--no-decode", action="store_true", help="skip the T=32 decode measurement")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip timing the router statistics and the capacity-limited forward")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the skewed-routing and many-experts workloads")
    ap.add_argument("--packed-only", action="store_true",
                    help="time only moe_forward_packed (not moe_forward on the caller's layout)")
    ap.add_argument("--cpu-sample", type=int, default=8192, help="tokens in the oracle's timed sample")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first run a 1 GiB device-to-device copy (reference for traffic counters)")
    ap.add_argument("--summarize-trace", metavar="DIR",
                    help="print a summary of a rocprofv3 --kernel-trace --stats csv directory and exit")
    ap.add_argument("--summarize-clock", metavar="DIR",
                    help="print the engine clock under each kernel from a GRBM_GUI_ACTIVE/GRBM_COUNT pass")
    ap.add_argument("--summarize-counters", metavar="DIR", nargs="+",
                    help="print a summary of rocprofv3 --pmc csv directories (FETCH_SIZE / WRITE_SIZE "
                         "scaled by the 1 GiB calibration copy) and exit")
    ap.add_argument("--traffic-json", metavar="FILE",
                    help="with --summarize-counters: also write the per-kernel HBM traffic, keyed by "
                         "the hash of the kernel's sources")
    return ap.parse_args()


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def upload(inp, dev, copies):
    import numpy as np
    import torch

    def up(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    x = up(inp.x)
    wg = up(inp.Wg)
    w = []
    for c in range(copies):
        if c == 0:
            w.append((up(inp.W1), up(inp.W3), up(inp.W2)))
        else:
            w.append(tuple(t.clone() for t in w[0]))
    return x, wg, w


def _time_calls(fn, reps, stream, warm=3):
    """Mean ms per call over `reps` calls, after `warm` untimed ones: the first calls after
    the GPU has idled (host work, synchronisation) run at a lower engine clock."""
    import torch
    for i in range(warm):
        fn(i)
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for i in range(reps):
        fn(i)
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def time_extras(moe, x, wg, wsets, K, y, stream, reps):
    """The optional paths on the same resident inputs: router statistics with the
    load-balancing loss, the capacity-limited forward (capacity factor 1.0) and
    the expert-choice forward (capacity factor K: the same expert work as top-K)."""
    T = x.shape[0]
    n = wg.shape[1]
    stats_ms = _time_calls(lambda i=0: moe.route_stats(x, wg, K, 0.01), reps, stream)
    st = moe.route_stats(x, wg, K, 0.01)

    def cap_step(i=0):
        w1, w3, w2 = wsets[i % 2]
        moe.forward_capacity(x, wg, w1, w3, w2, K, 1.0, y=y)

    cap_ms = _time_calls(cap_step, reps, stream)
    rc = moe.route_capacity(x, wg, K, 1.0, outputs=("offsets",))
    kept = int(rc["offsets"][-1].item())

    def ec_step(i=0):
        w1, w3, w2 = wsets[i % 2]
        moe.forward_expert_choice(x, wg, w1, w3, w2, float(K), y=y)

    ec_ms = _time_calls(ec_step, reps, stream)
    ec_route_ms = _time_calls(lambda i=0: moe.route_expert_choice(x, wg, float(K), outputs=("slot_pos",)),
                              reps, stream)
    return {
        "route_stats": {"ms_per_call": round(stats_ms, 4), "aux_loss_alpha_0.01": round(float(st["aux_loss"][0]), 6)},
        "forward_capacity_cf1": {"ms_per_step": round(cap_ms, 4), "tokens_per_s": round(T / (cap_ms * 1e-3), 1),
                                 "capacity": moe.expert_capacity(T, n, K, 1.0),
                                 "dropped_assignments": T * K - kept},
        "forward_expert_choice_cf_K": {"ms_per_step": round(ec_ms, 4), "tokens_per_s": round(T / (ec_ms * 1e-3), 1),
                                       "tokens_per_expert": moe.expert_choice_capacity(T, n, float(K)),
                                       "routing_ms": round(ec_route_ms, 4)},
    }


def _stage_events(stream):
    import torch
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
    for e in evs:
        e.record(stream)  # creates the underlying hipEvent_t
    return evs


def _time_layer(step, traced_step, steps, warmup, stream):
    """Mean ms per step over `steps` plain calls (two events around the loop), then
    the same calls with the library's stage events (per-stage durations)."""
    import numpy as np
    import torch
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    start.record(stream)
    for i in range(steps):
        step(i)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = start.elapsed_time(end)
    events = [_stage_events(stream) for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        traced_step(i, [e.cuda_event for e in events[i]])
    torch.cuda.synchronize()
    stage_ms = np.array([[ev[j].elapsed_time(ev[j + 1]) for j in range(5)] for ev in events])
    traced_ms = np.array([ev[0].elapsed_time(ev[5]) for ev in events])
    return dict(ms_per_step=total_ms / steps, wall_s=wall, stage_ms=stage_ms.mean(axis=0),
                stage_ms_min=stage_ms.min(axis=0),
                traced_step_ms={"median": round(float(np.median(traced_ms)), 4),
                                "min": round(float(traced_ms.min()), 4), "max": round(float(traced_ms.max()), 4)})


def time_workload(name, steps, warmup, with_extras=False, layouts=("packed", "caller")):
    """One workload on resident inputs: moe_forward_packed on weights packed once
    (moe_pack_up / moe_pack_down, outside the timed region) and moe_forward on the
    caller's [n][d][f] / [n][f][d] layout.  Two weight copies alternate between steps."""
    import numpy as np
    import torch

    import sparse_mixture_experts_22_amd as moe
    from synth import CONFIGS, make_config_inputs

    c = CONFIGS[name]
    T, d, f, n, K = c["T"], c["d"], c["f"], c["n"], c["K"]
    dev = torch.device("cuda:0")
    t0 = time.time()
    inp = make_config_inputs(name)
    x, wg, wsets = upload(inp, dev, copies=2)
    del inp
    log(f"[bench] {name}: inputs ready in {time.time() - t0:.1f}s")
    y = torch.empty((T, d), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    out = dict(name=name, T=T, d=d, f=f, n=n, K=K)
    if "caller" in layouts:
        def step(i):
            w1, w3, w2 = wsets[i % 2]
            moe.forward(x, wg, w1, w3, w2, K, y=y)

        def traced(i, evs):
            w1, w3, w2 = wsets[i % 2]
            moe.forward_traced(x, wg, w1, w3, w2, K, evs, y=y)

        out["caller"] = _time_layer(step, traced, steps, warmup, stream)
        assert torch.isfinite(y).all().item()
        if with_extras:
            out["extras"] = time_extras(moe, x, wg, wsets, K, y, stream, max(3, steps // 4))
    if "packed" in layouts:
        psets = [(moe.pack_up(w1, w3), moe.pack_down(w2)) for (w1, w3, w2) in wsets]
        torch.cuda.synchronize()

        def pstep(i):
            p13, p2 = psets[i % 2]
            moe.forward_packed(x, wg, p13, p2, f, K, y=y)

        def ptraced(i, evs):
            p13, p2 = psets[i % 2]
            moe.forward_packed_traced(x, wg, p13, p2, f, K, evs, y=y)

        out["packed"] = _time_layer(pstep, ptraced, steps, warmup, stream)
        assert torch.isfinite(y).all().item()
        del psets
    rt = moe.route(x, wg, K, outputs=("counts", "topk_idx"))
    torch.cuda.synchronize()
    out["counts"] = rt["counts"].cpu().numpy()
    top1 = rt["topk_idx"][:, 0].cpu().numpy()
    out["top1_share"] = np.bincount(top1, minlength=n) / float(T)
    del x, wg, wsets, y
    torch.cuda.empty_cache()
    return out


def layer_flops(r):
    return 2.0 * r["T"] * r["d"] * r["n"] + 6.0 * r["T"] * r["K"] * r["d"] * r["f"]


def mfma_record(r, layout, kernel, traffic_kernel=None):
    """Roofline of the up projection (the dominant kernel: 2/3 of the FLOPs) and
    the layer and per-GEMM fractions of the bf16 MFMA peak for one layout."""
    t = r[layout]
    T, d, f, n, K = r["T"], r["d"], r["f"], r["n"], r["K"]
    up_flops = 4.0 * T * K * d * f           # a = xW1 and b = xW3 on the T*K assignments
    down_flops = 2.0 * T * K * f * d
    up_ms, down_ms = float(t["stage_ms"][2]), float(t["stage_ms"][3])
    achieved = up_flops / (up_ms * 1e-3) / 1e12
    lt = layer_flops(r) / (t["ms_per_step"] * 1e-3) / 1e12
    return {
        "roofline": {"kernel": kernel, "bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic(traffic_kernel) if traffic_kernel else None,
                     "flops_per_launch": up_flops, "avg_launch_ms": round(up_ms, 4)},
        "ms_per_step": round(t["ms_per_step"], 4),
        "tokens_per_s": round(T / (t["ms_per_step"] * 1e-3), 1),
        "layer_tflops": round(lt, 1),
        "layer_frac_of_mfma_peak": round(lt / PEAK_BF16_TFLOPS, 4),
        "up_proj_frac_of_mfma_peak": round(achieved / PEAK_BF16_TFLOPS, 4),
        "down_proj_frac_of_mfma_peak": round(down_flops / (down_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "stages_ms": {s: round(float(v), 4) for s, v in zip(STAGES, t["stage_ms"])},
        "traced_step_ms": t["traced_step_ms"],
    }


def workload_record(r):
    """Both layouts of a prefill-size workload, with the routing's per-expert loads."""
    rec = {"workload": r["name"], "T": r["T"], "d": r["d"], "f": r["f"], "n": r["n"], "K": r["K"],
           "flops_per_step": layer_flops(r)}
    if "packed" in r:
        rec["packed"] = mfma_record(r, "packed", "packed_gemm_kernel<1> (gate/up projection + SwiGLU)",
                                    "packed_gemm_kernel<1>" if r["name"] == "mixtral_prefill" else None)
    if "caller" in r:
        rec["caller_layout"] = mfma_record(r, "caller", "grouped_gemm_kernel<1> (gate/up projection + SwiGLU)",
                                           "grouped_gemm_kernel<1>" if r["name"] == "mixtral_prefill" else None)
    rec["expert_counts"] = r["counts"].tolist()
    rec["top1_share"] = [round(float(v), 4) for v in r["top1_share"]]
    return rec


def decode_record(r, layout):
    t = r[layout]
    T, d, f, n, K = r["T"], r["d"], r["f"], r["n"], r["K"]
    touched = int((r["counts"] > 0).sum())
    up_bytes = touched * 2.0 * d * f * 2 + T * d * 2 + T * K * f * 2
    layer_bytes = touched * 3.0 * d * f * 2 + d * n * 2 + T * d * 2 + T * d * 4
    up_ms = float(t["stage_ms"][2])
    achieved = up_bytes / (up_ms * 1e-3) / 1e9
    layer_gbs = layer_bytes / (t["ms_per_step"] * 1e-3) / 1e9
    kernel = "skinny_kernel<1>" if layout == "caller" else "packed_stream_kernel<1>"
    return {
        "workload": "mixtral_decode", "T": T, "d": d, "f": f, "n": n, "K": K,
        "value": round(T / (t["ms_per_step"] * 1e-3), 1), "unit": "tokens/s",
        "ms_per_step": round(t["ms_per_step"], 4),
        "roofline": {"kernel": kernel + " (gate/up projection + SwiGLU)", "bound": "hbm",
                     "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": measured_traffic(kernel) if r["name"] == "mixtral_decode" else None,
                     "bytes_per_launch": up_bytes, "avg_launch_ms": round(up_ms, 4)},
        "layer_gbs": round(layer_gbs, 1), "layer_frac_of_hbm_peak": round(layer_gbs / PEAK_HBM_GBS, 4),
        "experts_touched": touched,
        "stages_ms": {s: round(float(v), 4) for s, v in zip(STAGES, t["stage_ms"])},
        "traced_step_ms": t["traced_step_ms"],
    }


def time_decode_q4(steps, warmup):
    """The decode batch with 4-bit expert weights (quantized on the GPU from the
    bf16 weights; two quantized copies alternate between steps)."""
    import numpy as np
    import torch

    import sparse_mixture_experts_22_amd as moe
    from synth import CONFIGS, make_config_inputs

    name = "mixtral_decode"
    c = CONFIGS[name]
    T, d, f, n, K = c["T"], c["d"], c["f"], c["n"], c["K"]
    dev = torch.device("cuda:0")
    inp = make_config_inputs(name)
    x, wg, wsets = upload(inp, dev, copies=1)
    del inp
    qsets = []
    for cp in range(2):
        w1, w3, w2 = wsets[0]
        if cp == 1:  # a second, distinct copy: perturb nothing, just separate storage
            w1, w3, w2 = w1.clone(), w3.clone(), w2.clone()
        qsets.append(tuple(moe.quantize_q4(w) for w in (w1, w3, w2)))
    del wsets
    torch.cuda.synchronize()
    y = torch.empty((T, d), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    # The host work above leaves the GPU idle for seconds, and the engine clock
    # takes tens of milliseconds of work to come back up; a 0.14 ms layer needs
    # about 200 calls for that, so the warm-up is at least that long.
    for i in range(max(warmup, 200)):
        q1, q3, q2 = qsets[i % 2]
        moe.forward_q4(x, wg, q1, q3, q2, d, f, K, y=y)
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for i in range(steps):
        q1, q3, q2 = qsets[i % 2]
        moe.forward_q4(x, wg, q1, q3, q2, d, f, K, y=y)
    b.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    counts = moe.route(x, wg, K, outputs=("counts",))["counts"].cpu().numpy()
    touched = int((counts > 0).sum())
    # algorithmic bytes: codes + scales of the touched experts, x, W_g, fp32 y
    wbytes = touched * 3 * (d * f // 2 + (d // 128) * f * 2)
    layer_bytes = wbytes + T * d * 2 + d * n * 2 + T * d * 4
    gbs = layer_bytes / (ms * 1e-3) / 1e9
    return {"workload": name + " (4-bit expert weights)", "T": T, "value": round(T / (ms * 1e-3), 1),
            "unit": "tokens/s", "ms_per_step": round(ms, 4), "weight_bytes": wbytes,
            "layer_gbs": round(gbs, 1), "layer_frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
            "experts_touched": touched}


def cpu_baseline(names, sample):
    """The fp64 oracle as it stands, per workload on its first `sample` tokens
    (all of them where the workload is no larger), on this host's cores."""
    import numpy as np

    import oracle
    from synth import make_config_inputs

    blas, threads = "unknown", None
    try:
        from threadpoolctl import threadpool_info
        pools = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        threads = max([int(i.get("num_threads", 1)) for i in pools] or [1])
        blas = ", ".join(f"{i.get('internal_api')} {i.get('version')}" for i in pools)
    except Exception:
        pass
    usable = len(os.sched_getaffinity(0))
    host_cpu = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            host_cpu = next(l.split(":", 1)[1].strip() for l in fh if l.startswith("model name"))
    except (OSError, StopIteration):
        pass
    per = {}
    for name in names:
        inp = make_config_inputs(name)
        ns = min(sample, inp.T)
        x = inp.f64("x")[:ns]
        t0 = time.perf_counter()
        y = oracle.forward(x, inp.f64("Wg"), lambda e: inp.expert_f64("W1", e),
                           lambda e: inp.expert_f64("W3", e), lambda e: inp.expert_f64("W2", e), inp.K)
        el = time.perf_counter() - t0
        assert np.isfinite(y).all()
        per[name] = {"tokens_per_s": round(ns / el, 2), "seconds": round(el, 2), "tokens": ns,
                     "of_tokens": inp.T}
        log(f"[bench] oracle {name}: {ns} tokens in {el:.1f}s")
        del inp, x, y
    head = names[0]
    return {"value": per[head]["tokens_per_s"], "unit": "tokens/s", "cores": threads or usable, "kind": "oracle",
            "sample": f"first {per[head]['tokens']} of the {per[head]['of_tokens']} tokens of {head}: fp64 routing "
                      f"and every touched expert (weights widened per expert), {per[head]['seconds']} s",
            "usable_cores": usable, "blas_threads": threads, "blas": blas,
            "env": {k: os.environ.get(k) for k in ("OPENBLAS_NUM_THREADS", "OMP_NUM_THREADS", "MKL_NUM_THREADS")},
            "host_cpu": host_cpu, "per_config": per}


# ---------------------------------------------------------------- profiles
ROOT = os.path.dirname(os.path.abspath(__file__))
TRAFFIC_JSON = os.path.join(ROOT, "profiles", "traffic_counters.json")
CALIB_BYTES = 1 << 30  # the --calibrate-copy copy: 1 GiB read, 1 GiB written
# Sources that determine each measured kernel's code (a change voids its counters), by the
# kernel's name without template arguments: every instance of a template shares them.
_Q = ["csrc/moe_internal.h", "build.py"]
KERNEL_SOURCES = {
    "grouped_gemm_kernel": ["csrc/gemm_prefill.hip", "csrc/tile_sched.h"] + _Q,
    "packed_gemm_kernel": ["csrc/gemm_packed.hip", "csrc/tile_sched.h"] + _Q,
    "packed_stream_kernel": ["csrc/gemm_packed.hip", "csrc/tile_sched.h"] + _Q,
    "skinny_kernel": ["csrc/gemm_skinny.hip"] + _Q,
    "skinny_q4_kernel": ["csrc/quant4.hip"] + _Q,
}


def kernel_sources(kernel):
    """Source files of `kernel` ("skinny_q4_kernel<1, 7>" -> those of skinny_q4_kernel), or None."""
    return KERNEL_SOURCES.get(kernel.split("<")[0])


def sources_hash(kernel):
    import hashlib
    h = hashlib.sha256()
    for rel in kernel_sources(kernel):
        with open(os.path.join(ROOT, "sparse_mixture_experts_22_amd", rel), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` in the default workloads (mixtral_prefill for the grouped
    GEMMs, mixtral_decode for the skinny kernels) from the committed counter summary, or None
    when that summary is missing or was taken on different kernel sources."""
    try:
        with open(TRAFFIC_JSON) as fh:
            rec = json.load(fh)["kernels"][kernel]
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("sources_sha256") != sources_hash(kernel):
        return None
    return rec["hbm_bytes"]


def short_kernel_name(name):
    import re
    name = name.replace("(anonymous namespace)::", "").replace("moe::", "")
    if name.startswith("void "):
        name = name[5:]
    return re.sub(r"\(.*", "", name)


def summarize_trace(d):
    """Per-kernel rows of a rocprofv3 --kernel-trace --stats run: the profiler's
    call count, average, min, max and share, plus the median duration of the
    individual dispatches (robust to the cold first calls that lift the average)."""
    import collections
    import csv
    import glob
    path = glob.glob(os.path.join(d, "*kernel_stats.csv"))[0]
    rows = list(csv.DictReader(open(path)))
    durations = collections.defaultdict(list)
    for tpath in glob.glob(os.path.join(d, "*kernel_trace.csv")):
        for r in csv.DictReader(open(tpath)):
            durations[short_kernel_name(r["Kernel_Name"])].append(
                (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    print(f"{'kernel':58s} {'calls':>5s} {'avg_us':>10s} {'median_us':>10s} {'min_us':>10s} {'max_us':>10s} "
          f"{'%':>6s}")
    for r in rows:
        name = short_kernel_name(r["Name"])
        v = sorted(durations.get(name, []))
        med = f"{v[len(v) // 2]:10.1f}" if v else f"{'-':>10s}"
        print(f"{name[:58]:58s} {int(r['Calls']):5d} {float(r['AverageNs']) / 1e3:10.1f} {med} "
              f"{float(r['MinNs']) / 1e3:10.1f} {float(r['MaxNs']) / 1e3:10.1f} {float(r['Percentage']):6.2f}")


def summarize_counters(dirs, traffic_json=None):
    import collections
    import csv
    import glob
    per = collections.defaultdict(lambda: collections.defaultdict(list))
    copies = collections.defaultdict(list)
    for d in dirs:
        for path in glob.glob(os.path.join(d, "*counter_collection.csv")):
            for r in csv.DictReader(open(path)):
                name = short_kernel_name(r["Kernel_Name"])
                key = f"{name} grid={int(r['Grid_Size'])}"
                v = float(r["Counter_Value"])
                per[key][r["Counter_Name"]].append(v)
                if name == "__amd_rocclr_copyBuffer":
                    copies[r["Counter_Name"]].append(v)
    # The largest copy of the run is the 1 GiB calibration copy (every other copy is smaller).
    fetch_factor = CALIB_BYTES / (max(copies["FETCH_SIZE"]) * 1024) if copies.get("FETCH_SIZE") else None
    write_factor = CALIB_BYTES / (max(copies["WRITE_SIZE"]) * 1024) if copies.get("WRITE_SIZE") else None
    print(f"calibration: 1 GiB device copy -> FETCH_SIZE {max(copies.get('FETCH_SIZE', [0])):.0f} KiB, "
          f"WRITE_SIZE {max(copies.get('WRITE_SIZE', [0])):.0f} KiB; "
          f"scale factors fetch {fetch_factor}, write {write_factor}")
    out = {"fetch_factor": fetch_factor, "write_factor": write_factor, "kernels": {}}
    for key in sorted(per):
        cs = {c: sum(v) / len(v) for c, v in per[key].items()}
        line = f"{key}: n={len(next(iter(per[key].values())))} " + " ".join(
            f"{c}={v:.6g}" for c, v in sorted(cs.items()))
        kname = key.split(" grid=")[0]
        if "FETCH_SIZE" in cs and "WRITE_SIZE" in cs and fetch_factor and write_factor:
            rb = cs["FETCH_SIZE"] * 1024 * fetch_factor
            wb = cs["WRITE_SIZE"] * 1024 * write_factor
            line += f" -> read {rb / 1e9:.4f} GB, written {wb / 1e9:.4f} GB per launch"
            if kernel_sources(kname) and int(key.split("grid=")[1]) >= out["kernels"].get(kname, {}).get("grid", 0):
                out["kernels"][kname] = {"grid": int(key.split("grid=")[1]),"fetch_kib": cs["FETCH_SIZE"], "write_kib": cs["WRITE_SIZE"],
                                       "read_bytes": rb, "write_bytes": wb, "hbm_bytes": rb + wb,
                                       "sources_sha256": sources_hash(kname)}
        print(line)
    if traffic_json:
        with open(traffic_json, "w") as fh:
            json.dump(out, fh, indent=1)
            fh.write("\n")


def summarize_clock(d):
    """Engine clock under each kernel, from a counter pass with GRBM_GUI_ACTIVE
    and GRBM_COUNT: both are clock counts summed over the device's 8 XCDs, so
    count / (8 x dispatch duration) is the clock in GHz (GUI_ACTIVE counts the
    busy cycles, GRBM_COUNT every cycle)."""
    import collections
    import csv
    import glob
    per = collections.defaultdict(lambda: collections.defaultdict(list))
    for path in glob.glob(os.path.join(d, "*counter_collection.csv")):
        for r in csv.DictReader(open(path)):
            dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
            if dur <= 0:
                continue
            per[short_kernel_name(r["Kernel_Name"])][r["Counter_Name"]].append(float(r["Counter_Value"]) / dur)
    print(f"{'kernel':44s} {'n':>4s} {'GHz (GRBM_COUNT)':>17s} {'GHz (GUI_ACTIVE)':>17s}")
    for name, cs in sorted(per.items()):
        cnt = sorted(cs.get("GRBM_COUNT", []))
        act = sorted(cs.get("GRBM_GUI_ACTIVE", []))
        if not cnt or not act:
            continue
        print(f"{name[:44]:44s} {len(cnt):4d} {cnt[len(cnt) // 2] / 8e9:17.3f} {act[len(act) // 2] / 8e9:17.3f}")


def main():
    args = parse()
    if args.summarize_trace:
        summarize_trace(args.summarize_trace)
        return
    if args.summarize_counters:
        summarize_counters(args.summarize_counters, args.traffic_json)
        return
    if args.summarize_clock:
        summarize_clock(args.summarize_clock)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this benchmark measures one GPU only (every box here has one); "
                                   "run with --gpus 1", "n_gpus": args.gpus}))
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    import sparse_mixture_experts_22_amd as moe
    moe.lib()  # fails loudly if the HIP library is missing

    if args.calibrate_copy:
        a = torch.empty(1 << 28, dtype=torch.float32, device="cuda:0")
        b = torch.empty_like(a)
        a.fill_(1.0)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        del a, b
    layouts = ("packed",) if args.packed_only else ("packed", "caller")
    main_r = time_workload(args.workload, args.steps, args.warmup, with_extras=not args.no_extras, layouts=layouts)
    log(f"[bench] {args.workload}: " + ", ".join(
        f"{lay} {main_r[lay]['ms_per_step']:.3f} ms/step" for lay in layouts))
    head = main_r["packed"]
    rec = {
        "metric": METRIC,
        "value": round(main_r["T"] / (head["ms_per_step"] * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(head["ms_per_step"], 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded N(0,1) activations, random-init N(0,1/fan_in) weights",
        "config": {"workload": args.workload, "T": main_r["T"], "d": main_r["d"], "f": main_r["f"],
                   "n": main_r["n"], "K": main_r["K"], "parallelism": "single GPU",
                   "weights": "bf16, packed once into MFMA fragment order (moe_pack_up / moe_pack_down) "
                              "outside the timed region; each step is one moe_forward_packed call "
                              "(routing included)"},
    }
    if args.workload == "mixtral_decode":
        dr = decode_record(main_r, "packed")
        rec["roofline"] = dr["roofline"]
        rec["stages_ms"] = dr["stages_ms"]
        if "caller" in main_r:
            rec["caller_layout"] = decode_record(main_r, "caller")
    else:
        wr = workload_record(main_r)
        pk = wr["packed"]
        rec["roofline"] = pk["roofline"]
        for k in ("layer_tflops", "layer_frac_of_mfma_peak", "up_proj_frac_of_mfma_peak",
                  "down_proj_frac_of_mfma_peak", "stages_ms", "traced_step_ms"):
            rec[k] = pk[k]
        if "caller_layout" in wr:
            rec["caller_layout"] = wr["caller_layout"]
        rec["expert_counts"] = wr["expert_counts"]
    if "extras" in main_r:
        rec["extras"] = main_r["extras"]
    if not args.no_decode and args.workload != "mixtral_decode":
        dr_raw = time_workload("mixtral_decode", max(args.steps, 20), args.warmup, layouts=layouts)
        rec["decode"] = decode_record(dr_raw, "packed")
        if "caller" in dr_raw:
            rec["decode_caller_layout"] = decode_record(dr_raw, "caller")
        log("[bench] decode: " + ", ".join(f"{lay} {dr_raw[lay]['ms_per_step']:.3f} ms/step" for lay in layouts))
    if not args.no_decode and not args.no_extras:
        rec["decode_q4"] = time_decode_q4(max(args.steps, 20), args.warmup)
        log(f"[bench] decode (4-bit weights): {rec['decode_q4']['ms_per_step']:.3f} ms/step")
    if not args.no_configs:
        for key, name in (("skewed", "mixtral_skewed"), ("many_experts", "many_experts")):
            if name == args.workload:
                continue
            r = time_workload(name, args.steps, args.warmup, layouts=layouts)
            rec[key] = workload_record(r)
            log(f"[bench] {name}: " + ", ".join(f"{lay} {r[lay]['ms_per_step']:.3f} ms/step" for lay in layouts))
    if not args.no_cpu_baseline:
        log("[bench] timing the fp64 oracle ...")
        names = [args.workload] + [w for w in ("mixtral_decode", "mixtral_skewed", "many_experts")
                                   if w != args.workload and not (args.no_configs and w != "mixtral_decode")]
        rec["cpu_baseline"] = cpu_baseline(names, args.cpu_sample)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
