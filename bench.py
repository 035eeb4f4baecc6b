"""Benchmark of the routed 4-bit MoE FFN layer on one MI355X.

One step = the layer's work for a prompt and its first generated token: one
prefill forward over the configuration's prompt length followed by one decode
forward of a single token, as configured (expert budget, WARM residency with
decay shift 5 paging from the pinned host store; --policy picks LRU or LFU).  Inputs are synthetic and already resident in HBM when the
timed region starts.  Prints one JSON line.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                  [--no-cpu-baseline]
  python bench.py --trace-summary TRACE_DIR [--workload NAME]
      per-kernel duration table (markdown) of a rocprofv3 --kernel-trace run of
      this script: the events-timed paged region, the events-timed all-resident
      region (both delimited by the one-element cumsum markers recorded around
      them) and the whole run; also writes profiles/kernels_<workload>.json
      (average duration per expert-kernel kind and region), which later runs
      quote beside their own event timings while the kernel code is unchanged.
  python bench.py --pmc-summary FETCH_DIR WRITE_DIR [--workload NAME]
      turns two rocprofv3 --pmc runs of this script (FETCH_SIZE, then
      WRITE_SIZE) into profiles/traffic_<workload>.json (HBM bytes per launch of
      each expert-kernel kind), which later runs use for the rooflines'
      `traffic` while the kernel code is unchanged.
  python bench.py --counter-summary DIR [DIR ...] [--kind KIND]
      median per dispatch of every counter in rocprofv3 --pmc runs of this
      script, for one expert-kernel kind (prefill_gate_up, prefill_down,
      decode_gate_up, decode_down) in the all-resident region (markdown).
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import statistics
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# row limit of the hybrid comparison run (the best of 2, 3 and 4 on the
# Qwen3-shaped layer: 351k, 403k, 369k tokens/s)
HYBRID_ROWS = 3
METRIC = "MoE-layer tokens/s (decode B=1, prefill 1180) + expert-weight HBM GB/s vs peak"
HBM_PEAK_GBPS = 8000.0
MFMA_PEAK_TFLOPS = {"f16": 2500.0, "bf16": 2500.0}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # the HIP runtime's first ~10 paged steps hold multi-millisecond host stalls
    # inside hipMemcpyAsync (measured; they stop once it has warmed up)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--workload", default="qwen3_30b_a3b")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--hybrid-rows", type=int, default=0,
                    help="hybrid layer whose prefill computes the missed experts with at most this many "
                         "tokens on the host (0: every miss is paged)")
    ap.add_argument("--cpu-steps", type=int, default=6)
    ap.add_argument("--no-policies", action="store_true", help="skip the paged decode policy runs")
    ap.add_argument("--policy", default="warm", choices=["lru", "lfu", "warm"],
                    help="residency policy of the paged layer (warm: decay_shift 5)")
    ap.add_argument("--cpu-baseline-only", action="store_true", help=argparse.SUPPRESS)
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--trace-summary", metavar="TRACE_DIR")
    ap.add_argument("--counter-summary", nargs="+", metavar="DIR")
    ap.add_argument("--kind", default="prefill_gate_up", choices=["prefill_gate_up", "prefill_down",
                                                                   "decode_gate_up", "decode_down"],
                    help="expert-kernel kind of --counter-summary")
    return ap.parse_args()


KERNEL_SRCS = [os.path.join(ROOT, "expert_paged_quantized_amd", "csrc", f)
               for f in ("kernels_expert.hip", "kernels_decode.hip", "kernels_route.hip", "moe_common.h")]
CALIB_BYTES = 256 << 20                        # plain device copy timed in the same run

def _gate_up_arg(name):
    """The second template argument (gate+up or down) of an expert kernel's
    demangled name, e.g. 'moe_decode_dot_kernel<1, true, 1, 1, false>'."""
    args = name[name.find("<") + 1:name.find(">")].split(",")
    return args[1].strip() if len(args) > 1 else ""


# Expert-kernel kinds the profile summaries report, by their demangled name.
KINDS = {
    "prefill_gate_up": lambda n: "moe_prefill_kernel" in n and _gate_up_arg(n) == "true",
    "prefill_down": lambda n: "moe_prefill_kernel" in n and _gate_up_arg(n) == "false",
    "decode_gate_up": lambda n: "moe_decode" in n and _gate_up_arg(n) == "true",
    "decode_down": lambda n: "moe_decode" in n and _gate_up_arg(n) == "false",
}


def code_hash(text):
    """Hash of C++ source with comments and whitespace removed: it changes with
    the code, not with its comments."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return hashlib.sha256(" ".join(text.split()).encode()).hexdigest()[:16]


def kernel_source_hash():
    """One hash over the code of every kernel source file."""
    return code_hash("\n".join(open(f).read() for f in KERNEL_SRCS))


def traffic_path(workload):
    return os.path.join(ROOT, "profiles", f"traffic_{workload}.json")


def durations_path(workload):
    return os.path.join(ROOT, "profiles", f"kernels_{workload}.json")


def load_profile_json(path):
    """A stored profile summary, only while the kernel code it was taken on is unchanged."""
    if not os.path.exists(path):
        return None
    d = json.load(open(path))
    return d if d.get("kernel_source_sha256_16") == kernel_source_hash() else None


def _short(n):
    return n[n.find("strata::") + 8:].split("(")[0] if "strata::" in n else n[:60]


def trace_summary(trace_dir, workload):
    """Markdown tables of kernel durations from a rocprofv3 kernel trace of this
    script, per marked region (see the module docstring), and
    profiles/kernels_<workload>.json: the average duration per expert-kernel
    kind in each events-timed region, for bench.py to quote beside its own
    event timings."""
    f = glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True)
    assert f, f"no kernel_trace.csv under {trace_dir}"
    rows = sorted(csv.DictReader(open(f[0])), key=lambda r: int(r["Start_Timestamp"]))
    marks = [i for i, r in enumerate(rows) if "scan" in r["Kernel_Name"].lower()]

    def dur(r):
        return (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3

    def table(sel, title):
        agg = {}
        for r in sel:
            agg.setdefault(_short(r["Kernel_Name"]), []).append(dur(r))
        out = [f"### {title}", "", "| kernel | calls | total us | avg us | min us | max us |",
               "|---|---|---|---|---|---|"]
        for k, v in sorted(agg.items(), key=lambda kv: -sum(kv[1])):
            out.append(f"| `{k}` | {len(v)} | {sum(v):.1f} | {statistics.mean(v):.2f} | {min(v):.2f} | "
                       f"{max(v):.2f} |")
        return "\n".join(out) + "\n"

    def kinds(sel):
        out = {}
        for kind, test in KINDS.items():
            v = [dur(r) for r in sel if test(r["Kernel_Name"])]
            if v:
                out[kind] = {"launches": len(v), "avg_us": round(statistics.mean(v), 3),
                             "total_us": round(sum(v), 2)}
        return out

    parts, regions = [], {}
    if len(marks) >= 4:
        paged, res = rows[marks[0] + 1:marks[1]], rows[marks[2] + 1:marks[3]]
        parts.append(table(paged, "Events-timed paged region (as configured)"))
        parts.append(table(res, "Events-timed all-resident region"))
        regions = {"paged": kinds(paged), "all_resident": kinds(res)}
    parts.append(table(rows, "Whole run"))
    print("\n".join(parts))
    with open(durations_path(workload), "w") as fo:
        json.dump({"workload": workload, "kernel_source_sha256_16": kernel_source_hash(),
                   "source": "rocprofv3 --kernel-trace of bench.py (events-timed regions)",
                   "regions": regions}, fo, indent=1)


def region_rows(d, counter):
    """Counter rows of one --pmc run, in dispatch order, and the slice of them
    between the third and fourth region markers (the all-resident events-timed
    steps)."""
    f = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    assert f, f"no counter_collection.csv under {d}"
    rows = [r for r in csv.DictReader(open(f[0])) if r["Counter_Name"] == counter]
    rows.sort(key=lambda r: int(r["Dispatch_Id"]))
    marks = [i for i, r in enumerate(rows) if "scan" in r["Kernel_Name"].lower()]
    assert len(marks) >= 4, "expected the four region markers of the events-timed passes"
    return rows, rows[marks[2] + 1:marks[3]]


def counter_summary(dirs, kind="prefill_gate_up"):
    """Median per dispatch of every counter of rocprofv3 --pmc runs, for one
    expert-kernel kind in the all-resident events-timed region."""
    out = [f"| counter | median per dispatch ({kind}) | dispatches |", "|---|---|---|"]
    for d in dirs:
        f = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        assert f, f"no counter_collection.csv under {d}"
        names = sorted({r["Counter_Name"] for r in csv.DictReader(open(f[0]))})
        for c in names:
            _, region = region_rows(d, c)
            v = [float(r["Counter_Value"]) for r in region if KINDS[kind](r["Kernel_Name"])]
            if v:
                out.append(f"| {c} | {statistics.median(v):,.0f} | {len(v)} |")
    print("\n".join(out))


def pmc_summary(fetch_dir, write_dir, workload):
    """Mean FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of each expert-kernel
    kind in the all-resident region, each scaled by what the counter reads for
    the calibration copy (CALIB_BYTES read and written by one copy kernel in
    the same process); written to profiles/traffic_<workload>.json."""
    kinds = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows, region = region_rows(d, counter)
        per = {}
        for r in rows:
            per.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        # the calibration copy (a same-dtype device copy, run by the HIP
        # runtime's copy kernel) is by far the largest copyBuffer dispatch
        cal = max(max(vs) for k, vs in per.items() if "copyBuffer" in k)
        factor = CALIB_BYTES / (cal * 1024.0)
        for kind, test in KINDS.items():
            v = [float(r["Counter_Value"]) for r in region if test(r["Kernel_Name"])]
            if not v:
                continue
            kinds.setdefault(kind, {})[counter] = {
                "kib_per_dispatch": sum(v) / len(v), "dispatches": len(v),
                "calibration_kib": cal, "factor": round(factor, 4)}
    for kind, c in kinds.items():
        c["traffic_bytes_per_launch"] = round(sum(x["kib_per_dispatch"] * 1024.0 * x["factor"]
                                                  for x in c.values() if isinstance(x, dict)))
    res = {"workload": workload, "region": "all-resident events-timed steps",
           "kernel_source_sha256_16": kernel_source_hash(), "kinds": kinds}
    with open(traffic_path(workload), "w") as f:
        json.dump(res, f, indent=1)
    print(json.dumps(res))


def flops_gate_up(cfg, rows):
    return 2.0 * rows * cfg.hidden * 2 * cfg.ffn


def flops_down(cfg, rows):
    return 2.0 * rows * cfg.ffn * cfg.hidden


def w1_bytes(cfg):
    """Packed gate+up bytes of one expert (codes, scales and biases; NVFP4
    matrix scales)."""
    H, F, G = cfg.hidden, cfg.ffn, cfg.group
    per = H * F // 2 + (4 * F * (H // G) if cfg.quant.startswith("int4") else F * (H // G))
    return 2 * per + (8 if cfg.quant == "nvfp4_g16" else 0)


def gate_up_bytes(cfg, distinct, rows):
    """Algorithmic HBM bytes of one gate+up launch: the packed gate+up weights
    of every expert it runs once (routed distinct + shared), each routed row's
    activations once (16-bit), h written once (16-bit)."""
    return (distinct + cfg.num_shared) * w1_bytes(cfg) + rows * cfg.hidden * 2 + rows * cfg.ffn * 2


def main():
    args = parse()
    if args.pmc_summary:
        pmc_summary(args.pmc_summary[0], args.pmc_summary[1], args.workload)
        return
    if args.trace_summary:
        trace_summary(args.trace_summary, args.workload)
        return
    if args.counter_summary:
        counter_summary(args.counter_summary, args.kind)
        return
    if args.cpu_baseline_only:
        from synth import CONFIGS, make_layer
        cfg = CONFIGS[args.workload]
        print(json.dumps(cpu_baseline(make_layer(cfg), cfg, args.cpu_steps)), flush=True)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the layer is not "
              "sharded in this build", file=sys.stderr)
        sys.exit(2)
    import torch

    import expert_paged_quantized_amd as epq
    from synth import CONFIGS, make_layer, make_tokens

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    props = torch.cuda.get_device_properties(dev)
    cfg = CONFIGS[args.workload]
    Tp, Td = cfg.prefill_T, 1
    K, W = args.steps, args.warmup
    log(f"[bench] {cfg.name}: generating weights")
    t0 = time.time()
    lw = make_layer(cfg)
    log(f"[bench] generated in {time.time() - t0:.1f}s; creating layers")
    paged = epq.MoELayer.from_weights(lw, budget=cfg.budget, max_tokens=Tp, policy=args.policy,
                                      decay_shift=5 if args.policy == "warm" else 0,
                                      hybrid=args.hybrid_rows > 0, hybrid_rows=args.hybrid_rows)
    resident = epq.MoELayer.from_weights(lw, budget=cfg.num_experts, max_tokens=Tp)

    n = W + K
    xs_p = [torch.from_numpy(make_tokens(cfg, Tp, step=2 * i).view(np.int16)).view(torch.bfloat16).to(dev)
            for i in range(n)]
    xs_d = [torch.from_numpy(make_tokens(cfg, Td, step=2 * i + 1).view(np.int16)).view(torch.bfloat16).to(dev)
            for i in range(n)]
    y_p = torch.empty((Tp, cfg.hidden), dtype=torch.bfloat16, device=dev)
    y_d = torch.empty((Td, cfg.hidden), dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()

    def run(layer, i):
        layer.forward(xs_p[i], y=y_p)
        layer.forward(xs_d[i], y=y_d)

    mark = torch.ones(4, device=dev)
    region_stats = {}

    def timed_region(layer, events=False, per_step_sync=True):
        for i in range(W):
            run(layer, i)
        torch.cuda.synchronize()
        layer.set_timing(events)
        layer.timing()  # reset
        per = []
        if events:  # a one-element cumsum marks the timed steps in a kernel trace
            mark.cumsum(0)
        torch.cuda.synchronize()
        s0 = layer.stats()
        t_all = time.perf_counter()
        for i in range(W, n):
            a = time.perf_counter()
            run(layer, i)
            if per_step_sync:
                torch.cuda.synchronize()
                per.append(time.perf_counter() - a)
        torch.cuda.synchronize()
        dt = time.perf_counter() - t_all
        s1 = layer.stats()
        region_stats["delta"] = {k: s1[k] - s0[k] for k in ("hits", "misses", "bytes_h2d", "waves", "forwards")}
        if events:
            mark.cumsum(0)
        tm = layer.timing()
        layer.set_timing(False)
        return dt, per, tm

    # (1) headline: as configured, no instrumentation
    log("[bench] timed region: as configured")
    dt, per, _ = timed_region(paged)
    st_timed = region_stats["delta"]  # cache counters of the K timed steps
    # (2) the same inputs with HIP events on every kernel (kernel durations)
    log("[bench] timed region: kernel events")
    dt_ev, _, tm = timed_region(paged, events=True)
    # (3) all experts resident: the GPU path alone
    log("[bench] timed region: all resident")
    dt_r, _, _ = timed_region(resident, per_step_sync=False)
    _, per_r, tm_r = timed_region(resident, events=True)
    st = paged.stats()
    # (4) the same budget and policy as a hybrid layer (the host computes the
    # few-token missed experts of each prefill and every decode miss), beside
    # the paged headline
    hybrid = None
    if args.hybrid_rows == 0 and cfg.budget < cfg.num_experts:
        log(f"[bench] timed region: hybrid, row limit {HYBRID_ROWS}")
        hl = epq.MoELayer.from_weights(lw, budget=cfg.budget, max_tokens=Tp, policy=args.policy,
                                       decay_shift=5 if args.policy == "warm" else 0, hybrid=True,
                                       hybrid_rows=HYBRID_ROWS)
        dt_h, per_h, _ = timed_region(hl)
        dh = dict(region_stats["delta"])
        s1 = hl.stats()
        hybrid = {"value": round(K * (Tp + Td) / dt_h, 1), "unit": "tokens/s", "hybrid_rows": HYBRID_ROWS,
                  "ms_per_step": round(dt_h / K * 1e3, 4),
                  "step_ms_median": round(float(np.median(per_h)) * 1e3, 3),
                  "pages_per_step": round(dh["bytes_h2d"] / max(cfg.expert_bytes(), 1) / K, 2),
                  "host_experts_total": s1["host_experts"], "host_ms_total": round(s1["host_ns"] / 1e6, 2),
                  "note": "host experts and host time since the layer's creation (warm-up included)"}
        hl.close()

    rows = Tp * cfg.top_k + cfg.num_shared * Tp
    up_fl = flops_gate_up(cfg, rows) * K
    mfma_dtype = "bf16" if cfg.quant == "mxfp4_g32" else "f16"
    peak = MFMA_PEAK_TFLOPS[mfma_dtype]
    # the kernel at the workload's shape: one gate+up launch per prefill over
    # all its experts (all-resident region); the paged steps run the same
    # kernel once per wave over that wave's experts (reported beside it)
    up_ms, up_n = tm_r["prefill_gate_up"]
    ach = up_fl / (up_ms * 1e-3) / 1e12
    pg_ms, pg_n = tm["prefill_gate_up"]
    ach_pg = up_fl / (pg_ms * 1e-3) / 1e12
    # arithmetic intensity of the launch against the ridge of the two peaks
    _, dbg_p = resident.forward(xs_p[W], y=y_p, dbg=True)
    distinct = int((dbg_p["counts"] > 0).sum().item())
    gu_bytes = gate_up_bytes(cfg, distinct, rows)
    ai = flops_gate_up(cfg, rows) / gu_bytes
    ridge = peak * 1e12 / (HBM_PEAK_GBPS * 1e9)
    attainable = min(1.0, ai / ridge)
    roof = {"bound": "mfma", "kernel": "moe_prefill_kernel (gate+up, SwiGLU epilogue), one launch per "
                                       "prefill over all its experts (all-resident region)",
            "achieved": round(ach, 2), "peak": peak, "unit": "TFLOP/s", "frac": round(ach / peak, 4),
            "traffic": None, "launches": int(up_n), "avg_launch_us": round(up_ms / max(up_n, 1) * 1e3, 2),
            "algorithmic_flops_per_launch": flops_gate_up(cfg, rows),
            "algorithmic_bytes_per_launch": gu_bytes, "distinct_experts": distinct,
            "arithmetic_intensity": round(ai, 1), "ridge": round(ridge, 1),
            "attainable_frac": round(attainable, 4), "frac_of_attainable": round(ach / peak / attainable, 4),
            "hbm_GBps_on_algorithmic_bytes": round(gu_bytes / (up_ms / max(up_n, 1) * 1e-3) / 1e9, 1),
            "paged_region": {"launches": int(pg_n), "avg_launch_us": round(pg_ms / max(pg_n, 1) * 1e3, 2),
                             "achieved": round(ach_pg, 2), "frac": round(ach_pg / peak, 4),
                             "note": "the same kernel once per wave of the paged steps (same FLOPs in all)"}}
    # stored profiler figures of the same kernel code (profiles/, hash-checked)
    tr = load_profile_json(traffic_path(cfg.name))
    if tr and "prefill_gate_up" in tr["kinds"]:
        t_b = tr["kinds"]["prefill_gate_up"]["traffic_bytes_per_launch"]
        roof["traffic"] = t_b
        roof["traffic_over_algorithmic"] = round(t_b / gu_bytes, 3)
        roof["traffic_unit"] = "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)"
    kd = load_profile_json(durations_path(cfg.name))
    if kd and "prefill_gate_up" in kd["regions"].get("all_resident", {}):
        rp_us = kd["regions"]["all_resident"]["prefill_gate_up"]["avg_us"]
        roof["rocprof_avg_launch_us"] = rp_us
        roof["rocprof_frac"] = round(flops_gate_up(cfg, rows) / (rp_us * 1e-6) / 1e12 / peak, 4)
        roof["duration_sources"] = ("avg_launch_us: HIP events on each dispatch in this run; "
                                    "rocprof_avg_launch_us: profiles/kernels_<workload>.json, same kernel code")

    # decode kernels: all-resident layer; cold = 1 GiB streamed (read) between
    # forwards, so the last-level cache holds other, clean data; warm = the
    # same forward repeated back to back
    log("[bench] decode cold/warm passes")
    flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)

    def decode_pass(cold):
        resident.set_timing(True)
        resident.timing()
        nbytes, cnt = 0, 0
        for i in range(W, n):
            if cold:
                flush.sum()
            else:
                resident.forward(xs_d[i], y=y_d)
            _, dbg = resident.forward(xs_d[i], y=y_d, dbg=True)
            torch.cuda.synchronize()
            nbytes += int((dbg["counts"] > 0).sum().item()) * cfg.expert_bytes() + cfg.num_shared * cfg.expert_bytes()
            cnt += 1
        t = resident.timing()
        resident.set_timing(False)
        runs = cnt if cold else 2 * cnt
        ms = (t["decode_gate_up"][0] + t["decode_down"][0]) * (cnt / runs)
        return nbytes / (ms * 1e-3) / 1e9, nbytes / cnt, ms / cnt

    dec_gbps, dec_bytes, dec_ms = decode_pass(cold=True)
    warm_gbps, _, warm_ms = decode_pass(cold=False)
    del flush

    # decode B=1 wall time, all resident: eager forwards against the same
    # forward replayed from a HIP graph (no host launch work per kernel; each
    # replay first copies the new token into the graph's input buffer)
    def decode_b1():
        x_st = xs_d[W].clone()
        y_st = torch.empty_like(x_st)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            resident.forward(x_st, y=y_st)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            resident.forward(x_st, y=y_st)
        out = {}
        for mode in ("eager", "graph"):
            def one(x):
                if mode == "eager":
                    resident.forward(x, y=y_d)
                else:
                    x_st.copy_(x)
                    g.replay()
            per = []
            for i in range(W, n):
                a = time.perf_counter()
                one(xs_d[i])
                torch.cuda.synchronize()
                per.append(time.perf_counter() - a)
            torch.cuda.synchronize()
            a = time.perf_counter()
            for i in range(W, n):
                one(xs_d[i])
            torch.cuda.synchronize()
            bb = (time.perf_counter() - a) / K
            out[mode] = {"us_per_token_synced_median": round(statistics.median(per) * 1e6, 1),
                         "tokens_per_s_back_to_back": round(1.0 / bb, 1)}
        del g
        return out

    log("[bench] decode B=1 latency: eager and graph replay")
    dec_b1 = decode_b1()

    # decode at each batch size the configuration lists (B tokens per
    # forward, fresh tokens each time): all resident (wall time with a
    # synchronisation after each forward, decode-kernel time by HIP events,
    # expert bytes per forward) and paged as configured (B tokens per forward
    # through the residency policy)
    def decode_batches():
        out = {}
        nf = 48
        for B in cfg.decode_T:
            xb = [torch.from_numpy(make_tokens(cfg, B, step=900000 + 1000 * B + i).view(np.int16))
                  .view(torch.bfloat16).to(dev) for i in range(2 * nf)]
            yb = torch.empty((B, cfg.hidden), dtype=torch.bfloat16, device=dev)
            for i in range(8):
                resident.forward(xb[i], y=yb)
            torch.cuda.synchronize()
            resident.set_timing(True)
            resident.timing()
            per, nbytes = [], 0
            for i in range(nf, 2 * nf):
                a = time.perf_counter()
                resident.forward(xb[i], y=yb)
                torch.cuda.synchronize()
                per.append(time.perf_counter() - a)
            t = resident.timing()
            resident.set_timing(False)
            for i in range(nf, 2 * nf):  # the same forwards again, for their distinct experts
                _, dbg = resident.forward(xb[i], y=yb, dbg=True)
                nbytes += (int((dbg["counts"] > 0).sum().item()) + cfg.num_shared) * cfg.expert_bytes()
            kms = t["decode_gate_up"][0] + t["decode_down"][0]
            med = statistics.median(per)
            pl = epq.MoELayer.from_weights(lw, budget=cfg.budget, max_tokens=max(cfg.decode_T),
                                           policy=args.policy, decay_shift=5 if args.policy == "warm" else 0)
            for i in range(nf):
                pl.forward(xb[i], y=yb)
            torch.cuda.synchronize()
            s0 = pl.stats()
            a = time.perf_counter()
            for i in range(nf, 2 * nf):
                pl.forward(xb[i], y=yb)
            torch.cuda.synchronize()
            dtp = time.perf_counter() - a
            s1 = pl.stats()
            pl.close()
            hits, miss = s1["hits"] - s0["hits"], s1["misses"] - s0["misses"]
            out[str(B)] = {"all_resident_tokens_per_s": round(B / med, 1),
                           "all_resident_us_per_forward_synced_median": round(med * 1e6, 1),
                           "decode_kernel_us_per_forward": round(kms * 1e3 / nf, 2),
                           "expert_bytes_per_forward": nbytes // nf,
                           "decode_kernel_GBps": round(nbytes / (kms * 1e-3) / 1e9, 1),
                           "paged_tokens_per_s": round(nf * B / dtp, 1),
                           "paged_hit_rate": round(hits / max(hits + miss, 1), 3),
                           "paged_misses_per_forward": round(miss / nf, 2)}
        return out

    dec_batches = None
    if len(cfg.decode_T) > 1 and not args.no_policies:
        log(f"[bench] decode at B = {cfg.decode_T}")
        dec_batches = decode_batches()
    read_ceiling = epq.measure_hbm_read(0, 1 << 30, 5)
    decode_roof = {"bound": "hbm", "kernel": "decode gate+up and down (expert-weight bytes)",
                   "achieved": round(dec_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                   "frac": round(dec_gbps / HBM_PEAK_GBPS, 4), "traffic": None,
                   "measured_read_ceiling": round(read_ceiling, 1),
                   "frac_of_measured_ceiling": round(dec_gbps / read_ceiling, 4),
                   "expert_bytes_per_forward": dec_bytes,
                   "kernel_us_per_forward": round(dec_ms * 1e3, 2),
                   "mall": "cold (1 GiB streamed between forwards)",
                   "warm": {"achieved": round(warm_gbps, 1), "kernel_us_per_forward": round(warm_ms * 1e3, 2)}}
    if tr and "decode_gate_up" in tr["kinds"] and "decode_down" in tr["kinds"]:
        t_b = tr["kinds"]["decode_gate_up"]["traffic_bytes_per_launch"] + \
            tr["kinds"]["decode_down"]["traffic_bytes_per_launch"]
        decode_roof["traffic"] = t_b
        decode_roof["traffic_over_algorithmic"] = round(t_b / dec_bytes, 3)
        decode_roof["traffic_unit"] = ("HBM bytes per decode forward, gate+up + down launches (rocprofv3 "
                                       "FETCH_SIZE + WRITE_SIZE, copy-calibrated; warm-region dispatches)")
    if kd and "decode_gate_up" in kd["regions"].get("all_resident", {}):
        ra = kd["regions"]["all_resident"]
        decode_roof["rocprof_kernel_us_per_forward"] = round(ra["decode_gate_up"]["avg_us"] +
                                                             ra.get("decode_down", {}).get("avg_us", 0.0), 2)

    # calibration copy for the HBM byte counters (FETCH_SIZE / WRITE_SIZE):
    # CALIB_BYTES read and written by one device-to-device copy
    cal_src = torch.empty(CALIB_BYTES // 4, dtype=torch.float32, device=dev)
    cal_dst = torch.empty_like(cal_src)
    cal_dst.copy_(cal_src)
    torch.cuda.synchronize()
    del cal_src, cal_dst

    # pinned host -> device rate on this machine (the paging link), measured by the library
    h2d_gbps = epq.measure_h2d(0, 256 << 20, 3)

    # paged decode streams (B=1, fresh x per token) under each residency policy
    policies = None if args.no_policies else decode_policies(epq, torch, lw, cfg, dev, make_tokens)

    # the step's resources (ro99/strata README, contribution rules: the step
    # time is bounded by max over resources of work / rate, plus the serial
    # part): host link (expert bytes paged), HBM (algorithmic bytes),
    # matrix cores (prefill FLOPs), and the serial kernels (router, routing,
    # combine) measured with events in the paged region
    ms_step = dt / K * 1e3
    link_bytes = st_timed["bytes_h2d"] / K
    link = {"bytes_per_step": round(link_bytes), "achieved_GBps": round(link_bytes / (ms_step * 1e-3) / 1e9, 2),
            "peak_GBps": round(h2d_gbps, 2), "peak_source": "pinned hipMemcpyAsync of 256 MB, this run",
            "frac": round(link_bytes / (ms_step * 1e-3) / 1e9 / h2d_gbps, 4),
            "pages_per_step": round(st_timed["misses"] / K, 2)}
    _, dbg_d = resident.forward(xs_d[W], y=y_d, dbg=True)
    distinct_d = int((dbg_d["counts"] > 0).sum().item())
    eb = cfg.expert_bytes()
    rows_d = Td * (cfg.top_k + cfg.num_shared)
    ksplit_planes = 1  # activations and o rows; o planes of a split-K down GEMM add reads
    hbm_bytes = ((distinct + cfg.num_shared + distinct_d + cfg.num_shared) * eb   # expert records
                 + 2 * cfg.num_experts * cfg.hidden * 2                        # router weights, 2 forwards
                 + (Tp + Td) * cfg.hidden * 2 * (2 if cfg.quant == "mxfp4_g32" else 3)  # x, fp16 copy, y
                 + (rows + rows_d) * (cfg.hidden * 2 + cfg.ffn * 4 + cfg.hidden * 8 * ksplit_planes)
                 + link_bytes)                                                  # pages written to HBM
    fl_step = flops_gate_up(cfg, rows) + flops_down(cfg, rows)
    serial_ms = sum(tm[k][0] for k in ("router", "group", "combine")) / K
    terms = {"host_link_ms": link_bytes / (h2d_gbps * 1e9) * 1e3,
             "hbm_ms": hbm_bytes / (HBM_PEAK_GBPS * 1e9) * 1e3,
             "mfma_ms": fl_step / (peak * 1e12) * 1e3}
    arg = max(terms, key=terms.get)
    tau = {"terms_ms": {k: round(v, 4) for k, v in terms.items()}, "serial_ms": round(serial_ms, 4),
           "serial_kernels": "router + routing (top-k, permute) + combine, HIP events, paged region",
           "tau_ms": round(max(terms.values()) + serial_ms, 4), "measured_ms_per_step": round(ms_step, 4),
           "argmax_r": arg.replace("_ms", ""),
           "hbm_bytes_per_step": round(hbm_bytes), "flops_per_step": fl_step}

    tokens_per_step = Tp + Td
    value = K * tokens_per_step / dt
    res = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": K,
        "warmup": W, "ms_per_step": round(dt / K * 1e3, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": mfma_dtype, "data": "synthetic",
        "config": {"workload": f"{cfg.name}: one MoE FFN layer, H={cfg.hidden} F={cfg.ffn} "
                               f"E={cfg.num_experts} top-{cfg.top_k} shared={cfg.num_shared} "
                               f"{cfg.quant} {cfg.router} router"
                               + (f" Zipf({cfg.zipf_s}) bias" if cfg.zipf_s else "")
                               + f"; budget {cfg.budget}/{cfg.num_experts} slots, {args.policy.upper()}; "
                               f"step = prefill {Tp} tokens + decode {Td} token"
                               + (f"; hybrid: the host computes the missed experts of at most "
                                  f"{args.hybrid_rows} tokens in prefill and every miss in decode"
                                  if args.hybrid_rows else ""),
                   "prefill_T": Tp, "decode_T": Td, "budget": cfg.budget, "hybrid_rows": args.hybrid_rows,
                   "parallelism": "single GPU"},
        "roofline": roof,
        "decode_roofline": decode_roof,
        "decode_b1_all_resident": dec_b1,
        "decode_batches": dec_batches,
        "step_ms_median": round(statistics.median(per) * 1e3, 3),
        "step_ms_range": [round(min(per) * 1e3, 3), round(max(per) * 1e3, 3)],
        "all_resident": {"value": round(K * tokens_per_step / dt_r, 1),
                         "step_ms_median": round(statistics.median(per_r) * 1e3, 4),
                         "kernel_ms_per_step": {k: round(v[0] / K, 4) for k, v in tm_r.items()}},
        "kernel_ms_per_step": {k: round(v[0] / K, 4) for k, v in tm.items()},
        "events_pass_ms_per_step": round(dt_ev / K * 1e3, 4),
        "link": link, "tau": tau,
        "cache": st, "h2d_GBps": round(h2d_gbps, 2),
        "paged_decode": policies,
        "hybrid": hybrid,
        "gpu": {"name": props.name, "cus": props.multi_processor_count},
    }

    paged.close()
    resident.close()
    if not args.no_cpu_baseline:
        # the oracle runs in a process of its own (no GPU runtime there)
        r = subprocess.run([sys.executable, os.path.abspath(__file__), "--cpu-baseline-only",
                            "--workload", args.workload, "--cpu-steps", str(args.cpu_steps)],
                           capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"cpu baseline failed: {r.stderr[-2000:]}")
        res["cpu_baseline"] = json.loads(r.stdout.strip().splitlines()[-1])
    print(json.dumps(res), flush=True)


DECODE_WARM, DECODE_TIMED = 64, 256
POLICY_RUNS = [("lru", dict(policy="lru")),
               ("lfu", dict(policy="lfu")),
               ("warm_d5", dict(policy="warm", decay_shift=5)),
               ("warm_d5_prefetch2", dict(policy="warm", decay_shift=5, prefetch=2)),
               # host threads compute the non-resident experts of each token
               ("hybrid_lfu", dict(policy="lfu", hybrid=True)),
               ("hybrid_warm_d5_prefetch2", dict(policy="warm", decay_shift=5, prefetch=2, hybrid=True))]


def decode_policies(epq, torch, lw, cfg, dev, make_tokens):
    """Decode B=1 through the residency manager: DECODE_WARM untimed then
    DECODE_TIMED timed forwards, each on a fresh token, per policy; the first
    DECODE_WARM forwards of a new layer started cold and started from a
    profile saved after another stream of the same workload; and a change of
    work (DECODE_TIMED tokens of one topic, then DECODE_TIMED of another,
    timed together after DECODE_WARM of the first)."""
    log("[bench] paged decode policies")
    n = DECODE_WARM + DECODE_TIMED
    xs = [torch.from_numpy(make_tokens(cfg, 1, step=500000 + i).view(np.int16)).view(torch.bfloat16).to(dev)
          for i in range(n)]
    xs_prev = [torch.from_numpy(make_tokens(cfg, 1, step=600000 + i).view(np.int16)).view(torch.bfloat16)
               .to(dev) for i in range(DECODE_TIMED)]
    y = torch.empty((1, cfg.hidden), dtype=torch.bfloat16, device=dev)

    def stream(layer, xs_run):
        torch.cuda.synchronize()
        s0 = layer.stats()
        t0 = time.perf_counter()
        for x in xs_run:
            layer.forward(x, y=y)
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        s1 = layer.stats()
        d = {k: s1[k] - s0[k] for k in ("hits", "misses", "bytes_h2d", "prefetched", "prefetch_hits",
                                        "host_experts", "host_ns")}
        out = {"tokens_per_s": round(len(xs_run) / dt, 1), "us_per_token": round(dt / len(xs_run) * 1e6, 2),
               "hit_rate": round(d["hits"] / max(1, d["hits"] + d["misses"] + d["host_experts"]), 4),
               "misses_per_token": round(d["misses"] / len(xs_run), 3),
               "h2d_MB_per_token": round(d["bytes_h2d"] / len(xs_run) / 1e6, 3),
               "prefetched": d["prefetched"], "prefetch_hits": d["prefetch_hits"]}
        if d["host_experts"]:
            hb = d["host_experts"] * cfg.expert_bytes()
            out.update({"host_experts_per_token": round(d["host_experts"] / len(xs_run), 3),
                        "host_us_per_token": round(d["host_ns"] / len(xs_run) / 1e3, 2),
                        "host_GBps": round(hb / max(d["host_ns"], 1), 2)})
        return out

    out = {"budget": cfg.budget, "experts": cfg.num_experts, "warmup_tokens": DECODE_WARM,
           "timed_tokens": DECODE_TIMED, "runs": {}}
    for name, kw in POLICY_RUNS:
        layer = epq.MoELayer.from_weights(lw, budget=cfg.budget, max_tokens=1, **kw)
        stream(layer, xs[:DECODE_WARM])
        out["runs"][name] = stream(layer, xs[DECODE_WARM:])
        layer.close()
    # warm start: a profile learned on another stream of the same workload
    src = epq.MoELayer.from_weights(lw, budget=cfg.budget, max_tokens=1, policy="warm", decay_shift=5)
    stream(src, xs_prev)
    prof = src.save_profile()
    src.close()
    ws = {}
    for name, p in (("cold", None), ("profile", prof)):
        layer = epq.MoELayer.from_weights(lw, budget=cfg.budget, max_tokens=1, policy="warm", decay_shift=5,
                                          profile=p)
        ws[name] = stream(layer, xs[:DECODE_WARM])
        layer.close()
    out["warm_start_first_tokens"] = ws
    # a change of work: topic 1 then topic 2 (each adds a fixed direction to x)
    xa = [torch.from_numpy(make_tokens(cfg, 1, step=700000 + i, topic=1).view(np.int16)).view(torch.bfloat16)
          .to(dev) for i in range(DECODE_WARM + DECODE_TIMED)]
    xb = [torch.from_numpy(make_tokens(cfg, 1, step=800000 + i, topic=2).view(np.int16)).view(torch.bfloat16)
          .to(dev) for i in range(DECODE_TIMED)]
    shift = {}
    for name, kw in POLICY_RUNS[:3]:
        layer = epq.MoELayer.from_weights(lw, budget=cfg.budget, max_tokens=1, **kw)
        stream(layer, xa[:DECODE_WARM])
        shift[name] = stream(layer, xa[DECODE_WARM:] + xb)
        layer.close()
    out["topic_shift"] = shift
    return out


def cpu_baseline(lw, cfg, n_steps):
    """The CPU oracle, untouched, timed on a bounded sample of the same workload:
    the first `n_steps` steps (prefill + one decode token each) of the inputs."""
    import threadpoolctl

    from oracle import moe as om
    from synth import make_tokens
    cores = min(len(os.sched_getaffinity(0)), 16)
    with threadpoolctl.threadpool_limits(limits=cores):
        xs = [(make_tokens(cfg, cfg.prefill_T, step=2 * i), make_tokens(cfg, 1, step=2 * i + 1))
              for i in range(n_steps)]
        log(f"[bench] cpu baseline: oracle on {n_steps} steps, {cores} threads")
        a = time.perf_counter()
        for xp, xd in xs:
            om.moe_forward(lw, xp)
            om.moe_forward(lw, xd)
        dt = time.perf_counter() - a
    tok = n_steps * (cfg.prefill_T + 1)
    return {"value": round(tok / dt, 2), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{n_steps} whole steps (prefill {cfg.prefill_T} + decode 1 token each) of the "
                      f"same inputs; {dt:.1f} s; fp64 oracle, dequantising per forward"}


if __name__ == "__main__":
    main()
