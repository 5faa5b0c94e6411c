"""Throughput of the MoE-layer forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu]

One step = one mok_moe_forward over the workload's whole batch: router projection + top-k,
dispatch plan, pull gather + gate/up GEMM with SwiGLU, down GEMM with the routing-weight
scale, shared experts and the fixed-order combine. Inputs are seeded synthetic tensors
already resident in HBM. Prints ONE JSON line.

`stage_ms` (other than the gate/up stage) comes from a separate untimed pass that times every
stage: the library ties each stage's events to the start of its first kernel and the end of
its last. `hbm` gives the same for the memory-bound stages (plan, combine, MXFP8 weight quantisation and
row gather): algorithmic bytes over the stage's HIP-event time against 8 TB/s.

`roofline` is taken live for the dominant kernel (the gate/up stage: grouped gate/up GEMM
with the fused pull gather and SwiGLU, routed + shared): HIP events that the library attaches
to that launch on the forward's own stream (its start and end; the only events in the timed
steps), averaged over the timed steps, against the
algorithmic FLOPs of one launch (4 * d * I per routed row + 4 * d * I_shared * n_shared per
own token). `roofline.traffic` is the HBM bytes of one launch of that kernel as measured by
the rocprofv3 counter passes summarised in profiles/ (FETCH_SIZE and WRITE_SIZE, each scaled
by what the counter reads for a plain copy of known size); it is null when the summary is
missing or was taken from different kernel sources. `cpu_baseline` is the CPU oracle timed on
a bounded sample of the same workload.

    python bench.py --summarize DIR

writes that summary from the rocprofv3 output directory DIR (layout and commands listed in
the summary itself).
"""
from __future__ import annotations

import argparse
import csv
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer fwd tokens/s + routed-expert TFLOP/s on 1 MI355X (bf16, MXFP8)"
PEAK = {"bf16": 2.5e15, "mxfp8": 5.0e15, "fp32": 157.3e12}
HBM_PEAK = 8.0e12


# sources whose machine code the counter passes describe
KERNEL_SOURCES = ["routing_grouped_expert_gemm_amd/csrc/expert_gemm.hip",
                  "routing_grouped_expert_gemm_amd/csrc/device_common.h",
                  "routing_grouped_expert_gemm_amd/csrc/launch.h",
                  "routing_grouped_expert_gemm_amd/_build.py"]
UP_KERNEL = "k_expert_stage<(mok::Elem)"   # + element, then "true" for the gate/up stage


def kernel_sources_sha256() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def profile_path(workload: str) -> str:
    return os.path.join(ROOT, "profiles", f"expert_gemm_up_{workload}.txt")


def profiled_traffic(workload: str):
    """HBM bytes per launch of the gate/up kernel from the committed counter summary, or None
    if there is none for this workload or it was taken from other kernel sources."""
    try:
        with open(profile_path(workload)) as fh:
            kv = dict(line.split(": ", 1) for line in fh.read().splitlines() if ": " in line)
    except OSError:
        return None
    if kv.get("kernel_sources_sha256", "").strip() != kernel_sources_sha256():
        return None
    try:
        return int(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def _is_up_kernel(name: str, elem: int) -> bool:
    return f"{UP_KERNEL}{elem}, true," in name


def summarize(d: str) -> str:
    """Write profiles/expert_gemm_up_<workload>.txt from a rocprofv3 output directory holding
    trace/ (kernel trace + stats of a bench run, its JSON line in trace.json), FETCH_SIZE/ and
    WRITE_SIZE/ (counter passes over a short bench run) and copy_FETCH_SIZE/, copy_WRITE_SIZE/
    (the same counters over a 1 GiB device copy)."""
    bench_line = json.loads(open(os.path.join(d, "trace.json")).read().strip().splitlines()[-1])
    wl = bench_line["config"]["workload"]
    elem = {"bf16": 1, "f32": 0, "mxfp8": 2}[bench_line["dtype"]]
    stats = list(csv.DictReader(open(os.path.join(d, "trace", "trace_kernel_stats.csv"))))

    def counter(sub, name_pred):
        rows = list(csv.DictReader(open(os.path.join(d, sub, f"{sub}_counter_collection.csv"))))
        vals = [float(r["Counter_Value"]) for r in rows if name_pred(r["Kernel_Name"])]
        return sum(vals) / len(vals), len(vals)

    up = lambda n: _is_up_kernel(n, elem)
    copy = lambda n: "copyBuffer" in n
    fetch_kib, n_f = counter("FETCH_SIZE", up)
    write_kib, n_w = counter("WRITE_SIZE", up)
    copy_fetch, _ = counter("copy_FETCH_SIZE", copy)
    copy_write, _ = counter("copy_WRITE_SIZE", copy)
    copy_kib = 1 << 20                               # 1 GiB read and 1 GiB written per copy
    f_fetch, f_write = copy_kib / copy_fetch, copy_kib / copy_write
    traffic = int(round((fetch_kib * f_fetch + write_kib * f_write) * 1024))
    up_stat = [r for r in stats if up(r["Name"])][0]
    prof_ms = float(up_stat["AverageNs"]) * 1e-6
    ev_ms = bench_line["stage_ms"]["up"]
    # the same dispatches as the events: the gate/up launches of the timed steps, which follow
    # the warm-up steps in launch order (the untimed per-stage pass comes after them)
    trace = [r for r in csv.DictReader(open(os.path.join(d, "trace", "trace_kernel_trace.csv")))
             if up(r["Kernel_Name"])]
    trace.sort(key=lambda r: int(r["Start_Timestamp"]))
    w, k = bench_line["warmup"], bench_line["steps"]
    timed = trace[w:w + k]
    timed_ms = sum(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in timed) / len(timed) * 1e-6
    lines = [
        f"# gate/up expert GEMM stage (routed + shared, fused pull gather and SwiGLU), workload {wl}",
        "#",
        "# commands (from the repository root; D = gpurun_out/prof_" + wl + "):",
        f"#   rocprofv3 --kernel-trace --stats -d D/trace -o trace --output-format csv -- "
        f"python3 bench.py --steps 10 --warmup 3 --no-cpu --workload {wl} > D/trace.json",
        f"#   rocprofv3 --pmc FETCH_SIZE --kernel-include-regex 'mok::' -d D/FETCH_SIZE -o FETCH_SIZE "
        f"--output-format csv -- python3 bench.py --steps 2 --warmup 1 --no-cpu --workload {wl}",
        f"#   rocprofv3 --pmc WRITE_SIZE --kernel-include-regex 'mok::' -d D/WRITE_SIZE -o WRITE_SIZE "
        f"--output-format csv -- python3 bench.py --steps 2 --warmup 1 --no-cpu --workload {wl}",
        "#   rocprofv3 --pmc FETCH_SIZE -d D/copy_FETCH_SIZE -o copy_FETCH_SIZE --output-format csv "
        "-- python3 bench.py --copy-probe-mib 1024",
        "#   rocprofv3 --pmc WRITE_SIZE -d D/copy_WRITE_SIZE -o copy_WRITE_SIZE --output-format csv "
        "-- python3 bench.py --copy-probe-mib 1024",
        "#   python3 bench.py --summarize D",
        "",
        "## kernel trace (--kernel-trace --stats), mok kernels, average per dispatch",
        f"{'kernel':<100} {'calls':>6} {'avg_us':>10} {'min_us':>10} {'max_us':>10}",
    ]
    for r in stats:
        if "mok::" not in r["Name"]:
            continue
        lines.append(f"{r['Name'][:100]:<100} {r['Calls']:>6} {float(r['AverageNs']) / 1e3:>10.1f} "
                     f"{float(r['MinNs']) / 1e3:>10.1f} {float(r['MaxNs']) / 1e3:>10.1f}")
    lines += [
        "",
        f"gate/up kernel average (profiler, all {up_stat['Calls']} dispatches): {prof_ms:.4f} ms",
        f"gate/up kernel average (profiler, the {len(timed)} dispatches of the timed steps): {timed_ms:.4f} ms",
        f"gate/up kernel average (bench.py HIP events, timed steps of the same run): {ev_ms:.4f} ms",
        f"agreement (same dispatches): {100 * (ev_ms - timed_ms) / timed_ms:+.1f} %; against the "
        f"all-dispatch average: {100 * (ev_ms - prof_ms) / prof_ms:+.1f} %",
        f"bench line of the traced run: ms_per_step {bench_line['ms_per_step']}, value "
        f"{bench_line['value']} tokens/s, roofline frac {bench_line['roofline']['frac']}",
        "",
        "## HBM bytes (--pmc), gate/up kernel, per dispatch",
        f"FETCH_SIZE KiB: {fetch_kib:.1f} (mean of {n_f} dispatches)",
        f"WRITE_SIZE KiB: {write_kib:.1f} (mean of {n_w} dispatches)",
        f"copy calibration: 1 GiB device copy reads FETCH_SIZE {copy_fetch:.1f} KiB, WRITE_SIZE "
        f"{copy_write:.1f} KiB -> factors {f_fetch:.4f} (fetch), {f_write:.4f} (write)",
        f"traffic_bytes_per_launch: {traffic}",
        f"kernel_sources_sha256: {kernel_sources_sha256()}",
    ]
    path = profile_path(wl)
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    return path


class HipEvents:
    """hipEvent_t pairs through the HIP runtime (the library records them on its stream).

    Created with hipEventDisableSystemFence: they only time, and the results are read after a
    device synchronisation, so recording them need not write back and invalidate the caches (a
    system-scope fence, which would also slow the kernel that follows)."""
    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self, n: int):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.ev = (ctypes.c_void_p * n)()
        for i in range(n):
            h = ctypes.c_void_p()
            assert self.hip.hipEventCreateWithFlags(ctypes.byref(h), self.DISABLE_SYSTEM_FENCE) == 0
            self.ev[i] = h

    def elapsed_ms(self, a: int, b: int) -> float:
        out = ctypes.c_float(0)
        assert self.hip.hipEventElapsedTime(ctypes.byref(out), self.ev[a], self.ev[b]) == 0
        return out.value

    def ptr(self):
        return ctypes.cast(self.ev, ctypes.c_void_p).value


def algorithmic_work(wl, n_routes: int) -> dict:
    I_sh = wl.n_shared * wl.I_shared
    up = 4.0 * wl.d * wl.I * n_routes + 4.0 * wl.d * I_sh * wl.T_own
    down = 2.0 * wl.d * wl.I * n_routes + 2.0 * wl.d * I_sh * wl.T_own
    return dict(routed_flop=6.0 * wl.d * wl.I * n_routes, shared_flop=6.0 * wl.d * I_sh * wl.T_own,
                up_flop=up, down_flop=down)


def hbm_stages(wl, n_routes: int, stage_ms: dict, ring: bool) -> dict:
    """Achieved HBM rate of the memory-bound stages: algorithmic bytes (each operand read once,
    each result written once) over the stage's HIP-event time, against the 8 TB/s peak.
      plan:    the top-k indices (4 B per route of the pool) read, the local route ids
               (4 B per local route) written;
      combine: per token the shared row and the k route rows read, y written (full layer);
      quant:   every bf16 weight element read (2 B), its E4M3 code and 1/32 of a scale byte
               written (MXFP8);
      gather:  per routed row and own token the bf16 x row read, its codes and scales written
               (MXFP8, stage-ordered; also holds the device work-list build)."""
    eb = 4 if wl.dtype == "fp32" else 2
    routes_pool = wl.T_pool * wl.k
    I_sh = wl.n_shared * wl.I_shared
    bytes_ = {"plan": 4 * routes_pool + 4 * n_routes}
    if wl.full_layer:
        bytes_["combine"] = wl.T_pool * wl.d * eb * (wl.k + 2)
    if wl.dtype == "mxfp8":
        n_w = wl.E_l * 3 * wl.d * wl.I + 3 * wl.d * I_sh
        bytes_["quant"] = n_w * (2 + 1 + 1 / 32)
        if not ring:
            bytes_["gather"] = (n_routes + wl.T_own) * wl.d * (2 + 1 + 1 / 32)
    out = {}
    for name, b in bytes_.items():
        t = stage_ms[name] * 1e-3
        if t <= 0:
            continue
        gbs = b / t / 1e9
        out[name] = {"bytes": int(b), "ms": round(stage_ms[name], 4), "achieved": round(gbs, 1),
                     "unit": "GB/s", "frac": round(gbs * 1e9 / HBM_PEAK, 4)}
    return out


def cpu_baseline(wl, inputs_cpu, sample_tokens: int) -> dict:
    """The oracle (as it stands) on the first `sample_tokens` tokens of the workload."""
    import numpy as np
    import oracle
    import synth
    sub = synth.scaled(wl, T_pool=sample_tokens, tokens_per_rank=sample_tokens,
                       T_own=min(wl.T_own, sample_tokens))
    x = inputs_cpu["x"][:sample_tokens]
    t0 = time.perf_counter()
    if wl.routing == "router":
        out = oracle.moe_forward(sub, x, w_router=inputs_cpu["w_router"], wg=inputs_cpu["wg"],
                                 wu=inputs_cpu["wu"], wd=inputs_cpu["wd"], sg=inputs_cpu["sg"],
                                 su=inputs_cpu["su"], sd=inputs_cpu["sd"])
    else:
        idx, w = oracle.topk(inputs_cpu["logits"][:sample_tokens], wl.k)
        out = oracle.moe_forward(sub, x, wg=inputs_cpu["wg"], wu=inputs_cpu["wu"],
                                 wd=inputs_cpu["wd"], sg=inputs_cpu["sg"], su=inputs_cpu["su"],
                                 sd=inputs_cpu["sd"], topk_in=(idx, w))
    dt = time.perf_counter() - t0
    assert np.isfinite(out["y_shared"]).all()
    cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return {"value": sample_tokens / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"first {sample_tokens} of {wl.T_pool} tokens, whole forward "
                      f"(routing, plan, float64 expert and shared FFNs, combine); {dt:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--ring", action="store_true", help="persistent ring work loop")
    ap.add_argument("--minibatch", type=int, default=None)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--cpu-sample", type=int, default=8192)
    ap.add_argument("--summarize", default=None, metavar="DIR",
                    help="write the profiles/ summary from a rocprofv3 output directory and exit")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (calibrates the HBM "
                         "byte counters of a profiler run) and exit")
    args = ap.parse_args()
    if args.summarize:
        print(summarize(args.summarize))
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): this build has no "
              "multi-GPU path; see the sharding notes in DESIGN.md", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_probe_mib:
        n = args.copy_probe_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n, "copies": 3}))
        return

    import routing_grouped_expert_gemm_amd as mok
    import synth
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from _layer import gpu_layer, gpu_topk, make_inputs

    wl = synth.WORKLOADS[args.workload or synth.EP1]
    dev = "cuda:0"
    torch.cuda.set_device(0)
    inp = make_inputs(wl, dev)
    topk = gpu_topk(inp["logits"], wl.k) if wl.routing == "logits" else None
    flags = 0 if args.ring else mok.MOK_FLAG_NO_RING
    layer = gpu_layer(wl, inp, topk=topk, flags=flags, mb=args.minibatch, keep=True)
    stream = torch.cuda.current_stream()
    n2 = 2 * mok.MOK_N_STAGES
    UP = mok.MOK_STAGE_UP

    def event_table(events, only_up):
        """Per-step stage_events arrays: all stages, or only the gate/up pair (others NULL)."""
        n_steps = len(events.ev) // (2 if only_up else n2)
        tables = []
        for i in range(n_steps):
            t = (ctypes.c_void_p * n2)()
            if only_up:
                t[2 * UP], t[2 * UP + 1] = events.ev[2 * i], events.ev[2 * i + 1]
            else:
                for q in range(n2):
                    t[q] = events.ev[n2 * i + q]
            tables.append(t)
        return tables

    def step(table=None):
        layer.args.stage_events = None if table is None else ctypes.cast(table, ctypes.c_void_p).value
        layer.forward(stream)

    for _ in range(args.warmup):
        step()
    # timed steps: events only on the gate/up launch (the roofline kernel); the library ties
    # them to that kernel's dispatch, so they queue no marker on the stream
    ev_up = HipEvents(2 * args.steps)
    up_tables = event_table(ev_up, True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(up_tables[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms = 1e3 * elapsed / args.steps
    assert layer.device_error(stream) == 0
    up_ms = sum(ev_up.elapsed_ms(2 * i, 2 * i + 1) for i in range(args.steps)) / args.steps
    # per-stage times: a separate, untimed pass with every stage event
    n_stage = min(args.steps, 10)
    ev_all = HipEvents(n2 * n_stage)
    all_tables = event_table(ev_all, False)
    for i in range(n_stage):
        step(all_tables[i])
    torch.cuda.synchronize()

    n_routes = int(layer.inter["offsets"][-1])
    work = algorithmic_work(wl, n_routes)
    stage_ms = {}
    names = ["route", "plan", "quant", "up", "down", "combine", "gather"]
    assert len(names) == mok.MOK_N_STAGES
    for s, name in enumerate(names):
        vals = [ev_all.elapsed_ms(n2 * i + 2 * s, n2 * i + 2 * s + 1) for i in range(n_stage)]
        stage_ms[name] = sum(vals) / len(vals)
    stage_ms["up"] = up_ms                      # the timed steps' own measurement
    up_s = stage_ms["up"] * 1e-3
    peak = PEAK[wl.dtype]
    achieved = work["up_flop"] / up_s
    tokens = wl.T_own if not wl.full_layer else wl.T_pool
    value = tokens / (ms * 1e-3)
    gemm_s = (stage_ms["up"] + stage_ms["down"]) * 1e-3
    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": {"bf16": "bf16", "mxfp8": "mxfp8", "fp32": "f32"}[wl.dtype],
        "data": "synthetic (seeded counter-based generator; random-init weights)",
        "config": {"workload": wl.name, "T_pool": wl.T_pool, "d": wl.d, "E": wl.E, "k": wl.k,
                   "I": wl.I, "E_local": wl.E_l, "n_shared": wl.n_shared,
                   "I_shared": wl.I_shared, "minibatch_rows": layer.args.minibatch_rows,
                   "work_loop": "ring" if args.ring else "stage-ordered"},
        "routed_rows": n_routes,
        "routed_tflops": round(work["routed_flop"] / (ms * 1e-3) / 1e12, 2),
        "gemm_tflops": round((work["routed_flop"] + work["shared_flop"]) / gemm_s / 1e12, 2),
        "stage_ms": {k: round(v, 4) for k, v in stage_ms.items()},
        "roofline": {"bound": "mfma", "kernel": "gate/up stage (k_expert_stage up)",
                     "achieved": round(achieved / 1e12, 2), "peak": peak / 1e12,
                     "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                     "traffic": profiled_traffic(wl.name)},
        "hbm": hbm_stages(wl, n_routes, stage_ms, args.ring),
    }
    if not args.no_cpu:
        import synth as _s  # noqa: F401
        cpu_inp = {k: (v.cpu() if v is not None else None) for k, v in inp.items()}
        out["cpu_baseline"] = cpu_baseline(wl, cpu_inp, min(args.cpu_sample, wl.T_pool))
    print(json.dumps(out))


if __name__ == "__main__":
    main()
