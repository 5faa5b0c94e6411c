"""Throughput of the MoE-layer forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--ring] [--no-cpu]

One step = one mok_moe_forward over the workload's whole batch: router projection + top-k
(or top-k of given logits), dispatch plan, pull gather + gate/up GEMM with SwiGLU, down GEMM
with the routing-weight scale, shared experts and (full layer) the fixed-order combine. Inputs
are seeded synthetic tensors already resident in HBM. Prints ONE JSON line.

Default run: the headline is the EP=1 bf16 layer (T=8192, d=2048, 64 experts, top-6) with
stage-ordered expert launches; the same line carries
  "ring":  that layer with the persistent ring work loop (the library default), and
  "mxfp8": the MXFP8 EP=64 share (262144-row pool, d=7168, 4 local experts + 1 shared),
  "mxfp4": the same share with MXFP4 operands (each with a "ring" object: the ring work loop,
           whose items include the row gather and quantisation), and
  "backward": the EP=1 layer's backward (mok_moe_backward), and
  "dispatch": pull gather against the push baseline on that share's routing,
each timed the same way (W warm-up steps, K timed steps between device synchronisations).
--workload NAME measures that workload alone (used by the profiling runs).

`stage_ms` (other than the roofline kernel's) comes from a separate, untimed pass that times
every stage with HIP events the library ties to the start of each stage's first kernel and the
end of its last; before each step of that pass a 1 GiB scratch buffer is read, so the
stage times are cold-cache times (the 256 MB last-level cache holds nothing of the step
before). A read, not a write: overwriting the buffer would leave ~1 GiB of dirty lines whose
write-back competes with the first stages of the step. `hbm` gives, for the memory-bound stages, algorithmic bytes over those times against
8 TB/s.

`roofline` is taken live for the dominant kernel: the gate/up stage (grouped gate/up GEMM with
the fused pull gather and SwiGLU, routed + shared) when stage-ordered, the whole ring loop
(gate/up and down tiles) with --ring. Its time comes from HIP events the library attaches to
that launch on the forward's own stream (the only events in the timed steps); `achieved` is the
launch's algorithmic FLOPs (gate/up: 4*d*I per routed row + 4*d*I_s*n_s per own token; down:
half that) over it. `roofline.traffic` is the HBM bytes of one launch of that kernel from the
rocprofv3 counter passes summarised in profiles/ (FETCH_SIZE and WRITE_SIZE, each scaled by
what the counter reads for a plain 1 GiB copy); null when the summary is missing or was taken
from other kernel sources. `cpu_baseline` is the CPU oracle timed on the same workload.

    python bench.py --summarize DIR

writes the profiles/ summaries from a rocprofv3 output directory DIR (layout and commands are
listed in the summaries themselves).
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
PEAK = {"bf16": 2.5e15, "mxfp8": 5.0e15, "mxfp4": 10.1e15, "fp32": 157.3e12}
HBM_PEAK = 8.0e12


# sources whose machine code the counter passes describe
KERNEL_SOURCES = ["routing_grouped_expert_gemm_amd/csrc/expert_gemm.hip",
                  "routing_grouped_expert_gemm_amd/csrc/device_common.h",
                  "routing_grouped_expert_gemm_amd/csrc/lds_dma.h",
                  "routing_grouped_expert_gemm_amd/csrc/worklist.h",
                  "routing_grouped_expert_gemm_amd/csrc/launch.h",
                  "routing_grouped_expert_gemm_amd/_build.py"]
ELEM = {"f32": 0, "bf16": 1, "mxfp8": 2, "mxfp4": 3}
ELEM_NAME = {0: "fp32", 1: "bf16", 2: "mxfp8", 3: "mxfp4"}
FLUSH_BYTES = 1 << 30        # scratch read before each step of the per-stage pass


def cache_scratch(dev):
    """A 1 GiB device buffer (4x the last-level cache), written once."""
    import torch
    scratch = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)
    scratch.fill_(1)
    torch.cuda.synchronize()
    return scratch


def evict_caches(scratch) -> None:
    """Reads the scratch buffer on the current stream: afterwards no cache holds anything of the
    earlier work, and no dirty line is left whose write-back would compete with what follows."""
    import torch
    scratch.view(torch.int64).sum()


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


# ------------------------------------------------------------------ profile summaries

def kernel_key(name: str) -> str:
    """Short, stable name of a mok kernel from its demangled name (None for other kernels)."""
    if "mok::" not in name:
        return None
    n = name.replace("void ", "").strip()
    if n.endswith(")"):                  # drop the parameter list: from the "(" matching the end
        depth = 0
        for i in range(len(n) - 1, -1, -1):
            depth += {")": 1, "(": -1}.get(n[i], 0)
            if depth == 0:
                n = n[:i]
                break
    n = n.replace("mok::", "").strip()
    if n.startswith("k_expert_stage<"):
        parts = n[len("k_expert_stage<"):].split(",")
        el = ELEM_NAME[int(parts[0].split(")")[-1])]
        return f"k_expert_stage<{el}, {'gate/up' if parts[1].strip() == 'true' else 'down'}>"
    if n.startswith("k_ring<"):
        el = ELEM_NAME[int(n[len("k_ring<"):].split(",")[0].split(")")[-1])]
        return f"k_ring<{el}>"
    return n


def algorithmic_bytes(wl, n_routes: int) -> dict:
    """Bytes each memory-bound kernel must move per forward (each operand read once, each
    result written once); the GEMM stages are priced in FLOPs instead."""
    es = 4 if wl.dtype == "fp32" else 2
    T, d, E, k = wl.T_pool, wl.d, wl.E, wl.k
    I_sh = wl.n_shared * wl.I_shared
    # keyed by kernel name without template arguments where those vary with the shape
    out = {"k_plan_count": 4 * T * k, "k_plan_scatter": 4 * T * k + 4 * n_routes,
           "k_topk": 4 * T * E + 8 * T * k}
    if wl.routing == "router":
        out["k_router_logits"] = T * d * es + E * d * es + 4 * T * E
        out["k_route"] = T * d * es + E * d * es + 4 * T * E + 8 * T * k   # logits + top-k
    if wl.full_layer:
        out["k_combine"] = T * d * es * (k + 2)
    if wl.dtype in ("mxfp8", "mxfp4"):
        cb = 0.5 if wl.dtype == "mxfp4" else 1.0      # code bytes per element
        n_w = wl.E_l * 3 * d * wl.I + 3 * d * I_sh
        out["k_quantize_mx"] = n_w * (2 + cb + 1 / 32)
        out["k_gather_quantize"] = (n_routes + wl.T_own) * d * (2 + cb + 1 / 32)
    return out


def _csv(path):
    with open(path) as fh:
        return list(csv.DictReader(fh))


def _per_forward(rows, key_of, value_of):
    """Per-kernel totals over a run divided by its forwards (or backwards): one k_plan_count
    each."""
    tot, n = {}, {}
    for r in rows:
        k = key_of(r)
        if k is None:
            continue
        tot[k] = tot.get(k, 0.0) + value_of(r)
        n[k] = n.get(k, 0) + 1
    fwd = n.get("k_plan_count", 1)
    return {k: v / fwd for k, v in tot.items()}, {k: v / fwd for k, v in n.items()}


def summarize(d: str) -> list:
    """Write the profiles/ summaries of one workload from a rocprofv3 output directory d:
      trace.json + trace/    kernel trace + stats of a bench run (its JSON line in trace.json)
      FETCH_SIZE/ WRITE_SIZE/             counter passes over a short bench run
      copy_FETCH_SIZE/ copy_WRITE_SIZE/   the same counters over a plain 1 GiB device copy
      ctr_p1/ ... (optional)  SQ/TCP/TCC counter sets over the expert GEMM stages
    into profiles/kernels_<wl>.txt (every kernel: time, counter bytes, algorithmic rate),
    profiles/expert_gemm_up_<wl>.txt (the gate/up launch: time agreement with bench.py's events
    and the HBM traffic bench.py reports) and, with ctr_p*, expert_gemm_counters_<wl>.txt."""
    import synth
    line = json.loads(open(os.path.join(d, "trace.json")).read().strip().splitlines()[-1])
    if line.get("mode") == "dispatch":
        return [summarize_dispatch(d, line)]
    if line.get("mode") == "backward":
        return [summarize_backward(d, line)]
    wl_name = line["config"]["workload"]
    wl = synth.WORKLOADS[wl_name]
    n_routes = line["routed_rows"]
    elem = ELEM[line["dtype"]]
    up_key = f"k_expert_stage<{ELEM_NAME[elem]}, gate/up>"
    name_col = lambda r: kernel_key(r["Kernel_Name"])
    trace = _csv(os.path.join(d, "trace", "trace_kernel_trace.csv"))
    dur = lambda r: (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-6   # ms
    t_fwd, calls = _per_forward(trace, name_col, dur)

    def counter(sub, pred=None):
        rows = _csv(os.path.join(d, sub, f"{sub}_counter_collection.csv"))
        if pred is not None:
            vals = [float(r["Counter_Value"]) for r in rows if pred(r["Kernel_Name"])]
            return sum(vals) / len(vals)
        return _per_forward(rows, name_col, lambda r: float(r["Counter_Value"]))[0]

    copy_fetch = counter("copy_FETCH_SIZE", lambda n: "copyBuffer" in n)
    copy_write = counter("copy_WRITE_SIZE", lambda n: "copyBuffer" in n)
    f_fetch, f_write = (1 << 20) / copy_fetch, (1 << 20) / copy_write   # 1 GiB each way
    fetch = {k: v * f_fetch * 1024 for k, v in counter("FETCH_SIZE").items()}
    write = {k: v * f_write * 1024 for k, v in counter("WRITE_SIZE").items()}
    alg = algorithmic_bytes(wl, n_routes)
    work = algorithmic_work(wl, n_routes)
    cmd = (f"--workload {wl_name}")
    D = f"gpurun_out/prof_{wl_name}"
    cmds = [
        f"#   rocprofv3 --kernel-trace --stats -d {D}/trace -o trace --output-format csv -- "
        f"python3 bench.py --steps 10 --warmup 3 --no-cpu {cmd} > {D}/trace.json",
        f"#   rocprofv3 --pmc FETCH_SIZE --kernel-include-regex 'mok::' -d {D}/FETCH_SIZE -o "
        f"FETCH_SIZE --output-format csv -- python3 bench.py --steps 2 --warmup 1 --no-cpu {cmd}",
        f"#   rocprofv3 --pmc WRITE_SIZE --kernel-include-regex 'mok::' -d {D}/WRITE_SIZE -o "
        f"WRITE_SIZE --output-format csv -- python3 bench.py --steps 2 --warmup 1 --no-cpu {cmd}",
        f"#   rocprofv3 --pmc FETCH_SIZE -d {D}/copy_FETCH_SIZE -o copy_FETCH_SIZE --output-format "
        f"csv -- python3 bench.py --copy-probe-mib 1024",
        f"#   rocprofv3 --pmc WRITE_SIZE -d {D}/copy_WRITE_SIZE -o copy_WRITE_SIZE --output-format "
        f"csv -- python3 bench.py --copy-probe-mib 1024",
        f"#   python3 bench.py --summarize {D}",
    ]
    written = []
    # ---- every kernel
    lines = [f"# every libmok kernel of one forward, workload {wl_name} ({line['dtype']}, "
             f"stage-ordered), per forward", "#", "# commands (from the repository root):"] + cmds + [
        "#",
        "# time: kernel durations from the trace, summed per forward (warm-up, timed and the",
        "#   cold-cache per-stage steps of the traced run together: 'calls' launches each);",
        "# fetch/write: FETCH_SIZE / WRITE_SIZE summed per forward, scaled by the copy",
        f"#   calibration (1 GiB copy reads FETCH_SIZE {copy_fetch:.0f} KiB, WRITE_SIZE "
        f"{copy_write:.0f} KiB: factors {f_fetch:.4f}, {f_write:.4f});",
        "# alg: the bytes the kernel must move (each operand read once, each result written once)",
        "#   and alg/time against 8 TB/s; GEMM stages: algorithmic FLOPs/time against the dtype's",
        "#   dense MFMA peak.",
        "",
        f"{'kernel':<36} {'calls':>5} {'time_us':>9} {'fetch_MB':>9} {'write_MB':>9} "
        f"{'alg_MB':>9} {'alg_GB/s':>9} {'counter_GB/s':>12} {'of_peak':>8}",
    ]
    peak = PEAK[ELEM_NAME[elem]]
    outside = []
    for k in sorted(t_fwd, key=lambda k: -t_fwd[k]):
        if calls[k] < 0.5:               # launched once per run (input preparation)
            outside.append(k)
            continue
        t = t_fwd[k]
        fb, wb = fetch.get(k, 0.0), write.get(k, 0.0)
        row = f"{k:<36} {calls[k]:>5.1f} {t * 1e3:>9.1f} {fb / 1e6:>9.1f} {wb / 1e6:>9.1f} "
        a = alg.get(k, alg.get(k.split("<")[0]))
        if a is not None:
            row += (f"{a / 1e6:>9.1f} {a / (t * 1e-3) / 1e9:>9.0f} "
                    f"{(fb + wb) / (t * 1e-3) / 1e9:>12.0f} {a / (t * 1e-3) / HBM_PEAK:>8.3f}")
        elif k.startswith("k_expert_stage"):
            f = work["up_flop"] if "gate/up" in k else work["down_flop"]
            row += (f"{'-':>9} {'-':>9} {(fb + wb) / (t * 1e-3) / 1e9:>12.0f} "
                    f"{f / (t * 1e-3) / peak:>8.3f}")
        else:
            row += f"{'-':>9} {'-':>9} {(fb + wb) / (t * 1e-3) / 1e9:>12.0f} {'-':>8}"
        lines.append(row)
    if outside:
        lines.append(f"(not part of the forward, launched once per run: {', '.join(outside)})")
    lines += ["", f"bench line of the traced run: ms_per_step {line['ms_per_step']}, value "
              f"{line['value']} tokens/s, routed rows {n_routes}",
              f"kernel_sources_sha256: {kernel_sources_sha256()}"]
    path = os.path.join(ROOT, "profiles", f"kernels_{wl_name}.txt")
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    written.append(path)
    # ---- the gate/up launch (roofline kernel): time agreement and traffic per launch
    ups = sorted((r for r in trace if name_col(r) == up_key), key=lambda r: int(r["Start_Timestamp"]))
    w, k = line["warmup"], line["steps"]
    timed = ups[w:w + k]
    timed_ms = sum(dur(r) for r in timed) / len(timed)
    all_ms = sum(dur(r) for r in ups) / len(ups)
    ev_ms = line["stage_ms"]["up"]
    traffic = int(round(fetch[up_key] + write[up_key]))     # one gate/up launch per forward
    alg_up = ((wl.E_l * 2 * wl.I + 2 * wl.n_shared * wl.I_shared) * wl.d +
              (n_routes + wl.T_own) * wl.d) * {"mxfp8": 1, "mxfp4": 0.5}.get(wl.dtype, 2)
    lines = [
        f"# gate/up expert GEMM stage (routed + shared, fused pull gather and SwiGLU), workload {wl_name}",
        "#", "# commands (from the repository root):"] + cmds + [
        "",
        f"gate/up kernel average (profiler, all {len(ups)} dispatches): {all_ms:.4f} ms",
        f"gate/up kernel average (profiler, the {len(timed)} dispatches of the timed steps): {timed_ms:.4f} ms",
        f"gate/up kernel average (bench.py HIP events, timed steps of the same run): {ev_ms:.4f} ms",
        f"agreement (same dispatches): {100 * (ev_ms - timed_ms) / timed_ms:+.1f} %",
        f"roofline of the traced run: {line['roofline']['achieved']} TFLOP/s, frac "
        f"{line['roofline']['frac']} of {line['roofline']['peak']} TFLOP/s",
        "",
        "## HBM bytes (--pmc), gate/up kernel, per dispatch",
        f"FETCH_SIZE: {fetch[up_key] / 1e6:.1f} MB, WRITE_SIZE: {write[up_key] / 1e6:.1f} MB (copy-calibrated)",
        f"algorithmic operand bytes (A rows + weights once): {alg_up / 1e6:.1f} MB; fetch / algorithmic = "
        f"{fetch[up_key] / alg_up:.2f}",
        f"traffic_bytes_per_launch: {traffic}",
        f"kernel_sources_sha256: {kernel_sources_sha256()}",
    ]
    path = profile_path(wl_name)
    with open(path, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    written.append(path)
    # ---- optional counter sets over the expert GEMM stages
    sets = sorted(x for x in os.listdir(d) if x.startswith("ctr_p") and os.path.isdir(os.path.join(d, x)))
    if sets:
        acc = {}
        for sub in sets:
            for r in _csv(os.path.join(d, sub, f"{sub}_counter_collection.csv")):
                kk = name_col(r)
                if kk and kk.startswith("k_expert_stage"):
                    acc.setdefault((kk, r["Counter_Name"]), []).append(float(r["Counter_Value"]))
        lines = [f"# expert GEMM stages, workload {wl_name}: hardware counters, mean per dispatch",
                 "#", "# commands (from the repository root; one run per counter set):",
                 f"#   rocprofv3 --pmc <set> --kernel-include-regex k_expert_stage -d {D}/ctr_pN -o "
                 f"ctr_pN --output-format csv -- python3 bench.py --steps 2 --warmup 1 --no-cpu {cmd}",
                 f"#   python3 bench.py --summarize {D}", ""]
        for kk in sorted({a for a, _ in acc}):
            m = {c: sum(v) / len(v) for (a, c), v in acc.items() if a == kk}
            lines.append(kk)
            lines += [f"  {c:<36} {m[c]:>12.4g}" for c in sorted(m)]
            if "SQ_CYCLES" in m:
                cyc = m["SQ_CYCLES"] / 32
                der = []
                if "SQ_VALU_MFMA_BUSY_CYCLES" in m:
                    der.append(("MFMA busy (of 1024 SIMDs x kernel cycles)",
                                m["SQ_VALU_MFMA_BUSY_CYCLES"] / (1024 * cyc)))
                if "TCC_HIT_sum" in m and "TCC_MISS_sum" in m:
                    der.append(("L2 hit rate", m["TCC_HIT_sum"] / (m["TCC_HIT_sum"] + m["TCC_MISS_sum"])))
                if "TCP_TCC_READ_REQ_LATENCY_sum" in m and "TCP_TCC_READ_REQ_sum" in m:
                    der.append(("L2 read latency seen by the L1 (cycles)",
                                m["TCP_TCC_READ_REQ_LATENCY_sum"] / m["TCP_TCC_READ_REQ_sum"]))
                if "TCP_PENDING_STALL_CYCLES_sum" in m:
                    der.append(("L1 stalled on pending L2 data", m["TCP_PENDING_STALL_CYCLES_sum"] / (256 * cyc)))
                if "SQ_LDS_BANK_CONFLICT" in m and "SQ_ACTIVE_INST_LDS" in m:
                    der.append(("LDS bank-conflict cycles / LDS-active cycles",
                                m["SQ_LDS_BANK_CONFLICT"] / m["SQ_ACTIVE_INST_LDS"]))
                if "SQ_WAIT_INST_ANY" in m and "SQ_WAVE_CYCLES" in m:
                    der.append(("waves waiting on a dependency", m["SQ_WAIT_INST_ANY"] / m["SQ_WAVE_CYCLES"]))
                lines.append(f"  derived (kernel cycles = SQ_CYCLES / 32 = {cyc:.3g}):")
                lines += [f"    {a:<48} {v:.3g}" for a, v in der]
        path = os.path.join(ROOT, "profiles", f"expert_gemm_counters_{wl_name}.txt")
        with open(path, "w") as fh:
            fh.write("\n".join(lines) + "\n")
        written.append(path)
    return written


def summarize_backward(d: str, line: dict) -> str:
    """profiles/kernels_backward_<wl>.txt: every kernel of one mok_moe_backward (per backward:
    the run's totals over its k_bwd_describe launches), the grouped GEMMs against the bf16 peak."""
    import synth
    wl = synth.WORKLOADS[line["workload"]]
    n = line["routed_rows"]
    I_sh = wl.n_shared * wl.I_shared
    per_row = lambda c: c * wl.d * wl.I * n + c * wl.d * I_sh * wl.T_own
    gemm = {"k_ggemm<false, false, true>": ("recompute G, U; SwiGLU backward in the epilogue",
                                            per_row(4.0)),
            "k_ggemm<false, true, false>": ("dgrad: D = dP Wd; dx = [dG dU] [Wg; Wu] (bf16 rows)",
                                            per_row(6.0)),
            "k_ggemm<true, true, false>": ("wgrad: dWg, dWu, dWd (ragged K)", per_row(6.0))}
    trace = _csv(os.path.join(d, "trace", "trace_kernel_trace.csv"))
    key = lambda r: kernel_key(r["Kernel_Name"])
    dur = lambda r: (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-6   # ms
    tot, cnt = {}, {}
    for r in trace:
        k = key(r)
        if k is not None:
            tot[k] = tot.get(k, 0.0) + dur(r)
            cnt[k] = cnt.get(k, 0) + 1
    n_bwd = cnt.get("k_bwd_describe", 1)             # one per backward
    t_b = {k: v / n_bwd for k, v in tot.items()}
    calls = {k: v / n_bwd for k, v in cnt.items()}
    D = "gpurun_out/prof_backward"
    lines = [f"# every libmok kernel of one mok_moe_backward, workload {wl.name} (bf16), per backward",
             "#", "# commands (from the repository root):",
             f"#   rocprofv3 --kernel-trace --stats -d {D}/trace -o trace --output-format csv -- "
             f"python3 bench.py --backward --steps 10 --warmup 3 > {D}/trace.json",
             f"#   python3 bench.py --summarize {D}",
             "#",
             "# time: kernel durations from the trace, summed per backward over the run (the bench's",
             "#   forward, run once to get the routing, is listed apart); grouped GEMMs: algorithmic",
             "#   FLOPs (16 d I per routed row, 16 d I_s n_s per own token in all) / time against",
             "#   the 2.5 PFLOP/s dense bf16 peak.",
             "",
             f"{'kernel':<40} {'calls':>5} {'time_us':>9} {'TFLOP/s':>9} {'of_peak':>8}  product"]
    total = 0.0
    outside = []
    for k in sorted(t_b, key=lambda k: -t_b[k]):
        if calls[k] < 0.5:
            outside.append(k)
            continue
        t = t_b[k]
        total += t
        row = f"{k:<40} {calls[k]:>5.1f} {t * 1e3:>9.1f}"
        if k in gemm:
            what, f = gemm[k]
            row += f" {f / (t * 1e-3) / 1e12:>9.1f} {f / (t * 1e-3) / PEAK['bf16']:>8.3f}  {what}"
        lines.append(row)
    if outside:
        lines.append(f"(launched once per run, not per backward: {', '.join(outside)})")
    lines += ["", f"kernel time per backward: {total:.3f} ms; bench line of the traced run: "
              f"{line['ms']} ms per backward, {line['achieved_tflops']} TFLOP/s, frac "
              f"{line['frac']}, routed rows {n}"]
    path = os.path.join(ROOT, "profiles", f"kernels_backward_{wl.name}.txt")
    with open(path, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    return path


def summarize_dispatch(d: str, line: dict) -> str:
    """profiles/kernels_dispatch_<wl>.txt: the pull gather and the push baseline (and the plan
    the pull needs), per step, with copy-calibrated counter bytes."""
    import synth
    wl = synth.WORKLOADS[line["workload"]]
    n, row = line["routed_rows"], line["row_bytes"]
    name_col = lambda r: kernel_key(r["Kernel_Name"])
    trace = _csv(os.path.join(d, "trace", "trace_kernel_trace.csv"))
    dur = lambda r: (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-6
    t_step, calls = _per_forward(trace, name_col, dur)

    def counter(sub, pred=None):
        rows = _csv(os.path.join(d, sub, f"{sub}_counter_collection.csv"))
        if pred is not None:
            vals = [float(r["Counter_Value"]) for r in rows if pred(r["Kernel_Name"])]
            return sum(vals) / len(vals)
        return _per_forward(rows, name_col, lambda r: float(r["Counter_Value"]))[0]

    copy_fetch = counter("copy_FETCH_SIZE", lambda n_: "copyBuffer" in n_)
    copy_write = counter("copy_WRITE_SIZE", lambda n_: "copyBuffer" in n_)
    f_fetch, f_write = (1 << 20) / copy_fetch, (1 << 20) / copy_write
    fetch = {k: v * f_fetch * 1024 for k, v in counter("FETCH_SIZE").items()}
    write = {k: v * f_write * 1024 for k, v in counter("WRITE_SIZE").items()}
    routes = wl.T_pool * wl.k
    alg = {"k_pull_gather": 2 * n * row + 4 * n, "k_push_dispatch": 2 * n * row + 4 * routes + 4 * n,
           "k_plan_count": 4 * routes, "k_plan_scatter": 4 * routes + 4 * n}
    D = f"gpurun_out/prof_dispatch"
    lines = [f"# pull gather against the push-dispatch baseline, {wl.name} routing "
             f"({n} local routes of {routes}, rows of {row} B), per step",
             "#", "# commands (from the repository root):",
             f"#   rocprofv3 --kernel-trace --stats -d {D}/trace -o trace --output-format csv -- "
             f"python3 bench.py --dispatch --steps 10 --warmup 3 > {D}/trace.json",
             f"#   rocprofv3 --pmc FETCH_SIZE --kernel-include-regex 'mok::' -d {D}/FETCH_SIZE -o "
             f"FETCH_SIZE --output-format csv -- python3 bench.py --dispatch --steps 2 --warmup 1",
             f"#   rocprofv3 --pmc WRITE_SIZE --kernel-include-regex 'mok::' -d {D}/WRITE_SIZE -o "
             f"WRITE_SIZE --output-format csv -- python3 bench.py --dispatch --steps 2 --warmup 1",
             f"#   (copy calibration: the copy-probe passes of the layer profiles, copied here)",
             f"#   python3 bench.py --summarize {D}", "#",
             f"# calibration: 1 GiB copy reads FETCH_SIZE {copy_fetch:.0f} KiB, WRITE_SIZE "
             f"{copy_write:.0f} KiB (factors {f_fetch:.4f}, {f_write:.4f})",
             "# alg: row bytes read + written once and the index bytes each kernel must touch", "",
             f"{'kernel':<20} {'calls':>5} {'time_us':>9} {'fetch_MB':>9} {'write_MB':>9} "
             f"{'alg_MB':>9} {'alg_GB/s':>9} {'counter_GB/s':>12} {'of_8TB/s':>9}"]
    for k in sorted(t_step, key=lambda k: -t_step[k]):
        if k not in alg and not k.startswith("k_plan"):
            continue
        t = t_step[k]
        fb, wb = fetch.get(k, 0.0), write.get(k, 0.0)
        row_s = f"{k:<20} {calls[k]:>5.1f} {t * 1e3:>9.1f} {fb / 1e6:>9.1f} {wb / 1e6:>9.1f} "
        if k in alg:
            a = alg[k]
            row_s += (f"{a / 1e6:>9.1f} {a / (t * 1e-3) / 1e9:>9.0f} {(fb + wb) / (t * 1e-3) / 1e9:>12.0f} "
                      f"{a / (t * 1e-3) / HBM_PEAK:>9.3f}")
        else:
            row_s += f"{'-':>9} {'-':>9} {(fb + wb) / (t * 1e-3) / 1e9:>12.0f} {'-':>9}"
        lines.append(row_s)
    lines += ["", "bench line of the traced run (cold-cache HIP-event times): "
              f"pull_gather {line['pull_gather']}, push_dispatch {line['push_dispatch']}, "
              f"plan {line['plan']}; push slot order identical in two runs: "
              f"{line['push_slot_order_same_in_two_runs']}"]
    path = os.path.join(ROOT, "profiles", f"kernels_dispatch_{wl.name}.txt")
    with open(path, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    return path


# ------------------------------------------------------------------ measurement

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
        self.ev = (ctypes.c_void_p * n)()
        for i in range(n):
            h = ctypes.c_void_p()
            assert self.hip.hipEventCreateWithFlags(ctypes.byref(h), self.DISABLE_SYSTEM_FENCE) == 0
            self.ev[i] = h

    def elapsed_ms(self, a: int, b: int) -> float:
        out = ctypes.c_float(0)
        assert self.hip.hipEventElapsedTime(ctypes.byref(out), self.ev[a], self.ev[b]) == 0
        return out.value


def algorithmic_work(wl, n_routes: int) -> dict:
    I_sh = wl.n_shared * wl.I_shared
    up = 4.0 * wl.d * wl.I * n_routes + 4.0 * wl.d * I_sh * wl.T_own
    down = 2.0 * wl.d * wl.I * n_routes + 2.0 * wl.d * I_sh * wl.T_own
    return dict(routed_flop=6.0 * wl.d * wl.I * n_routes, shared_flop=6.0 * wl.d * I_sh * wl.T_own,
                up_flop=up, down_flop=down)


def hbm_stages(wl, n_routes: int, stage_ms: dict, ring: bool) -> dict:
    """Achieved HBM rate of the memory-bound stages (cold-cache stage times): algorithmic bytes
    (each operand read once, each result written once) over the stage's HIP-event time, against
    8 TB/s.
      plan:    the top-k indices (4 B per route of the pool) read, the local route ids
               (4 B per local route) written;
      combine: per token the shared row and the k route rows read, y written (full layer);
      quant:   every bf16 weight element read (2 B), its E4M3 code and 1/32 of a scale byte
               written (MXFP8);
      gather:  per routed row and own token the bf16 x row read, its codes and scales written
               (MXFP8, stage-ordered; the stage also holds the device work-list build)."""
    eb = 4 if wl.dtype == "fp32" else 2
    routes_pool = wl.T_pool * wl.k
    I_sh = wl.n_shared * wl.I_shared
    bytes_ = {"plan": 4 * routes_pool + 4 * n_routes}
    if wl.full_layer:
        bytes_["combine"] = wl.T_pool * wl.d * eb * (wl.k + 2)
    if wl.dtype in ("mxfp8", "mxfp4"):
        cb = 0.5 if wl.dtype == "mxfp4" else 1.0      # code bytes per element
        n_w = wl.E_l * 3 * wl.d * wl.I + 3 * wl.d * I_sh
        bytes_["quant"] = n_w * (2 + cb + 1 / 32)
        if not ring:
            bytes_["gather"] = (n_routes + wl.T_own) * wl.d * (2 + cb + 1 / 32)
    out = {}
    for name, b in bytes_.items():
        t = stage_ms[name] * 1e-3
        if t <= 0:
            continue
        gbs = b / t / 1e9
        out[name] = {"bytes": int(b), "ms": round(stage_ms[name], 4), "achieved": round(gbs, 1),
                     "unit": "GB/s", "frac": round(gbs * 1e9 / HBM_PEAK, 4)}
    return out


def _cpu_info() -> tuple:
    model = "unknown"
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                model = ln.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    try:
        from threadpoolctl import threadpool_info
        blas = [p["num_threads"] for p in threadpool_info() if p.get("user_api") == "blas"]
        if blas:
            threads = max(threads, max(blas))
    except Exception:
        pass
    return model, threads


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
    model, threads = _cpu_info()
    return {"value": sample_tokens / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "cpu": model,
            "sample": f"first {sample_tokens} of {wl.T_pool} tokens, whole forward (routing "
                      f"(C), plan (C), float64 numpy expert and shared FFNs, combine); {dt:.1f} s"}


def measure(wl, mode: str, steps: int, warmup: int, minibatch=None, dev="cuda:0") -> dict:
    """Time `steps` forwards of workload wl after `warmup` (wall clock between device
    synchronisations; HIP events on the roofline kernel only), then a cold-cache per-stage pass.
    mode: "stage" (two stage launches), "ring" (the ring work loop) or "loop" (the stage order
    in one persistent launch). Returns the JSON fields of one measurement and the inputs (for
    the CPU baseline)."""
    import torch
    import routing_grouped_expert_gemm_amd as mok
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from _layer import gpu_layer, gpu_topk, make_inputs

    inp = make_inputs(wl, dev)
    topk = gpu_topk(inp["logits"], wl.k) if wl.routing == "logits" else None
    ring = mode == "ring"
    flags = {"stage": mok.MOK_FLAG_NO_RING, "ring": 0, "loop": mok.MOK_FLAG_STAGE_LOOP}[mode]
    layer = gpu_layer(wl, inp, topk=topk, flags=flags, mb=minibatch, keep=True)
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

    for _ in range(warmup):
        step()
    # timed steps: events only on the roofline launch; the library ties them to that kernel's
    # dispatch, so they queue no marker on the stream
    ev_up = HipEvents(2 * steps)
    up_tables = event_table(ev_up, True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(up_tables[i])
    torch.cuda.synchronize()
    ms = 1e3 * (time.perf_counter() - t0) / steps
    assert layer.device_error(stream) == 0
    up_ms = sum(ev_up.elapsed_ms(2 * i, 2 * i + 1) for i in range(steps)) / steps
    # per-stage times: a separate, untimed pass with every stage event, each step after a 1 GiB
    # scratch read (nothing of the previous step stays in the caches)
    n_stage = min(steps, 10)
    ev_all = HipEvents(n2 * n_stage)
    all_tables = event_table(ev_all, False)
    scratch = cache_scratch(dev)
    for i in range(n_stage):
        evict_caches(scratch)
        step(all_tables[i])
    torch.cuda.synchronize()
    del scratch

    n_routes = int(layer.inter["offsets"][-1])
    work = algorithmic_work(wl, n_routes)
    stage_ms = {}
    names = ["route", "plan", "quant", "up", "down", "combine", "gather"]
    assert len(names) == mok.MOK_N_STAGES
    for s_, name in enumerate(names):
        vals = [ev_all.elapsed_ms(n2 * i + 2 * s_, n2 * i + 2 * s_ + 1) for i in range(n_stage)]
        stage_ms[name] = sum(vals) / len(vals)
    stage_ms["up_cold"] = stage_ms["up"]
    stage_ms["up"] = up_ms                      # the timed steps' own measurement
    peak = PEAK[wl.dtype]
    if mode != "stage":
        # one persistent launch runs the gate/up and the down tiles (and, in the ring, the MX
        # row gather)
        roof_flop = work["up_flop"] + work["down_flop"]
        kernel = ("ring work loop (k_ring: gate/up and down tiles of every minibatch)" if ring
                  else "stage order in one persistent launch (k_ring over the stage tables)")
        gemm_s = up_ms * 1e-3
    else:
        roof_flop = work["up_flop"]
        kernel = "gate/up stage (k_expert_stage up)"
        gemm_s = (up_ms + stage_ms["down"]) * 1e-3
    achieved = roof_flop / (up_ms * 1e-3)
    tokens = wl.T_pool if wl.full_layer else wl.T_own
    res = {
        "value": round(tokens / (ms * 1e-3), 1), "unit": "tokens/s", "steps": steps,
        "warmup": warmup, "ms_per_step": round(ms, 4),
        "dtype": {"bf16": "bf16", "mxfp8": "mxfp8", "mxfp4": "mxfp4", "fp32": "f32"}[wl.dtype],
        "config": {"workload": wl.name, "T_pool": wl.T_pool, "T_own": wl.T_own, "d": wl.d,
                   "E": wl.E, "k": wl.k, "I": wl.I, "E_local": wl.E_l, "n_shared": wl.n_shared,
                   "I_shared": wl.I_shared, "minibatch_rows": layer.args.minibatch_rows,
                   "ring_rows": layer.args.ring_rows if ring else None,
                   "work_loop": {"stage": "stage-ordered", "ring": "ring",
                                 "loop": "stage-ordered, one persistent launch"}[mode]},
        "routed_rows": n_routes,
        "routed_tflops": round(work["routed_flop"] / (ms * 1e-3) / 1e12, 2),
        "gemm_tflops": round((work["routed_flop"] + work["shared_flop"]) / gemm_s / 1e12, 2),
        "stage_ms": {k: round(v, 4) for k, v in stage_ms.items()},
        "roofline": {"bound": "mfma", "kernel": kernel, "achieved": round(achieved / 1e12, 2),
                     "peak": peak / 1e12, "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                     "traffic": profiled_traffic(wl.name) if mode == "stage" else None},
        "hbm": hbm_stages(wl, n_routes, stage_ms, ring),
    }
    del layer
    return res, inp


def measure_dispatch(steps: int, warmup: int, dev="cuda:0") -> dict:
    """Pull (plan + gather in plan order) against push (atomic-slot scatter) on the EP=64 share's
    routing: 262144 pool rows of d = 7168 bf16, top-8 of 256 experts, 4 local experts. Both
    move the same rows into expert-contiguous buffers; times are HIP events on the stream,
    averaged over `steps` after `warmup`, each step after a 1 GiB scratch read."""
    import torch
    import routing_grouped_expert_gemm_amd as mok
    import synth
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from _layer import gpu_topk
    wl = synth.WORKLOADS[synth.EP64]
    T, d, k, E_l = wl.T_pool, wl.d, wl.k, wl.E_l
    x = synth.x_rows(wl, range(T), dev)
    idx, _ = gpu_topk(synth.pool_logits_rows(wl, range(T), dev), k)
    i32 = dict(dtype=torch.int32, device=dev)
    counts, offsets = torch.empty(E_l, **i32), torch.empty(E_l + 1, **i32)
    rank_counts = torch.empty((E_l, wl.n_ranks), **i32)
    route_ids = torch.empty(T * min(k, E_l), **i32)
    ws = torch.empty(mok.mok_dispatch_plan_workspace_bytes(T, k, E_l), dtype=torch.uint8, device=dev)
    pull_buf = torch.empty((T * min(k, E_l), d), dtype=x.dtype, device=dev)
    cap = T                                   # a token picks an expert at most once: no drops
    fill = torch.empty(E_l, **i32)
    push_buf = torch.empty((E_l, cap, d), dtype=x.dtype, device=dev)
    src = torch.empty((E_l, cap), **i32)
    scratch = cache_scratch(dev)

    def plan():
        mok.mok_dispatch_plan(idx, wl.E, wl.e0, E_l, wl.tokens_per_rank, counts, offsets,
                              rank_counts, route_ids, ws)

    ev = lambda: torch.cuda.Event(enable_timing=True)
    t = {"plan": 0.0, "pull_gather": 0.0, "push_dispatch": 0.0}
    orders = []
    for i in range(warmup + steps):
        e = [ev() for _ in range(6)]
        evict_caches(scratch)
        e[0].record(); plan(); e[1].record()
        evict_caches(scratch)
        e[2].record(); mok.mok_pull_gather(x, k, route_ids, offsets, pull_buf); e[3].record()
        evict_caches(scratch)
        e[4].record(); mok.mok_push_dispatch(x, idx, wl.e0, fill, push_buf, src); e[5].record()
        torch.cuda.synchronize()
        if i >= warmup:
            t["plan"] += e[0].elapsed_time(e[1]) / steps
            t["pull_gather"] += e[2].elapsed_time(e[3]) / steps
            t["push_dispatch"] += e[4].elapsed_time(e[5]) / steps
        if i >= warmup + steps - 2:
            orders.append(src[0, :int(fill[0])].clone())
    n = int(offsets[-1])
    assert torch.equal(fill.cpu(), counts.cpu())
    row = d * x.element_size()
    moved = 2 * n * row                       # every local route's row read once, written once
    same = bool(torch.equal(orders[0], orders[1]))
    res = {"workload": wl.name, "routed_rows": n, "row_bytes": row,
           "rows_bytes_moved": moved, "unit": "GB/s"}
    for name, ms in t.items():
        res[name] = {"ms": round(ms, 4)}
    for name in ("pull_gather", "push_dispatch"):
        gbs = moved / (t[name] * 1e-3) / 1e9
        res[name].update(achieved=round(gbs, 1), frac=round(gbs * 1e9 / HBM_PEAK, 4))
    pull_total = t["plan"] + t["pull_gather"]
    res["pull_with_plan"] = {"ms": round(pull_total, 4),
                             "achieved": round(moved / (pull_total * 1e-3) / 1e9, 1)}
    res["push_over_pull_time"] = round(t["push_dispatch"] / t["pull_gather"], 3)
    res["push_slot_order_same_in_two_runs"] = same
    return res


def measure_backward(steps: int, warmup: int, dev="cuda:0") -> dict:
    """Backward of the EP=1 bf16 layer (mok_moe_backward) with the forward's routing, HIP-event
    time per step (each step after a 1 GiB scratch read). Its GEMMs execute 16*d*I FLOPs per
    routed row (gate/up recompute 4, dgrad 6, wgrad 6) and 16*d*I_s*n_s per own token."""
    import torch
    import routing_grouped_expert_gemm_amd as mok
    import synth
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from _layer import gpu_layer, make_inputs
    wl = synth.WORKLOADS[synth.EP1]
    inp = make_inputs(wl, dev)
    fwd = gpu_layer(wl, inp, flags=mok.MOK_FLAG_NO_RING, keep=True)
    fwd.forward()
    dy = synth.normal_rows(0, 21, wl.d, range(wl.T_pool), 1.0, torch.bfloat16, dev)
    b = mok.MoeBackward(d=wl.d, E=wl.E, k=wl.k, I=wl.I, e0=wl.e0, E_l=wl.E_l,
                        tokens_per_rank=wl.tokens_per_rank, T_pool=wl.T_pool, own_begin=0,
                        T_own=wl.T_own, n_shared=wl.n_shared, I_shared=wl.I_shared, x=inp["x"],
                        topk_idx=fwd.inter["topk_idx"], topk_w=fwd.inter["topk_w"],
                        w_gate=inp["wg"], w_up=inp["wu"], w_down=inp["wd"], ws_gate=inp["sg"],
                        ws_up=inp["su"], ws_down=inp["sd"], dy=dy, device=dev)
    scratch = cache_scratch(dev)
    t = 0.0
    for i in range(warmup + steps):
        evict_caches(scratch)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        b.backward()
        e1.record()
        torch.cuda.synchronize()
        if i >= warmup:
            t += e0.elapsed_time(e1) / steps
    assert b.device_error() == 0
    n = int(fwd.inter["offsets"][-1])
    I_sh = wl.n_shared * wl.I_shared
    flop = 16.0 * wl.d * wl.I * n + 16.0 * wl.d * I_sh * wl.T_own
    ach = flop / (t * 1e-3)
    return {"workload": wl.name, "ms": round(t, 4), "tokens_per_s": round(wl.T_pool / (t * 1e-3), 1),
            "routed_rows": n,
            "gemm_flop": flop, "achieved_tflops": round(ach / 1e12, 2), "peak_tflops": 2500.0,
            "frac": round(ach / PEAK["bf16"], 4),
            "note": "cold-cache HIP-event time of one mok_moe_backward (plan, describe, 4 grouped "
                    "GEMM launches with the SwiGLU backward fused into the recompute, topk-weight "
                    "gradients, combine)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=None,
                    help="measure this workload alone (default: the headline and its extras)")
    ap.add_argument("--ring", action="store_true", help="persistent ring work loop")
    ap.add_argument("--stage-loop", action="store_true",
                    help="the stage order in one persistent launch")
    ap.add_argument("--minibatch", type=int, default=None)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--cpu-sample", type=int, default=8192)
    ap.add_argument("--summarize", default=None, metavar="DIR",
                    help="write the profiles/ summaries from a rocprofv3 output directory and exit")
    ap.add_argument("--dispatch", action="store_true",
                    help="only the pull-versus-push dispatch comparison (one JSON line)")
    ap.add_argument("--backward", action="store_true",
                    help="only the backward of the EP=1 layer (one JSON line)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (calibrates the HBM "
                         "byte counters of a profiler run) and exit")
    args = ap.parse_args()
    if args.summarize:
        for p_ in summarize(args.summarize):
            print(p_)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): this build has no "
              "multi-GPU path; the sharding plan is design only", file=sys.stderr)
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

    import synth
    torch.cuda.set_device(0)
    if args.backward:
        print(json.dumps({"mode": "backward", "steps": args.steps, "warmup": args.warmup,
                          **measure_backward(args.steps, args.warmup)}))
        return
    if args.dispatch:
        print(json.dumps({"mode": "dispatch", "steps": args.steps, "warmup": args.warmup,
                          **measure_dispatch(args.steps, args.warmup)}))
        return
    name = args.workload or synth.EP1
    wl = synth.WORKLOADS[name]
    mode = "ring" if args.ring else "loop" if args.stage_loop else "stage"
    res, inp = measure(wl, mode, args.steps, args.warmup, args.minibatch)
    out = {"metric": METRIC, "value": res["value"], "unit": "tokens/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": res["ms_per_step"],
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": res["dtype"],
           "data": "synthetic (seeded counter-based generator; random-init weights)",
           "config": res["config"]}
    for k in ("routed_rows", "routed_tflops", "gemm_tflops", "stage_ms", "roofline", "hbm"):
        out[k] = res[k]
    cpu_inp = None
    if not args.no_cpu:
        cpu_inp = {k: (v.cpu() if v is not None else None) for k, v in inp.items()}
    del inp
    if args.workload is None:
        torch.cuda.empty_cache()
        # the same layer with the persistent ring work loop (the library default)
        r, i2 = measure(wl, "ring", args.steps, args.warmup, args.minibatch)
        del i2
        out["ring"] = {k: r[k] for k in ("value", "ms_per_step", "routed_tflops", "config",
                                         "stage_ms", "roofline")}
        torch.cuda.empty_cache()
        # ... and with the stage order in one persistent launch
        r, i2 = measure(wl, "loop", args.steps, args.warmup, args.minibatch)
        del i2
        out["stage_loop"] = {k: r[k] for k in ("value", "ms_per_step", "routed_tflops", "config",
                                               "stage_ms", "roofline")}
        torch.cuda.empty_cache()
        # the MXFP8 share
        m, i3 = measure(synth.WORKLOADS[synth.EP64_MX], "stage", args.steps, args.warmup)
        del i3
        torch.cuda.empty_cache()
        out["mxfp8"] = {k: m[k] for k in ("value", "unit", "ms_per_step", "dtype", "config",
                                          "routed_rows", "routed_tflops", "gemm_tflops",
                                          "stage_ms", "roofline", "hbm")}
        # ... and with the ring work loop (gather items inside the loop)
        mr, i3 = measure(synth.WORKLOADS[synth.EP64_MX], "ring", args.steps, args.warmup)
        del i3
        torch.cuda.empty_cache()
        out["mxfp8"]["ring"] = {k: mr[k] for k in ("value", "ms_per_step", "routed_tflops",
                                                   "config", "roofline")}
        # the same share with MXFP4 operands
        m4, i4 = measure(synth.WORKLOADS[synth.EP64_MX4], "stage", args.steps, args.warmup)
        del i4
        torch.cuda.empty_cache()
        out["mxfp4"] = {k: m4[k] for k in ("value", "unit", "ms_per_step", "dtype", "config",
                                           "routed_rows", "routed_tflops", "gemm_tflops",
                                           "stage_ms", "roofline", "hbm")}
        m4r, i4 = measure(synth.WORKLOADS[synth.EP64_MX4], "ring", args.steps, args.warmup)
        del i4
        torch.cuda.empty_cache()
        out["mxfp4"]["ring"] = {k: m4r[k] for k in ("value", "ms_per_step", "routed_tflops",
                                                    "config", "roofline")}
        # the backward of the headline layer
        out["backward"] = measure_backward(min(args.steps, 10), min(args.warmup, 3))
        torch.cuda.empty_cache()
        # pull gather against the push baseline on the EP=64 share's routing
        out["dispatch"] = measure_dispatch(min(args.steps, 10), min(args.warmup, 3))
        torch.cuda.empty_cache()
    if cpu_inp is not None:
        out["cpu_baseline"] = cpu_baseline(wl, cpu_inp, min(args.cpu_sample, wl.T_pool))
    print(json.dumps(out))


if __name__ == "__main__":
    main()
