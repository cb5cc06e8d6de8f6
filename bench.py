#!/usr/bin/env python3
"""Benchmark of the SSD chunked forward (libssd) on one MI355X.

    python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--config 2] [--variant auto]

One step is one full forward (every kernel of the path) over the workload's synthetic inputs,
which are resident in HBM before timing starts. Before every step a read-only sweep over 2 GiB of
clean memory leaves no input in the 256 MB Infinity Cache or the L2s (cold-cache timing). Two
timed passes of K steps each, bracketed by device synchronisations: the first times each whole
forward with HIP events on its stream (the reported ms per step and tokens/s), the second also
records events around every kernel inside the forward (per-kernel durations; the roofline).

Prints ONE JSON line: tokens/s (mean and median step), ms per step, the whole forward's roofline
(its algorithmic bytes over its measured time, against MI355X's 8 TB/s; `roofline`), the dominant
kernel's (its algorithmic bytes per launch over its measured duration;
`dominant_kernel_roofline`), per-kernel times, the other bf16 workloads' cold-cache times and
roofline fractions (`workloads`), run metadata (`run`: ROCm, compiler, GPU, clocks, revision,
CPU), and the CPU oracle's throughput on the same workload (with the parity of the GPU result on
the units the oracle computed).

    python bench.py --summarize-profiles DIR

turns rocprofv3 output under DIR (a kernel-trace run, one FETCH_SIZE and one WRITE_SIZE counter
run with --copy-calibration, two SQ counter runs, plus DIR/bench.json from a plain bench run)
into the text summaries under profiles/ and the traffic record the bench line reports; see
PROFILE_COMMANDS.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_F16_PEAK_TFLOPS = 2516.6  # dense fp16/bf16 matrix cores
FP32_PEAK_TFLOPS = 157.3
METRIC = "SSD fwd tokens/s + % of MI355X HBM/MFMA roofline, L=8K H=80 P=64 N=128"


def algorithmic(shape, with_initial_state: bool):
    """Algorithmic bytes and flops of one forward (what the method must move and compute).

    bytes/token = H P (s_x + s_y) + 2 G N s_io + 4 H  (+ states in/out: 4 H P N per batch)
    flops/token = G (Q+1) N [C B^T, causal] + H (Q+1) P [masked intra product]
                  + 2 H P N [chunk state] + 2 H P N [inter readout] + 2 H P N / Q [passing]
    Returns per-token stream bytes, whole-forward bytes, and flops.
    """
    s_io = 2 if shape.io == "bf16" else 4
    H, P, N, G, Q = shape.nheads, shape.headdim, shape.dstate, shape.ngroups, shape.chunk_size
    tokens = shape.batch * shape.seqlen
    stream_per_token = H * P * 2 * s_io + 2 * G * N * s_io + 4 * H
    states = shape.batch * H * P * N * 4 * (2 if with_initial_state else 1)
    flops_per_token = G * (Q + 1) * N + H * (Q + 1) * P + 4 * H * P * N + 2 * H * P * N / Q
    return {
        "stream_bytes_per_token": stream_per_token,
        "bytes": stream_per_token * tokens + states,
        "flops": flops_per_token * tokens,
        "tokens": tokens,
    }


# Sources that define, plan or launch the fused forward's kernels (the traffic counters describe
# these; the unfused kernels and the decode step do not change them).
FUSED_SOURCES = ("ssd_api.cpp", "ssd_device.h", "ssd_fused.hip", "ssd_launch.h")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "mamba_ssd_chunked_cumsum_amd", "csrc")
    for name in FUSED_SOURCES:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, kernels) -> float | None:
    """L2-to-memory bytes per launch, summed over `kernels`, from committed counter runs taken on
    these sources (None if there are none, or a kernel is missing from them). FETCH_SIZE and
    WRITE_SIZE count what the L2s exchange with the memory side, part of which the Infinity Cache
    may serve: an upper bound on HBM bytes."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_hash") != kernel_source_hash():
        return None
    per = rec.get("kernels", {})
    if any(k not in per for k in kernels):
        return None
    return float(sum(per[k]["fetch_bytes"] + per[k]["write_bytes"] for k in kernels))


def cpu_baseline(inp, shape, y_gpu, f_gpu, max_seconds: float):
    """The C oracle (float64 recurrence, OpenMP over heads) timed on the host cores, on the whole
    workload or, when that would exceed max_seconds, on a spread sample of (batch, head) units.
    Also scores the GPU output on the units computed."""
    import numpy as np
    from oracle import metrics, native

    n_units = shape.batch * shape.nheads
    per_unit_probe = max(1, min(n_units, 4))
    probe = list(range(per_unit_probe))
    t = time.perf_counter()
    native.forward(**inp, units=probe)
    t_probe = (time.perf_counter() - t) / per_unit_probe
    k = n_units if t_probe * n_units <= max_seconds else max(8, int(max_seconds / t_probe))
    k = min(k, n_units)
    units = list(range(n_units)) if k == n_units else sorted(
        set(int(round(i * (n_units - 1) / (k - 1))) for i in range(k)))
    threads = native.max_threads()
    t = time.perf_counter()
    y_ref, f_ref = native.forward(**inp, units=units)
    elapsed = time.perf_counter() - t
    tokens_per_s = shape.seqlen * len(units) / shape.nheads / elapsed
    bs = [u // shape.nheads for u in units]
    hs = [u % shape.nheads for u in units]
    yg = np.stack([y_gpu[b, :, h] for b, h in zip(bs, hs)])
    yr = np.stack([y_ref[b, :, h] for b, h in zip(bs, hs)])
    fg = np.stack([f_gpu[b, h] for b, h in zip(bs, hs)])
    fr = np.stack([f_ref[b, h] for b, h in zip(bs, hs)])
    rep = metrics.parity_report(yg, yr, fg, fr, shape.io)
    sample = ("whole workload" if len(units) == n_units else
              f"{len(units)} of {n_units} (batch, head) units, all {shape.seqlen} tokens each")
    return {
        "value": tokens_per_s, "unit": "tokens/s", "cores": threads, "kind": "oracle",
        "sample": f"{sample}; float64 C recurrence, {elapsed:.2f} s",
    }, rep


SQ_PASSES = {
    "sq1": "SQ_WAVES SQ_INSTS_VALU SQ_INSTS_MFMA SQ_INSTS_SALU SQ_INSTS_LDS SQ_INSTS_VMEM "
           "SQ_WAVE_CYCLES SQ_BUSY_CYCLES GRBM_GUI_ACTIVE",
    "sq2": "SQ_VALU_MFMA_BUSY_CYCLES SQ_ACTIVE_INST_VALU SQ_WAIT_INST_ANY SQ_WAIT_ANY "
           "SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE SQ_ACTIVE_INST_LDS SQ_INSTS_VALU_MFMA_MOPS_F16 "
           "GRBM_GUI_ACTIVE",
}


def profile_commands(cfg: int = 2) -> list:
    """The commands whose output --summarize-profiles reads, for workload index cfg (the headline
    workload's commands carry no --config)."""
    c = "" if cfg == 2 else f" --config {cfg}"
    run = ("python3 bench.py --steps 2 --warmup 0 --no-cpu-baseline --no-backward --no-workloads"
           + c)
    return [
        f"python3 bench.py --steps 20 --warmup 3{c} > DIR/bench.json",
        "rocprofv3 --kernel-trace --stats -d DIR/prof_kt -o kt --output-format csv -- "
        f"python3 bench.py --steps 5 --warmup 1 --no-cpu-baseline --no-backward --no-workloads{c}",
        "rocprofv3 --pmc FETCH_SIZE -d DIR/prof_fetch -o fetch --output-format csv -- "
        f"{run} --copy-calibration",
        "rocprofv3 --pmc WRITE_SIZE -d DIR/prof_write -o write --output-format csv -- "
        f"{run} --copy-calibration",
        *[f"rocprofv3 --pmc {q} -d DIR/prof_{n} -o {n} --output-format csv -- {run}"
          for n, q in SQ_PASSES.items()],
        "python3 bench.py --summarize-profiles DIR",
    ]


PROFILE_COMMANDS = profile_commands()


def _short_kernel(name: str):
    import re
    m = re.search(r"ssd::(?:\(anonymous namespace\)::)?k_(\w+)", name)
    if m:
        return m.group(1)
    if "copyBuffer" in name:
        return "copy"
    return None


def _csv_rows(path):
    import csv
    import glob
    rows = []
    for f in sorted(glob.glob(path)):
        with open(f) as fh:
            rows.extend(csv.DictReader(fh))
    return rows


# The forward's kernels as the library's timer names them, and their rocprofv3 names (k_<name>).
_KERNEL_OBJ = {"run_states": "run_states", "chain": "state_chain", "fused_scan": "fused_scan",
               "chunk_cumsum": "chunk_cumsum", "bmm_chunk": "bmm_chunk",
               "chunk_state": "chunk_state", "state_passing": "state_passing",
               "chunk_scan": "chunk_scan", "quadratic": "quadratic"}


def summarize_profiles(d: str) -> None:
    """Write profiles/forward_<workload>.txt (kernel times and L2-to-memory bytes),
    profiles/forward_counters_<workload>.txt (SQ counters) and profiles/traffic_<workload>.json
    from the rocprofv3 runs under d (see PROFILE_COMMANDS)."""
    with open(os.path.join(d, "bench.json")) as f:
        bench = json.loads(f.read().strip().splitlines()[-1])
    workload = bench["config"]["workload"]
    from mamba_ssd_chunked_cumsum_amd import synth
    cfg = next(i for i, sh in enumerate(synth.CONFIGS) if sh.name == workload)
    commands = profile_commands(cfg)
    stats = {}
    for r in _csv_rows(os.path.join(d, "prof_kt", "*kernel_stats.csv")):
        k = _short_kernel(r["Name"])
        if k and k != "copy":
            stats[k] = (int(r["Calls"]), float(r["AverageNs"]), float(r["MinNs"]),
                        float(r["MaxNs"]))
    counters = {}
    for sub in ("prof_fetch", "prof_write", *[f"prof_{n}" for n in SQ_PASSES]):
        for r in _csv_rows(os.path.join(d, sub, "*counter_collection.csv")):
            k = _short_kernel(r["Kernel_Name"])
            if k:
                counters.setdefault((k, r["Counter_Name"]), []).append(float(r["Counter_Value"]))
    # copy calibration: the 1 GiB device-to-device copy reads and writes exactly 2^30 bytes
    gib = float(1 << 30)
    cf = max(counters.get(("copy", "FETCH_SIZE"), [0.0]))
    cw = max(counters.get(("copy", "WRITE_SIZE"), [0.0]))
    if cf <= 0 or cw <= 0:
        raise SystemExit("no 1 GiB copy dispatch found in the counter runs (--copy-calibration)")
    fetch_scale, write_scale = gib / (cf * 1024), gib / (cw * 1024)
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    src = kernel_source_hash()
    roof = bench["roofline"]
    dom = bench["dominant_kernel_roofline"]
    lines = [
        f"rocprofv3 summary: libssd forward kernels, workload {workload} "
        f"({json.dumps(bench['config'])})",
        f"kernel sources hash {src}; run {json.dumps(bench.get('run', {}))}",
        "",
        "commands (DIR = a scratch output folder; the last runs on any host):",
        *["  " + c for c in commands],
        "",
        f"copy calibration (1 GiB copy): FETCH_SIZE {cf:.0f} KiB -> x{fetch_scale:.3f}, "
        f"WRITE_SIZE {cw:.0f} KiB -> x{write_scale:.3f}",
        "FETCH_SIZE / WRITE_SIZE count bytes between the L2s and the memory side, part of which "
        "the Infinity Cache may serve: an upper bound on HBM bytes.",
        "",
        f"{'kernel':16s}{'calls':>7s}{'avg us':>10s}{'min us':>10s}{'max us':>10s}"
        f"{'bench us':>10s}{'fetch MB':>11s}{'write MB':>11s}",
    ]
    traffic = {}
    for k, (calls, avg, mn, mx) in sorted(stats.items(), key=lambda kv: -kv[1][1]):
        fk = counters.get((k, "FETCH_SIZE"))
        wk = counters.get((k, "WRITE_SIZE"))
        fb = (sum(fk) / len(fk)) * 1024 * fetch_scale if fk else float("nan")
        wb = (sum(wk) / len(wk)) * 1024 * write_scale if wk else float("nan")
        traffic[k] = (fb, wb)
        name = next((t for t, o in _KERNEL_OBJ.items() if o == k), k)
        bus = bench["kernel_ms"].get(name, float("nan")) * 1e3
        lines.append(f"{k:16s}{calls:7d}{avg / 1e3:10.1f}{mn / 1e3:10.1f}{mx / 1e3:10.1f}"
                     f"{bus:10.1f}{fb / 1e6:11.2f}{wb / 1e6:11.2f}")
    fwd = [_KERNEL_OBJ.get(k, k) for k in bench["kernel_ms"]]
    tot = sum(sum(traffic.get(k, (float("nan"),) * 2)) for k in fwd)
    dk = _KERNEL_OBJ.get(dom["kernel"], dom["kernel"])
    dfb, dwb = traffic.get(dk, (float("nan"), float("nan")))
    lines += [
        "",
        f"whole forward ({' + '.join(fwd)}): algorithmic bytes {roof['bytes'] / 1e6:.2f} MB, "
        f"L2-to-memory bytes {tot / 1e6:.2f} MB (ratio {tot / roof['bytes']:.2f})",
        f"dominant kernel {dk}: algorithmic bytes per launch {dom['bytes'] / 1e6:.2f} MB, "
        f"L2-to-memory bytes per launch {(dfb + dwb) / 1e6:.2f} MB "
        f"(ratio {(dfb + dwb) / dom['bytes']:.2f})",
        f"bench line: {bench['ms_per_step'] * 1e3:.1f} us per forward (median "
        f"{bench['ms_per_step_median'] * 1e3:.1f}), {bench['value'] / 1e6:.2f} M tokens/s, "
        f"forward roofline frac {roof['frac']:.3f}, dominant kernel frac {dom['frac']:.3f}",
    ]
    with open(os.path.join(ROOT, "profiles", f"forward_{workload}.txt"), "w") as f:
        f.write("\n".join(lines) + "\n")
    rec = {"workload": workload, "source_hash": src, "fetch_scale": fetch_scale,
           "write_scale": write_scale, "commands": commands,
           "kernels": {_KERNEL_OBJ_REV.get(k, k): {"fetch_bytes": fb, "write_bytes": wb}
                       for k, (fb, wb) in traffic.items()}}
    with open(os.path.join(ROOT, "profiles", f"traffic_{workload}.json"), "w") as f:
        json.dump(rec, f, indent=1)
    print("\n".join(lines))
    clines = _sq_summary(counters, stats, workload, src)
    if clines:
        with open(os.path.join(ROOT, "profiles", f"forward_counters_{workload}.txt"), "w") as f:
            f.write("\n".join(clines) + "\n")
        print("\n".join(clines))


_KERNEL_OBJ_REV = {o: t for t, o in _KERNEL_OBJ.items()}


def _sq_summary(counters, stats, workload, src):
    """Per-kernel SQ counter figures. Normalisation (MI355X: 8 XCDs, 256 CUs, 1024 SIMDs):
    GRBM_GUI_ACTIVE sums the XCDs' busy cycles, so a SIMD's cycles are GUI_ACTIVE / 8;
    SQ_VALU_MFMA_BUSY_CYCLES sums matrix-core busy cycles over SIMDs; SQ_ACTIVE_INST_VALU counts
    issue quad-cycles (4 cycles each) summed over waves; SQ_WAVE_CYCLES and SQ_WAIT_* count
    quad-cycles per wave, summed over waves."""
    names = sorted({k for (k, c) in counters if c.startswith("SQ_") and k != "copy"})
    if not names:
        return []
    out = [f"rocprofv3 SQ counters: libssd forward kernels, workload {workload}; kernel sources "
           f"hash {src}", "commands: the two 'rocprofv3 --pmc SQ_...' lines of the forward "
           f"summary (profiles/forward_{workload}.txt)", "",
           _sq_summary.__doc__.split("Normalisation")[1].strip().replace("\n    ", "\n"), ""]
    for k in names:
        v = {c: sum(x) / len(x) for (kk, c), x in counters.items() if kk == k}
        gui = v.get("GRBM_GUI_ACTIVE", 0.0)
        waves = v.get("SQ_WAVES", 0.0)
        simd_cycles = gui / 8 * 1024 if gui else 0.0
        out.append(f"{k}: {stats.get(k, (0, float('nan')))[1] / 1e3:.1f} us average "
                   f"(kernel trace), {waves:.0f} waves")
        if waves:
            per = ", ".join(f"{c[9:].lower()} {v[c] / waves:.0f}" for c in
                            ("SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_SALU", "SQ_INSTS_LDS",
                             "SQ_INSTS_VMEM") if c in v)
            out.append(f"   instructions per wave: {per}")
        if simd_cycles:
            if "SQ_VALU_MFMA_BUSY_CYCLES" in v:
                out.append(f"   matrix cores busy: {v['SQ_VALU_MFMA_BUSY_CYCLES'] / simd_cycles:.3f}"
                           " of SIMD cycles")
            if "SQ_ACTIVE_INST_VALU" in v:
                out.append(f"   vector ALU issuing: {4 * v['SQ_ACTIVE_INST_VALU'] / simd_cycles:.3f}"
                           " of SIMD cycles")
        if v.get("SQ_WAVE_CYCLES"):
            wc = v["SQ_WAVE_CYCLES"]
            for c, what in (("SQ_WAIT_INST_ANY", "waiting on a dependency (waitcnt)"),
                            ("SQ_WAIT_ANY", "waiting on anything")):
                if c in v:
                    out.append(f"   wave time {what}: {v[c] / wc:.3f}")
        if v.get("SQ_LDS_IDX_ACTIVE"):
            out.append(f"   LDS bank-conflict cycles / LDS active cycles: "
                       f"{v.get('SQ_LDS_BANK_CONFLICT', 0.0) / v['SQ_LDS_IDX_ACTIVE']:.3f}")
        if "SQ_INSTS_VALU_MFMA_MOPS_F16" in v and gui:
            t = stats.get(k, (0, 0.0))[1] * 1e-9
            if t:
                out.append(f"   fp16 matrix flops: {v['SQ_INSTS_VALU_MFMA_MOPS_F16'] * 512 / t / 1e12:.1f}"
                           " TFLOP/s (MOPS x 512 over the kernel's average duration)")
        out.append("")
    return out


def decode_bench(shape, dev, layers: int = 64, rounds: int = 5) -> dict:
    """ssd_step at the workload's layer shape (one token per sequence) over `layers` distinct
    states, one in-place step per state per round, as a decode pass through a stack of layers
    does: 64 states of the 2.7B-shaped layer are 335 MB, more than the 256 MB Infinity Cache, so
    each step reads and writes its state in HBM. Returns per-step time and bandwidth."""
    import torch

    from mamba_ssd_chunked_cumsum_amd import libssd

    Bt, H, P, N, G = shape.batch, shape.nheads, shape.headdim, shape.dstate, shape.ngroups
    io = torch.bfloat16 if shape.io == "bf16" else torch.float32
    g = torch.Generator(device=dev).manual_seed(7)
    states = torch.randn((layers, Bt, H, P, N), device=dev, generator=g)
    x = torch.randn((Bt, H, P), device=dev, generator=g).to(io)
    Bm = torch.randn((Bt, G, N), device=dev, generator=g).to(io)
    Cm = torch.randn((Bt, G, N), device=dev, generator=g).to(io)
    dt = torch.rand((Bt, H), device=dev, generator=g) * 0.1
    A = -1.0 - 15.0 * torch.rand((H,), device=dev, generator=g)
    D = torch.ones((H,), device=dev)
    y = torch.empty_like(x)

    def one_round():
        for k in range(layers):
            libssd.step(states[k], x, dt, A, Bm, Cm, D, out_state=states[k], out=y)

    # one round captured as a HIP graph and replayed: the launches then cost no host time (the
    # step launches nothing but its kernel, so it captures as is)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        one_round()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        one_round()
    graph.replay()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for _ in range(rounds):
        graph.replay()
    t1.record()
    torch.cuda.synchronize()
    us = t0.elapsed_time(t1) * 1e3 / (rounds * layers)
    e = 2 if shape.io == "bf16" else 4
    nbytes = (2 * Bt * H * P * N * 4 + 2 * Bt * H * P * e + 2 * Bt * G * N * e + Bt * H * 4
              + 2 * H * 4)
    return {"layers": layers, "us_per_step": us, "bytes_per_step": nbytes,
            "achieved_gbs": nbytes / (us * 1e-6) / 1e9,
            "frac": nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS,
            "note": "ssd_step, one token per sequence, in-place state, rounds of steps replayed "
                    "from a HIP graph"}


def short_sequence_bench(dev, flush, flush_out, steps: int = 10) -> dict:
    """The short-sequence dispatch: whole forwards (cold cache) of two short workloads under the
    auto variant and the alternatives it chose between. The tiny fp32 workload (auto: the one-
    kernel quadratic form) against the five unfused kernels; a batched bf16 prefill of 32
    sequences of 128 tokens at the 2.7B layer's head shape (auto: one run per sequence, no chain
    kernel) against the unfused kernels."""
    import numpy as np
    import torch

    import mamba_ssd_chunked_cumsum_amd as ssd
    from mamba_ssd_chunked_cumsum_amd import synth

    cases = [
        ("tiny_fp32 (1 x 256 tokens, 2 heads, headdim 16, dstate 16)", synth.config("tiny_fp32"),
         ("auto", "unfused")),
        ("batched_prefill_bf16 (32 x 128 tokens, 80 heads, headdim 64, dstate 128)",
         synth.SSDShape("batched_prefill", 32, 128, 80, 64, 128, 1, 128, init_state=True),
         ("auto", "unfused")),
    ]
    out = {}
    for name, shape, variants in cases:
        inp = synth.make_inputs(shape, seed=7)
        io = torch.bfloat16 if shape.io == "bf16" else torch.float32
        d = {k: (None if v is None else torch.from_numpy(v).to(dev)) for k, v in inp.items()}
        for k in ("x", "B", "C"):
            d[k] = d[k].to(io)
        y = torch.empty_like(d["x"])
        fin = torch.empty((shape.batch, shape.nheads, shape.headdim, shape.dstate),
                          dtype=torch.float32, device=dev)
        row = {}
        for v in variants:
            def call():
                ssd.forward(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], shape.chunk_size,
                            d["initial_state"], variant=v, out=y, final_out=fin)
            call()
            torch.cuda.synchronize()
            ms = []
            for _ in range(steps):
                if flush is not None:
                    torch.sum(flush, dim=0, dtype=torch.int64, out=flush_out)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                call()
                e1.record()
                torch.cuda.synchronize()
                ms.append(e0.elapsed_time(e1))
            row[v] = float(np.mean(ms))
        out[name] = {"ms_per_forward": row}
        del d, y, fin
    return out


def backward_bench(shape, d, flush, flush_out, steps: int = 3) -> dict:
    """ssd_backward at the workload's shape: output gradient dy of x's dtype and a final-state
    gradient, cold cache before every call. Reports ms per call and tokens/s; the bytes it must
    move (x, dy, B, C, dt in; dx, ddt, dB, dC out in fp32) and the flops of its four fp32
    chunked recurrences give its roofline (fp32 matrix cores: 157.3 TFLOP/s)."""
    import numpy as np
    import torch

    from mamba_ssd_chunked_cumsum_amd import libssd

    x = d["x"]
    g = torch.Generator(device=x.device).manual_seed(11)
    dy = torch.randn(x.shape, device=x.device, generator=g).to(x.dtype)
    dfinal = torch.randn((shape.batch, shape.nheads, shape.headdim, shape.dstate),
                         device=x.device, generator=g)

    def call():
        return libssd.backward(x, d["dt"], d["A"], d["B"], d["C"], d["D"], dy, shape.chunk_size,
                               d["initial_state"], dfinal)

    call()
    torch.cuda.synchronize()
    ms = []
    for _ in range(steps):
        if flush is not None:
            torch.sum(flush, dim=0, dtype=torch.int64, out=flush_out)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        out = call()
        e1.record()
        torch.cuda.synchronize()
        ms.append(e0.elapsed_time(e1))
        del out
    t = float(np.mean(ms)) if ms else float("nan")
    s_io = 2 if shape.io == "bf16" else 4
    tokens = shape.batch * shape.seqlen
    H, P, N, G = shape.nheads, shape.headdim, shape.dstate, shape.ngroups
    nbytes = tokens * (H * P * (2 * s_io + 4) + 2 * G * N * (s_io + 4) + 2 * H * 4)
    alg = algorithmic(shape, d["initial_state"] is not None)
    flops = 4 * alg["flops"]  # four chunked recurrences of the forward's size
    t_roof = max(nbytes / (HBM_PEAK_GBS * 1e9), flops / (FP32_PEAK_TFLOPS * 1e12))
    return {"ms_per_call": t, "tokens_per_s": tokens / (t / 1e3), "bytes": nbytes,
            "flops": flops, "bound": "fp32 matrix cores", "t_roofline_us": t_roof * 1e6,
            "frac": t_roof / (t / 1e3),
            "note": "ssd_backward (dx, ddt, dA, dB, dC, dD, initial-state gradient) from dy and "
                    "a final-state gradient; four fp32 chunked recurrences plus elementwise "
                    "kernels"}


def host_metadata() -> dict:
    """What the numbers were measured with, from the host side: ROCm and compiler, GPU clocks
    (rocm-smi), the library's revision (git, or the one recorded when it was built) and source
    hash, and the host CPU. Runs its helper programs as child processes, so it is called before
    this process touches the GPU (a child forked after that would inherit the initialised
    device)."""
    import platform

    # Under a profiler whose preloaded library has already opened the device (rocprofv3 with
    # counters does), even a child process would start from an initialised device: no children.
    profiled = "rocprof" in os.environ.get("LD_PRELOAD", "") or any(
        k.startswith("ROCPROF") for k in os.environ)

    def cmd(args, timeout=20):
        if profiled:
            return ""
        try:
            return subprocess.run(args, capture_output=True, text=True, timeout=timeout).stdout
        except (OSError, subprocess.SubprocessError):
            return ""

    info = {}
    try:
        with open("/opt/rocm/.info/version") as f:
            info["rocm"] = f.read().strip()
    except OSError:
        info["rocm"] = None
    info["hipcc"] = (cmd(["/opt/rocm/bin/hipcc", "--version"]).splitlines() or [None])[0]
    # Clocks: the highest supported level of each clock (rocm-smi --showclkfrq), and the level at
    # the moment of the query, which on an idle GPU is its low-power state (sclk ~95 MHz), not
    # the clock the kernels run at.
    clocks = {}
    for line in cmd(["rocm-smi", "--showclocks"]).splitlines():
        for key in ("sclk", "mclk", "fclk", "socclk"):
            if f"{key} clock level" in line and "(" in line:
                clocks[key + "_at_query"] = line.split("(")[-1].split(")")[0]
    section = None
    for line in cmd(["rocm-smi", "--showclkfrq"]).splitlines():
        text = line.split(":", 1)[-1].strip() if line.startswith("GPU[") else line.strip()
        if text.startswith("Supported ") and " frequencies" in text:
            section = text.split()[1]
            continue
        head, _, val = text.partition(":")
        val = val.replace("*", "").strip()
        if section and head.strip() and val.lower().endswith("mhz"):
            try:
                mhz = float(val[:-3])
            except ValueError:
                continue
            key = section + "_max"
            if mhz > float(str(clocks.get(key, "0Mhz"))[:-3] or 0):
                clocks[key] = f"{mhz:g}Mhz"
    info["clocks"] = clocks or None
    rev = cmd(["git", "-C", ROOT, "rev-parse", "HEAD"]).strip()
    build = {}
    try:
        with open(os.path.join(ROOT, "mamba_ssd_chunked_cumsum_amd", "_lib", "build_info.json")) as f:
            build = json.load(f)
    except (OSError, ValueError):
        pass
    info["git_rev"] = rev or build.get("git_rev")
    info["library_built_from"] = build or None
    info["kernel_sources_hash"] = kernel_source_hash()
    cpu = None
    try:
        with open("/proc/cpuinfo") as f:
            cpu = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), None)
    except OSError:
        pass
    info["cpu"] = cpu or platform.processor()
    info["cpu_threads"] = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") \
        else os.cpu_count()
    return info


def run_metadata(dev, host: dict) -> dict:
    """host_metadata() plus the GPU's name, architecture and compute units, and torch."""
    import torch

    props = torch.cuda.get_device_properties(dev)
    info = dict(host)
    info["gpu"] = props.name
    info["arch"] = getattr(props, "gcnArchName", None)
    info["compute_units"] = props.multi_processor_count
    info["torch"] = torch.__version__
    return info


def workload_bench(index: int, dev, flush, flush_out, steps: int = 5) -> dict:
    """One more workload's whole forward (auto variant, cold cache before every step): mean and
    median ms, tokens/s, per-kernel ms and its roofline fraction."""
    import numpy as np
    import torch

    import mamba_ssd_chunked_cumsum_amd as ssd
    from mamba_ssd_chunked_cumsum_amd import libssd, synth

    shape = synth.CONFIGS[index]
    inp = synth.make_inputs(shape, cfg_index=index)
    io = torch.bfloat16 if shape.io == "bf16" else torch.float32
    d = {k: (None if v is None else torch.from_numpy(v).to(dev)) for k, v in inp.items()}
    del inp
    for k in ("x", "B", "C"):
        d[k] = d[k].to(io)
    y = torch.empty_like(d["x"])
    fin = torch.empty((shape.batch, shape.nheads, shape.headdim, shape.dstate),
                      dtype=torch.float32, device=dev)

    def call(timer=None):
        ssd.forward(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], shape.chunk_size,
                    d["initial_state"], out=y, final_out=fin, timer=timer)

    call()
    torch.cuda.synchronize()
    ms, per = [], {}
    for k in range(2 * steps):
        if flush is not None:
            torch.sum(flush, dim=0, dtype=torch.int64, out=flush_out)
        tm = libssd.KernelTimer() if k >= steps else None
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        call(tm)
        e1.record()
        torch.cuda.synchronize()
        if tm is None:
            ms.append(e0.elapsed_time(e1))
        else:
            for name, t in tm.times_ms().items():
                per.setdefault(name, []).append(t)
    alg = algorithmic(shape, d["initial_state"] is not None)
    t = float(np.mean(ms))
    t_roof = max(alg["bytes"] / (HBM_PEAK_GBS * 1e9),
                 alg["flops"] / ((MFMA_F16_PEAK_TFLOPS if shape.io == "bf16"
                                  else FP32_PEAK_TFLOPS) * 1e12))
    return {"shape": {"batch": shape.batch, "seqlen": shape.seqlen, "nheads": shape.nheads,
                      "headdim": shape.headdim, "dstate": shape.dstate,
                      "ngroups": shape.ngroups, "chunk_size": shape.chunk_size,
                      "initial_state": d["initial_state"] is not None},
            "ms_per_forward": t, "ms_per_forward_median": float(np.median(ms)),
            "tokens_per_s": alg["tokens"] / (t / 1e3),
            "kernel_ms": {k: float(np.mean(v)) for k, v in per.items()},
            "t_roofline_us": t_roof * 1e6, "frac": t_roof / (t / 1e3),
            "bytes": alg["bytes"], "flops": alg["flops"]}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=2, help="workload index (0..4)")
    ap.add_argument("--variant", default="auto", choices=["auto", "fused", "unfused"])
    ap.add_argument("--precision", default="auto", choices=["auto", "fp16", "fp32"],
                    help="operand precision (auto: fp16 operands, run states split hi + lo)")
    ap.add_argument("--run-chunks", type=int, default=0)
    ap.add_argument("--no-flush", action="store_true",
                    help="skip the cache sweep before steps (inputs may then be served from the "
                         "256 MB Infinity Cache)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the timed ssd_backward calls reported under 'backward' and the "
                         "short-sequence forwards under 'short_sequence'")
    ap.add_argument("--cpu-seconds", type=float, default=30.0)
    ap.add_argument("--no-workloads", action="store_true",
                    help="skip the other bf16 workloads reported under 'workloads'")
    ap.add_argument("--summarize-profiles", metavar="DIR",
                    help="write profiles/ summaries from rocprofv3 output under DIR and exit")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one 1 GiB device-to-device copy (a known-size kernel for "
                         "scaling hardware byte counters)")
    args = ap.parse_args()
    if args.summarize_profiles:
        summarize_profiles(args.summarize_profiles)
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: libssd runs the SSD forward on one GPU; --gpus {args.gpus} "
              f"(WORLD_SIZE {world}) is not supported. Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    host = host_metadata()  # before anything touches the GPU

    import numpy as np
    import torch

    import mamba_ssd_chunked_cumsum_amd as ssd
    from mamba_ssd_chunked_cumsum_amd import libssd, synth

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    shape = synth.CONFIGS[args.config]
    inp = synth.make_inputs(shape, cfg_index=args.config)
    io = torch.bfloat16 if shape.io == "bf16" else torch.float32
    d = {}
    for k, v in inp.items():
        if v is None:
            d[k] = None
            continue
        t = torch.from_numpy(v).to(dev)
        d[k] = t.to(io) if k in ("x", "B", "C") else t
    y = torch.empty_like(d["x"])
    fin = torch.empty((shape.batch, shape.nheads, shape.headdim, shape.dstate),
                      dtype=torch.float32, device=dev)

    def step(timer=None):
        ssd.forward(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], shape.chunk_size,
                    d["initial_state"], variant=args.variant, precision=args.precision,
                    run_chunks=args.run_chunks, out=y, final_out=fin, timer=timer)

    # correctness run first, then the CPU oracle leg on the same inputs
    step()
    torch.cuda.synchronize()
    cpu = None
    parity = None
    if not args.no_cpu_baseline:
        y64 = y.float().cpu().numpy().astype(np.float64)
        f64 = fin.cpu().numpy().astype(np.float64)
        cpu, parity = cpu_baseline(inp, shape, y64, f64, args.cpu_seconds)
        del y64, f64

    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    for _ in range(args.warmup):
        step()
    # Before every timed step a read-only sweep over 2 GiB of clean memory evicts the inputs (and
    # everything else) from L2 and the Infinity Cache, so each step reads its inputs from HBM. A
    # write-based flush would leave the cache full of dirty lines whose write-back is charged to
    # the next kernel instead.
    flush = None
    if not args.no_flush:
        flush = torch.ones(1 << 29, dtype=torch.int32, device=dev)  # 2 GiB
        flush_out = torch.empty((), dtype=torch.int64, device=dev)
    timers = [libssd.KernelTimer() for _ in range(args.steps)]
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]

    # Two timed passes of K steps each: the first times whole forwards as a caller sees them (no
    # events between the library's kernels), the second records HIP events around every kernel on
    # the call's stream for the per-kernel durations (those events cost a few microseconds of gap
    # between kernels, so the second pass's forwards are not the ones reported).
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    for k in range(args.steps):
        if flush is not None:
            torch.sum(flush, dim=0, dtype=torch.int64, out=flush_out)
        starts[k].record()
        step()
        ends[k].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    step_ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]

    inst_starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    inst_ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    for k in range(args.steps):
        if flush is not None:
            torch.sum(flush, dim=0, dtype=torch.int64, out=flush_out)
        inst_starts[k].record()
        step(timers[k])
        inst_ends[k].record()
    torch.cuda.synchronize()
    inst_ms = [s.elapsed_time(e) for s, e in zip(inst_starts, inst_ends)]
    per_kernel = {}
    for tm in timers:
        for name, ms in tm.times_ms().items():
            per_kernel.setdefault(name, []).append(ms)
    kernel_ms = {k: float(np.mean(v)) for k, v in per_kernel.items()}
    ms_per_step = float(np.mean(step_ms))
    ms_median = float(np.median(step_ms))
    alg = algorithmic(shape, d["initial_state"] is not None)
    tokens = alg["tokens"]
    value = tokens / (ms_per_step / 1e3)
    t_roof = max(alg["bytes"] / (HBM_PEAK_GBS * 1e9),
                 alg["flops"] / ((MFMA_F16_PEAK_TFLOPS if shape.io == "bf16"
                                  else FP32_PEAK_TFLOPS) * 1e12))
    fwd_kernels = list(kernel_ms)  # the timer's names, as the traffic record keys them
    # The whole forward against the HBM roofline: its algorithmic bytes (inputs read once, y and
    # the final state written once) over the measured time of a forward.
    fwd_gbs = alg["bytes"] / (ms_per_step / 1e3) / 1e9
    roofline = {
        "bound": "hbm", "achieved": fwd_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
        "frac": fwd_gbs / HBM_PEAK_GBS,
        "traffic": measured_traffic(shape.name, fwd_kernels),
        "scope": "whole forward (" + " + ".join(kernel_ms) + ")",
        "bytes": alg["bytes"], "ms": ms_per_step,
    }
    dominant = max(kernel_ms, key=kernel_ms.get)
    # Algorithmic bytes of the dominant kernel: the fused scan (or the unfused chunk scan) streams
    # every input token's x, B, C, dt and writes y -- the per-token stream figure times the
    # tokens of one launch. Other kernels are charged the same figure only if they dominate.
    kb = alg["stream_bytes_per_token"] * tokens
    achieved = kb / (kernel_ms[dominant] / 1e3) / 1e9
    out = {
        "metric": METRIC,
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if shape.io == "bf16" else "f32",
        "data": "synthetic",
        "config": {
            "workload": shape.name, "batch": shape.batch, "seqlen": shape.seqlen,
            "nheads": shape.nheads, "headdim": shape.headdim, "dstate": shape.dstate,
            "ngroups": shape.ngroups, "chunk_size": shape.chunk_size,
            "variant": args.variant, "precision": args.precision,
            "cache_flush": flush is not None,
        },
        "roofline": roofline,
        "dominant_kernel_roofline": {
            "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": measured_traffic(shape.name, [dominant]),
            "kernel": dominant, "kernel_ms": kernel_ms[dominant], "bytes": kb,
        },
        "forward_roofline": {
            "bytes": alg["bytes"], "flops": alg["flops"], "t_roofline_us": t_roof * 1e6,
            "frac": t_roof / (ms_per_step / 1e3),
            "frac_median": t_roof / (ms_median / 1e3),
            "gbs": fwd_gbs,
            "tflops": alg["flops"] / (ms_per_step / 1e3) / 1e12,
        },
        "ms_per_step_median": ms_median,
        "value_median": tokens / (ms_median / 1e3),
        "kernel_ms": kernel_ms,
        "step_ms_min": float(np.min(step_ms)),
        "ms_per_step_with_kernel_events": float(np.mean(inst_ms)),
        "wall_s_timed_loop": wall,
        "cpu_baseline": cpu,
        "parity": parity,
        "run": run_metadata(dev, host),
        "decode_step": decode_bench(shape, dev),
        "backward": None if args.no_backward else backward_bench(
            shape, d, flush, flush_out if flush is not None else None),
        "short_sequence": None if args.no_backward else short_sequence_bench(
            dev, flush, flush_out if flush is not None else None),
    }
    if not args.no_workloads:
        del d, y, fin
        torch.cuda.empty_cache()
        out["workloads"] = {
            synth.CONFIGS[i].name: workload_bench(i, dev, flush,
                                                  flush_out if flush is not None else None)
            for i in range(1, len(synth.CONFIGS))
            if i != args.config and synth.CONFIGS[i].io == "bf16"}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
