#!/usr/bin/env python3
"""Decode-step benchmark of the MI355X persistent megakernel.

Workload: Llama-3.2-1B-shaped decoder (16 layers, hidden 2048, 32 Q / 8 KV
heads of 64, SwiGLU 8192, vocab 128256, tied LM head, RoPE theta 5e5), bf16
synthetic weights ~N(0, 0.02), bf16 KV cache prefilled with N(0, 1) to
context 1024, batch 1; K greedy decode steps at positions 1024, 1025, ...
with the next token chained on the device.  One step = one kernel launch.

Prints one JSON line: steps/s (value, launch gaps included), ms and us per step,
the roofline of the megakernel (algorithmic bytes = weights + KV read per step,
over the kernel's own average launch duration from an event pair around every
launch, against the 8 TB/s HBM peak; measured HBM traffic from the committed
counter profile when it matches the kernel source), the one-kernel-per-op HIP
baseline on the same inputs, and the oracle's CPU time on a bounded sample.

  python bench.py [--gpus 1] [--steps 256] [--warmup 10] [--sched static|dynamic|event]
  python bench.py --batch 16    (mixed-context batch workload, tokens/s, with the one-kernel-per-op baseline
                                on the same inputs beside it; not the headline line)
  python bench.py --model moe   (64-expert top-8 MoE on the 1B attention shape, batch 16, context 2048)
  python bench.py --prefill 1024 (the prompt megakernel on a 1024-token prompt: tokens/s, TFLOP/s vs the
                                matrix-core peak, beside the same prompt as 1024 decode steps)
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode µs/step (steps/s) at batch 1, Llama-1B shape; achieved HBM GB/s vs peak"
HBM_PEAK_GBS = 8000.0
SCHEDS = {"static": 0, "dynamic": 1, "event": 2, "scheduler": 3}


def step_bytes(cfg, positions):
    """Algorithmic bytes of one decode step: every weight once + K and V rows 0..P of every layer."""
    kv = 4 * cfg.n_layers * cfg.n_kv * cfg.head_dim * (np.asarray(positions, np.int64) + 1)
    return cfg.weight_bytes() + int(kv.sum())


def traffic_file(batch=1):
    """The committed counter-traffic record of the 1B-shape workload at this batch."""
    return os.path.join(ROOT, "profiles", f"mk_step_kernel_llama1b_b{batch}_traffic.json")


def measured_traffic(batch=1):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE passes (scaled by the same
    counters on a plain copy of known size), or None if there is no record for this workload or the kernel
    source changed since they were taken."""
    import hashlib
    try:
        rec = json.load(open(traffic_file(batch)))
        src = b"".join(open(os.path.join(ROOT, f), "rb").read() for f in rec["source_files"])
    except (OSError, KeyError, ValueError):
        return None
    if hashlib.sha256(src).hexdigest() != rec.get("source_sha256"):
        return None
    return int(rec["traffic_bytes_per_launch"])


# every source the kernel's memory traffic depends on: the kernel, the planner (tiles, queues), the
# runtime's weight packing (tile order in HBM) and the compiler flags the library is built with
TRAFFIC_SOURCES = ["persistent_megakernel_decode_cu_amd/csrc/megakernel.hip",
                   "persistent_megakernel_decode_cu_amd/csrc/graph.cpp",
                   "persistent_megakernel_decode_cu_amd/csrc/runtime.cpp",
                   "persistent_megakernel_decode_cu_amd/csrc/runtime.h",
                   "persistent_megakernel_decode_cu_amd/csrc/mk_internal.h",
                   "persistent_megakernel_decode_cu_amd/build.py"]


def traffic_from_counters(fetch_csv, write_csv, kernel="mk::mk_step_kernel", copy_bytes=256 << 20,
                          workload="llama-3.2-1b-shape, batch 1, decode from position 1024, max_ctx 2048"):
    """HBM bytes per launch of `kernel` from two rocprofv3 --pmc runs of this bench with
    --copy-calibration (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch), each scaled by what the
    same counter reads for the plain device copy of copy_bytes (its three largest dispatches)."""
    import csv
    import hashlib

    def read(path, counter):
        mk_vals, copy_vals = [], []
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] != counter:
                    continue
                v = float(r["Counter_Value"])
                if r["Kernel_Name"].startswith(kernel):
                    mk_vals.append(v)
                elif "copyBuffer" in r["Kernel_Name"]:
                    copy_vals.append(v)
        copy_vals = sorted(copy_vals)[-3:]
        return float(np.median(mk_vals)), float(np.median(copy_vals)), len(mk_vals)

    f_mk, f_copy, n = read(fetch_csv, "FETCH_SIZE")
    w_mk, w_copy, _ = read(write_csv, "WRITE_SIZE")
    fs, ws = (copy_bytes / 1024) / f_copy, (copy_bytes / 1024) / w_copy
    src = b"".join(open(os.path.join(ROOT, f), "rb").read() for f in TRAFFIC_SOURCES)
    rd, wr = int(f_mk * 1024 * fs), int(w_mk * 1024 * ws)
    return {"kernel": kernel, "workload": workload,
            "source_sha256": hashlib.sha256(src).hexdigest(), "source_files": TRAFFIC_SOURCES,
            "fetch_size_kib_median": f_mk, "write_size_kib_median": w_mk, "copy_bytes": copy_bytes,
            "copy_fetch_size_kib": f_copy, "copy_write_size_kib": w_copy,
            "fetch_scale": round(fs, 4), "write_scale": round(ws, 4),
            "hbm_read_bytes_per_launch": rd, "hbm_write_bytes_per_launch": wr,
            "traffic_bytes_per_launch": rd + wr, "launches": n}


def host_info():
    """The host CPU model and the GPU clocks as amd-smi reports them (raw, trimmed), for the record."""
    import subprocess
    info = {"cpu_model": None, "cpu_threads": len(os.sched_getaffinity(0)), "gpu_clocks": None}
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                info["cpu_model"] = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    if "rocprof" in os.environ.get("LD_PRELOAD", "") or "ROCPROF_OUTPUT_PATH" in os.environ:
        return info  # under the profiler: a child process would inherit its GPU-initialising preload
    for cmd in (["amd-smi", "metric", "--clock", "--json"], ["rocm-smi", "--showclocks", "--json"]):
        try:
            r = subprocess.run(cmd, capture_output=True, text=True, timeout=30)
        except (OSError, subprocess.TimeoutExpired):
            continue
        if r.returncode == 0 and r.stdout.strip():
            try:
                raw = json.loads(r.stdout)
                # amd-smi: {"gpu_data": [{"gpu": 0, "clock": {"gfx_0": {"clk": {"value": .., "unit": "MHz"},
                # "max_clk": ..}, "mem_0": ..}}]} -> current / max MHz of the compute and memory clocks
                clk = {}
                for g in raw.get("gpu_data", []) if isinstance(raw, dict) else []:
                    for dom, v in g.get("clock", {}).items():
                        if dom.startswith(("gfx", "mem")) and isinstance(v, dict):
                            cur, mx = v.get("clk"), v.get("max_clk")
                            clk[dom] = [cur.get("value") if isinstance(cur, dict) else cur,
                                        mx.get("value") if isinstance(mx, dict) else mx]
                info["gpu_clocks"] = {"MHz_current_max": clk} if clk else raw
            except ValueError:
                info["gpu_clocks"] = r.stdout.strip()[:2000]
            info["gpu_clocks_tool"] = " ".join(cmd)
            break
    return info


def cpu_baseline(cfg, w, kc, vc, tok, P0, budget_s=10.0):
    """The oracle (plain C, double precision, OpenMP over output rows) on the same inputs."""
    import oracle
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    k2, v2 = kc.copy(), vc.copy()
    t = np.array(tok, np.int32)
    first = None
    n = 0
    t0 = time.perf_counter()
    while True:
        r = oracle.decode_step(cfg, w, t, [P0 + n], k2, v2)
        if first is None:
            first = r
        t = r["next"].copy()
        n += 1
        if time.perf_counter() - t0 > budget_s and n >= 2:
            break
    dt = time.perf_counter() - t0
    out = dict(value=n / dt, unit="steps/s", cores=threads, kind="oracle",
               sample=f"{n} greedy decode steps of the same workload from position {P0} ({dt:.1f} s)")
    # the same oracle on one thread: one step (OpenMP's thread count set through its runtime)
    try:
        import ctypes
        gomp = ctypes.CDLL("libgomp.so.1")
        gomp.omp_set_num_threads(1)
        t1 = time.perf_counter()
        oracle.decode_step(cfg, w, t, [P0 + n], k2, v2)
        out["single_thread"] = {"value": 1.0 / (time.perf_counter() - t1), "unit": "steps/s", "cores": 1,
                                "sample": "1 decode step"}
        gomp.omp_set_num_threads(threads)
    except OSError:
        pass
    return out, first


def baseline_leg(mk, torch, cfg, desc, kv, tok, P0, C, K, W, mk_ms):
    """The one-kernel-per-op HIP baseline on the same inputs (weights, KV cache, first tokens and
    positions): K greedy steps with plain launches, then the same steps replayed from a HIP graph."""
    P0 = np.atleast_1d(np.asarray(P0, np.int32))
    B = len(P0)
    hb = mk.mkb_create(desc, B, C)
    logits = torch.empty(B, cfg.vocab, dtype=torch.float32, device="cuda")
    tokb = torch.tensor(np.asarray(tok, np.int32), device="cuda")
    posb = torch.tensor(P0, device="cuda")
    tok_h, pos_h = tokb.clone(), posb.clone()
    stream = torch.cuda.current_stream()

    def reset():
        tokb.copy_(tok_h)
        posb.copy_(pos_h)
        torch.cuda.synchronize()

    def step():
        mk.mkb_decode_step(hb, tokb.data_ptr(), posb.data_ptr(), kv.data_ptr(), logits.data_ptr(),
                           torch.cuda.current_stream().cuda_stream, 1)

    def timed(fn):
        reset()
        for _ in range(W):
            fn()
        reset()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(K):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / K

    ms_stream = timed(step)
    launches = mk.mkb_launches_per_step(hb)
    g = torch.cuda.CUDAGraph()
    reset()
    with torch.cuda.graph(g):
        step()
    ms_graph = timed(g.replay)
    del g
    mk.mkb_destroy(hb)
    best = min(ms_stream, ms_graph)
    return {"us_per_step_stream": round(ms_stream * 1000, 2), "us_per_step_graph": round(ms_graph * 1000, 2),
            "launches_per_step": launches, "megakernel_speedup_vs_best": round(best / mk_ms, 3)}


TRACE_OPS = {1: "QKV+RoPE", 2: "attention", 3: "O-proj", 4: "gate/up", 5: "down", 6: "LM head", 7: "router",
             8: "expert gate/up", 9: "expert down", 10: "RMSNorm (prompt)", 11: "QKV+RoPE (prompt)",
             12: "attention (prompt)", 13: "O-proj (prompt)", 14: "gate/up (prompt)", 15: "down (prompt)",
             16: "LM head (prompt)"}


def trace_summary(tr, ex, title, command):
    """Markdown summary of one traced step (mk_read_trace, 16 words per task: workgroup, t_fetch,
    t_inputs_ready, t_staged, t_computed, t_end, t_stored, t_last_page, first page, last wave's epilogue
    issued, last wave's stores acknowledged, wave 0's epilogue issued, the loader's first and last page
    issued, its last page published; 100 MHz ticks): where each operation's time goes, when each layer's
    phases end, and how long each dependency hop takes."""
    tasks = ex["tasks"]
    us = 0.01  # one tick of the 100 MHz clock in microseconds
    (fetch, ready, staged, computed, end, stored, last_pg, epi, acked) = (
        tr[:, i].astype(np.int64) for i in (1, 2, 3, 4, 5, 6, 7, 9, 10))
    t0 = int(fetch.min())
    ops = tasks["op"]
    lines = [f"# {title}", "", f"Command: `{command}`", "",
             f"Step span (first task fetched to last task ended): {(int(end.max()) - t0) * us:.1f} µs over "
             f"{len(tasks)} tasks on {ex['header']['W']} workgroups.", "",
             "## Per operation (µs; median over the step's tasks, p90 in brackets)", "",
             "Columns: waiting for the input event; staging the inputs; compute (page waits included) and, of it, "
             "how long after staging wave 0 got its last page; the epilogue until the last wave issued its "
             "stores; until the last wave's stores were acknowledged; until the signal was issued (done "
             "barrier, counter add); inputs ready to end.", "",
             "| op | tasks | wait | stage | compute | last page after staging | epilogue issued | stores acked | "
             "barrier + signal | busy |", "|---|---|---|---|---|---|---|---|---|---|"]

    def med(a):
        return f"{np.median(a) * us:.2f} [{np.percentile(a, 90) * us:.2f}]" if len(a) else "-"

    for op in sorted(set(int(o) for o in ops)):
        s = ops == op
        lp = last_pg[s] - staged[s]
        lp = lp[last_pg[s] > 0]
        lines.append(f"| {TRACE_OPS.get(op, op)} | {int(s.sum())} | {med(ready[s] - fetch[s])} | "
                     f"{med(staged[s] - ready[s])} | {med(computed[s] - staged[s])} | {med(np.maximum(lp, 0))} | "
                     f"{med(epi[s] - computed[s])} | {med(acked[s] - epi[s])} | {med(end[s] - acked[s])} | "
                     f"{med(end[s] - ready[s])} |")
    # the loader's side: when the task's pages were issued and its last page published
    iss0, iss1, pubd = (tr[:, i].astype(np.int64) for i in (12, 13, 14))
    lines += ["", "## Loader (µs from the task's inputs being ready; negative: before)", "",
              "Columns: loader wave 0 issued the task's first page; issued its last page; published its last "
              "page (its loads had landed); that last page's issue-to-publish latency; the time compute wave 0 "
              "spent waiting for pages (attention and several-sequence GEMV tasks only).", "",
              "| op | tasks with pages | first page issued | last page issued | last page published | "
              "last page latency | wave 0 waiting for pages |", "|---|---|---|---|---|---|---|"]
    pwait = tr[:, 15].astype(np.int64)
    for op in sorted(set(int(o) for o in ops)):
        s = (ops == op) & (iss0 > 0) & (pubd > 0)
        lines.append(f"| {TRACE_OPS.get(op, op)} | {int(s.sum())} | {med(iss0[s] - ready[s])} | "
                     f"{med(iss1[s] - ready[s])} | {med(pubd[s] - ready[s])} | {med(pubd[s] - iss1[s])} | "
                     f"{med(pwait[s])} |")
    # per layer: when each phase's last task ended (from the step's first fetch)
    layers = tasks["layer"]
    L = ex["header"]["L"]
    phase_ops = [o for o in (1, 2, 3, 4, 5, 7, 8, 9, 10, 11, 12, 13, 14, 15) if (ops == o).any()]
    lines += ["", "## Layer phases (µs from the step's first fetch: the end of each phase's last task)", "",
              "| layer | " + " | ".join(TRACE_OPS[o] for o in phase_ops) + " | layer time |",
              "|---|" + "---|" * (len(phase_ops) + 1)]
    prev = None
    layer_times = []
    for l in range(L):
        row = []
        for o in phase_ops:
            s = (layers == l) & (ops == o)
            row.append((int(end[s].max()) - t0) * us if s.any() else float("nan"))
        last = max(r for r in row if r == r)
        lt = last - prev if prev is not None else last
        layer_times.append(lt)
        prev = last
        if l < 3 or l >= L - 2:
            lines.append(f"| {l} | " + " | ".join(f"{r:.1f}" for r in row) + f" | {lt:.1f} |")
        elif l == 3:
            lines.append("| … |" + " |" * (len(phase_ops) + 1))
    s = (ops == 6) | (ops == 16)
    if s.any():
        lm_end = (int(end[s].max()) - t0) * us
        lines += ["", f"Median layer time {np.median(layer_times[1:] or layer_times):.1f} µs; LM head phase "
                      f"{lm_end - prev:.1f} µs after the last layer (ends at {lm_end:.1f} µs)."]
    # dependency hops: an event's last producer ends -> its consumers see the event
    prod_end = {}
    for i, k in enumerate(tasks):
        if k["sig_ev"] != 0xFFFFFFFF:
            e = int(k["sig_ev"])
            prod_end[e] = max(prod_end.get(e, 0), int(end[i]))
    hops = {}
    for i, k in enumerate(tasks):
        e = int(k["wait_ev"])
        if e != 0xFFFFFFFF and e in prod_end:
            hops.setdefault(int(k["op"]), []).append(int(ready[i]) - prod_end[e])
    lines += ["", "## Dependency hops (µs: the awaited event's last producer ended → the consumer saw the event;",
              "negative when the consumer saw it before the producer's own end record)", "",
              "| consumer | median | p10 | p90 |", "|---|---|---|---|"]
    for op, v in sorted(hops.items()):
        v = np.asarray(v)
        lines.append(f"| {TRACE_OPS.get(op, op)} | {np.median(v) * us:.2f} | {np.percentile(v, 10) * us:.2f} | "
                     f"{np.percentile(v, 90) * us:.2f} |")
    return "\n".join(lines) + "\n"


def traced_step_summary(mk, torch, model, B, C, opt_kw, run_args, title, command, out_path, steps=4):
    """Builds a handle with per-task tracing on, runs a few chained steps, writes the trace summary."""
    tok0, positions, kv, logits = run_args
    h = mk.mk_build_graph(model.desc, B, C, mk.options(trace=1, **opt_kw))
    ex = mk.parse_export(mk.mk_export_graph(h))
    sp = torch.cuda.current_stream().cuda_stream
    nxt = mk.mk_next_tokens(h)
    for s in range(steps):
        mk.mk_decode_step(h, tok0.data_ptr() if s == 0 else nxt, positions[s].data_ptr(), kv.data_ptr(),
                          logits.data_ptr(), sp)
    torch.cuda.synchronize()
    err = mk.mk_check_device_error(h)
    if err:
        raise SystemExit(f"device error: {err}")
    tr = mk.mk_read_trace(h, int(ex["header"]["n_tasks"]))
    mk.mk_destroy(h)
    text = trace_summary(tr, ex, title, command)
    with open(out_path, "w") as f:
        f.write(text)
    return text


def moe_step_bytes(cfg, positions, experts):
    """Algorithmic bytes of one MoE decode step: the dense part (attention, norms, LM head), every layer's
    router, each expert that at least one sequence selected in that layer once, and the K/V rows read.
    experts: [L][B][top_k] selected ids of that step."""
    h, fe = cfg.hidden, cfg.expert_ffn
    touched = sum(len(np.unique(experts[l])) for l in range(cfg.n_layers))
    return step_bytes(cfg, positions) + 2 * cfg.n_layers * cfg.n_experts * h + 2 * 3 * h * fe * touched


def _hip_copy_async(torch, dst, src_ptr, nbytes, stream_ptr):
    import ctypes
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipMemcpyAsync.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p]
    rc = hip.hipMemcpyAsync(ctypes.c_void_p(dst), ctypes.c_void_p(src_ptr), nbytes, 3, ctypes.c_void_p(stream_ptr))
    if rc != 0:
        raise SystemExit(f"hipMemcpyAsync failed ({rc})")


def bench_batch(args, torch, synth, mk):
    """Several sequences per step.  Dense: Llama-1B shape, per-sequence contexts uniform in [256, 4096] from
    the token seed, KV cache room for 4352 positions.  MoE: 64 experts of SwiGLU 1024, top-8, on the 1B
    attention shape, every sequence at context 2048.  K greedy steps, every sequence advancing by one."""
    cfg = synth.configs.MOE_1B if args.model == "moe" else synth.configs.LLAMA_1B
    moe = cfg.n_experts > 0
    # MoE: every sequence at context 2048; dense: contexts uniform in [256, 4096]
    B, K, W = args.batch, args.steps, args.warmup
    C = 2048 + (max(K, W) + 63) // 64 * 64 if moe else 4352
    t_gen = time.perf_counter()
    w = synth.make_weights(cfg)
    kc, vc = synth.make_kv(cfg, B, C)
    tok = synth.make_tokens(cfg, B)
    P0 = np.full(B, 2048, np.int32) if moe else synth.make_positions(B, 256, 4096)
    t_gen = time.perf_counter() - t_gen
    if int(P0.max()) + max(K, W) > C:
        raise SystemExit("steps exceed the KV cache")
    dev = {k: torch.from_numpy(v.view(np.int16)).cuda() for k, v in w.items()}
    model = mk.Model(cfg, dev)
    opt_kw = dict(sched=SCHEDS[args.sched], policy=0 if args.policy == "rr" else 1, attn_splits=args.attn_splits,
                  cooperative=1 if args.cooperative else 0)
    h = mk.mk_build_graph(model.desc, B, C, mk.options(**opt_kw))
    graph = mk.parse_export(mk.mk_export_graph(h))
    kv = torch.from_numpy(np.concatenate([kc.reshape(-1), vc.reshape(-1)]).view(np.int16)).cuda()
    del kc, vc
    logits = torch.empty(B, cfg.vocab, dtype=torch.float32, device="cuda")
    n = max(K, W)
    positions = torch.tensor(np.stack([P0 + s for s in range(n)]), dtype=torch.int32, device="cuda")
    tok0 = torch.tensor(tok, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    nxt = mk.mk_next_tokens(h)

    def run(n_, first=True):
        for s in range(n_):
            tptr = tok0.data_ptr() if (s == 0 and first) else nxt
            mk.mk_decode_step(h, tptr, positions[s].data_ptr(), kv.data_ptr(), logits.data_ptr(), sp)

    run(W)
    torch.cuda.synchronize()
    err = mk.mk_check_device_error(h)
    if err:
        raise SystemExit(f"device error: {err}")
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    run(K)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / K
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    if moe:
        # each step's selections, copied out after the launch's closing event
        sel = torch.empty(K, cfg.n_layers * B * cfg.top_k, dtype=torch.int32, device="cuda")
        eids = mk.mk_expert_ids(h)
    for s_ in range(K):
        ev[s_][0].record(stream)
        mk.mk_decode_step(h, nxt, positions[s_].data_ptr(), kv.data_ptr(), logits.data_ptr(), sp)
        ev[s_][1].record(stream)
        if moe:
            _hip_copy_async(torch, sel[s_].data_ptr(), eids, sel.shape[1] * 4, sp)
    torch.cuda.synchronize()
    ms_launch = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    err = mk.mk_check_device_error(h)
    if err:
        raise SystemExit(f"device error: {err}")
    if moe:
        sel = sel.cpu().numpy().reshape(K, cfg.n_layers, B, cfg.top_k)
        per_step = [moe_step_bytes(cfg, P0 + s, sel[s]) for s in range(K)]
        experts_touched = float(np.mean([sum(len(np.unique(sel[s, l])) for l in range(cfg.n_layers))
                                         for s in range(K)]) / cfg.n_layers)
    else:
        per_step = [step_bytes(cfg, P0 + s) for s in range(K)]
    bytes_mean = np.mean(per_step)
    achieved = bytes_mean / (ms_launch * 1e-3) / 1e9
    mk.mk_destroy(h)
    out = {
        "metric": f"decode tokens/s at batch {B}, " + ("64-expert top-8 MoE on the Llama-1B attention shape, "
                                                        "context 2048" if moe else "Llama-1B shape, mixed contexts"),
        "value": round(B * 1000.0 / ms, 1), "unit": "tokens/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": round(ms, 5), "us_per_step": round(ms * 1000.0, 2), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{cfg.name} greedy decode, batch {B}, "
                               + ("every context 2048" if moe else "contexts uniform in [256, 4096]")
                               + ", bf16 weights and KV cache, one kernel launch per step",
                   "batch": B, "max_ctx": C, "first_positions": P0.tolist(), "sched": args.sched,
                   "workgroups": int(graph["header"]["W"]), "tasks_per_step": int(graph["header"]["n_tasks"]),
                   "attn_splits": int(graph["header"]["attn_splits"])},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None if moe or args.sched != "static" else measured_traffic(B),
                     "algorithmic_bytes_per_step": int(bytes_mean), "kernel_us_per_launch": round(ms_launch * 1000, 2)},
        "input_generation_s": round(t_gen, 1),
    }
    if args.copy_calibration:  # reference dispatches for the HBM byte counters
        src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda").random_(0, 255)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        out["copy_calibration_bytes"] = 256 << 20
        del src, dst
    if moe:
        out["config"]["experts"] = {"n_experts": cfg.n_experts, "top_k": cfg.top_k, "expert_ffn": cfg.expert_ffn,
                                    "mean_distinct_experts_per_layer": round(experts_touched, 2)}
    elif not args.no_baseline:
        # same weights, the same KV cache (the baseline rewrites the slots the megakernel wrote), same first
        # tokens and positions
        out["multi_kernel_baseline"] = baseline_leg(mk, torch, cfg, model.desc, kv, tok, P0, C, K, W, ms)
    if args.trace:
        traced_step_summary(mk, torch, model, B, C, opt_kw, (tok0, positions, kv, logits),
                            f"Trace of one decode step: {out['config']['workload']}", " ".join(["python"] + sys.argv),
                            args.trace)
        out["trace_summary"] = args.trace
    del dev, model
    print(json.dumps(out), flush=True)


def prefill_flops(cfg, T, pos0=0):
    """Algorithmic flops of one prompt: the projections of every token (2 per weight), causal attention
    (QK^T and PV, 2 d flops each per query head and visible key) and the LM head of the last token."""
    h, d = cfg.hidden, cfg.head_dim
    proj = cfg.n_layers * (h * (cfg.n_q + 2 * cfg.n_kv) * d + cfg.n_q * d * h + 3 * h * cfg.ffn)
    keys = sum(pos0 + t + 1 for t in range(T))
    attn = cfg.n_layers * cfg.n_q * 4 * d * keys
    return 2 * proj * T + attn + 2 * cfg.vocab * h


def bench_prefill(args, torch, synth, mk):
    """The prompt (prefill) megakernel: one launch runs a prompt of T tokens at positions 0 .. T-1 through
    the Llama-1B shape (K/V of every layer written, last token's logits and next token).  Synthetic prompt
    tokens uniform over the vocabulary, the same prompt every launch."""
    cfg = synth.configs.LLAMA_1B
    T, K, W = args.prefill, args.steps, args.warmup
    C = max(2048, (T + 63) // 64 * 64)
    t_gen = time.perf_counter()
    w = synth.make_weights(cfg)
    kc, vc = synth.make_kv(cfg, 1, C)
    toks = synth.make_prompt(cfg, T)
    t_gen = time.perf_counter() - t_gen
    dev = {k: torch.from_numpy(v.view(np.int16)).cuda() for k, v in w.items()}
    model = mk.Model(cfg, dev)
    opt_kw = dict(sched=SCHEDS[args.sched], policy=0 if args.policy == "rr" else 1,
                  cooperative=1 if args.cooperative else 0)
    h = mk.mk_build_prefill(model.desc, T, C, mk.options(**opt_kw))
    graph = mk.parse_export(mk.mk_export_graph(h))
    kv = torch.from_numpy(np.concatenate([kc.reshape(-1), vc.reshape(-1)]).view(np.int16)).cuda()
    logits = torch.empty(cfg.vocab, dtype=torch.float32, device="cuda")
    tok = torch.tensor(toks, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    for _ in range(W):
        mk.mk_prefill(h, tok.data_ptr(), 0, kv.data_ptr(), logits.data_ptr(), sp)
    torch.cuda.synchronize()
    err = mk.mk_check_device_error(h)
    if err:
        raise SystemExit(f"device error: {err}")
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    t0 = time.perf_counter()
    for s_ in range(K):
        ev[s_][0].record(stream)
        mk.mk_prefill(h, tok.data_ptr(), 0, kv.data_ptr(), logits.data_ptr(), sp)
        ev[s_][1].record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1000.0 / K
    ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    err = mk.mk_check_device_error(h)
    if err:
        raise SystemExit(f"device error: {err}")
    mk.mk_destroy(h)
    flops = prefill_flops(cfg, T)
    tflops = flops / (ms * 1e-3) / 1e12
    wbytes = cfg.weight_bytes()
    # the same prompt as T decode steps of the decode megakernel (batch 1, one launch per token): the
    # per-step time at the prompt's mid context, times T
    hd = mk.mk_build_graph(model.desc, 1, C, mk.options())
    kvd = kv.clone()
    pos = torch.arange(T // 2, T // 2 + 16, dtype=torch.int32, device="cuda")
    for s_ in range(4):
        mk.mk_decode_step(hd, tok.data_ptr(), pos[s_].data_ptr(), kvd.data_ptr(), 0, sp)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for s_ in range(16):
        mk.mk_decode_step(hd, tok.data_ptr() + 4 * s_, pos[s_].data_ptr(), kvd.data_ptr(), 0, sp)
    e1.record(stream)
    torch.cuda.synchronize()
    dec_us = e0.elapsed_time(e1) * 1000.0 / 16
    mk.mk_destroy(hd)
    del kvd
    out = {
        "metric": f"prompt (prefill) tokens/s, Llama-1B shape, {T}-token prompt, one launch; achieved TFLOP/s vs "
                  "the bf16 matrix-core peak",
        "value": round(T * 1000.0 / ms, 1), "unit": "tokens/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": round(ms, 4), "wall_ms_per_prompt": round(wall_ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{cfg.name} prompt of {T} tokens at positions 0..{T - 1}, bf16 weights and KV "
                               "cache, one kernel launch per prompt",
                   "prompt_tokens": T, "max_ctx": C, "sched": args.sched, "workgroups": int(graph["header"]["W"]),
                   "tasks_per_prompt": int(graph["header"]["n_tasks"])},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 1), "peak": 2500.0, "unit": "TFLOP/s",
                     "frac": round(tflops / 2500.0, 4), "traffic": None,
                     "algorithmic_flops_per_prompt": int(flops), "kernel_us_per_launch": round(ms * 1000, 2),
                     "weight_bytes": int(wbytes), "weights_gbs": round(wbytes / (ms * 1e-3) / 1e9, 1)},
        "as_decode_steps": {"us_per_step": round(dec_us, 1), "ms_for_prompt": round(dec_us * T / 1000.0, 2),
                            "speedup": round(dec_us * T / 1000.0 / ms, 2)},
        "input_generation_s": round(t_gen, 1),
    }
    if args.trace:
        ht = mk.mk_build_prefill(model.desc, T, C, mk.options(trace=1, **opt_kw))
        ex = mk.parse_export(mk.mk_export_graph(ht))
        for _ in range(2):
            mk.mk_prefill(ht, tok.data_ptr(), 0, kv.data_ptr(), logits.data_ptr(), sp)
        torch.cuda.synchronize()
        err = mk.mk_check_device_error(ht)
        if err:
            raise SystemExit(f"device error: {err}")
        tr = mk.mk_read_trace(ht, int(ex["header"]["n_tasks"]))
        mk.mk_destroy(ht)
        with open(args.trace, "w") as f:
            f.write(trace_summary(tr, ex, f"Trace of one prompt launch: {out['config']['workload']}",
                                  " ".join(["python"] + sys.argv)))
        out["trace_summary"] = args.trace
    if not args.no_cpu_baseline:
        from oracle import prefill as oprefill
        n = min(T, 128)
        t0 = time.perf_counter()
        oprefill.prefill(cfg, w, toks[:n], 0, kc.copy(), vc.copy())
        dt = time.perf_counter() - t0
        out["cpu_baseline"] = {"value": round(n / dt, 2), "unit": "tokens/s", "cores": os.cpu_count(),
                               "kind": "oracle", "sample": f"the oracle's double-precision prefill of the first "
                                                           f"{n} prompt tokens (numpy matrix products)"}
    del dev, model
    print(json.dumps(out), flush=True)


def bench_micro(mk):
    """The costs the megakernel trades against each other, measured on this GPU."""
    us_stream, us_graph = mk.mkm_launch_latency(2000)
    hop_x, xa, xb = mk.mkm_pingpong(20000, same_xcd=False)
    hop_s, sa, sb = mk.mkm_pingpong(20000, same_xcd=True)
    fill = {f"{n_wg}wg_depth{d}": round(mk.mkm_lds_fill(8 << 20 if n_wg > 1 else 64 << 20, n_wg, d), 1)
            for n_wg in (1, 256) for d in (4, 8, 16)}
    out = {
        "metric": "microbenchmarks", "n_gpus": 1,
        "empty_kernel_launch_us": {"stream": round(us_stream, 3), "hip_graph": round(us_graph, 3)},
        "dependency_hop_ns": {"cross_xcd": round(hop_x, 1), "xcds": [xa, xb], "same_xcd": round(hop_s, 1),
                              "same_xcds": [sa, sb]},
        "workgroup_barrier_ns": round(mk.mkm_barrier(200000), 2),
        "lds_fill_GBps": fill,
        "stream_read_GBps": round(mk.mkm_stream_read(4 << 30), 1),
    }
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--sched", choices=list(SCHEDS), default="static",
                    help="static per-CU queues, dynamic global queue, event-driven ready queue filled by the "
                         "activating workers, or filled by scheduler waves from activated-event queues")
    ap.add_argument("--policy", choices=["rr", "lpt"], default="rr")
    ap.add_argument("--attn-splits", type=int, default=0)
    ap.add_argument("--cooperative", action="store_true", help="cooperative launch instead of the default plain one")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-baseline", action="store_true", help="skip the one-kernel-per-op baseline")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 256 MiB device copy three times (reference for the HBM byte counters)")
    ap.add_argument("--model", choices=["1b", "8b", "moe"], default="1b",
                    help="8b: the Llama-3-8B shape at batch 1, context 8192; moe: 64 experts of SwiGLU 1024, "
                         "top-8, on the 1B attention shape, in the batch workload (default batch 16); neither "
                         "is the headline line")
    ap.add_argument("--batch", type=int, default=1,
                    help="sequences per step; above 1: the mixed-context batch workload (contexts uniform in "
                         "[256, 4096], room for 4352), reported in tokens/s")
    ap.add_argument("--prefill", type=int, default=0, metavar="T",
                    help="the prompt (prefill) megakernel on a T-token prompt instead of the decode step")
    ap.add_argument("--micro", action="store_true",
                    help="run the measurement microbenchmarks (launch latency, dependency hop, barrier, LDS fill, "
                         "streaming read) and print their JSON line instead of the step benchmark")
    ap.add_argument("--trace", metavar="OUT_MD",
                    help="after the timed steps, run a few steps of a handle built with per-task tracing and write "
                         "the per-operation / per-layer / dependency-hop summary of the last one to OUT_MD")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the measured-traffic record from two rocprofv3 counter-collection CSVs and exit")
    args = ap.parse_args()
    if args.traffic_from:
        wl = None if args.batch == 1 else (f"llama-3.2-1b-shape, batch {args.batch}, contexts uniform in [256, 4096] "
                                           "from the token seed, max_ctx 4352")
        rec = traffic_from_counters(*args.traffic_from, **({"workload": wl} if wl else {}))
        with open(traffic_file(args.batch), "w") as f:
            json.dump(rec, f, indent=1)
        print(json.dumps(rec))
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only (--gpus 1): the megakernel has no "
                                   "multi-GPU sharding", "n_gpus": args.gpus}))
        sys.exit(2)

    import torch
    import synth
    import persistent_megakernel_decode_cu_amd as mk

    if args.prefill:
        return bench_prefill(args, torch, synth, mk)
    if args.micro:
        return bench_micro(mk)
    if args.model == "8b" and args.batch > 1:
        raise SystemExit("the batch workload runs on the 1B shape or the MoE only")
    if args.model == "moe" and args.batch == 1:
        args.batch = 16
    if args.batch > 1:
        return bench_batch(args, torch, synth, mk)
    cfg = synth.configs.LLAMA_1B
    P0, C, K, W = 1024, 2048, args.steps, args.warmup
    if args.model == "8b":
        cfg = synth.configs.LLAMA_8B
        P0, C = 8192, 8448
        args.no_baseline = True
    if P0 + max(K, W) > C:
        raise SystemExit("steps exceed the KV cache")
    t_gen = time.perf_counter()
    w = synth.make_weights(cfg)
    kc, vc = synth.make_kv(cfg, 1, C)
    tok = synth.make_tokens(cfg, 1)
    t_gen = time.perf_counter() - t_gen

    dev = {k: torch.from_numpy(v.view(np.int16)).cuda() for k, v in w.items()}
    model = mk.Model(cfg, dev)
    opt_kw = dict(sched=SCHEDS[args.sched], policy=0 if args.policy == "rr" else 1, attn_splits=args.attn_splits,
                  cooperative=1 if args.cooperative else 0)
    h = mk.mk_build_graph(model.desc, 1, C, mk.options(**opt_kw))
    graph = mk.parse_export(mk.mk_export_graph(h))
    kv = torch.from_numpy(np.concatenate([kc.reshape(-1), vc.reshape(-1)]).view(np.int16)).cuda()
    logits = torch.empty(cfg.vocab, dtype=torch.float32, device="cuda")
    positions = torch.arange(P0, P0 + max(K, W), dtype=torch.int32, device="cuda")
    tok0 = torch.tensor(tok, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    nxt = mk.mk_next_tokens(h)

    def run(n):
        for s in range(n):
            tptr = tok0.data_ptr() if s == 0 else nxt
            mk.mk_decode_step(h, tptr, positions[s:s + 1].data_ptr(), kv.data_ptr(), logits.data_ptr(), sp)

    # first step alone: parity sanity check against the oracle below
    run(1)
    torch.cuda.synchronize()
    err = mk.mk_check_device_error(h)
    if err:
        raise SystemExit(f"device error: {err}")
    first_logits = logits.cpu().numpy().copy()
    # warmup (the KV slots it writes are rewritten by the timed steps)
    run(W)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    run(K)
    e1.record(stream)
    torch.cuda.synchronize()
    ms_total = e0.elapsed_time(e1)
    # the same steps again with an event pair around every launch: the kernel's own duration
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    for s_ in range(K):
        ev[s_][0].record(stream)
        tptr = nxt
        mk.mk_decode_step(h, tptr, positions[s_:s_ + 1].data_ptr(), kv.data_ptr(), logits.data_ptr(), sp)
        ev[s_][1].record(stream)
    torch.cuda.synchronize()
    launch_ms = np.array([a.elapsed_time(b) for a, b in ev])
    ms_launch = float(np.mean(launch_ms))
    err = mk.mk_check_device_error(h)
    if err:
        raise SystemExit(f"device error: {err}")
    ms = ms_total / K
    pos_list = list(range(P0, P0 + K))
    bytes_mean = np.mean([step_bytes(cfg, [p]) for p in pos_list])
    achieved = bytes_mean / (ms_launch * 1e-3) / 1e9
    traffic = measured_traffic(1) if args.model == "1b" else None

    out = {
        "metric": METRIC if args.model == "1b" else "decode µs/step (steps/s) at batch 1, Llama-3-8B shape; achieved HBM GB/s vs peak",
        "value": round(1000.0 / ms, 2),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms, 5),
        "us_per_step": round(ms * 1000.0, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "arithmetic": "bf16 weights and KV cache; fp32 activations between tasks; fp32 accumulation",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name} greedy decode, batch 1, positions {P0}..{P0 + K - 1}, bf16 weights "
                               f"and KV cache, one kernel launch per step",
                   "batch": 1, "first_position": P0, "max_ctx": C, "sched": args.sched, "policy": args.policy,
                   "launch": "cooperative" if args.cooperative else "plain",
                   "workgroups": int(graph["header"]["W"]), "tasks_per_step": int(graph["header"]["n_tasks"]),
                   "attn_splits": int(graph["header"]["attn_splits"])},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "algorithmic_bytes_per_step": int(bytes_mean), "kernel_us_per_launch": round(ms_launch * 1000, 2),
                     "throughput_GBps_incl_launch_gaps": round(bytes_mean / (ms * 1e-3) / 1e9, 1),
                     "kernel_us_p10_median_p90": [round(float(np.percentile(launch_ms, q)) * 1000, 2)
                                                  for q in (10, 50, 90)]},
    }
    mk.mk_destroy(h)
    if args.trace:
        pos2 = positions.reshape(-1, 1)
        traced_step_summary(mk, torch, model, 1, C, opt_kw, (tok0, pos2, kv, logits),
                            f"Trace of one decode step: {out['config']['workload']}", " ".join(["python"] + sys.argv),
                            args.trace)
        out["trace_summary"] = args.trace
    # context: the practical read ceiling of this GPU (a plain 4 GiB streaming read)
    read_peak = mk.mkm_stream_read(4 << 30)
    out["roofline"]["measured_read_peak_GBps"] = round(read_peak, 1)
    out["roofline"]["frac_of_measured_read_peak"] = round(achieved / read_peak, 4)

    if args.copy_calibration:
        n = 256 << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").random_(0, 255)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        out["copy_calibration_bytes"] = n
        del src, dst

    if not args.no_baseline:
        kvb = torch.from_numpy(np.concatenate([kc.reshape(-1), vc.reshape(-1)]).view(np.int16)).cuda()
        out["multi_kernel_baseline"] = baseline_leg(mk, torch, cfg, model.desc, kvb, tok, P0, C, K, W, ms)
        del kvb
    del dev, model

    if not args.no_cpu_baseline:
        cb, first = cpu_baseline(cfg, w, kc, vc, tok, P0, budget_s=10.0 if args.model == "1b" else 20.0)
        hi = host_info()
        cb["cpu_model"] = hi["cpu_model"]
        out["cpu_baseline"] = cb
        out["parity_first_step"] = {
            "max_abs_dlogit": float(np.abs(first_logits.astype(np.float64) - first["logits"][0]).max()),
            "argmax_equal": bool(int(np.argmax(first_logits)) == int(first["next"][0]))}
    out["input_generation_s"] = round(t_gen, 1)
    out["host"] = host_info()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
