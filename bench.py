#!/usr/bin/env python3
"""Benchmark of the int4 (q4f16_1) decode path on one MI355X.

Workload (one "step" = one decode token): a Phi-3-mini-shaped 32-layer stack at
batch 1 -- per layer QKV 9216x3072 -> O 3072x3072 (input: the V slice, i.e.
single-position attention) -> add+RMSNorm -> gate_up 16384x3072 + SiLU-multiply
-> down 3072x8192 -> add+RMSNorm, all weights int4 group-32 (2,038,431,744 bytes
per token), eps 1e-5, gammas ~N(1, 0.1). Each token consumes the previous
token's output: token i+1 starts from residual = h_i and normalised state =
h_i (a unit-RMS vector, as an embedding row would be after the input norm), so
the timed steps form one dependency chain while the residual stream restarts
every token, as it does in decode. Weights
(synthetic, seeded) are resident in HBM before timing starts; 2.04 GB per token
streams past the 256 MB Infinity Cache by itself.

Printed: one JSON line with the effective weight bandwidth (GB/s), the
microseconds per token, the roofline of the dominant kernel (measured with HIP
events on the stream it runs on) and the CPU oracle timed on a bounded sample.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import datagen  # noqa: E402

HBM_PEAK_GBS = 8000.0
F16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense f16 matrix-core peak
METRIC = "effective weight GB/s (% of HBM peak) and µs/token for int4 dequant-GEMV decode stack"

# Threads of the all-cores oracle leg: every host core, at most the 16 the GPU
# box grants one GPU's jobs.
HOST_THREADS = max(1, min(16, os.cpu_count() or 1))

# The pages' own decode rates for Phi-3-mini q4f16_1 (BENCH.md, "Why a third
# baseline"; Zero TVM Documentation, "vs WebLLM"): a browser on an Apple GPU,
# a whole decode step with attention and the LM head. Context, not a target.
BROWSER_CONTEXT = {
    "what": "Phi-3-mini q4f16_1 decode tokens/s in a browser (context only, other hardware, "
            "a whole decode step with attention and LM head)",
    "hardware": "Apple M2 Max, Chrome 150, WebGPU",
    "zero_tvm_tok_s": 83.20,
    "webllm_0_2_80_tok_s": 60.07,
}

PHI3 = dict(d=3072, f=8192, n_qkv=9216, v_off=6144, dv=3072, layers=32, eps=1e-5)
BPW = 0.5625  # bytes per int4 weight: 4 bits + one f16 scale per 32 weights


def layer_shapes(p):
    return [(p["n_qkv"], p["d"]), (p["d"], p["dv"]), (2 * p["f"], p["d"]), (p["d"], p["f"])]


def stack_weight_bytes(p, n_layers=None):
    n_layers = p["layers"] if n_layers is None else n_layers
    return int(n_layers * sum(n * k * BPW for n, k in layer_shapes(p)))


def stack_seed(layer, j):
    """Seed of matrix j (0..7: W/S of QKV, O, gate_up, down) of one layer."""
    return datagen.SEED_BASE + 3_000_000 + 16 * layer + j


def host_layer(p, layer):
    """Packed words and scales of one layer, as host arrays (for the oracle)."""
    mats = []
    for j, (n, k) in enumerate(layer_shapes(p)):
        mats.append(datagen.words(stack_seed(layer, 2 * j), n, k))
        mats.append(datagen.scales(stack_seed(layer, 2 * j + 1), n, k))
    return mats


def host_state(p, n_layers):
    d = p["d"]
    base = datagen.SEED_BASE + 3_900_000
    gi = datagen.gammas(base + 1, n_layers, d)
    gp = datagen.gammas(base + 2, n_layers, d)
    gf = datagen.gammas(base + 3, 1, d)[0]
    r0 = datagen.activations(base + 4, 1, d)[0]
    h0 = datagen.activations(base + 5, 1, d)[0]
    return gi, gp, gf, r0, h0


def build_stack(q4, torch, p, n_layers=None, device="cuda"):
    """Upload a seeded stack. Returns (q4.Stack, device state dict)."""
    n_layers = p["layers"] if n_layers is None else n_layers
    layers = []
    for L in range(n_layers):
        mats = host_layer(p, L)
        layers.append([torch.from_numpy(m.view(np.int32) if m.dtype == np.uint32 else m)
                       .to(device) for m in mats])
    gi, gp, gf, r0, h0 = host_state(p, n_layers)
    g = [torch.from_numpy(a).to(device) for a in (gi, gp, gf)]
    stack = q4.Stack(layers, g[0], g[1], g[2], p["d"], p["f"], p["n_qkv"], p["v_off"], p["dv"],
                     p["eps"])
    st = dict(r0=torch.from_numpy(r0).to(device), h0=torch.from_numpy(h0).to(device),
              gammas=g, host=(gi, gp, gf, r0, h0))
    return stack, st


def time_dominant_kernel(q4, torch, stack, st, p, reps=3):
    """The gate_up matvec as the stack runs it (RMSNorm prologue, SiLU-multiply
    epilogue; the largest matrix of a layer), launched over the 32 layers'
    gate_up weights back to back (a 906 MB rotation). Each launch records its
    own dispatch start and end on HIP events (q4_timer_arm: the kernel's
    execution on the stream it runs on, as a profiler's kernel trace measures
    it); the mean over the launches is returned."""
    d, f = p["d"], p["f"]
    x = st["r0"]
    gamma = st["gammas"][1][0]
    y = torch.empty(f, dtype=torch.float16, device="cuda")
    n = len(stack.layers)
    durs = []
    for _ in range(reps):
        torch.cuda._sleep(20_000_000)  # keeps the stream busy while launches queue
        for L in range(n):
            q4.timer_arm(L)
            q4.gemv_ex(stack.layers[L][4], stack.layers[L][5], x, y=y, kind=q4.EPI_SILU_MUL,
                       norm_gamma=gamma, eps=p["eps"])
        durs += [q4.timer_read(L) for L in range(n)]
    us = float(np.mean(durs))
    bytes_per_launch = 2 * f * d * BPW
    return us, bytes_per_launch


COUNTER_PROFILE = os.path.join(ROOT, "profiles", "traffic_gate_up_phi3.md")
COPY_BYTES = 256 << 20  # plain device copy used to calibrate the byte counters


def kernel_source_hash():
    """Hash of the sources that define the dominant kernel: counters taken on an
    older kernel are not reported for the current one."""
    import hashlib
    h = hashlib.sha256()
    for f in ("q4_gemv.hip", "q4_dequant.h", "q4_common.h"):
        with open(os.path.join(ROOT, "int4_weight_only_q4_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def counter_workload(q4, torch, stack, st, p):
    """What the counter runs profile: a plain device copy of COPY_BYTES (three
    times; it calibrates FETCH_SIZE / WRITE_SIZE), then the dominant kernel over
    the 32 layers' gate_up weights, launched as time_dominant_kernel does."""
    src = torch.ones(COPY_BYTES // 4, dtype=torch.int32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print("copy calibration done", file=sys.stderr, flush=True)
    x, gamma = st["r0"], st["gammas"][1][0]
    y = torch.empty(p["f"], dtype=torch.float16, device="cuda")
    for L in range(len(stack.layers)):
        q4.gemv_ex(stack.layers[L][4], stack.layers[L][5], x, y=y, kind=q4.EPI_SILU_MUL,
                   norm_gamma=gamma, eps=p["eps"])
    torch.cuda.synchronize()
    print("dominant kernel launches done", file=sys.stderr, flush=True)


def _counter_rows(d):
    """(kernel name, counter value) rows of the rocprofv3 CSV counter output under d."""
    import csv
    import glob
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit("no counter_collection.csv under %s" % d)
    rows = []
    for fn in files:
        with open(fn) as fh:
            for r in csv.DictReader(fh):
                rows.append((r["Kernel_Name"], r["Counter_Name"], float(r["Counter_Value"])))
    return rows


def summarize_counters(fetch_dir, write_dir):
    """Per-dispatch FETCH_SIZE / WRITE_SIZE (KiB) of the copy and of the dominant
    kernel, the copy-calibrated HBM bytes per launch, written to COUNTER_PROFILE."""
    res = {}
    for cname, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = [r for r in _counter_rows(d) if r[1] == cname]
        # the calibration copy is the largest copy dispatch of the run (weight
        # uploads before it are smaller)
        copy = sorted(v for k, _, v in rows if "copy" in k.lower())[-3:]
        dom = [v for k, _, v in rows if "k_gemv<32, 3, 2, 1, 1," in k]
        if not copy or not dom:
            raise SystemExit("%s: missing copy (%d) or dominant-kernel (%d) dispatches" % (
                cname, len(copy), len(dom)))
        copy_kib = float(np.median(copy))
        factor = (COPY_BYTES / 1024.0) / copy_kib
        res[cname] = dict(copy_kib=round(copy_kib, 1), factor=round(factor, 4),
                          dominant_kib=round(float(np.mean(dom)), 1), dispatches=len(dom))
    traffic = 1024.0 * (res["FETCH_SIZE"]["dominant_kib"] * res["FETCH_SIZE"]["factor"] +
                        res["WRITE_SIZE"]["dominant_kib"] * res["WRITE_SIZE"]["factor"])
    algo = 2 * PHI3["f"] * PHI3["d"] * BPW
    rec = dict(kernel="gate_up 16384x3072 matvec (k_gemv<32, 3, 2, 1, 1, false>)",
               source_hash=kernel_source_hash(), traffic_bytes_per_launch=int(traffic),
               algorithmic_bytes_per_launch=int(algo), ratio=round(traffic / algo, 4), **res)
    cmd = ("export REPO=$PWD && cd /tmp && export TMPDIR=/tmp && timeout -s KILL 150 "
           "rocprofv3 --pmc {C} "
           "--output-format csv -d $OUT/pmc_{c} -o pmc -- "
           "python3 $REPO/bench.py --counters")
    text = [
        "# HBM traffic of the dominant kernel: gate_up 16384x3072 matvec, Phi-3-mini stack",
        "",
        "Two counter runs (one counter group each), from the repository root on one MI355X "
        "(OUT: an output directory):",
        "",
        "```",
        cmd.format(C="FETCH_SIZE", c="fetch"),
        cmd.format(C="WRITE_SIZE", c="write"),
        "python3 bench.py --summarize-counters $OUT/pmc_fetch $OUT/pmc_write",
        "```",
        "",
        "`bench.py --counters` runs a plain %d MiB device copy three times, then the "
        "gate_up kernel over the 32 layers' weights (the launch `bench.py` times). Each "
        "counter is scaled by (copy bytes / what the counter reads for the copy)." % (COPY_BYTES >> 20),
        "",
        "| counter | copy KiB | factor | gate_up KiB per dispatch | dispatches |",
        "|---|---|---|---|---|",
    ]
    for cname in ("FETCH_SIZE", "WRITE_SIZE"):
        r = res[cname]
        text.append("| %s | %.1f | %.4f | %.1f | %d |" % (cname, r["copy_kib"], r["factor"],
                                                        r["dominant_kib"], r["dispatches"]))
    text += ["",
             "Calibrated HBM bytes per launch: %d (algorithmic: %d, ratio %.3f)." % (
                 int(traffic), int(algo), traffic / algo),
             "",
             "Machine-readable (read by bench.py; ignored once the kernel sources change):",
             "",
             json.dumps(rec), ""]
    with open(COUNTER_PROFILE, "w") as fh:
        fh.write("\n".join(text))
    print(json.dumps(rec))


def committed_traffic():
    """Calibrated HBM bytes per launch of the dominant kernel from the committed
    counter summary, or None if absent or taken on other kernel sources."""
    try:
        with open(COUNTER_PROFILE) as fh:
            for line in fh:
                if line.startswith("{"):
                    rec = json.loads(line)
                    if rec.get("source_hash") == kernel_source_hash():
                        return int(rec["traffic_bytes_per_launch"])
    except (OSError, ValueError, KeyError):
        pass
    return None


STACK_TRACE_PROFILE = os.path.join(ROOT, "profiles", "kernel_trace_phi3_stack_decode.md")
DOMINANT_KERNEL = "k_gemv<32, 3, 2, 1, 1, false>"  # gate_up: RMSNorm prologue, SiLU epilogue
DOMINANT_REPS = 3  # passes of time_dominant_kernel over the layers' gate_up weights
STACK_KERNEL_ROLES = {
    DOMINANT_KERNEL: "gate_up 16384x3072, RMSNorm prologue + SiLU-multiply epilogue",
    "k_gemv<32, 3, 2, 0, 1, false>": "QKV 9216x3072, RMSNorm prologue (layers 1..31)",
    "k_gemv<64, 4, 1, 2, 0, false>": "down 3072x8192, residual-add epilogue",
    "k_gemv<32, 3, 1, 2, 0, false>": "O 3072x3072, residual-add epilogue",
    "k_gemv<32, 3, 2, 0, 0, false>": "QKV 9216x3072 (layer 0, given h)",
    "k_add_rmsnorm_vec<2>": "final RMSNorm (and the trace norms of the parity check)",
}


def summarize_trace(trace_csv, status):
    """The per-kernel summary of a rocprofv3 kernel trace of `bench.py
    --no-cpu-baseline`, and the dominant kernel's mean dispatch duration inside
    the stack's tokens (every gate_up dispatch but the timing loop's last ones)
    against the timing loop's, written to STACK_TRACE_PROFILE with the hash of
    the kernel's sources."""
    import csv
    with open(trace_csv, newline="") as fh:
        rows = sorted(csv.DictReader(fh), key=lambda r: int(r["Start_Timestamp"]))

    def name(r):
        return r["Kernel_Name"].replace("void ", "").replace(
            "q4::(anonymous namespace)::", "").split("(")[0]

    def dur(r):
        return (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0

    p = PHI3
    per = {}
    for r in rows:
        per.setdefault(name(r), []).append(dur(r))
    gu = per.get(DOMINANT_KERNEL, [])
    loop_n = DOMINANT_REPS * p["layers"]
    if len(gu) <= loop_n:
        raise SystemExit("the trace holds %d dispatches of %s, not the stack's and the "
                         "timing loop's" % (len(gu), DOMINANT_KERNEL))
    bytes_per_launch = int(2 * p["f"] * p["d"] * BPW)

    def gbs(us):
        return bytes_per_launch / (us * 1e-6) / 1e9

    stack_us = float(np.mean(gu[:-loop_n]))
    loop_us = float(np.mean(gu[-loop_n:]))
    rec = dict(source_hash=kernel_source_hash(), kernel=DOMINANT_KERNEL,
               bytes_per_launch=bytes_per_launch,
               in_stack_dispatches=len(gu) - loop_n, in_stack_us=round(stack_us, 3),
               loop_dispatches=loop_n, loop_us=round(loop_us, 3), profiled_status=int(status))
    text = [
        "# Kernel trace: Phi-3-mini-shaped 32-layer int4 decode stack, batch 1 (bench.py)",
        "",
        "Commands (from the repository root, on one MI355X; OUT: an output directory; the "
        "summary from the trace CSV):",
        "",
        "```",
        "export REPO=$PWD && cd /tmp && export TMPDIR=/tmp && rocprofv3 --kernel-trace --stats "
        "--output-format csv -d $OUT/prof_bench -o bench -- python3 $REPO/bench.py "
        "--no-cpu-baseline; echo $?",
        "python3 bench.py --summarize-trace $OUT/prof_bench/bench_kernel_trace.csv STATUS",
        "```",
        "",
        "The profiled command exited with status %d%s." % (
            int(status), " (no fault at the profiler's exit)" if int(status) == 0 else ""),
        "Durations are the dispatch durations of the kernel trace over every dispatch of the "
        "run: the parity check, the eager warm-up and graph-check tokens, the warm-up and timed "
        "tokens replayed from the captured token graphs, and the dominant-kernel timing loop "
        "(the library's kernels with the largest total time).",
        "",
        "| kernel | role | dispatches | mean us | min us | max us |",
        "|---|---|---|---|---|---|",
    ]
    ours = {k: v for k, v in per.items() if k.startswith("k_")}  # the library's kernels
    for k, v in sorted(ours.items(), key=lambda kv: -sum(kv[1]))[:8]:
        text.append("| `%s` | %s | %d | %.3f | %.3f | %.3f |" % (
            k, STACK_KERNEL_ROLES.get(k, ""), len(v), np.mean(v), min(v), max(v)))
    text += [
        "",
        "Dominant kernel (the roofline line of bench.py): the gate_up matvec, %s B per launch."
        % format(bytes_per_launch, ","),
        "",
        "| dispatches | mean us per launch | GB/s | % of 8 TB/s |",
        "|---|---|---|---|",
        "| inside the stack's tokens (the first %d) | %.3f | %.0f | %.1f |" % (
            len(gu) - loop_n, stack_us, gbs(stack_us), 100 * gbs(stack_us) / HBM_PEAK_GBS),
        "| the timing loop, launched back to back over the layers' weights (the last %d) "
        "| %.3f | %.0f | %.1f |" % (loop_n, loop_us, gbs(loop_us), 100 * gbs(loop_us) / HBM_PEAK_GBS),
        "",
        "Under the kernel trace the whole stack runs slower than without it, so in-stack "
        "durations here are upper bounds. bench.py reports the in-stack figure beside its "
        "roofline line while the kernel's sources are unchanged (the hash below).",
        "",
        json.dumps(rec),
        "",
    ]
    with open(STACK_TRACE_PROFILE, "w") as fh:
        fh.write("\n".join(text))
    print(json.dumps(rec))


def in_stack_line(bytes_per_launch):
    """The roofline line's kernel as it runs inside the stack: the mean of its
    dispatches over the stack's tokens in the committed kernel trace (the line
    itself times it back to back over the layers' weights), or None."""
    rec = committed_in_stack()
    if rec is None or rec.get("bytes_per_launch") != int(bytes_per_launch):
        return None
    us = rec["in_stack_us"]
    achieved = bytes_per_launch / (us * 1e-6) / 1e9
    return {"us_per_launch": us, "achieved": round(achieved, 1),
            "frac": round(achieved / HBM_PEAK_GBS, 4), "dispatches": rec["in_stack_dispatches"],
            "source": "rocprofv3 kernel trace of this command (committed summary), "
                      "upper bound: the profiler slows the stack"}


def committed_in_stack():
    """The dominant kernel's mean dispatch duration inside the stack from the
    committed kernel-trace summary, or None if absent or taken on other kernel
    sources."""
    try:
        with open(STACK_TRACE_PROFILE) as fh:
            for line in fh:
                if line.startswith("{"):
                    rec = json.loads(line)
                    if rec.get("source_hash") == kernel_source_hash():
                        return rec
    except (OSError, ValueError):
        pass
    return None


GEMV_TABLE_PROFILE = os.path.join(ROOT, "profiles", "gemv_table_phi3_qwen3_moe.md")
MOE_KERNELS = ("the gate_up stage one expert kernel; the down stage one kernel with the "
               "routing-weighted combine up to 32 (token, slot) pairs, else an expert kernel "
               "and a finishing kernel")
QWEN3 = dict(qkv=(6144, 2560), o=(2560, 4096), gate_up=(19456, 2560), down=(2560, 9728),
             lm_head=(151936, 2560))


def _rotation(torch, n, k, seed, min_bytes=512 << 20):
    """Distinct device copies of one seeded n x k matrix, together more than
    min_bytes, so that cycling through them reads HBM rather than the 256 MB
    Infinity Cache."""
    W = torch.from_numpy(datagen.words(seed, n, k).view(np.int32)).cuda()
    S = torch.from_numpy(datagen.scales(seed + 1, n, k)).cuda()
    copies = max(2, -(-min_bytes // int(n * k * BPW)))
    return [(W, S)] + [(W.clone(), S.clone()) for _ in range(copies - 1)]


def _time(q4, torch, launch, count, timed_kernels=True):
    """(us per call back to back, us per matvec kernel from its dispatch events)."""
    for i in range(4):
        launch(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(10_000_000)
    e0.record()
    for i in range(count):
        launch(i)
    e1.record()
    torch.cuda.synchronize()
    per_call = e0.elapsed_time(e1) * 1e3 / count
    per_kernel = None
    if timed_kernels:
        n = min(count, 64)
        torch.cuda._sleep(10_000_000)
        for i in range(n):
            q4.timer_arm(i)
            launch(i)
        per_kernel = float(np.mean([q4.timer_read(i) for i in range(n)]))
    return per_call, per_kernel


def _time_graph(q4, torch, launch, count, reps=5):
    """us per call from a captured HIP graph of `count` calls, replayed `reps`
    times (no host launch overhead; the calls enqueue kernels only: no
    allocation, copy or memset, the workspace of the capture stream being
    sized by eager warm-up calls on that stream)."""
    # warm-up and capture on one stream: the library's workspace is per stream
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        for i in range(4):
            launch(i)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=st):
        for i in range(count):
            launch(i)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / (reps * count)


def gemv_table(q4, torch, o=None, threads=HOST_THREADS):
    """Per-GEMV throughput at the single-GEMV, Phi-3-mini, Qwen3-4B (M = 1 and
    8) and MoE workloads, weights rotated past the Infinity Cache; with the
    oracle `o`, the oracle's time for the same matmul (or MoE layer) on one
    host thread and on `threads` threads beside each GPU row."""
    rows = []
    base = datagen.SEED_BASE + 5_000_000

    def add(workload, shape, m, weight_bytes, launch, count=200, note="", per_call=False,
            oracle_us=None):
        call_us, kern_us = _time(q4, torch, launch, count)
        us = call_us if per_call or kern_us is None else kern_us
        gbs = weight_bytes / (us * 1e-6) / 1e9
        row = dict(workload=workload, shape=shape, m=m, weight_bytes=int(weight_bytes),
                   us_kernel=round(kern_us, 3) if kern_us is not None else None,
                   us_per_call=round(call_us, 3), gbs=round(gbs, 1),
                   pct_peak=round(100 * gbs / HBM_PEAK_GBS, 1), note=note)
        if o is not None and oracle_us is not None:
            row["oracle_us_1t"] = round(oracle_us(1)[0], 1)
            row["oracle_us_all"] = round(oracle_us(threads)[0], 1)
        rows.append(row)
        print("  %-22s %-12s M=%-2d %8.3f us/kernel %8.3f us/call %8.1f GB/s%s" % (
            workload, shape, m, us, call_us, gbs,
            "  oracle %.0f / %.0f us" % (row["oracle_us_1t"], row["oracle_us_all"])
            if "oracle_us_1t" in row else ""), file=sys.stderr, flush=True)

    def gemv_rows(workload, shapes, ms, seed0):
        for j, (name, (n, k)) in enumerate(shapes):
            rot = _rotation(torch, n, k, seed0 + 10 * j)
            wb = n * k * BPW
            Wh = datagen.words(seed0 + 10 * j, n, k) if o is not None else None
            Sh = datagen.scales(seed0 + 10 * j + 1, n, k) if o is not None else None
            for m in ms:
                xh = datagen.activations(seed0 + 10 * j + 2, m, k)
                x = torch.from_numpy(xh).cuda()
                y = torch.empty((m, n), dtype=torch.float16, device="cuda")
                if m == 1:
                    def launch(i, rot=rot, x=x, y=y):
                        W, S = rot[i % len(rot)]
                        q4.gemv(W, S, x[0], y=y[0])
                else:
                    def launch(i, rot=rot, x=x, y=y):
                        W, S = rot[i % len(rot)]
                        q4.gemv_batched(W, S, x, y=y)
                add(workload, "%s %dx%d" % (name, n, k), m, wb, launch,
                    count=max(20, min(200, int(4e9 / wb))),
                    oracle_us=lambda t, Wh=Wh, Sh=Sh, xh=xh: oracle_rows_us(o, Wh, Sh, xh, t))
            del rot, Wh, Sh
            torch.cuda.empty_cache()

    gemv_rows("single GEMV", [("W", (512, 256))], [1], base)
    gemv_rows("Phi-3-mini layer", [("QKV", (9216, 3072)), ("O", (3072, 3072)),
                                   ("gate_up", (16384, 3072)), ("down", (3072, 8192))], [1],
              base + 1000)
    gemv_rows("Qwen3-4B", list(QWEN3.items()), [1, 2, 4, 8], base + 2000)

    # the MLX affine format (w = s * q + b, group 64) at the Qwen3-4B shapes
    for j, (name, (n, k)) in enumerate([("qkv", (6144, 2560)), ("gate_up", (19456, 2560)),
                                        ("down", (2560, 9728))]):
        Wh = torch.from_numpy(datagen.words(base + 2600 + 10 * j, n, k).view(np.int32)).cuda()
        Sh = torch.from_numpy(datagen.scales(base + 2601 + 10 * j, n, k // 2)).cuda()
        Bh = torch.from_numpy(datagen.normal_f16(base + 2602 + 10 * j, (n, k // 64), 0.0, 0.05)).cuda()
        copies = max(2, -(-(512 << 20) // int(n * k * BPW)))
        rot = [(Wh, Sh, Bh)] + [(Wh.clone(), Sh.clone(), Bh.clone()) for _ in range(copies - 1)]
        wb = n * k * BPW
        for m in (1, 2, 4, 8):
            x = torch.from_numpy(datagen.activations(base + 2603 + 10 * j, m, k)).cuda()
            y = torch.empty((m, n), dtype=torch.float16, device="cuda")

            def launch(i, rot=rot, x=x, y=y, m=m):
                W, S, B = rot[i % len(rot)]
                q4.gemv_affine(W, S, B, x[0] if m == 1 else x, y=y[0] if m == 1 else y)
            add("Qwen3-4B MLX affine", "%s %dx%d" % (name, n, k), m, wb, launch,
                count=max(20, min(200, int(4e9 / wb))),
                note="w = s*q + b, group 64 (scales and biases f16: 4.5 bits per weight)")
        del rot
        torch.cuda.empty_cache()

    # LM head with f32 logits and the greedy token (the whole call: matvec and
    # argmax kernels); the Qwen3-4B head is tied to the embedding matrix
    for j, (workload, n, k, ms) in enumerate([("Phi-3-mini LM head", 32064, 3072, [1]),
                                             ("Qwen3-4B LM head", 151936, 2560, [1, 2, 4, 8])]):
        rot = _rotation(torch, n, k, base + 2500 + 10 * j)
        wb = n * k * BPW
        for m in ms:
            x = torch.from_numpy(datagen.activations(base + 2502 + 10 * j, m, k)).cuda()
            logits = torch.empty((m, n), dtype=torch.float32, device="cuda")
            tok = torch.empty(m, dtype=torch.int32, device="cuda")

            def launch(i, rot=rot, x=x, logits=logits, tok=tok, m=m):
                W, S = rot[i % len(rot)]
                q4.lm_head_argmax(W, S, x[0] if m == 1 else x, logits=logits[0] if m == 1
                                  else logits, tokens=tok)
            add(workload + " + argmax", "%dx%d" % (n, k), m, wb, launch,
                count=max(20, min(200, int(4e9 / wb))), per_call=True,
                note="f32 logits; GB/s over the whole call (matvec + argmax)")
        del rot
        torch.cuda.empty_cache()

    # RoPE + paged KV append fused into the Phi-3 QKV matvec, and decode
    # attention over the paged cache (Phi-3: 32 heads of 96, 16-slot pages);
    # every cache is one layer's, rotated past 512 MB as the layers' caches
    # would be in a decode step. Attention bytes = L * heads * 96 * 2 (K, V) * 2.
    d = q4.attn_desc(32, 32, 96, 16, 257)
    table = torch.arange(257, dtype=torch.int32, device="cuda")
    rot = _rotation(torch, 9216, 3072, base + 2800)
    x = torch.from_numpy(datagen.activations(base + 2802, 1, 3072)).cuda()
    kv = q4.kv_cache(d)
    qo = torch.empty(3072, dtype=torch.float16, device="cuda")
    pos1 = torch.tensor([1234], dtype=torch.int32, device="cuda")

    def launch(i, rot=rot, x=x, kv=kv, qo=qo):
        W, S = rot[i % len(rot)]
        q4.qkv_rope_append(W, S, x[0], d, pos1, table, kv, q_out=qo)
    add("Phi-3-mini QKV + RoPE + KV append", "9216x3072", 1, 9216 * 3072 * BPW, launch,
        count=200, note="fused epilogue: Q rotated out, K and V into the cache slot")
    del rot, kv
    torch.cuda.empty_cache()
    for L in (256, 1024, 4112):
        npages = -(-L // 16)
        dl = q4.attn_desc(32, 32, 96, 16, npages)
        cache_bytes = npages * q4.kv_page_bytes(dl)
        first = torch.from_numpy(datagen.normal_f16(base + 2900, (npages, 2, 32, 16, 96))).cuda()
        caches = [first] + [first.clone() for _ in range(max(2, -(-(512 << 20) // cache_bytes)) - 1)]
        tab = torch.arange(npages, dtype=torch.int32, device="cuda")
        q = torch.from_numpy(datagen.activations(base + 2950, 1, 3072)).cuda()
        out = torch.empty(3072, dtype=torch.float16, device="cuda")
        posL = torch.tensor([L - 1], dtype=torch.int32, device="cuda")

        def launch(i, caches=caches, tab=tab, q=q, out=out, posL=posL, dl=dl, L=L):
            q4.attention_decode(q[0], caches[i % len(caches)], tab, posL, L, dl, out=out)
        launch(0)
        torch.cuda.synchronize()
        eager = out.clone()
        call_us = _time_graph(q4, torch, launch, 2 * len(caches))
        launch(0)
        torch.cuda.synchronize()
        if not torch.equal(out, eager):
            raise RuntimeError("graph replay of the attention differs from the eager call")
        wb = L * 32 * 96 * 2 * 2
        gbs = wb / (call_us * 1e-6) / 1e9
        rows.append(dict(workload="attention decode (32 heads x 96, paged)", shape="L=%d" % L, m=1,
                         weight_bytes=int(wb), us_kernel=None, us_per_call=round(call_us, 3),
                         gbs=round(gbs, 1), pct_peak=round(100 * gbs / HBM_PEAK_GBS, 1),
                         note="K and V bytes read; %d caches rotated; split attention + "
                              "combine; timed from a HIP graph of the calls" % len(caches)))
        print("  attention L=%-5d %8.3f us/call %8.1f GB/s" % (L, call_us, gbs), file=sys.stderr,
              flush=True)
        del caches, first
        torch.cuda.empty_cache()

    # MoE layer: 128 experts, top-8; gate_up stage (SiLU-multiply) + down stage
    # with the routing-weighted combine. Two copies of the expert stack are
    # alternated and the routing is drawn from a pool of 256, so the touched
    # experts are not hot in cache; GB/s counts the unique experts touched.
    E, hidden, f, topk = 128, 2048, 768, 8
    stacks = []
    for c in range(2):
        Wg = torch.from_numpy(datagen.words(base + 3000 + c, E * 2 * f, hidden)
                              .view(np.int32).reshape(E, 2 * f, hidden // 8)).cuda()
        Sg = torch.from_numpy(datagen.scales(base + 3100 + c, E * 2 * f, hidden)
                              .reshape(E, 2 * f, hidden // 32)).cuda()
        Wd = torch.from_numpy(datagen.words(base + 3200 + c, E * hidden, f)
                              .view(np.int32).reshape(E, hidden, f // 8)).cuda()
        Sd = torch.from_numpy(datagen.scales(base + 3300 + c, E * hidden, f)
                              .reshape(E, hidden, f // 32)).cuda()
        stacks.append((Wg, Sg, Wd, Sd))
    expert_bytes = (2 * f * hidden + hidden * f) * BPW
    moe_host = None
    if o is not None:  # the first copy of the expert stack on the host
        moe_host = (datagen.words(base + 3000, E * 2 * f, hidden).reshape(E, 2 * f, hidden // 8),
                    datagen.scales(base + 3100, E * 2 * f, hidden).reshape(E, 2 * f, hidden // 32),
                    datagen.words(base + 3200, E * hidden, f).reshape(E, hidden, f // 8),
                    datagen.scales(base + 3300, E * hidden, f).reshape(E, hidden, f // 32))
    for t in (1, 4, 16):
        ids_h, w_h = datagen.routing_pool(base + 4000 + t, 256, t, E, topk)
        ids = torch.from_numpy(ids_h).cuda()
        rw = torch.from_numpy(w_h).cuda()
        x = torch.from_numpy(datagen.activations(base + 4100 + t, t, hidden)).cuda()
        uniq = float(np.mean([len(np.unique(ids_h[i])) for i in range(len(ids_h))]))

        u = torch.empty((t, topk, f), dtype=torch.float16, device="cuda")
        y = torch.empty((t, hidden), dtype=torch.float16, device="cuda")

        def launch(i, ids=ids, rw=rw, x=x, u=u, y=y):
            Wg, Sg, Wd, Sd = stacks[i & 1]
            q4.moe_gemv(Wg, Sg, ids[i % 256], x, ldx=hidden, x_slot_stride=0, epi_silu=True,
                        y=u)
            q4.moe_gemv(Wd, Sd, ids[i % 256], u, ldx=topk * f, x_slot_stride=f,
                        route_w=rw[i % 256], y=y)

        call_us = _time_graph(q4, torch, launch, 32)
        wb = uniq * expert_bytes
        gbs = wb / (call_us * 1e-6) / 1e9
        row = dict(workload="MoE layer (128 experts, top-8)", shape="T=%d" % t, m=t,
                   weight_bytes=int(wb), us_kernel=None, us_per_call=round(call_us, 3),
                   gbs=round(gbs, 1), pct_peak=round(100 * gbs / HBM_PEAK_GBS, 1),
                   note="%.2f unique experts per layer on average; both stages, timed from a "
                        "HIP graph of 32 layers (%s)" % (uniq, MOE_KERNELS))
        if o is not None:
            row["oracle_us_1t"], row["oracle_us_all"] = (
                round(oracle_moe_us(o, moe_host, ids_h[0], w_h[0],
                                    datagen.activations(base + 4100 + t, t, hidden), f, thr), 1)
                for thr in (1, threads))
        rows.append(row)
        print("  MoE T=%-2d %8.3f us/layer %8.1f GB/s (unique experts %.2f)%s" % (
            t, call_us, gbs, uniq, "  oracle %.0f / %.0f us" % (
                row["oracle_us_1t"], row["oracle_us_all"]) if o is not None else ""),
            file=sys.stderr, flush=True)
    # Phi-3-mini decode token, 32 layers, with the real attention step over L
    # cached positions (each layer its own cache; the step appends at L - 1)
    stack, stt = build_stack(q4, torch, PHI3)
    r_out = torch.empty(PHI3["d"], dtype=torch.float16, device="cuda")
    h_out = torch.empty(PHI3["d"], dtype=torch.float16, device="cuda")
    for L in (1024, 4096):
        npages = -(-L // 16)
        g = q4.attn_desc(32, 32, 96, 16, npages)
        first = torch.from_numpy(datagen.normal_f16(base + 3500, (npages, 2, 32, 16, 96))).cuda()
        caches = [first] + [first.clone() for _ in range(PHI3["layers"] - 1)]
        tab = torch.arange(npages, dtype=torch.int32, device="cuda")
        posL = torch.tensor([L - 1], dtype=torch.int32, device="cuda")

        def launch(i, g=g, caches=caches, tab=tab, posL=posL, L=L):
            stack.decode_attn(g, caches, tab, posL, L, stt["r0"], stt["h0"], r_out, h_out)
        call_us = _time_graph(q4, torch, launch, 10)
        wb = stack_weight_bytes(PHI3) + PHI3["layers"] * L * 32 * 96 * 2 * 2
        gbs = wb / (call_us * 1e-6) / 1e9
        rows.append(dict(workload="Phi-3-mini decode token with attention (32 layers)",
                         shape="L=%d" % L, m=1, weight_bytes=int(wb), us_kernel=None,
                         us_per_call=round(call_us, 3), gbs=round(gbs, 1),
                         pct_peak=round(100 * gbs / HBM_PEAK_GBS, 1),
                         note="q4_stack_decode_attn: 6 or 7 kernels per layer, timed from a "
                              "HIP graph of the calls; bytes = weights + K and V of every layer"))
        print("  decode token + attention L=%-5d %9.1f us/token %8.1f GB/s" % (L, call_us, gbs),
              file=sys.stderr, flush=True)
        del caches, first
        torch.cuda.empty_cache()
    del stack
    torch.cuda.empty_cache()
    return rows


PREFILL = [("Phi-3-mini prefill", "QKV", 9216, 3072, 1024),
           ("Phi-3-mini prefill", "O", 3072, 3072, 1024),
           ("Phi-3-mini prefill", "gate_up", 16384, 3072, 1024),
           ("Phi-3-mini prefill", "down", 3072, 8192, 1024),
           ("Qwen3-4B prefill chunk", "gate_up", 19456, 2560, 256),
           ("Qwen3-4B prefill chunk", "down", 2560, 9728, 256),
           ("Qwen3-4B prefill chunk", "o", 2560, 4096, 256)]


def prefill_table(q4, torch):
    """Prefill matmul (q4_gemm) throughput at the Phi-3-mini (M = 1024) and
    Qwen3-4B (M = 256, the pages' chunk shapes) matrices, both weight modes,
    and the 16-row decode launches (q4_gemv_batched) at M = 64 beside q4_gemm
    at M = 64 for the crossover. Weights rotated past the Infinity Cache."""
    rows = []
    base = datagen.SEED_BASE + 6_000_000

    def add(workload, shape, m, n, k, launch, note):
        # whole calls back to back: a K-split call is two kernels (tiles, combine)
        call_us, _ = _time(q4, torch, launch, 40, timed_kernels=False)
        us = call_us
        tf = 2.0 * m * n * k / (us * 1e-6) / 1e12
        rows.append(dict(workload=workload, shape=shape, m=m, us_kernel=round(us, 2),
                         us_per_call=round(call_us, 2), tflops=round(tf, 1),
                         pct_f16_peak=round(100 * tf / F16_MFMA_PEAK_TFLOPS, 1), note=note))
        print("  %-24s %-18s M=%-5d %9.2f us %8.1f TFLOP/s  %s" % (workload, shape, m, us, tf,
                                                                     note), file=sys.stderr,
              flush=True)

    for j, (workload, name, n, k, m) in enumerate(PREFILL):
        rot = _rotation(torch, n, k, base + 10 * j)
        x = torch.from_numpy(datagen.activations(base + 10 * j + 2, m, k)).cuda()
        y = torch.empty((m, n), dtype=torch.float16, device="cuda")
        for mode, label in ((q4.GEMM_EXACT, "exact weights"), (q4.GEMM_F16_WEIGHT, "f16 weights")):
            def launch(i, rot=rot, x=x, y=y, mode=mode):
                W, S = rot[i % len(rot)]
                q4.gemm(W, S, x, y=y, weights=mode)
            add(workload, "%s %dx%d" % (name, n, k), m, n, k, launch, "q4_gemm, " + label)
        if j == 0:
            for mm in (16, 64):
                xs, ys = x[:mm], y[:mm]

                def launch(i, rot=rot, xs=xs, ys=ys):
                    W, S = rot[i % len(rot)]
                    q4.gemv_batched(W, S, xs, y=ys)
                add(workload, "%s %dx%d" % (name, n, k), mm, n, k, launch,
                    "q4_gemv_batched (16-row decode launches)")

                def launch(i, rot=rot, xs=xs, ys=ys):
                    W, S = rot[i % len(rot)]
                    q4.gemm(W, S, xs, y=ys)
                add(workload, "%s %dx%d" % (name, n, k), mm, n, k, launch,
                    "q4_gemm, exact weights")
        # context: torch's dense f16 matmul (hipBLASLt) of the same shape, weights
        # already f16 (four times the weight bytes, no dequantisation)
        xd = x.clone()
        wd = torch.randn(k, n, dtype=torch.float16, device="cuda")

        def launch(i, xd=xd, wd=wd, y=y):
            torch.mm(xd, wd, out=y)
        call_us, _ = _time(q4, torch, launch, 40, timed_kernels=False)
        tf = 2.0 * m * n * k / (call_us * 1e-6) / 1e12
        rows.append(dict(workload=workload, shape="%s %dx%d" % (name, n, k), m=m,
                         us_kernel=round(call_us, 2), us_per_call=round(call_us, 2),
                         tflops=round(tf, 1), pct_f16_peak=round(100 * tf / F16_MFMA_PEAK_TFLOPS, 1),
                         note="reference: torch.mm dense f16 (not int4)"))
        print("  %-24s %-18s M=%-5d %9.2f us %8.1f TFLOP/s  reference: torch.mm dense f16" % (
            workload, "%s %dx%d" % (name, n, k), m, call_us, tf), file=sys.stderr, flush=True)
        del rot, wd, xd
        torch.cuda.empty_cache()

    # the MLX affine format (w = s * q + b, group 64) at the chunk shapes of the
    # pages' GEMM microbench (qwen3mlx, M = 256)
    for j, (name, n, k) in enumerate([("gate_up", 19456, 2560), ("down", 2560, 9728),
                                      ("o", 2560, 4096)]):
        m = 256
        Wh = torch.from_numpy(datagen.words(base + 700 + 10 * j, n, k).view(np.int32)).cuda()
        Sh = torch.from_numpy(datagen.scales(base + 701 + 10 * j, n, k // 2)).cuda()
        Bh = torch.from_numpy(datagen.normal_f16(base + 702 + 10 * j, (n, k // 64), 0.0,
                                                 0.05)).cuda()
        copies = max(2, -(-(512 << 20) // int(n * k * BPW)))
        rot = [(Wh, Sh, Bh)] + [(Wh.clone(), Sh.clone(), Bh.clone()) for _ in range(copies - 1)]
        x = torch.from_numpy(datagen.activations(base + 703 + 10 * j, m, k)).cuda()
        y = torch.empty((m, n), dtype=torch.float16, device="cuda")

        def launch(i, rot=rot, x=x, y=y):
            W, S, B = rot[i % len(rot)]
            q4.gemm_affine(W, S, B, x, y=y)
        add("Qwen3-4B MLX affine prefill chunk", "%s %dx%d" % (name, n, k), m, n, k, launch,
            "q4_gemm_affine, exact weights")
        del rot
        torch.cuda.empty_cache()
    return rows


def write_prefill_table(rows, out_dir):
    """The prefill table as markdown, to out_dir/prefill_table.md."""
    text = ["# Prefill matmul (q4_gemm, q4_gemm_affine) on the matrix cores: Phi-3-mini "
            "M = 1024, Qwen3-4B M = 256 (q4f16_1 and MLX affine)",
            "",
            "Command (from the repository root, on one MI355X): `python3 bench.py --prefill-table`",
            "",
            "Weights are seeded synthetic int4 group-32 (codes U{0..15}, scales U[0.005, 0.05]), "
            "cycled through device copies totalling more than 512 MB; activations N(0, 1) f16. "
            "`us` is the mean time per call over 40 calls back to back (a call whose grid would "
            "fill under half the GPU splits K: tile kernel + combine kernel); "
            "TFLOP/s = 2 M N K / us; the peak is the dense f16 "
            "matrix-core figure (2.5 PFLOP/s). Exact weights feed the codes q - 7 to the "
            "matrix cores and scale each 32-value group sum by s in f32; f16 weights feed "
            "f16((q - 7) s). The reference rows time torch.mm on dense f16 weights of the "
            "same shape (back-to-back calls, event timing), for context only.",
            "",
            "| workload | matrix | M | us | TFLOP/s | % of f16 peak | path |",
            "|---|---|---|---|---|---|---|"]
    for r in rows:
        text.append("| %s | %s | %d | %.2f | %.1f | %.1f | %s |" % (
            r["workload"], r["shape"], r["m"], r["us_kernel"], r["tflops"], r["pct_f16_peak"],
            r["note"]))
    os.makedirs(out_dir, exist_ok=True)
    with open(os.path.join(out_dir, "prefill_table.md"), "w") as fh:
        fh.write("\n".join(text) + "\n")


def write_gemv_table(rows):
    text = ["# Per-GEMV throughput: single GEMV, Phi-3-mini, Qwen3-4B (M = 1, 2, 4, 8), LM heads with "
            "argmax, QKV + RoPE + KV append, decode attention, and MoE shapes",
            "",
            "Command (from the repository root, on one MI355X): `python3 bench.py --gemv-table`",
            "",
            "Weights are seeded synthetic int4 group-32 (codes U{0..15}, scales U[0.005, 0.05]); "
            "each matrix is cycled through enough distinct device copies to exceed 512 MB, so "
            "HBM, not the 256 MB Infinity Cache, is measured. `us/kernel` is the matvec "
            "kernel's own dispatch time (q4_timer_arm events, mean of 64 launches); `us/call` "
            "is the time per call of 20-200 calls back to back (one event pair, includes "
            "the gaps between launches). GB/s = weight bytes (0.5625 B per weight) / "
            "us/kernel, except for the rows that run several kernels per call (the LM head + "
            "argmax: 2 kernels at M = 1, 4 at M = 8; attention: 1 or 2; the MoE layer: 3 to "
            "5), where it is bytes / us/call (attention: the K and V bytes read). For those "
            "rows us/kernel is the first matvec kernel alone. `oracle us` is the plain C "
            "oracle (binary64) on the same matmul or MoE layer on the host of the same run: "
            "one thread, then all host threads (the oracle single-threaded per part); "
            "empty where it was not run.",
            "",
            "Context only (other hardware, a whole decode step with attention and the LM "
            "head): %s, %s: Zero TVM %.2f tok/s, WebLLM 0.2.80 %.2f tok/s." % (
                BROWSER_CONTEXT["what"].split(" (")[0], BROWSER_CONTEXT["hardware"],
                BROWSER_CONTEXT["zero_tvm_tok_s"], BROWSER_CONTEXT["webllm_0_2_80_tok_s"]),
            "",
            "| workload | shape | M | weight bytes | us/kernel | us/call | GB/s | % of 8 TB/s "
            "| oracle us, 1 thread | oracle us, all threads | note |",
            "|---|---|---|---|---|---|---|---|---|---|---|"]
    fmt = lambda v: "%.1f" % v if v is not None else ""
    for r in rows:
        text.append("| %s | %s | %d | %d | %s | %.3f | %.1f | %.1f | %s | %s | %s |" % (
            r["workload"], r["shape"], r["m"], r["weight_bytes"],
            "%.3f" % r["us_kernel"] if r["us_kernel"] is not None else "",
            r["us_per_call"], r["gbs"], r["pct_peak"], fmt(r.get("oracle_us_1t")),
            fmt(r.get("oracle_us_all")), r["note"]))
    text.append("")
    with open(GEMV_TABLE_PROFILE, "w") as fh:
        fh.write("\n".join(text))


def verify_one_token(q4, torch, stack, st, p, o, layers_checked=(0, 1)):
    """Teacher-forced check of single layers of one token against the oracle."""
    d = p["d"]
    n = len(stack.layers)
    trace = torch.empty((n, 2, d), dtype=torch.float16, device="cuda")
    r_out = torch.empty(d, dtype=torch.float16, device="cuda")
    h_out = torch.empty(d, dtype=torch.float16, device="cuda")
    stack.decode(st["r0"], st["h0"], r_out, h_out, trace=trace)
    torch.cuda.synchronize()
    tr = trace.cpu().numpy()
    gi, gp, gf, r0, h0 = st["host"]
    worst = 0.0
    dims = (p["d"], p["f"], p["n_qkv"], p["v_off"], p["dv"])
    for L in layers_checked:
        r_in, h_in = (r0, h0) if L == 0 else (tr[L - 1, 0], tr[L - 1, 1])
        g_next = gi[L + 1] if L + 1 < n else gf
        _, _, h64 = o.layer(dims, host_layer(p, L), gp[L], g_next, r_in, h_in, eps=p["eps"])
        err = np.abs(tr[L, 1].astype(np.float64) - h64)
        tol = 1e-2 + 5e-3 * np.abs(h64)
        if not np.all(err <= tol):
            raise SystemExit("parity check failed at layer %d (max abs err %.3g)" % (L, err.max()))
        worst = max(worst, float(err.max()))
    return worst


def token_graphs(torch, stack, hs, r_out):
    """Two captured HIP graphs of one decode token each (the 129 kernel
    launches of q4_stack_decode): graph a reads (residual, normalised) =
    (hs[a], hs[a]) and writes hs[1 - a] (r_out takes the residual). They are
    captured on a side stream whose library workspace was reserved first
    (q4_workspace_reserve), so the graphs hold kernels only. Returns (stream,
    [graph0, graph1])."""
    import int4_weight_only_q4_amd as q4
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    q4.workspace_reserve(q4.stack_workspace_bytes(stack), stream=st)
    torch.cuda.synchronize()
    graphs = []
    for a in (0, 1):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=st):
            stack.decode(hs[a], hs[a], r_out, hs[1 - a])
        graphs.append(g)
    torch.cuda.synchronize()
    return st, graphs


def check_graph_tokens(torch, stack, graphs, hs, r_out, n=3):
    """n tokens replayed from the graphs equal n eager tokens from the same
    state bit for bit; leaves the state in hs[n & 1]."""
    d = hs[0].numel()
    start = hs[0].clone()
    e = [start.clone(), torch.empty_like(start)]
    r_tmp = torch.empty(d, dtype=torch.float16, device="cuda")
    for i in range(n):
        stack.decode(e[i & 1], e[i & 1], r_tmp, e[(i + 1) & 1])
    torch.cuda.synchronize()
    for i in range(n):
        graphs[i & 1].replay()
    torch.cuda.synchronize()
    if not torch.equal(hs[n & 1].view(torch.int16), e[n & 1].view(torch.int16)):
        raise SystemExit("graph-replayed tokens differ from eager tokens")


def measured_copy_gbs(torch, nbytes=1 << 30, reps=20):
    """HBM bytes moved per second (read + write) by a plain device-to-device
    copy of `nbytes`: the box's measured ceiling, reported beside the nominal
    peak for information (it is not the roofline's peak)."""
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    secs = e0.elapsed_time(e1) * 1e-3 / reps
    del src, dst
    torch.cuda.empty_cache()
    return 2 * nbytes / secs / 1e9


def host_info(threads):
    """The host the oracle legs ran on: CPU model (/proc/cpuinfo), os.cpu_count()
    (what std::thread::hardware_concurrency reports), the CPUs this process may
    run on (what nproc prints) and the threads the all-cores leg used."""
    model = ""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        nproc = len(os.sched_getaffinity(0))
    except AttributeError:
        nproc = None
    return {"cpu_model": model, "os_cpu_count": os.cpu_count(), "nproc": nproc,
            "threads": threads}


def _split(n, parts):
    """n items as `parts` contiguous (start, end) ranges (empty ones dropped)."""
    b = [n * i // parts for i in range(parts + 1)]
    return [(b[i], b[i + 1]) for i in range(parts) if b[i + 1] > b[i]]


def _in_threads(fn, items, threads):
    """fn over items in `threads` host threads (the oracle is one single-threaded
    C call per item; ctypes releases the GIL during it)."""
    if threads == 1:
        return [fn(it) for it in items]
    with cf.ThreadPoolExecutor(max_workers=threads) as ex:
        return list(ex.map(fn, items))


def oracle_rows_us(o, W, S, X, threads, target_s=0.25):
    """Oracle microseconds for one matmul of all N rows of W against the M
    activation rows X, extrapolated from a contiguous block of rows sized for
    about target_s of work per thread; the block is split into `threads`
    contiguous parts, each run by the single-threaded oracle (gemv for M = 1,
    gemv_batched otherwise) in a thread of its own. Returns (us, rows timed)."""
    n = W.shape[0]

    def run(rng):
        r0, r1 = rng
        if X.shape[0] == 1:
            o.gemv(W[r0:r1], S[r0:r1], X[0])
        else:
            o.gemv_batched(W[r0:r1], S[r0:r1], X)

    r = min(n, 4)
    t0 = time.perf_counter()
    run((0, r))
    per_row = max((time.perf_counter() - t0) / r, 1e-9)
    rows = int(min(n, max(r, target_s * threads / per_row)))
    t0 = time.perf_counter()
    _in_threads(run, _split(rows, threads), threads)
    return (time.perf_counter() - t0) / rows * n * 1e6, rows


def oracle_moe_us(o, mats, ids, route_w, x, f, threads):
    """Oracle microseconds for one MoE layer (the gate_up stage with the
    SiLU-multiply, its output rounded to binary16 as stored between the stages,
    then the down stage with the routing-weighted sum) over the tokens of ids
    [T][top-k]; the tokens are split over `threads` threads, each running the
    single-threaded oracle's stages on its tokens."""
    Wg, Sg, Wd, Sd = mats
    t, topk = ids.shape
    hidden = x.shape[1]

    def run(rng):
        a, b = rng
        u = o.moe_stage(Wg, Sg, ids[a:b], None, x[a:b], hidden, 0, 2 * f, hidden, True)
        u16 = np.ascontiguousarray(u.astype(np.float16))
        o.moe_stage(Wd, Sd, ids[a:b], route_w[a:b], u16, topk * f, f, hidden, f, False)

    t0 = time.perf_counter()
    _in_threads(run, _split(t, min(threads, t)), min(threads, t))
    return (time.perf_counter() - t0) * 1e6


def cpu_baseline(p, o, seconds=10.0, threads=HOST_THREADS):
    """The oracle (plain C, binary64, single-threaded per call) on the decode
    stack's layers:
      single thread: whole layers of one token, chained, until about `seconds`
        of CPU time has been spent;
      all cores: the 32 layers of one token's weights spread over `threads`
        threads, each layer run by the single-threaded oracle from the same
        input state (the chain cannot be split across cores, the layers' weight
        streams can).
    The main value is the all-cores rate; both are weight GB/s."""
    gi, gp, gf, r0, h0 = host_state(p, p["layers"])
    dims = (p["d"], p["f"], p["n_qkv"], p["v_off"], p["dv"])
    r, h = r0, h0
    done, spent = 0, 0.0
    while spent < seconds and done < p["layers"]:
        mats = host_layer(p, done)
        t0 = time.perf_counter()
        r, h, _ = o.layer(dims, mats, gp[done], gi[done + 1] if done + 1 < p["layers"] else gf,
                          r, h, eps=p["eps"])
        spent += time.perf_counter() - t0
        done += 1
    one_gbs = stack_weight_bytes(p, done) / spent / 1e9
    nl = p["layers"]
    mats_all = [host_layer(p, L) for L in range(nl)]

    def run_layers(rng):
        for L in range(*rng):
            o.layer(dims, mats_all[L], gp[L], gi[L + 1] if L + 1 < nl else gf, r0, h0,
                    eps=p["eps"])

    t0 = time.perf_counter()
    _in_threads(run_layers, _split(nl, threads), threads)
    wall = time.perf_counter() - t0
    all_gbs = stack_weight_bytes(p) / wall / 1e9
    return {"value": round(all_gbs, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": "the 32 decode layers of one token (%.1f MB of int4 weights) over %d "
                      "threads, each layer one single-threaded call of the C oracle in "
                      "binary64: %.2f s wall (%.1f us per token's weights)" % (
                          stack_weight_bytes(p) / 1e6, threads, wall, wall * 1e6),
            "single_thread": {"value": round(one_gbs, 4), "unit": "GB/s", "cores": 1,
                              "sample": "%d of 32 layers of one token chained (%.1f MB), "
                                        "%.1f s" % (done, stack_weight_bytes(p, done) / 1e6,
                                                    spent),
                              "us_per_token": round(stack_weight_bytes(p) / (one_gbs * 1e3), 1)},
            "host": host_info(threads)}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--eager", action="store_true",
                    help="launch each token's kernels from the host instead of replaying "
                         "a captured graph of them")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--out-dir", default=os.path.join(ROOT, "bench_out"),
                    help="directory for the markdown of --prefill-table")
    ap.add_argument("--gemv-table", action="store_true",
                    help="measure the per-GEMV table (Phi-3, Qwen3 M=1/2/4/8, MoE) and exit")
    ap.add_argument("--prefill-table", action="store_true",
                    help="measure the prefill matmul table (q4_gemm) and exit")
    ap.add_argument("--counters", action="store_true",
                    help="run only the workload of the rocprofv3 counter passes")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write the traffic summary from two rocprofv3 --pmc CSV outputs")
    ap.add_argument("--summarize-trace", nargs=2, metavar=("TRACE_CSV", "STATUS"),
                    help="write the stack's kernel-trace summary from a rocprofv3 --kernel-trace "
                         "CSV of this command and the profiled command's exit status")
    args = ap.parse_args()
    if args.summarize_trace:
        summarize_trace(*args.summarize_trace)
        return
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: the int4 decode path is built and timed on a single "
              "MI355X (how the path would shard over several GPUs is described, not built); "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import int4_weight_only_q4_amd as q4

    q4.lib()
    assert torch.cuda.is_available(), "no GPU"
    if args.gemv_table:
        import oracle
        rows = gemv_table(q4, torch, None if args.no_cpu_baseline else oracle.load())
        write_gemv_table(rows)
        print(json.dumps({"gemv_table": rows}), flush=True)
        return
    if args.prefill_table:
        rows = prefill_table(q4, torch)
        write_prefill_table(rows, args.out_dir)
        print(json.dumps({"prefill_table": rows}), flush=True)
        return
    p = PHI3
    print("building the %d-layer stack (%.3f GB of int4 weights)..." % (
        p["layers"], stack_weight_bytes(p) / 1e9), file=sys.stderr, flush=True)
    stack, st = build_stack(q4, torch, p)
    torch.cuda.synchronize()
    if args.counters:
        counter_workload(q4, torch, stack, st, p)
        return

    import oracle
    o = oracle.load()
    worst = verify_one_token(q4, torch, stack, st, p, o)
    print("parity (teacher-forced layers 0,1): max abs err %.3g" % worst, file=sys.stderr,
          flush=True)

    d = p["d"]
    r_out = torch.empty(d, dtype=torch.float16, device="cuda")
    hs = [st["h0"].clone(), torch.empty(d, dtype=torch.float16, device="cuda")]
    stack.decode(st["r0"], st["h0"], r_out, hs[0])      # first token from the seeded state

    # token i+1 starts from (residual, normalised) = (h_i, h_i); the state
    # alternates between hs[0] and hs[1]
    tok = 0
    if args.eager:
        run_stream = torch.cuda.current_stream()

        def run(count):
            nonlocal tok
            for _ in range(count):
                a = tok & 1
                stack.decode(hs[a], hs[a], r_out, hs[1 - a])
                tok += 1
    else:
        _, graphs = token_graphs(torch, stack, hs, r_out)
        check_graph_tokens(torch, stack, graphs, hs, r_out)
        tok = 3
        run_stream = torch.cuda.current_stream()  # replay() launches on the current stream

        def run(count):
            nonlocal tok
            for _ in range(count):
                graphs[tok & 1].replay()
                tok += 1

    run(args.warmup)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(run_stream)
    run(args.steps)
    e1.record(run_stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    wall_ms = (t1 - t0) * 1e3 / args.steps
    gpu_ms = e0.elapsed_time(e1) / args.steps
    ms = max(wall_ms, gpu_ms)
    h_last = hs[tok & 1].float()
    if not torch.isfinite(h_last).all() or float(h_last.abs().max()) == 0.0:
        raise SystemExit("timed output is not finite / all zero")

    wb = stack_weight_bytes(p)
    gbs = wb / (ms * 1e-3) / 1e9
    dom_us, dom_bytes = time_dominant_kernel(q4, torch, stack, st, p)
    dom_gbs = dom_bytes / (dom_us * 1e-6) / 1e9
    copy_gbs = measured_copy_gbs(torch)

    rec = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": "Phi-3-mini-shaped 32-layer int4 (q4f16_1) decode stack, batch 1",
            "layers": p["layers"], "d": p["d"], "ffn": p["f"], "qkv_rows": p["n_qkv"],
            "weight_bytes_per_token": wb,
            "us_per_token": round(ms * 1e3, 2),
            "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
            "launch": ("eager: 129 kernel launches per token" if args.eager else
                       "one HIP graph per token (its 129 kernels), replayed"),
            "gpu_event_ms_per_token": round(gpu_ms, 6),
            "wall_ms_per_token": round(wall_ms, 6),
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "gate_up 16384x3072 matvec, RMSNorm prologue + SiLU-multiply epilogue",
            "achieved": round(dom_gbs, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(dom_gbs / HBM_PEAK_GBS, 4),
            "us_per_launch": round(dom_us, 3),
            "bytes_per_launch": int(dom_bytes),
            "traffic": committed_traffic(),
            "measured_copy_gbs": round(copy_gbs, 1),
            "measured_copy_note": "1 GiB device-to-device copy, read + write bytes per "
                                  "second; informational, the peak is the nominal 8 TB/s",
            "in_stack": in_stack_line(dom_bytes),
        },
    }
    rec["context"] = dict(BROWSER_CONTEXT)
    rec["context"]["this_stack_tok_s"] = round(1e3 / ms, 1)
    rec["context"]["this_stack_note"] = ("tokens/s of the stack measured here: 32 layers' "
                                         "matmuls and norms, identity attention, no LM head")
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(p, o, args.cpu_seconds)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
