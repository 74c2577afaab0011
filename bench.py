#!/usr/bin/env python3
"""Throughput of the double-binary-factorised product on one MI355X.

Workload (the metric's configuration): a DBF-compressed attention projection,
N = M = 4096, R = 2048, ell = 1, Bernoulli signs, log-normal fp16 scales,
x ~ N(0,1) fp16 (synthetic, seeded).  One step is one ``dbf_forward`` call
over a batch of T = 256 tokens (the prefill case, matrix-core path); the same
JSON line also reports the decode case (T = 1, the sign-GEMV path), a grouped
decode over 256 distinct layers in one dispatch, the 64-adapter serving batch
(T = 2048, R = 64, ell = 2, Zipf ids), the layer's QAT backward at T = 256
(every gradient and the soft-sign straight-through latent gradients), the
transposed product, and every configuration's single call.

Every timed call reads factors that are not in any cache: calls rotate over
distinct device copies of the layer whose total size exceeds twice the 256 MB
Infinity Cache.  Times come from HIP events on the stream the library
launches on.  Prints ONE JSON line on stdout.

The roofline object is for the dominant kernel of the timed call: each of the
two launches is also timed alone (DBF_RUN_STAGE1 / DBF_RUN_STAGE2; stage 1
reads x in place on this layer, so DBF_RUN_PREP launches nothing; 64 calls
captured in a HIP graph and replayed between HIP events, so the host's launch
rate does not set the time), and the slower of the two matrix-core stages is
reported against the fp16 matrix-core peak.  Its HBM traffic comes from the rocprofv3 FETCH_SIZE /
WRITE_SIZE summary committed under profiles/ (scaled by what the counters
read for a device copy of known size), and is reported only while the kernel
source still matches the one the counters were taken on.

Other modes: --copy-calibration runs a 256 MiB device copy (for the counter
calibration run); --summarize-pmc FETCH_DIR WRITE_DIR prints the traffic
summary from two rocprofv3 --pmc output directories.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "DBF sign-matmul tokens/s + effective GB/s (4096², R=2048, T=1/256), % roofline"
HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0
FP32_PEAK_TFLOPS = 157.3  # published dense fp32 (matrix core; also the packed vector rate)
N_, R_, M_ = 4096, 2048, 4096
GEMM_SRC = os.path.join(ROOT, "double_binary_rank_amd", "csrc", "dbf_tile.hip")
GEMV_SRC = os.path.join(ROOT, "double_binary_rank_amd", "csrc", "dbf_gemv.hip")
TRAFFIC_MD = os.path.join(ROOT, "profiles", "k_tile_traffic_attn4096_R2048_T256.md")
# kernel-trace summaries the roofline objects take their launch durations from
PREFILL_TRACE_MD = os.path.join(ROOT, "profiles", "k_tile_prefill_attn4096_R2048_T256.md")
DECODE_TRACE_MD = os.path.join(ROOT, "profiles", "k_gemv_fused_grouped_decode_256x_attn4096_R2048.md")
DECODE_TRAFFIC_MD = os.path.join(ROOT, "profiles",
                                 "k_gemv_fused_traffic_grouped_decode_256x_attn4096_R2048.md")
COPY_MIB = 256


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def alg_bytes(N, R, M, ell, T, accumulate=False, ids=False):
    b = -(-(N * R + R * M) // 8) + 2 * ell * (N + R + M) + 2 * M * T + 2 * N * T
    if accumulate:
        b += 2 * N * T
    if ids:
        b += 4 * T
    return b


def alg_flops(N, R, M, ell, T):
    return 2 * T * ell * R * (N + M)


def time_calls(fn, n_calls, warmup):
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for i in range(n_calls):
        fn(i)
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / 1e3  # seconds for n_calls


def time_graph(fn, n_calls, reps, warmup):
    """Seconds per call of fn(0..n_calls-1) captured once into a HIP graph
    and replayed `reps` times between events (no host launch gaps: a single
    short kernel launched from Python would be timed at the host's rate)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(n_calls):
            fn(i)
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(n_calls):
            fn(i)
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(reps):
        g.replay()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / 1e3 / (reps * n_calls)


def call_percentiles(fn, n_calls, warmup):
    """p10 / median / p90 of per-call GPU time (µs): an event is recorded on
    the stream between consecutive calls (outside the timed region)."""
    for i in range(warmup):
        fn(i)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n_calls + 1)]
    torch.cuda.synchronize()
    ev[0].record()
    for i in range(n_calls):
        fn(i)
        ev[i + 1].record()
    torch.cuda.synchronize()
    d = np.array([ev[i].elapsed_time(ev[i + 1]) * 1e3 for i in range(n_calls)])
    return {"p10": float(np.percentile(d, 10)), "median": float(np.median(d)),
            "p90": float(np.percentile(d, 90)), "calls": n_calls}


def host_cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def replicate(t: torch.Tensor, k: int):
    return [t.clone() for _ in range(k)]


def file_sha256(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def committed_json(path, tag, src):
    """The `tag:` JSON line of a committed profile summary, or None when the
    file is absent or was taken on kernel source other than `src`."""
    try:
        with open(path) as f:
            for line in f:
                if line.startswith(tag + ":"):
                    d = json.loads(line.split(":", 1)[1])
                    return d if d.get("source_sha256") == file_sha256(src) else None
    except (OSError, ValueError):
        return None
    return None


def committed_mean_us(path, kernel, src):
    """Mean launch duration (us) of the kernel whose name starts with
    `kernel` in a committed kernel-trace summary of the current source."""
    d = committed_json(path, "trace_json", src)
    if not d:
        return None
    for k, v in d.get("mean_us", {}).items():
        if k.startswith(kernel):
            return v
    return None


def committed_traffic(stage):
    """HBM bytes per launch of the stage kernel from the committed counter
    summary, or None when absent or taken on different kernel source."""
    try:
        with open(TRAFFIC_MD) as f:
            for line in f:
                if line.startswith("traffic_json:"):
                    d = json.loads(line.split(":", 1)[1])
                    if d.get("source_sha256") != file_sha256(GEMM_SRC):
                        return None
                    return d["stages"][str(stage)]["bytes_per_launch"]
    except (OSError, KeyError, ValueError):
        return None
    return None


def _pmc_rows(d):
    rows = []
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        rows += list(csv.DictReader(open(f)))
    return rows


def summarize_pmc(fetch_dir, write_dir):
    """Per-dispatch FETCH_SIZE / WRITE_SIZE (KiB) of the stage kernels and of
    the calibration copy, scaled by the copy's known size."""
    def per_kernel(d, counter):
        acc = {}
        for r in _pmc_rows(d):
            if r["Counter_Name"] != counter:
                continue
            name = r["Kernel_Name"]
            key = ("stage1" if "k_tile<1" in name else "stage2" if "k_tile<2" in name
                   else "prep" if "k_prep_v" in name
                   else "copy" if "copy" in name.lower() or "elementwise" in name else None)
            if key:
                acc.setdefault(key, []).append(float(r["Counter_Value"]))
        # the calibration copy is the largest copy dispatch (the set-up also
        # copies the layer instances, 2 MiB each)
        return {k: (max(v) if k == "copy" else sum(v) / len(v)) for k, v in acc.items()}

    fe, wr = per_kernel(fetch_dir, "FETCH_SIZE"), per_kernel(write_dir, "WRITE_SIZE")
    copy_kib = COPY_MIB * 1024.0
    f_fac, w_fac = copy_kib / fe["copy"], copy_kib / wr["copy"]
    stages = {}
    for st, k in (("1", "stage1"), ("2", "stage2"), ("prep", "prep")):
        if k not in fe or k not in wr:
            continue
        fb, wb = fe[k] * 1024 * f_fac, wr[k] * 1024 * w_fac
        stages[st] = {"fetch_kib_raw": fe[k], "write_kib_raw": wr[k], "fetch_bytes": fb,
                      "write_bytes": wb, "bytes_per_launch": fb + wb}
    return {"source_sha256": file_sha256(GEMM_SRC), "copy_mib": COPY_MIB,
            "copy_fetch_kib_raw": fe["copy"], "copy_write_kib_raw": wr["copy"],
            "fetch_factor": f_fac, "write_factor": w_fac, "stages": stages}


def trace_means(trace_dir):
    """Mean duration (us) per kernel name in a rocprofv3 --kernel-trace run
    (names shortened to the template, without the argument list)."""
    rows = []
    for f in glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True):
        rows += list(csv.DictReader(open(f)))
    per = {}
    for r in rows:
        name = r["Kernel_Name"].replace("dbf::(anonymous namespace)::", "").replace("void ", "")
        name = name.replace("dbf::", "").split("(")[0].strip()
        per.setdefault(name, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    return {k: float(np.mean(v)) for k, v in per.items()}


def summarize_pmc_kernel(fetch_dir, write_dir, kernel, src):
    """FETCH_SIZE / WRITE_SIZE per launch of the kernel whose name contains
    `kernel`, scaled like summarize_pmc by the calibration copy, tagged with
    the kernel source's sha256."""
    def per(d, counter):
        k_v, c_v = [], []
        for r in _pmc_rows(d):
            if r["Counter_Name"] != counter:
                continue
            name = r["Kernel_Name"]
            if kernel in name:
                k_v.append(float(r["Counter_Value"]))
            elif "copy" in name.lower() or "elementwise" in name:
                c_v.append(float(r["Counter_Value"]))
        return sum(k_v) / len(k_v), max(c_v)
    fk, fc = per(fetch_dir, "FETCH_SIZE")
    wk, wc = per(write_dir, "WRITE_SIZE")
    copy_kib = COPY_MIB * 1024.0
    ff, wf = copy_kib / fc, copy_kib / wc
    return {"kernel": kernel, "source": os.path.relpath(src, ROOT), "source_sha256": file_sha256(src),
            "copy_mib": COPY_MIB, "fetch_kib_raw": fk, "write_kib_raw": wk,
            "copy_fetch_kib_raw": fc, "copy_write_kib_raw": wc, "fetch_factor": ff,
            "write_factor": wf, "fetch_bytes": fk * 1024 * ff, "write_bytes": wk * 1024 * wf,
            "bytes_per_launch": fk * 1024 * ff + wk * 1024 * wf}


def summarize_trace(trace_dir, top=12):
    """Markdown table of kernel durations from a rocprofv3 --kernel-trace
    run: calls, mean, p10, median, p90, min, max and share of the summed
    time per kernel name, from the per-dispatch timestamps."""
    rows = []
    for f in glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True):
        rows += list(csv.DictReader(open(f)))
    per = {}
    for r in rows:
        d = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        per.setdefault(r["Kernel_Name"], []).append(d)
    total = sum(sum(v) for v in per.values()) or 1.0
    lines = ["| kernel | calls | mean us | p10 us | median us | p90 us | min us | max us | share |",
             "|---|---|---|---|---|---|---|---|---|"]
    for name, v in sorted(per.items(), key=lambda kv: -sum(kv[1]))[:top]:
        a = np.array(v)
        short = name if len(name) <= 70 else name[:67] + "..."
        lines.append(f"| `{short}` | {len(a)} | {a.mean():.2f} | {np.percentile(a, 10):.2f} | "
                     f"{np.median(a):.2f} | {np.percentile(a, 90):.2f} | {a.min():.2f} | "
                     f"{a.max():.2f} | {100 * a.sum() / total:.1f}% |")
    return "\n".join(lines)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", default="", help="comma list of cases to run (profiling)")
    ap.add_argument("--configs", default="",
                    help="with the configs case: comma list of its entries to run, e.g. "
                         "mlp_up_2bpw_T1 (profiling)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help=f"also run a {COPY_MIB} MiB device copy (counter calibration)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--pmc-kernel", metavar="NAME",
                    help="with --summarize-pmc: summarise this kernel (name substring) alone")
    ap.add_argument("--pmc-source", metavar="SRC", help="with --pmc-kernel: its source file")
    ap.add_argument("--summarize-trace", metavar="TRACE_DIR",
                    help="print a kernel duration table from a rocprofv3 --kernel-trace run")
    ap.add_argument("--trace-source", metavar="SRC",
                    help="with --summarize-trace: also print a trace_json line of mean "
                         "durations tagged with this kernel source file's sha256")
    args = ap.parse_args()
    if args.summarize_pmc:
        if args.pmc_kernel:
            print("traffic_json: " + json.dumps(summarize_pmc_kernel(
                *args.summarize_pmc, args.pmc_kernel, args.pmc_source)))
        else:
            print("traffic_json: " + json.dumps(summarize_pmc(*args.summarize_pmc)))
        return
    if args.summarize_trace:
        print(summarize_trace(args.summarize_trace))
        if args.trace_source:
            print("\ntrace_json: " + json.dumps({
                "source": os.path.relpath(args.trace_source, ROOT),
                "source_sha256": file_sha256(args.trace_source),
                "mean_us": trace_means(args.summarize_trace)}))
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import double_binary_rank_amd as dbf
    import oracle
    import synth

    only = set(filter(None, args.only.split(",")))
    want = (lambda c: not only or c in only)
    dev = "cuda"
    torch.cuda.set_device(0)
    out = {}

    # ----------------------------------------------------- layer set-up --
    T = 256
    L = synth.make_config_layer(3, T)
    pl = dbf.PackedLayer.from_signs(L.S1, L.S2, L.alpha, L.beta, L.gamma, device=dev)
    n_inst = 256  # 256 x 2 MiB of packed signs = 512 MiB > 2 x MALL
    B1s = replicate(pl.B1, n_inst)
    B2s = replicate(pl.B2, n_inst)
    x256 = torch.as_tensor(L.x).to(dev)
    xs = replicate(x256, 16)
    y256 = torch.empty((T, N_), dtype=torch.float16, device=dev)
    ws = torch.empty(dbf.dbf_workspace_bytes(N_, R_, M_, 1, T), dtype=torch.uint8, device=dev)
    log("layer set-up done")

    # parity of the timed configuration (T = 256) against the oracle
    yref = oracle.forward(L.x, L.S1, L.S2, L.alpha, L.beta, L.gamma)
    ychk = pl.forward(x256, ws=ws)
    torch.cuda.synchronize()
    err256 = oracle.max_norm_error(ychk.float().cpu().numpy(), yref)
    log(f"parity T=256 err={err256:.3e}")

    def call256(i):
        k = i % n_inst
        dbf.dbf_forward(xs[i % len(xs)], B1s[k], B2s[k], pl.alpha, pl.beta, pl.gamma, N_, R_, M_,
                        y=y256, ws=ws)

    # ---------------------------------------------------- prefill T=256 --
    flops = alg_flops(N_, R_, M_, 1, T)
    byts = alg_bytes(N_, R_, M_, 1, T)
    t_call = value = achieved_tflops = float("nan")
    roof = None
    decode_roof = None
    if want("prefill"):
        sec = time_calls(call256, args.steps, args.warmup)
        t_call = sec / args.steps
        value = T / t_call
        achieved_tflops = flops / t_call / 1e12
        log(f"prefill T=256: {t_call * 1e6:.2f} us/call, {achieved_tflops:.1f} TFLOP/s")
        out["prefill_T256_call_us"] = call_percentiles(call256, 200, 10)
        # the whole call replayed from a HIP graph (no host launch gaps)
        t_g = time_graph(call256, 64, max(args.steps // 16, 4), 2)
        out["prefill_T256_graph"] = {"us_per_call": t_g * 1e6, "tokens_per_s": T / t_g,
                                     "TFLOPs": flops / t_g / 1e12}
        log(f"prefill T=256 replayed from a graph: {t_g * 1e6:.2f} us/call, "
            f"{T / t_g / 1e6:.2f} M tokens/s")
        log("prefill per-call us: " + ", ".join(
            f"{k} {v:.2f}" for k, v in out["prefill_T256_call_us"].items() if k != "calls"))

        # each launch alone: stage 1 (z = beta * B2 (gamma x), reading x in
        # place; the prep phase launches nothing on this layer) and stage 2
        # (y = alpha * B1 z), which reads the z stage 1 left in ws
        def phase_call(ph):
            def f(i):
                k = i % n_inst
                dbf.dbf_forward(xs[i % len(xs)], B1s[k], B2s[k], pl.alpha, pl.beta, pl.gamma, N_,
                                R_, M_, y=y256, ws=ws, phases=ph)
            return f

        t_ph = {}
        for ph in ("stage1", "stage2"):
            call256(0)
            torch.cuda.synchronize()
            t_ph[ph] = time_graph(phase_call(ph), 64, max(args.steps // 16, 4), 2)
        f_st = {"stage1": 2 * T * R_ * M_, "stage2": 2 * T * N_ * R_}
        dom = max(f_st, key=lambda k: t_ph[k])
        kname = {"stage1": "k_tile<1", "stage2": "k_tile<2"}[dom]
        # the launch duration: the committed rocprof mean of this kernel when
        # it was taken on the current source, else the live graph replay
        prof_us = committed_mean_us(PREFILL_TRACE_MD, kname, GEMM_SRC)
        dur_us = prof_us if prof_us is not None else t_ph[dom] * 1e6
        ach = f_st[dom] / (dur_us * 1e-6) / 1e12
        roof = {"bound": "mfma", "achieved": ach, "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": ach / MFMA_F16_PEAK_TFLOPS, "traffic": committed_traffic(dom[-1]),
                "kernel": kname + ", ...> (" + dom + " of the T=256 call)",
                "launch_us": dur_us, "launch_us_source": "rocprof" if prof_us is not None else "live",
                "launch_us_live": t_ph[dom] * 1e6, "alg_flops_per_launch": f_st[dom],
                "phase_launch_us": {k: v * 1e6 for k, v in t_ph.items()}}
        log("phase launches: " + ", ".join(f"{k} {v * 1e6:.2f} us" for k, v in t_ph.items())
            + f"; dominant {dom}: {ach:.1f} TFLOP/s")

    # ---------------- the same layer at longer prefills (T = 1024, 4096) --
    # calls and each stage alone replayed from HIP graphs over the cold
    # copies of the signs; parity on a sample of token rows
    if want("sweep"):
        sweep = {}
        for Ts in (1024, 4096):
            gx = torch.Generator(device=dev)
            gx.manual_seed(3000 + Ts)
            xT = torch.randn(Ts, M_, device=dev, dtype=torch.float16, generator=gx)
            yT = torch.empty((Ts, N_), dtype=torch.float16, device=dev)
            wsT = torch.empty(dbf.dbf_workspace_bytes(N_, R_, M_, 1, Ts), dtype=torch.uint8,
                              device=dev)

            def callT(i, ph=None):
                k = i % n_inst
                dbf.dbf_forward(xT, B1s[k], B2s[k], pl.alpha, pl.beta, pl.gamma, N_, R_, M_, y=yT,
                                ws=wsT, phases=ph)

            callT(0)
            torch.cuda.synchronize()
            rows = np.linspace(0, Ts - 1, 8).astype(np.int64)
            xs_h = xT[torch.as_tensor(rows, device=dev)].cpu().numpy()
            ys_h = yT[torch.as_tensor(rows, device=dev)].float().cpu().numpy()
            errT = oracle.max_norm_error(ys_h, oracle.forward(xs_h, L.S1, L.S2, L.alpha, L.beta,
                                                              L.gamma))
            tT = time_graph(callT, 16, 4, 1)
            fT = alg_flops(N_, R_, M_, 1, Ts)
            st = {}
            for ph in ("stage1", "stage2"):
                tp = time_graph(lambda i, ph=ph: callT(i, ph), 16, 4, 1)
                fs = 2.0 * Ts * R_ * (M_ if ph == "stage1" else N_)
                st[ph] = {"us": tp * 1e6, "TFLOPs": fs / tp / 1e12,
                          "mfma_frac": fs / tp / 1e12 / MFMA_F16_PEAK_TFLOPS}
            sweep[f"T{Ts}"] = {"us_per_call_graph": tT * 1e6, "tokens_per_s": Ts / tT,
                               "TFLOPs": fT / tT / 1e12,
                               "mfma_frac": fT / tT / 1e12 / MFMA_F16_PEAK_TFLOPS,
                               "stages": st, "parity_err_8_rows": errT}
            log(f"prefill T={Ts}: {tT * 1e6:.1f} us/call (graph), {fT / tT / 1e12:.0f} TFLOP/s; "
                + ", ".join(f"{k} {v['us']:.1f} us = {100 * v['mfma_frac']:.1f} %"
                            for k, v in st.items()) + f"; err {errT:.2e}")
            del xT, yT, wsT
        out["prefill_T_sweep"] = sweep

    # ------------------------------------------------------ decode T=1 --
    if want("decode"):
        x1 = x256[:1].contiguous()
        y1 = torch.empty((1, N_), dtype=torch.float16, device=dev)
        ws1 = torch.empty(dbf.dbf_workspace_bytes(N_, R_, M_, 1, 1), dtype=torch.uint8, device=dev)
        ychk = pl.forward(x1, ws=ws1)
        torch.cuda.synchronize()
        err1 = oracle.max_norm_error(ychk.float().cpu().numpy(), yref[:1])

        def call1(i):
            k = i % n_inst
            dbf.dbf_forward(x1, B1s[k], B2s[k], pl.alpha, pl.beta, pl.gamma, N_, R_, M_, y=y1,
                            ws=ws1)

        n1 = max(args.steps, 256)
        t1 = time_calls(call1, n1, args.warmup) / n1
        # the same calls captured in a HIP graph: the GPU's time per call,
        # free of the host's launch rate
        t1g = time_graph(call1, 64, max(args.steps // 16, 4), 2)
        b1 = alg_bytes(N_, R_, M_, 1, 1)
        out["decode_T1"] = {
            "T": 1, "us_per_call": t1 * 1e6, "tokens_per_s": 1 / t1,
            "us_per_call_graph": t1g * 1e6, "effective_GBs_graph": b1 / t1g / 1e9,
            "call_us": call_percentiles(call1, 200, 10),
            "effective_GBs": b1 / t1 / 1e9, "hbm_frac": b1 / t1 / 1e9 / HBM_PEAK_GBS,
            "alg_bytes_per_call": b1, "parity_err": err1,
        }
        log(f"decode T=1: {t1 * 1e6:.2f} us/call, {b1 / t1 / 1e9:.1f} GB/s; graph replay "
            f"{t1g * 1e6:.2f} us/call, {b1 / t1g / 1e9:.1f} GB/s")

    # ------------------------- grouped decode: 256 layers, 1 token each --
    if want("grouped"):
        G = n_inst
        tab = lambda ts: dbf.pointer_table(ts, dev)  # noqa: E731
        tB1, tB2 = tab(B1s), tab(B2s)
        # every layer instance has its own copy of the scales too, so the
        # call streams all the bytes it is credited with
        aS, bS, gS = replicate(pl.alpha, G), replicate(pl.beta, G), replicate(pl.gamma, G)
        ta, tb, tg = tab(aS), tab(bS), tab(gS)
        xg = x256[:1].repeat(G, 1).contiguous()
        ids = torch.arange(G, dtype=torch.int32, device=dev)
        yg = torch.empty((G, N_), dtype=torch.float16, device=dev)
        wsg = torch.empty(dbf.dbf_workspace_bytes(N_, R_, M_, 1, G), dtype=torch.uint8, device=dev)

        def callg(i):
            dbf.dbf_forward_multi_adapter(xg, ids, tB1, tB2, ta, tb, tg, G, N_, R_, M_, 1, y=yg,
                                          ws=wsg)

        callg(0)
        torch.cuda.synchronize()
        yg_h = yg.float().cpu().numpy()
        errg = oracle.max_norm_error(yg_h[:1], yref[:1])
        # the G instances are copies of one layer on copies of one token, so
        # every row must be the same, bit for bit
        rows_equal = bool((yg_h == yg_h[:1]).all())
        errg_all = oracle.max_norm_error(yg_h, np.repeat(yref[:1], G, axis=0))
        ng = max(args.steps // 10, 10)
        tg_ = time_calls(callg, ng, 3) / ng
        tgg = time_graph(callg, 8, max(args.steps // 40, 3), 2)
        bg = G * alg_bytes(N_, R_, M_, 1, 1, ids=True)
        out["grouped_decode_256_layers"] = {
            "layers": G, "T_per_layer": 1, "us_per_call": tg_ * 1e6, "tokens_per_s": G / tg_,
            "effective_GBs": bg / tg_ / 1e9, "hbm_frac": bg / tg_ / 1e9 / HBM_PEAK_GBS,
            "us_per_call_graph": tgg * 1e6, "hbm_frac_graph": bg / tgg / 1e9 / HBM_PEAK_GBS,
            "alg_bytes_per_call": bg, "parity_err_token0": errg, "parity_err_all_rows": errg_all,
            "rows_bit_identical": rows_equal,
        }
        log(f"grouped decode: {tg_ * 1e6:.1f} us/call, {bg / tg_ / 1e9:.1f} GB/s; graph replay "
            f"{tgg * 1e6:.1f} us/call, {bg / tgg / 1e9:.1f} GB/s")
        # the decode-side roofline: the one k_gemv_fused launch of the call
        prof_us = committed_mean_us(DECODE_TRACE_MD, "k_gemv_fused", GEMV_SRC)
        dur_us = prof_us if prof_us is not None else tgg * 1e6
        tr = committed_json(DECODE_TRAFFIC_MD, "traffic_json", GEMV_SRC)
        decode_roof = {"bound": "hbm", "achieved": bg / (dur_us * 1e-6) / 1e9, "peak": HBM_PEAK_GBS,
                       "unit": "GB/s", "frac": bg / (dur_us * 1e-6) / 1e9 / HBM_PEAK_GBS,
                       "traffic": tr["bytes_per_launch"] if tr else None,
                       "kernel": "k_gemv_fused (256 one-token layers, one launch per call)",
                       "launch_us": dur_us,
                       "launch_us_source": "rocprof" if prof_us is not None else "live",
                       "launch_us_live": tgg * 1e6, "alg_bytes_per_launch": bg}

    # ------------------------------------------ multi-adapter batch cfg5 --
    if want("multi"):
        B = synth.make_multi_adapter()
        layers = [dbf.PackedLayer.from_signs(a.S1, a.S2, a.alpha, a.beta, a.gamma, device=dev)
                  for a in B.adapters]
        tab = lambda ts: dbf.pointer_table(ts, dev)  # noqa: E731
        mt = [tab([getattr(p, f) for p in layers]) for f in ("B1", "B2", "alpha", "beta", "gamma")]
        xm = torch.as_tensor(B.x).to(dev)
        idm = torch.as_tensor(B.ids).to(dev)
        Tm = xm.shape[0]
        ym = torch.empty((Tm, 4096), dtype=torch.float16, device=dev)
        wsm = torch.empty(dbf.dbf_workspace_bytes(4096, 64, 4096, 2, Tm), dtype=torch.uint8,
                          device=dev)

        def callm(i):
            dbf.dbf_forward_multi_adapter(xm, idm, *mt, 64, 4096, 64, 4096, 2, y=ym, ws=wsm)

        callm(0)
        torch.cuda.synchronize()
        errm = oracle.max_norm_error(ym.float().cpu().numpy(),
                                     oracle.forward_multi_adapter(B.x, B.ids, B.adapters))
        y_eager = ym.clone()
        nm = max(args.steps // 2, 20)
        tm = time_calls(callm, nm, args.warmup) / nm
        # the same call captured in a HIP graph (its three launches without
        # the host's launch gaps); the replays must leave y bit for bit as
        # the eager call did
        tmg = time_graph(callm, 16, max(args.steps // 16, 4), 2)
        graph_same = bool(torch.equal(ym, y_eager))
        bm = 64 * (-(-(2 * 4096 * 64) // 8) + 2 * 2 * (4096 + 64 + 4096)) + 2 * 4096 * Tm * 2 + 4 * Tm
        fm = alg_flops(4096, 64, 4096, 2, Tm)
        out["multi_adapter_64"] = {
            "T": Tm, "adapters": 64, "us_per_call": tm * 1e6, "tokens_per_s": Tm / tm,
            "effective_GBs": bm / tm / 1e9, "hbm_frac": bm / tm / 1e9 / HBM_PEAK_GBS,
            "mfma_frac": fm / tm / 1e12 / MFMA_F16_PEAK_TFLOPS, "alg_bytes_per_call": bm,
            "us_per_call_graph": tmg * 1e6, "hbm_frac_graph": bm / tmg / 1e9 / HBM_PEAK_GBS,
            "graph_bit_identical": graph_same, "parity_err": errm,
        }
        log(f"multi-adapter: {tm * 1e6:.1f} us/call, {bm / tm / 1e9:.1f} GB/s; graph replay "
            f"{tmg * 1e6:.1f} us/call")

    # ------------------------------- the other configurations, timed --
    if want("configs"):
        cfgs = {}
        for cfg, Tc in ((1, 4), (2, 1), (2, 8), (4, 1), (4, 16), (4, 256), (40, 1), (40, 16),
                        (40, 256)):
            name = f"{synth.CONFIGS[cfg].name}_T{Tc}"
            if args.configs and name not in args.configs.split(","):
                continue
            Lc = synth.make_config_layer(cfg, Tc)
            Nc, Rc, Mc = Lc.S1.shape[0], Lc.S1.shape[1], Lc.S2.shape[1]
            plc = dbf.PackedLayer.from_signs(Lc.S1, Lc.S2, Lc.alpha, Lc.beta, Lc.gamma,
                                             device=dev)
            lb = plc.B1.numel() + plc.B2.numel()
            k_inst = max(1, min(4096, -(-(512 << 20) // lb)))  # cold: >= 512 MiB of signs
            cB1, cB2 = replicate(plc.B1, k_inst), replicate(plc.B2, k_inst)
            xc = torch.as_tensor(Lc.x).to(dev)
            yc = torch.empty((Tc, Nc), dtype=torch.float16, device=dev)
            wsc = torch.empty(dbf.dbf_workspace_bytes(Nc, Rc, Mc, 1, Tc), dtype=torch.uint8,
                              device=dev)
            plc.forward(xc, y=yc, ws=wsc)
            torch.cuda.synchronize()
            if Nc * Rc * Mc <= 4096 * 64 * 4096:
                errc = oracle.max_norm_error(
                    yc.float().cpu().numpy(),
                    oracle.forward(Lc.x, Lc.S1, Lc.S2, Lc.alpha, Lc.beta, Lc.gamma))
                chk = "full"
            else:  # sampled: 4 tokens x 64 outputs
                ts = np.arange(min(Tc, 4))
                ns = np.random.default_rng(cfg + Tc).choice(Nc, 64, replace=False)
                want_s = oracle.forward_rows(Lc.x[ts], Lc.S1, Lc.S2, Lc.alpha, Lc.beta, Lc.gamma,
                                             ns)
                errc = oracle.max_norm_error(yc.float().cpu().numpy()[ts][:, ns], want_s)
                chk = "4 tokens x 64 outputs"

            def callc(i, cB1=cB1, cB2=cB2, plc=plc, xc=xc, yc=yc, wsc=wsc, k=k_inst, n=(Nc, Rc, Mc)):
                dbf.dbf_forward(xc, cB1[i % k], cB2[i % k], plc.alpha, plc.beta, plc.gamma, *n,
                                y=yc, ws=wsc)

            nc = max(args.steps, 100)
            tc = time_calls(callc, nc, args.warmup) / nc
            # the same calls replayed from a HIP graph: the GPU's time per
            # call, free of the host's launch rate
            tg = time_graph(callc, 64, max(args.steps // 16, 4), 2)
            bc, fc = alg_bytes(Nc, Rc, Mc, 1, Tc), alg_flops(Nc, Rc, Mc, 1, Tc)
            cfgs[name] = {
                "N": Nc, "R": Rc, "M": Mc, "T": Tc, "us_per_call": tc * 1e6,
                "tokens_per_s": Tc / tc, "effective_GBs": bc / tc / 1e9,
                "hbm_frac": bc / tc / 1e9 / HBM_PEAK_GBS,
                "mfma_frac": fc / tc / 1e12 / MFMA_F16_PEAK_TFLOPS,
                "us_per_call_graph": tg * 1e6, "effective_GBs_graph": bc / tg / 1e9,
                "hbm_frac_graph": bc / tg / 1e9 / HBM_PEAK_GBS,
                "mfma_frac_graph": fc / tg / 1e12 / MFMA_F16_PEAK_TFLOPS, "cold_instances": k_inst,
                "parity_err": errc, "parity_check": chk,
            }
            log(f"{name}: {tc * 1e6:.2f} us/call, {bc / tc / 1e9:.1f} GB/s, "
                f"{fc / tc / 1e12:.1f} TFLOP/s; graph replay {tg * 1e6:.2f} us/call, "
                f"{bc / tg / 1e9:.1f} GB/s, {fc / tg / 1e12:.1f} TFLOP/s; err {errc:.2e}")
            del cB1, cB2
        out["configs"] = cfgs

    # ------------------- transposed product dW^T g (input gradient) --
    if want("transposed"):
        plt = pl.transposed()
        tt_ = time_calls(lambda i: pl.transposed(), 20, 2) / 20  # both sign matrices
        gT = np.random.default_rng(7).standard_normal((T, N_)).astype(np.float16)
        gT = torch.as_tensor(gT).to(dev)
        yT = torch.empty((T, M_), dtype=torch.float16, device=dev)
        wsT = torch.empty(dbf.dbf_workspace_bytes(M_, R_, N_, 1, T), dtype=torch.uint8, device=dev)
        TB1s, TB2s = replicate(plt.B1, n_inst), replicate(plt.B2, n_inst)
        plt.forward(gT, y=yT, ws=wsT)
        torch.cuda.synchronize()
        errT = oracle.max_norm_error(
            yT.float().cpu().numpy(),
            oracle.forward_transposed(gT.cpu().numpy(), L.S1, L.S2, L.alpha, L.beta, L.gamma))

        def callT(i):
            k = i % n_inst
            dbf.dbf_forward(gT, TB1s[k], TB2s[k], plt.alpha, plt.beta, plt.gamma, M_, R_, N_,
                            y=yT, ws=wsT)

        tT = time_calls(callT, args.steps, args.warmup) / args.steps
        out["transposed_T256"] = {
            "T": T, "us_per_call": tT * 1e6, "tokens_per_s": T / tT,
            "achieved_TFLOPs": alg_flops(M_, R_, N_, 1, T) / tT / 1e12,
            "transpose_signs_us": tt_ * 1e6, "parity_err": errT,
        }
        log(f"transposed T=256: {tT * 1e6:.2f} us/call (sign transposes {tt_ * 1e6:.1f} us)")

    # ------------------------------ QAT backward, attention layer T=256 --
    if want("backward"):
        rngb = np.random.default_rng(8)
        gB = torch.as_tensor(oracle.fp16_rne(rngb.standard_normal((T, N_))).astype(np.float16)).to(dev)
        H1 = torch.as_tensor(rngb.standard_normal((N_, R_)), dtype=torch.float32).to(dev)
        H2 = torch.as_tensor(rngb.standard_normal((R_, M_)), dtype=torch.float32).to(dev)
        tau = 0.5
        B1ts = [dbf.dbf_transpose_signs(b, N_, R_) for b in B1s]
        B2ts = [dbf.dbf_transpose_signs(b, R_, M_) for b in B2s]
        wsB = torch.empty(dbf.dbf_backward_workspace_bytes(N_, R_, M_, 1, T), dtype=torch.uint8,
                          device=dev)

        def callB(i):
            k = i % n_inst
            return dbf.dbf_backward(x256, gB, B1s[k], B2s[k], B1ts[k], B2ts[k], pl.alpha, pl.beta,
                                    pl.gamma, N_, R_, M_, sign_grads=True, H1=H1, H2=H2, tau=tau,
                                    ws=wsB)

        gotB = callB(0)
        torch.cuda.synchronize()
        t_o = time.perf_counter()
        refB = oracle.backward(L.x, gB.cpu().numpy(), L.S1, L.S2, L.alpha, L.beta, L.gamma,
                               H1=H1.cpu().numpy(), H2=H2.cpu().numpy(), tau=tau)
        t_o = time.perf_counter() - t_o
        errB = {k: oracle.max_norm_error(v.float().cpu().numpy(), refB[k]) for k, v in gotB.items()}
        nB = max(args.steps // 4, 20)
        tB = time_calls(callB, nB, 3) / nB
        flB = 3 * alg_flops(N_, R_, M_, 1, T)  # U, P, W, Q and the two sign gradients
        out["backward_T256"] = {
            "T": T, "us_per_call": tB * 1e6, "tokens_per_s": T / tB,
            "achieved_TFLOPs": flB / tB / 1e12, "mfma_frac": flB / tB / 1e12 / MFMA_F16_PEAK_TFLOPS,
            "alg_flops_per_call": flB, "outputs": sorted(gotB), "parity_err": errB,
            "oracle_s_per_call": t_o,
        }
        log(f"backward T=256: {tB * 1e6:.1f} us/call, {flB / tB / 1e12:.1f} TFLOP/s, "
            f"max err {max(errB.values()):.2e}; fp64 oracle {t_o:.2f} s")

    # ------------- three same-input layers (q/k/v) in one call, T=1 / 256 --
    if want("grouped_layers"):
        J = 3
        layers_of = lambda i: [dbf.PackedLayer(B1s[(i * J + j) % n_inst], B2s[(i * J + j) % n_inst],  # noqa: E731
                                               pl.alpha, pl.beta, pl.gamma, N_, R_, M_)
                               for j in range(J)]
        res = {}
        for Tg in (1, 256):
            xg = x256[:Tg].contiguous()
            yg = torch.empty((J, Tg, N_), dtype=torch.float16, device=dev)
            wsg = torch.empty(dbf.dbf_grouped_workspace_bytes(N_, R_, M_, 1, Tg, J),
                              dtype=torch.uint8, device=dev)
            ys1 = [torch.empty((Tg, N_), dtype=torch.float16, device=dev) for _ in range(J)]
            ws1 = torch.empty(dbf.dbf_workspace_bytes(N_, R_, M_, 1, Tg), dtype=torch.uint8,
                              device=dev)
            lay = [layers_of(i) for i in range(64)]

            def grouped(i):
                dbf.dbf_forward_grouped(xg, lay[i % 64], y=yg, ws=wsg)

            def separate(i):
                for j, p_ in enumerate(lay[i % 64]):
                    p_.forward(xg, y=ys1[j], ws=ws1)

            grouped(0)
            separate(0)
            torch.cuda.synchronize()
            same = all(torch.equal(yg[j], ys1[j]) for j in range(J))
            tg_ = time_graph(grouped, 64, max(args.steps // 16, 4), 2)
            ts_ = time_graph(separate, 64, max(args.steps // 16, 4), 2)
            res[f"T{Tg}"] = {"grouped_us": tg_ * 1e6, "separate_us": ts_ * 1e6,
                             "speedup": ts_ / tg_, "bit_identical": same,
                             "tokens_per_s": J * Tg / tg_}
            log(f"grouped q/k/v T={Tg}: {tg_ * 1e6:.2f} us vs {ts_ * 1e6:.2f} us for three calls"
                f" (graph replay), identical={same}")
        out["grouped_qkv_3x_attn"] = res

    # ----- decoder-layer stack: non-uniform widths at 1.5 bits per weight --
    if want("stack"):
        n_dec, bpw = 2, 1.5
        proj = [("q", 4096, 4096, -0.5), ("k", 4096, 4096, -0.5), ("v", 4096, 4096, 0.0),
                ("o", 4096, 4096, 0.0), ("gate", 14336, 4096, -0.3), ("up", 14336, 4096, -0.3),
                ("down", 4096, 14336, 0.3)]
        gen = torch.Generator(device=dev)
        gen.manual_seed(11)

        def lognormal(n, mu):
            z = torch.randn(n, generator=gen, device=dev, dtype=torch.float32)
            return torch.exp(mu + 0.5 * z).to(torch.float16)[None].contiguous()

        def make(N, M, R, off):
            # signs Bernoulli(1/2); alpha, gamma ~ exp(N(-1, 0.5^2)); beta scaled so that
            # the projection's gain is near 1 (times a per-type offset)
            S1 = (torch.randint(0, 2, (N, R), generator=gen, device=dev, dtype=torch.int8) * 2 - 1)
            S2 = (torch.randint(0, 2, (R, M), generator=gen, device=dev, dtype=torch.int8) * 2 - 1)
            mu_b = off - math.log(math.exp(-2.25) * math.sqrt(R * M))
            return dbf.PackedLayer(dbf.dbf_pack_signs(S1), dbf.dbf_pack_signs(S2),
                                   lognormal(N, -1.0), lognormal(R, mu_b), lognormal(M, -1.0),
                                   N, R, M)

        full = [make(N, M, dbf.rank_for_bits(N, M, 2.0), off) for _ in range(n_dec)
                for (_, N, M, off) in proj]
        shapes = [(p_.N, p_.R, p_.M) for p_ in full]
        budget = bpw * sum(N * M for (N, _, M) in shapes)
        keep = dbf.plan_channels(shapes, [p_.channel_importance() for p_ in full], budget)
        nonuni = [p_.select_channels(k) for p_, k in zip(full, keep)]
        uni = [make(N, M, dbf.rank_for_bits(N, M, bpw), off) for _ in range(n_dec)
               for (_, N, M, off) in proj]
        del full
        bits = lambda ls: sum(dbf.layer_bits(q.N, q.R, q.M) for q in ls)  # noqa: E731
        weights = sum(N * M for (N, _, M) in shapes)
        wsS = torch.empty(max(dbf.dbf_grouped_workspace_bytes(14336, 6400, 14336, 1, 256, 3), 16),
                          dtype=torch.uint8, device=dev)

        def chain(ls, h, bufs, grouped):
            # per decoder layer: q, k, v on h; h += o(q); gate, up on h; h += down(up)
            for d in range(n_dec):
                b = 7 * d
                if grouped:
                    dbf.dbf_forward_grouped(h, ls[b:b + 3], y=bufs["qkv"], ws=wsS)
                    q = bufs["qkv"][0]
                else:
                    q = ls[b].forward(h, y=bufs["q"], ws=wsS)
                    ls[b + 1].forward(h, y=bufs["k"], ws=wsS)
                    ls[b + 2].forward(h, y=bufs["v"], ws=wsS)
                ls[b + 3].forward(q, y=h, accumulate=True, ws=wsS)
                if grouped:
                    dbf.dbf_forward_grouped(h, ls[b + 4:b + 6], y=bufs["gu"], ws=wsS)
                    u = bufs["gu"][1]
                else:
                    ls[b + 4].forward(h, y=bufs["g"], ws=wsS)
                    u = ls[b + 5].forward(h, y=bufs["u"], ws=wsS)
                ls[b + 6].forward(u, y=h, accumulate=True, ws=wsS)

        def timed(ls, Ts, grouped):
            x0 = torch.randn((Ts, 4096), generator=gen, device=dev).to(torch.float16)
            h = torch.empty_like(x0)
            e16 = lambda *sh: torch.empty(sh, dtype=torch.float16, device=dev)  # noqa: E731
            bufs = {"q": e16(Ts, 4096), "k": e16(Ts, 4096), "v": e16(Ts, 4096),
                    "g": e16(Ts, 14336), "u": e16(Ts, 14336), "qkv": e16(3, Ts, 4096),
                    "gu": e16(2, Ts, 14336)}

            def step(_i):
                h.copy_(x0)
                chain(ls, h, bufs, grouped)

            return time_graph(step, 8, max(args.steps // 20, 4), 2)

        res = {"decoder_layers": n_dec, "projections": [p_[0] for p_ in proj], "target_bpw": bpw}
        for name, ls, grouped in (("uniform", uni, False), ("uniform_grouped", uni, True),
                                  ("nonuniform", nonuni, False)):
            r = {"widths": [q.R for q in ls], "bpw": bits(ls) / weights}
            for Ts in (1, 256):
                t_ = timed(ls, Ts, grouped)
                r[f"T{Ts}_us"] = t_ * 1e6
                r[f"T{Ts}_tokens_per_s"] = Ts / t_
            res[name] = r
            log(f"stack {name}: {r['bpw']:.3f} bpw, decode {r['T1_us']:.1f} us/token, "
                f"prefill T=256 {r['T256_us']:.1f} us")
        # parity of the first pruned projection at T = 1
        xq = torch.randn((1, 4096), generator=gen, device=dev).to(torch.float16)
        p0 = nonuni[0]
        yq = p0.forward(xq)
        torch.cuda.synchronize()
        S1h = dbf.dbf_unpack_signs(p0.B1, p0.N, p0.R).cpu().numpy()
        S2h = dbf.dbf_unpack_signs(p0.B2, p0.R, p0.M).cpu().numpy()
        res["parity_err_first_projection"] = oracle.max_norm_error(
            yq.float().cpu().numpy(),
            oracle.forward(xq.cpu().numpy(), S1h, S2h, p0.alpha.cpu().numpy(),
                           p0.beta.cpu().numpy(), p0.gamma.cpu().numpy()))
        out["decoder_stack_2x7_1p5bpw"] = res

    # ----------------------- factorisation of a dense 4096 x 4096 matrix --
    if want("factorize"):
        Nf = Mf = 4096
        kf, outer, iters, n_pow = 2048, 2, 5, 8
        rngf = np.random.default_rng(9)
        Wf = torch.as_tensor(rngf.standard_normal((Nf, Mf)) * 0.02, dtype=torch.float32).to(dev)
        omf = torch.as_tensor(rngf.standard_normal((kf, Nf)), dtype=torch.float32).to(dev)
        wsf = torch.empty(dbf.dbf_factorize_workspace_bytes(Nf, Mf, kf), dtype=torch.uint8,
                          device=dev)
        run = lambda: dbf.dbf_factorize(Wf, kf, omf, outer=outer, admm_iters=iters,  # noqa: E731
                                        power_iters=n_pow, ws=wsf)
        run()
        torch.cuda.synchronize()
        s_, e_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s_.record()
        fres = run()
        e_.record()
        torch.cuda.synchronize()
        tf = s_.elapsed_time(e_) / 1e3
        n_ns = 2 * math.ceil(math.log2(kf + 1)) + 10
        ns = n_ns * 2 * 2 * kf ** 3
        gem = 2 * kf * Nf * Mf + 2 * Nf * kf * kf  # the start, the first least squares
        gem += outer * (2 * kf * kf * Mf + ns + 2 * Nf * Mf * kf + iters * 2 * Nf * kf * kf
                        + 2 * kf * kf * Nf + ns + 2 * kf * Mf * Nf + iters * 2 * kf * kf * Mf)
        gem += 2 * Nf * kf * Mf  # the error check
        # the fp64 oracle on a bounded sample: a 512 x 512 matrix, k = 256
        Ws = rngf.standard_normal((512, 512)) * 0.02
        oms = rngf.standard_normal((256, 512))
        t_o = time.perf_counter()
        ref_s = oracle.factorize(Ws, 256, oms, 1, 2)
        t_o = time.perf_counter() - t_o
        got_s = dbf.dbf_factorize(torch.as_tensor(Ws, dtype=torch.float32).to(dev), 256,
                                  torch.as_tensor(oms, dtype=torch.float32).to(dev), outer=1,
                                  admm_iters=2, power_iters=30)
        torch.cuda.synchronize()
        out["factorize_4096x4096_k2048"] = {
            "N": Nf, "M": Mf, "k": kf, "outer": outer, "admm_iters": iters, "power_iters": n_pow,
            "seconds": tf, "rel_err": float(fres["rel_err"]),
            "gemm_tflop_executed": gem / 1e12, "achieved_TFLOPs": gem / tf / 1e12,
            "fp32_peak_frac": gem / tf / 1e12 / FP32_PEAK_TFLOPS,
            "sample_512_k256": {"rel_err_gpu": float(got_s["rel_err"]),
                                "rel_err_oracle": ref_s["rel_err"], "oracle_seconds": t_o},
        }
        log(f"factorize 4096x4096 k=2048: {tf:.3f} s, rel err {float(fres['rel_err']):.4f}, "
            f"{gem / tf / 1e12:.1f} TFLOP/s executed; 512 sample: gpu "
            f"{float(got_s['rel_err']):.4f} vs oracle {ref_s['rel_err']:.4f} ({t_o:.1f} s)")

    # ------------------------------------------------ copy calibration --
    if args.copy_calibration:
        n = COPY_MIB << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy calibration: {COPY_MIB} MiB device copy x5")

    # ------------------------------------- achievable HBM: a device copy --
    if want("copy"):
        n = COPY_MIB << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        sec = time_calls(lambda i: dst.copy_(src), 20, 3) / 20
        out["device_copy"] = {"MiB": COPY_MIB, "GBs_read_plus_write": 2 * n / sec / 1e9,
                              "hbm_frac": 2 * n / sec / 1e9 / HBM_PEAK_GBS}
        log(f"device copy {COPY_MIB} MiB: {2 * n / sec / 1e9:.0f} GB/s read + write")
        del src, dst

    # ---- the vendor library's fp16 products on this machine (context only) --
    # torch's fp16 linear (hipBLASLt): a large square product for the matrix
    # cores' achievable rate, the dense fp16 layer the factorisation replaces
    # (4096 x 4096 at T = 256 and T = 1) and a dense product of one stage's
    # shape (T = 256, 2048 x 4096, i.e. the signs stored as fp16); and one
    # fp32 product of the factorisation's size (2048^3).  Weights rotate over
    # copies that exceed twice the Infinity Cache, as above.
    if want("vendor"):
        F = torch.nn.functional
        ven = {}

        def linear_case(name, T_, rows, cols, n_copies, calls, dtype=torch.float16):
            g = torch.Generator(device=dev)
            g.manual_seed(7)
            a = torch.randn(T_, cols, device=dev, dtype=dtype, generator=g)
            ws_ = [torch.randn(rows, cols, device=dev, dtype=dtype, generator=g)
                   for _ in range(n_copies)]
            o = torch.empty(T_, rows, device=dev, dtype=dtype)
            esz = a.element_size()
            peak = MFMA_F16_PEAK_TFLOPS if dtype == torch.float16 else FP32_PEAK_TFLOPS

            def f(i):
                torch.matmul(a, ws_[i % n_copies].t(), out=o)

            sec_eager = time_calls(f, calls, 5) / calls
            f(n_copies - 1)
            torch.cuda.synchronize()
            want_o = o.clone()
            o.zero_()
            # the same calls replayed from a HIP graph (free of the host's
            # launch rate); the last replayed call's result must equal the
            # eager one
            try:
                sec_graph = time_graph(f, n_copies, max(calls // n_copies, 2), 1)
                same = bool(torch.equal(o, want_o))
            except RuntimeError as exc:  # capture refused: keep the eager figure
                log(f"vendor {name}: no graph replay ({exc})")
                sec_graph, same = None, False
            sec = sec_graph if same else sec_eager
            fl = 2.0 * T_ * rows * cols
            by = esz * (T_ * cols + rows * cols + T_ * rows)
            ven[name] = {"T": T_, "rows": rows, "cols": cols, "dtype": str(dtype).split(".")[-1],
                         "us_per_call": sec * 1e6,
                         "us_per_call_eager": sec_eager * 1e6, "graph_replay": same,
                         "TFLOPs": fl / sec / 1e12, "mfma_frac": fl / sec / 1e12 / peak,
                         "GBs": by / sec / 1e9, "hbm_frac": by / sec / 1e9 / HBM_PEAK_GBS,
                         "weight_copies": n_copies}
            log(f"vendor {name}: {sec * 1e6:.2f} us/call ({'graph' if same else 'eager'}; "
                f"eager {sec_eager * 1e6:.2f}), {fl / sec / 1e12:.0f} TFLOP/s, {by / sec / 1e9:.0f} GB/s")
            del a, ws_, o

        linear_case("square_8192", 8192, 8192, 8192, 1, 20)
        linear_case("dense_layer_4096_T256", 256, 4096, 4096, 16, 64)
        linear_case("dense_layer_4096_T1", 1, 4096, 4096, 16, 256)
        linear_case("dense_layer_4096_T4096", 4096, 4096, 4096, 16, 32)
        linear_case("stage1_shape_dense_T256", 256, 2048, 4096, 32, 64)
        # fp32: the factorisation's products (2048^3, against the fp32 matrix peak)
        tf32 = torch.backends.cuda.matmul.allow_tf32
        torch.backends.cuda.matmul.allow_tf32 = False  # full fp32 products
        linear_case("sgemm_2048_fp32", 2048, 2048, 2048, 1, 20, torch.float32)
        torch.backends.cuda.matmul.allow_tf32 = tf32
        out["vendor_fp16_linear"] = ven

    # ------------------------------------------------------ CPU oracle --
    cpu = None
    cpu_ctx = None
    if not args.no_cpu_baseline:
        try:
            from threadpoolctl import threadpool_info
            cores = max((d.get("num_threads", 1) for d in threadpool_info()), default=1)
        except Exception:  # pragma: no cover
            cores = os.cpu_count()
        n_rep, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < 10.0:
            oracle.forward(L.x, L.S1, L.S2, L.alpha, L.beta, L.gamma)
            n_rep += 1
        dt = time.perf_counter() - t0
        cpu = {"value": n_rep * T / dt, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
               "sample": f"fp64 oracle on the same 4096x4096 R=2048 layer, T=256, "
                         f"{n_rep} calls in {dt:.1f} s"}
        log(f"cpu oracle: {cpu['value']:.0f} tokens/s on {cores} threads")
        cpu_ctx = {"host_cpu": host_cpu_model(), "host_threads": os.cpu_count()}
        try:
            from threadpoolctl import threadpool_limits
            with threadpool_limits(limits=1):
                n1, t1s = 0, time.perf_counter()
                while time.perf_counter() - t1s < 5.0:
                    oracle.forward(L.x, L.S1, L.S2, L.alpha, L.beta, L.gamma)
                    n1 += 1
                d1 = time.perf_counter() - t1s
            cpu_ctx["oracle_1_thread_tokens_per_s"] = n1 * T / d1
            log(f"cpu oracle, 1 thread: {n1 * T / d1:.0f} tokens/s")
        except ImportError:  # pragma: no cover
            pass
        # the factored form against the dense update built from the factors
        # (small configurations only: the dense update is N x M)
        dense = {}
        for cfg, tc, name in ((1, 4, "tiny_T4"), (2, 1, "lordba_T1")):
            Lc = synth.make_config_layer(cfg, tc)
            ta = time.perf_counter()
            yf = oracle.forward(Lc.x, Lc.S1, Lc.S2, Lc.alpha, Lc.beta, Lc.gamma)
            tf_ = time.perf_counter() - ta
            ta = time.perf_counter()
            dw = oracle.delta_w(Lc.S1, Lc.S2, Lc.alpha, Lc.beta, Lc.gamma)
            yd = np.asarray(Lc.x, np.float64) @ dw.T
            td_ = time.perf_counter() - ta
            dense[name] = {"factored_s": tf_, "dense_dW_s": td_,
                           "max_norm_diff": oracle.max_norm_error(yd, yf)}
            log(f"cpu {name}: factored {tf_ * 1e3:.2f} ms, dense dW {td_ * 1e3:.1f} ms")
        cpu_ctx["dense_vs_factored"] = dense

    line = {
        "metric": METRIC,
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": t_call * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "dbf_attn_proj_4096x4096_R2048_T256", "N": N_, "R": R_, "M": M_,
                   "ell": 1, "T": T, "cold_cache_instances": n_inst},
        "effective_GBs": byts / t_call / 1e9,
        "parity_err": err256,
        "achieved_TFLOPs_per_call": achieved_tflops,
        "roofline": roof,
        "decode_roofline": decode_roof,
        "cpu_baseline": cpu,
        "cpu_context": cpu_ctx,
        "cases": out,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
