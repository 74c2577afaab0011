#!/usr/bin/env python3
"""Throughput of the double-binary-factorised product on one MI355X.

Workload (the metric's configuration): a DBF-compressed attention projection,
N = M = 4096, R = 2048, ell = 1, Bernoulli signs, log-normal fp16 scales,
x ~ N(0,1) fp16 (synthetic, seeded).  One step is one ``dbf_forward`` call
over a batch of T = 256 tokens (the prefill case, matrix-core path); the same
JSON line also reports the decode case (T = 1, the sign-GEMV path), a grouped
decode over 256 distinct layers in one dispatch, and the 64-adapter serving
batch (T = 2048, R = 64, ell = 2, Zipf ids).

Every timed call reads factors that are not in any cache: calls rotate over
distinct device copies of the layer whose total size exceeds twice the 256 MB
Infinity Cache.  Times come from HIP events on the stream the library
launches on.  Prints ONE JSON line on stdout.
"""
from __future__ import annotations

import argparse
import json
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
N_, R_, M_ = 4096, 2048, 4096


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


def replicate(t: torch.Tensor, k: int):
    return [t.clone() for _ in range(k)]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", default="", help="comma list of cases to run (profiling)")
    args = ap.parse_args()
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
    if want("prefill"):
        sec = time_calls(call256, args.steps, args.warmup)
        t_call = sec / args.steps
        value = T / t_call
        achieved_tflops = flops / t_call / 1e12
        log(f"prefill T=256: {t_call * 1e6:.2f} us/call, {achieved_tflops:.1f} TFLOP/s")

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
        b1 = alg_bytes(N_, R_, M_, 1, 1)
        out["decode_T1"] = {
            "T": 1, "us_per_call": t1 * 1e6, "tokens_per_s": 1 / t1,
            "effective_GBs": b1 / t1 / 1e9, "hbm_frac": b1 / t1 / 1e9 / HBM_PEAK_GBS,
            "alg_bytes_per_call": b1, "parity_err": err1,
        }
        log(f"decode T=1: {t1 * 1e6:.2f} us/call, {b1 / t1 / 1e9:.1f} GB/s")

    # ------------------------- grouped decode: 256 layers, 1 token each --
    if want("grouped"):
        G = n_inst
        tab = lambda ts: dbf.pointer_table(ts, dev)  # noqa: E731
        tB1, tB2 = tab(B1s), tab(B2s)
        ta, tb, tg = tab([pl.alpha] * G), tab([pl.beta] * G), tab([pl.gamma] * G)
        xg = x256[:1].repeat(G, 1).contiguous()
        ids = torch.arange(G, dtype=torch.int32, device=dev)
        yg = torch.empty((G, N_), dtype=torch.float16, device=dev)
        wsg = torch.empty(dbf.dbf_workspace_bytes(N_, R_, M_, 1, G), dtype=torch.uint8, device=dev)

        def callg(i):
            dbf.dbf_forward_multi_adapter(xg, ids, tB1, tB2, ta, tb, tg, G, N_, R_, M_, 1, y=yg,
                                          ws=wsg)

        callg(0)
        torch.cuda.synchronize()
        errg = oracle.max_norm_error(yg[:1].float().cpu().numpy(), yref[:1])
        ng = max(args.steps // 10, 10)
        tg_ = time_calls(callg, ng, 3) / ng
        bg = G * alg_bytes(N_, R_, M_, 1, 1, ids=True)
        out["grouped_decode_256_layers"] = {
            "layers": G, "T_per_layer": 1, "us_per_call": tg_ * 1e6, "tokens_per_s": G / tg_,
            "effective_GBs": bg / tg_ / 1e9, "hbm_frac": bg / tg_ / 1e9 / HBM_PEAK_GBS,
            "alg_bytes_per_call": bg, "parity_err_token0": errg,
        }
        log(f"grouped decode: {tg_ * 1e6:.1f} us/call, {bg / tg_ / 1e9:.1f} GB/s")

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
        nm = max(args.steps // 2, 20)
        tm = time_calls(callm, nm, args.warmup) / nm
        bm = 64 * (-(-(2 * 4096 * 64) // 8) + 2 * 2 * (4096 + 64 + 4096)) + 2 * 4096 * Tm * 2 + 4 * Tm
        fm = alg_flops(4096, 64, 4096, 2, Tm)
        out["multi_adapter_64"] = {
            "T": Tm, "adapters": 64, "us_per_call": tm * 1e6, "tokens_per_s": Tm / tm,
            "effective_GBs": bm / tm / 1e9, "hbm_frac": bm / tm / 1e9 / HBM_PEAK_GBS,
            "mfma_frac": fm / tm / 1e12 / MFMA_F16_PEAK_TFLOPS, "alg_bytes_per_call": bm,
            "parity_err": errm,
        }
        log(f"multi-adapter: {tm * 1e6:.1f} us/call, {bm / tm / 1e9:.1f} GB/s")

    # ------------------------------------------------------ CPU oracle --
    cpu = None
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
        "roofline": {"bound": "mfma", "achieved": achieved_tflops, "peak": MFMA_F16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved_tflops / MFMA_F16_PEAK_TFLOPS,
                     "traffic": None,
                     "kernel": "k_stage_f16 stage 1 + stage 2 (one dbf_forward call)"},
        "cpu_baseline": cpu,
        "cases": out,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
