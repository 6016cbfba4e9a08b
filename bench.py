#!/usr/bin/env python3
"""Benchmark of the SSD core on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

A step is one chunked forward (ssd_chunk_scan_prepare + ssd_chunk_scan_walk,
i.e. ssd_chunk_scan_fwd) over one batch of the 1.3B-layer workload
(batch 4, T 2048, 64 heads, P 64, N 128, one group, chunk 256, bf16
storage), with inputs resident in HBM. Three independent input / output /
workspace sets rotate (444 MB together, more than the 256 MB Infinity Cache),
so no step reads the previous step's data from the cache. The decode step is
timed after the forward: 1000 ssd_step calls on the 256 x 64 x 64 x 128 fp32
state, then 50 forwards with the fused layer prologue / epilogue
(ssd_chunk_scan_fwd_fused) and 20 backward passes (ssd_chunk_scan_bwd) of
the forward workload, reported beside the forward. Prints one JSON line.

The oracle is timed beside the GPU on a bounded sample of the same workload
(whole batch elements, about ten seconds of host work) for the cpu_baseline
field.
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "SSD fwd tokens/s + % bf16 MFMA roofline (h=64,P=64,N=128,T=2048); decode GB/s"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix cores
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "walk_l1p3b_traffic.txt")
WALK_SOURCES = [os.path.join(ROOT, "ssd_sequence_mixing_amd", "csrc", f)
                for f in ("ssd_fwd.hip", "ssd_common.h")]


def fwd_accounting(cfg, chunk):
    """Algorithmic work of one forward (what the method must do).

    Flops: the causal diagonal block with C B^T once per group, plus the chunk
    state (2NP per token and head) and state -> output (2NP):
        F/token = G (Q+1) N + H [(Q+1) P + 4 N P].
    Bytes: read X, dt, B, C, A, D; write Y and the final state. Workspace
    traffic (log-decays, C B^T tiles) is implementation traffic, not credited.
    """
    es = 2 if cfg.dtype == "bf16" else 4
    Bz, T, H, P, N, G, Q = cfg.batch, cfg.seqlen, cfg.nheads, cfg.headdim, cfg.dstate, cfg.ngroups, chunk
    tokens = Bz * T
    flops = tokens * (G * (Q + 1) * N + H * ((Q + 1) * P + 4 * N * P))
    x = tokens * H * P * es
    bc = tokens * G * N * es
    final = Bz * H * P * N * 4
    total = x + tokens * H * es + 2 * bc + 2 * H * 4 + x + final
    walk = x + 2 * bc + x + final  # the walk kernel's share: X, B, C in; Y, final state out
    return {"flops": flops, "bytes": total, "walk_bytes": walk, "tokens": tokens}


def decode_accounting(d):
    """One decode step: the fp32 state in and out, plus x, y, dt, B, C."""
    state = d.batch * d.nheads * d.headdim * d.dstate * 4
    small = (2 * d.batch * d.nheads * d.headdim + d.batch * d.nheads + 2 * d.batch * d.ngroups * d.dstate) * 2
    return {"bytes": 2 * state + small + 2 * d.nheads * 4,
            "flops": 5 * d.batch * d.nheads * d.headdim * d.dstate}


def walk_source_hash():
    h = hashlib.sha256()
    for p in WALK_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def read_traffic():
    """HBM bytes per walk launch measured with rocprofv3 counters (FETCH_SIZE +
    WRITE_SIZE, scaled by a copy-kernel calibration), if they were taken on the
    current kernel source; None otherwise."""
    try:
        vals = {}
        with open(TRAFFIC_FILE) as f:
            for line in f:
                if ":" in line:
                    k, v = line.split(":", 1)
                    vals[k.strip()] = v.strip()
        if vals.get("source_sha256") != walk_source_hash():
            return None
        return float(vals["hbm_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def cpu_baseline(inp, cfg, budget_s=10.0, max_passes=200):
    """Oracle throughput on this host: whole batch elements of the workload, one
    at a time, repeated over the batch until about budget_s of wall time."""
    import numpy as np

    import oracle
    per_b = [[np.ascontiguousarray(inp[k][b:b + 1], dtype=np.float64) for k in ("X32", "dt32", "B32", "C32")]
             for b in range(cfg.batch)]
    done_tokens, elapsed, used = 0, 0.0, 0
    while elapsed < budget_s and used < max_passes * cfg.batch:
        args = per_b[used % cfg.batch]
        t0 = time.perf_counter()
        oracle.fwd(args[0], args[1], inp["A"], args[2], args[3], inp["D"], cfg.ngroups)
        elapsed += time.perf_counter() - t0
        done_tokens += cfg.seqlen
        used += 1
    return {"value": done_tokens / elapsed, "unit": "tokens/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"{used} single-sequence forwards cycling over the {cfg.batch} batch elements of the "
                      f"same workload ({done_tokens} tokens x {cfg.nheads} heads), fp64 sequential "
                      f"recurrence, {elapsed:.2f} s wall"}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--chunk", type=int, default=0, help="override the workload's chunk length")
    ap.add_argument("--workload", default="l1p3b_bf16",
                    choices=["l1p3b_bf16", "l125m_bf16", "long16k_bf16"],
                    help="forward workload (default: the 1.3B-layer shape the metric is quoted on; "
                         "the others are the 125M-layer shape and the 16K-token shape)")
    ap.add_argument("--sets", type=int, default=3, help="rotating input/output/workspace sets")
    ap.add_argument("--decode-steps", type=int, default=1000)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-fused", action="store_true")
    ap.add_argument("--backward-steps", type=int, default=20)
    ap.add_argument("--traffic-probe", action="store_true",
                    help="for counter runs: 5 walk launches, then 5 element-wise negations of a "
                         "512 MiB bf16 buffer (a copy of known size, to calibrate the counters); "
                         "prints one line and exits")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures the SSD core on a single GPU; multi-GPU runs are not implemented "
              "(heads shard across GPUs with no communication inside the core).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import ssd_inputs as si
    import ssd_sequence_mixing_amd as ssd

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    lib = ssd.load()
    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)

    def up(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    cfg = si.CONFIGS[args.workload]
    chunk = args.chunk or cfg.chunk
    code = ssd.SSD_BF16 if cfg.dtype == "bf16" else ssd.SSD_F32
    Bz, T, H, P, N, G = cfg.batch, cfg.seqlen, cfg.nheads, cfg.headdim, cfg.dstate, cfg.ngroups
    need = ssd.ssd_chunk_scan_fwd_workspace_bytes(Bz, T, H, P, N, G, chunk, code)
    stream = torch.cuda.current_stream()
    sptr = stream.cuda_stream

    sets, first_inp = [], None
    for k in range(args.sets):
        inp = si.make_fwd_inputs(dataclasses.replace(cfg, seed=cfg.seed + 1000 * k))
        if k == 0:
            first_inp = inp
        t = {n: up(inp[n]) for n in ("X", "dt", "B", "C", "A", "D")}
        t["Y"] = torch.empty_like(t["X"])
        t["F"] = torch.empty((Bz, H, P, N), dtype=torch.float32, device=dev)
        t["W"] = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
        p = {n: v.data_ptr() for n, v in t.items()}
        t["prep"] = (p["dt"], p["A"], p["B"], p["C"], chunk, Bz, T, H, P, N, G, code, p["W"], need, sptr)
        t["walk"] = (p["X"], p["B"], p["C"], p["D"], None, chunk, p["Y"], p["F"], Bz, T, H, P, N, G, code,
                     p["W"], need, sptr)
        sets.append(t)

    if args.traffic_probe:
        for i in range(5):
            t = sets[i % len(sets)]
            if lib.ssd_chunk_scan_prepare(*t["prep"]) or lib.ssd_chunk_scan_walk(*t["walk"]):
                raise RuntimeError("forward failed")
        torch.cuda.synchronize()
        n_copy = 512 * 2 ** 20
        src = torch.ones(n_copy // 2, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        print(json.dumps({"traffic_probe": True, "walk_launches": 5, "copy_bytes_read": n_copy,
                          "copy_bytes_written": n_copy,
                          "walk_algorithmic_bytes": fwd_accounting(cfg, chunk)["walk_bytes"]}), flush=True)
        return

    def step(t):
        st = lib.ssd_chunk_scan_prepare(*t["prep"])
        st = st or lib.ssd_chunk_scan_walk(*t["walk"])
        if st:
            raise ssd.SSDError(st, "forward")

    for i in range(args.warmup):
        step(sets[i % len(sets)])
    torch.cuda.synchronize()

    # Timed region: K whole steps, bracketed by two events and nothing between
    # the launches (an event recorded between two kernels adds a few us of gap).
    K = args.steps
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall0 = time.perf_counter()
    start.record(stream)
    for i in range(K):
        step(sets[i % len(sets)])
    end.record(stream)
    torch.cuda.synchronize()
    wall_s = time.perf_counter() - t_wall0
    ms_total = start.elapsed_time(end)
    ms_step = ms_total / K

    # Per-kernel durations: the same K steps again, with an event on the launch
    # stream before and after each kernel.
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    for i in range(K):
        t = sets[i % len(sets)]
        e = evs[i]
        e[0].record(stream)
        if lib.ssd_chunk_scan_prepare(*t["prep"]):
            raise RuntimeError("prepare failed")
        e[1].record(stream)
        if lib.ssd_chunk_scan_walk(*t["walk"]):
            raise RuntimeError("walk failed")
        e[2].record(stream)
    torch.cuda.synchronize()
    prep_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    walk_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))

    acc = fwd_accounting(cfg, chunk)
    t_s = ms_step / 1e3
    tokens_per_s = acc["tokens"] / t_s
    tflops = acc["flops"] / t_s / 1e12
    hbm_gbs = acc["bytes"] / t_s / 1e9
    mfma_frac = tflops / MFMA_BF16_PEAK_TFLOPS
    hbm_frac = hbm_gbs / HBM_PEAK_GBS
    roof_time = max(acc["flops"] / (MFMA_BF16_PEAK_TFLOPS * 1e12), acc["bytes"] / (HBM_PEAK_GBS * 1e9))
    walk_gbs = acc["walk_bytes"] / (walk_ms / 1e3) / 1e9
    traffic = read_traffic() if args.workload == "l1p3b_bf16" else None

    out = {
        "metric": METRIC,
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": {"l1p3b_bf16": "ssd_fwd 1.3B-layer shape", "l125m_bf16": "ssd_fwd 125M-layer shape",
                                "long16k_bf16": "ssd_fwd 16K-token shape"}[args.workload],
                   "batch": Bz, "seqlen": T, "nheads": H,
                   "headdim": P, "dstate": N, "ngroups": G, "chunk": chunk, "storage": cfg.dtype,
                   "rotating_sets": len(sets)},
        "roofline": {"bound": "hbm", "kernel": "k_chunk_walk", "achieved": walk_gbs,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": walk_gbs / HBM_PEAK_GBS,
                     "traffic": traffic, "algorithmic_bytes_per_launch": acc["walk_bytes"],
                     "avg_launch_ms": walk_ms},
        "forward": {"ms_prepare": prep_ms, "ms_walk": walk_ms, "wall_s": wall_s,
                    "tflops": tflops, "mfma_frac": mfma_frac, "hbm_gbs": hbm_gbs, "hbm_frac": hbm_frac,
                    "roof_frac": roof_time / t_s, "algorithmic_flops": acc["flops"],
                    "algorithmic_bytes": acc["bytes"]},
    }

    if not args.no_decode:
        dc = si.DECODE
        d = si.make_decode_inputs(dc)
        state = up(d["state0"])
        A_d, D_d = up(d["A"]), up(d["D"])
        dsets = [{k: up(v) for k, v in s.items() if not k.endswith("32")} for s in d["sets"]]
        y = torch.empty_like(dsets[0]["x"])
        dcode = ssd.SSD_BF16
        dargs = [(state.data_ptr(), s["x"].data_ptr(), s["dt"].data_ptr(), A_d.data_ptr(),
                  s["B"].data_ptr(), s["C"].data_ptr(), D_d.data_ptr(), y.data_ptr(), dc.batch,
                  dc.nheads, dc.headdim, dc.dstate, dc.ngroups, dcode, sptr) for s in dsets]
        for i in range(10):
            lib.ssd_step(*dargs[i % len(dargs)])
        torch.cuda.synchronize()
        ds, de = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ds.record(stream)
        for i in range(args.decode_steps):
            if lib.ssd_step(*dargs[i % len(dargs)]):
                raise RuntimeError("ssd_step failed")
        de.record(stream)
        torch.cuda.synchronize()
        us = ds.elapsed_time(de) * 1e3 / args.decode_steps
        dacc = decode_accounting(dc)
        gbs = dacc["bytes"] / (us / 1e6) / 1e9
        out["decode"] = {"workload": "ssd_step batch 256, 64 heads, P 64, N 128, fp32 state",
                         "steps": args.decode_steps, "us_per_step": us, "GB/s": gbs,
                         "hbm_frac": gbs / HBM_PEAK_GBS, "bytes_per_step": dacc["bytes"],
                         "kernel": "k_step"}
        del state, dsets

    if not args.no_fused:
        # the forward with the layer's fused prologue and epilogue (causal conv1d +
        # SiLU on X, softplus(dt + bias), Y * SiLU(z)) on the same workload
        t = sets[0]
        rng = np.random.default_rng(8)
        cw = up((0.5 * rng.standard_normal((H * P, 4))).astype(np.float32))
        cb = up((0.1 * rng.standard_normal(H * P)).astype(np.float32))
        dtb = up((0.5 * rng.standard_normal(H)).astype(np.float32))
        zz = torch.empty_like(t["X"]).normal_()
        Yf = torch.empty_like(t["X"])
        Ff = torch.empty((Bz, H, P, N), dtype=torch.float32, device=dev)
        def fused():
            return ssd.ssd_chunk_scan_fwd_fused(t["X"], t["dt"], t["A"], t["B"], t["C"], t["D"], chunk,
                                                conv_w=cw, conv_b=cb, dt_bias=dtb, dt_softplus=1, z=zz, Y=Yf,
                                                final_state=Ff, workspace=t["W"], stream=stream)
        for _ in range(5):
            fused()
        torch.cuda.synchronize()
        fs, fe = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        fs.record(stream)
        for _ in range(50):
            fused()
        fe.record(stream)
        torch.cuda.synchronize()
        ms_f = fs.elapsed_time(fe) / 50
        out["fused"] = {"workload": out["config"]["workload"] + ", conv1d(4)+SiLU on X, softplus(dt+bias), "
                                    "Y*SiLU(z)", "ms_per_call": ms_f, "tokens_per_s": Bz * T / (ms_f / 1e3),
                        "vs_plain_forward": ms_f / ms_step}
        del zz, Yf, Ff

    bwd_ok = not args.no_backward and cfg.dtype == "bf16"
    if bwd_ok:
        try:
            ssd.ssd_chunk_scan_bwd_workspace_bytes(Bz, T, H, P, N, G, chunk, code)
        except ssd.SSDError:
            bwd_ok = False  # no backward kernel for this shape (e.g. N 256)
            out["backward"] = None
    if bwd_ok:
        # one backward (ssd_chunk_scan_bwd) of the same workload; its states per
        # 64-token tile (2 x 134 MB at the 1.3B shape) already exceed the cache
        t = sets[0]
        rng = np.random.default_rng(7)
        dY = up(si.bf16_round_bits(rng.standard_normal((Bz, T, H, P)).astype(np.float32)))
        nb = ssd.ssd_chunk_scan_bwd_workspace_bytes(Bz, T, H, P, N, G, chunk, code)
        bws = torch.empty(nb, dtype=torch.uint8, device=dev)
        def bwd():
            return ssd.ssd_chunk_scan_bwd(t["X"], t["dt"], t["A"], t["B"], t["C"], t["D"], chunk, dY,
                                          workspace=bws, stream=stream)
        for _ in range(3):
            bwd()
        torch.cuda.synchronize()
        bs, be = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        bs.record(stream)
        for _ in range(args.backward_steps):
            bwd()
        be.record(stream)
        torch.cuda.synchronize()
        ms_b = bs.elapsed_time(be) / args.backward_steps
        es = 2
        bbytes = 2 * (2 * Bz * T * H * P * es + Bz * T * H * es + 2 * Bz * T * G * N * es)
        out["backward"] = {"workload": out["config"]["workload"], "ms_per_call": ms_b,
                           "tokens_per_s": Bz * T / (ms_b / 1e3),
                           "algorithmic_bytes": bbytes, "GB/s": bbytes / (ms_b / 1e3) / 1e9,
                           "hbm_frac": bbytes / (ms_b / 1e3) / 1e9 / HBM_PEAK_GBS,
                           "kernels": "k_state_pass x2, k_bwd_tile, k_bwd_fin, k_bwd_sum_bc (+ k_prepare)"}
        del bws, dY

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(first_inp, cfg)
    else:
        out["cpu_baseline"] = None

    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
