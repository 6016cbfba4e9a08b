#!/usr/bin/env python3
"""Benchmark of the SSD core on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

A step is one chunked forward (ssd_chunk_scan_prepare + ssd_chunk_scan_walk,
i.e. ssd_chunk_scan_fwd) over one batch of the 1.3B-layer workload
(batch 4, T 2048, 64 heads, P 64, N 128, one group, chunk 256, bf16
storage), with inputs resident in HBM. Three independent input / output /
workspace sets rotate (444 MB together, more than the 256 MB Infinity Cache),
so no step reads the previous step's data from the cache. After W untimed
steps, the K timed steps run back to back between two events; events at the
boundaries of R equal sub-blocks give the median per-step time beside the
mean.

The other measurements run before the forward's, in this order: 50 forwards
with the fused layer prologue / epilogue (ssd_chunk_scan_fwd_fused), 20
backward passes (ssd_chunk_scan_bwd) of the forward workload (and 5 of the
16K-token one), the 125M-layer and 16K-token forwards (timed like the main
one after 20 warmup steps, with a quarter of the steps, under "shapes") and
1000 ssd_step calls on the
256 x 64 x 64 x 128 fp32 state (decode). Every input is made before the first
of them, so the GPU work runs back to back, and the forward comes last,
straight after the decode steps: from an idle GPU the same forward takes ~10%
longer for the first few tens of milliseconds, longer than a short timed run
lasts.
Prints one JSON line.

The oracle is timed beside the GPU on a bounded sample of the same workload
(whole batch elements, about ten seconds of host work on all host threads,
and one batch element on a single thread) for the cpu_baseline field.
"""
from __future__ import annotations

import argparse
import dataclasses
import glob
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
# the walk of the bf16 shapes with P 64 and N <= 128 (k_walk_rs)
WALK_KERNEL = "k_walk_rs"
WALK_SOURCES = [os.path.join(ROOT, "ssd_sequence_mixing_amd", "csrc", f)
                for f in ("ssd_walk_rs.hip", "ssd_common.h")]
WORKLOAD_NAMES = {"l1p3b_bf16": "ssd_fwd 1.3B-layer shape", "l125m_bf16": "ssd_fwd 125M-layer shape",
                  "long16k_bf16": "ssd_fwd 16K-token shape"}


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


def bwd_accounting(cfg):
    """Algorithmic bytes of one backward: X, dY, dt, B, C in; dX, ddt, dB, dC out
    (A, D, dA, dD are a few hundred bytes)."""
    es = 2 if cfg.dtype == "bf16" else 4
    x = cfg.batch * cfg.seqlen * cfg.nheads * cfg.headdim * es
    dt = cfg.batch * cfg.seqlen * cfg.nheads * es
    bc = cfg.batch * cfg.seqlen * cfg.ngroups * cfg.dstate * es
    return (2 * x + dt + 2 * bc) + (x + dt + 2 * bc)


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


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


_SINGLE_THREAD_SNIPPET = """
import json, sys, time
sys.path.insert(0, {root!r})
import numpy as np
import ssd_inputs as si
import oracle
cfg = si.CONFIGS[{workload!r}]
inp = si.make_fwd_inputs(cfg)
args = [np.ascontiguousarray(inp[k][:1], dtype=np.float64) for k in ("X32", "dt32", "B32", "C32")]
t0 = time.perf_counter()
oracle.fwd(args[0], args[1], inp["A"], args[2], args[3], inp["D"], cfg.ngroups)
dt = time.perf_counter() - t0
print(json.dumps({{"seconds": dt, "tokens": cfg.seqlen, "threads": oracle.num_threads()}}))
"""


def cpu_single_thread(workload: str):
    """The oracle on one batch element of the workload with one OpenMP thread,
    in a child process (the thread count is fixed when the oracle loads)."""
    import subprocess
    env = dict(os.environ, OMP_NUM_THREADS="1")
    try:
        p = subprocess.run([sys.executable, "-c", _SINGLE_THREAD_SNIPPET.format(root=ROOT, workload=workload)],
                           env=env, capture_output=True, text=True, timeout=120)
        r = json.loads(p.stdout.strip().splitlines()[-1])
    except Exception as e:  # noqa: BLE001  (reported, not fatal)
        return {"error": str(e)[:200]}
    return {"value": r["tokens"] / r["seconds"], "unit": "tokens/s", "cores": r["threads"],
            "sample": f"one sequence of the workload ({r['tokens']} tokens) on one thread, "
                      f"{r['seconds']:.2f} s wall"}


def device_info(torch):
    """GPU model, ROCm / HIP versions and the current clock levels."""
    prop = torch.cuda.get_device_properties(0)
    info = {"name": prop.name, "arch": getattr(prop, "gcnArchName", None),
            "compute_units": prop.multi_processor_count, "hbm_bytes": prop.total_memory,
            "hip_runtime": torch.version.hip}
    try:
        with open("/opt/rocm/.info/version") as f:
            info["rocm"] = f.read().strip()
    except OSError:
        info["rocm"] = None
    # current clock levels from the driver's sysfs tables (the line marked *);
    # read as files, so no program is started from a process that uses the GPU
    clocks = {}
    for card in sorted(glob.glob("/sys/class/drm/card*/device")):
        for name in ("pp_dpm_sclk", "pp_dpm_mclk", "pp_dpm_fclk"):
            try:
                with open(os.path.join(card, name)) as f:
                    cur = [l.strip() for l in f if l.strip().endswith("*")]
                if cur:
                    clocks[f"{os.path.basename(os.path.dirname(card))}/{name[7:]}"] = cur[0]
            except OSError:
                pass
    info["clocks"] = clocks or None
    return info


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
            "kind": "oracle", "cpu_model": cpu_model(),
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
    ap.add_argument("--no-shapes", action="store_true", help="skip the 125M-layer and 16K-token shapes")
    ap.add_argument("--repeats", type=int, default=10,
                    help="sub-blocks of the timed steps for the median per-step time")
    ap.add_argument("--backward-steps", type=int, default=20)
    ap.add_argument("--traffic-probe", action="store_true",
                    help="for counter runs: 5 forwards (or, with --probe-backward, 5 backward passes), "
                         "then 5 element-wise negations of a 512 MiB bf16 buffer (a copy of known size, "
                         "to calibrate the counters); prints one line and exits")
    ap.add_argument("--probe-backward", action="store_true",
                    help="with --traffic-probe: run ssd_chunk_scan_bwd instead of the forward")
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

    stream = torch.cuda.current_stream()
    sptr = stream.cuda_stream

    def make_sets(cfg, chunk, nsets):
        code = ssd.SSD_BF16 if cfg.dtype == "bf16" else ssd.SSD_F32
        Bz, T, H, P, N, G = cfg.batch, cfg.seqlen, cfg.nheads, cfg.headdim, cfg.dstate, cfg.ngroups
        need = ssd.ssd_chunk_scan_fwd_workspace_bytes(Bz, T, H, P, N, G, chunk, code)
        sets, first_inp = [], None
        for k in range(nsets):
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
        return sets, first_inp

    def step(t):
        st = lib.ssd_chunk_scan_prepare(*t["prep"])
        st = st or lib.ssd_chunk_scan_walk(*t["walk"])
        if st:
            raise ssd.SSDError(st, "forward")

    def time_forward(sets, K, warmup, R):
        """K whole steps between two events, with events only at the boundaries
        of R equal sub-blocks (an event between two kernels adds a few us of gap,
        so none sits between the launches of a sub-block); then the same K steps
        with an event around each kernel, for the per-kernel durations."""
        for i in range(warmup):
            step(sets[i % len(sets)])
        torch.cuda.synchronize()
        R = max(1, min(R, K))
        bounds = [round(K * j / R) for j in range(R + 1)]
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(R + 1)]
        torch.cuda.synchronize()
        t_wall0 = time.perf_counter()
        evs[0].record(stream)
        for j in range(R):
            for i in range(bounds[j], bounds[j + 1]):
                step(sets[i % len(sets)])
            evs[j + 1].record(stream)
        torch.cuda.synchronize()
        wall_s = time.perf_counter() - t_wall0
        ms_total = evs[0].elapsed_time(evs[R])
        per_block = [evs[j].elapsed_time(evs[j + 1]) / (bounds[j + 1] - bounds[j]) for j in range(R)]
        kev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
        for i in range(K):
            t, e = sets[i % len(sets)], kev[i]
            e[0].record(stream)
            if lib.ssd_chunk_scan_prepare(*t["prep"]):
                raise RuntimeError("prepare failed")
            e[1].record(stream)
            if lib.ssd_chunk_scan_walk(*t["walk"]):
                raise RuntimeError("walk failed")
            e[2].record(stream)
        torch.cuda.synchronize()
        return {"ms_step": ms_total / K, "median_ms_step": float(np.median(per_block)),
                "ms_step_blocks": [float(v) for v in per_block], "wall_s": wall_s,
                "ms_prepare": float(np.mean([e[0].elapsed_time(e[1]) for e in kev])),
                "ms_walk": float(np.mean([e[1].elapsed_time(e[2]) for e in kev]))}

    def shape_summary(cfg, chunk, tm):
        acc = fwd_accounting(cfg, chunk)
        t_s = tm["ms_step"] / 1e3
        roof_time = max(acc["flops"] / (MFMA_BF16_PEAK_TFLOPS * 1e12), acc["bytes"] / (HBM_PEAK_GBS * 1e9))
        return acc, {"tokens_per_s": acc["tokens"] / t_s, "ms_per_step": tm["ms_step"],
                     "median_ms_per_step": tm["median_ms_step"], "ms_prepare": tm["ms_prepare"],
                     "ms_walk": tm["ms_walk"], "roof_frac": roof_time / t_s,
                     "walk_hbm_frac": acc["walk_bytes"] / (tm["ms_walk"] / 1e3) / 1e9 / HBM_PEAK_GBS}

    cfg = si.CONFIGS[args.workload]
    chunk = args.chunk or cfg.chunk
    code = ssd.SSD_BF16 if cfg.dtype == "bf16" else ssd.SSD_F32
    Bz, T, H, P, N, G = cfg.batch, cfg.seqlen, cfg.nheads, cfg.headdim, cfg.dstate, cfg.ngroups
    sets, first_inp = make_sets(cfg, chunk, args.sets)

    if args.traffic_probe:
        if args.probe_backward:
            t = sets[0]
            dY = torch.empty_like(t["X"]).normal_()
            for _ in range(5):
                ssd.ssd_chunk_scan_bwd(t["X"], t["dt"], t["A"], t["B"], t["C"], t["D"], chunk, dY, stream=stream)
        else:
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
        es = 2 if cfg.dtype == "bf16" else 4
        bwd_bytes = bwd_accounting(cfg)
        print(json.dumps({"traffic_probe": True, "backward": args.probe_backward, "launches": 5,
                          "copy_bytes_read": n_copy, "copy_bytes_written": n_copy,
                          "walk_algorithmic_bytes": fwd_accounting(cfg, chunk)["walk_bytes"],
                          "backward_algorithmic_bytes": bwd_bytes}), flush=True)
        return

    K = args.steps
    # The other GPU workloads first: the forward is timed last, on a GPU whose
    # clocks have left their idle state (see the module docstring). Every input
    # is made before any of them runs, so that the GPU work runs back to back
    # with no long host-side pause between the sections.
    sections = {}
    shape_names = [] if args.no_shapes else [n for n in ("l125m_bf16", "long16k_bf16") if n != args.workload]
    shape_sets = {n: make_sets(si.CONFIGS[n], si.CONFIGS[n].chunk, 3 if n == "l125m_bf16" else 2)[0]
                  for n in shape_names}
    if not args.no_decode:
        dc = si.DECODE
        d = si.make_decode_inputs(dc)
        state = up(d["state0"])
        A_d, D_d = up(d["A"]), up(d["D"])
        dsets = [{k: up(v) for k, v in s.items() if not k.endswith("32")} for s in d["sets"]]
        y = torch.empty_like(dsets[0]["x"])
        del d
    # the backward's output gradient dY ~ N(0, 1), rounded to bf16, per timed workload
    bwd_dy = {}
    if not args.no_backward and cfg.dtype == "bf16":
        for bc in [cfg] + ([si.CONFIGS["long16k_bf16"]] if "long16k_bf16" in shape_names else []):
            rng = np.random.default_rng(7)
            bwd_dy[bc.name] = up(si.bf16_round_bits(
                rng.standard_normal((bc.batch, bc.seqlen, bc.nheads, bc.headdim)).astype(np.float32)))
    torch.cuda.synchronize()

    if not args.no_fused:
        # the forward with the layer's fused prologue and epilogue (causal conv1d +
        # SiLU on X, softplus(dt + bias), Y * SiLU(z)) on the same workload. The
        # step sizes arrive before their activation: raw N(0, 1) with bias -4,
        # so softplus(raw + bias) has the plain workload's distribution.
        t = sets[0]
        rng = np.random.default_rng(8)
        cw = up((0.5 * rng.standard_normal((H * P, 4))).astype(np.float32))
        cb = up((0.1 * rng.standard_normal(H * P)).astype(np.float32))
        dtb = up(np.full(H, -4.0, dtype=np.float32))
        dt_raw = up(si.bf16_round_bits(rng.standard_normal((Bz, T, H)).astype(np.float32)))
        zz = torch.empty_like(t["X"]).normal_()
        Yf = torch.empty_like(t["X"])
        Ff = torch.empty((Bz, H, P, N), dtype=torch.float32, device=dev)
        # arguments marshalled once, as for the forward: the timed loop is C calls only
        fargs = (t["X"].data_ptr(), cw.data_ptr(), cb.data_ptr(), dt_raw.data_ptr(), dtb.data_ptr(), 1,
                 t["A"].data_ptr(), t["B"].data_ptr(), t["C"].data_ptr(), t["D"].data_ptr(), zz.data_ptr(), chunk,
                 Yf.data_ptr(), Ff.data_ptr(), Bz, T, H, P, N, G, code, t["W"].data_ptr(), t["W"].numel(), sptr)

        def fused():
            st = lib.ssd_chunk_scan_fwd_fused(*fargs)
            if st:
                raise ssd.SSDError(st, "ssd_chunk_scan_fwd_fused")
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
        es = 2 if cfg.dtype == "bf16" else 4
        fbytes = fwd_accounting(cfg, chunk)["bytes"] + Bz * T * H * P * es  # plus z
        sections["fused"] = {"workload": WORKLOAD_NAMES[args.workload] + ", conv1d(4)+SiLU on X, softplus(dt+bias) "
                                         "with raw dt ~ N(0,1) and bias -4, Y*SiLU(z)", "ms_per_call": ms_f,
                             "tokens_per_s": Bz * T / (ms_f / 1e3),
                        "algorithmic_bytes": fbytes, "hbm_frac": fbytes / (ms_f / 1e3) / 1e9 / HBM_PEAK_GBS}
        del zz, Yf, Ff, dt_raw

    bwd_ok = not args.no_backward and cfg.dtype == "bf16"
    if bwd_ok:
        try:
            ssd.ssd_chunk_scan_bwd_workspace_bytes(Bz, T, H, P, N, G, chunk, code)
        except ssd.SSDError:
            bwd_ok = False  # no backward kernel for this shape (e.g. N 256)
            sections["backward"] = None
    def time_backward(bcfg, t, bchunk, steps):
        """ssd_chunk_scan_bwd on input set t of workload bcfg: `steps` calls
        between two events, after 3 untimed ones (arguments marshalled once)."""
        bcode = ssd.SSD_BF16 if bcfg.dtype == "bf16" else ssd.SSD_F32
        b_, t_, h_, p_, n_, g_ = bcfg.batch, bcfg.seqlen, bcfg.nheads, bcfg.headdim, bcfg.dstate, bcfg.ngroups
        dY = bwd_dy[bcfg.name]
        nb = ssd.ssd_chunk_scan_bwd_workspace_bytes(b_, t_, h_, p_, n_, g_, bchunk, bcode)
        bws = torch.empty(nb, dtype=torch.uint8, device=dev)
        g = {"dX": torch.empty_like(t["X"]), "ddt": torch.empty_like(t["dt"]), "dB": torch.empty_like(t["B"]),
             "dC": torch.empty_like(t["C"]), "dA": torch.empty_like(t["A"]), "dD": torch.empty_like(t["D"])}
        bargs = (t["X"].data_ptr(), t["dt"].data_ptr(), t["A"].data_ptr(), t["B"].data_ptr(), t["C"].data_ptr(),
                 t["D"].data_ptr(), bchunk, None, dY.data_ptr(), None, g["dX"].data_ptr(), g["ddt"].data_ptr(),
                 g["dA"].data_ptr(), g["dB"].data_ptr(), g["dC"].data_ptr(), g["dD"].data_ptr(), None,
                 b_, t_, h_, p_, n_, g_, bcode, bws.data_ptr(), nb, sptr)

        def bwd():
            st = lib.ssd_chunk_scan_bwd(*bargs)
            if st:
                raise ssd.SSDError(st, "ssd_chunk_scan_bwd")
        for _ in range(3):
            bwd()
        torch.cuda.synchronize()
        bs, be = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        bs.record(stream)
        for _ in range(steps):
            bwd()
        be.record(stream)
        torch.cuda.synchronize()
        ms_b = bs.elapsed_time(be) / steps
        bbytes = bwd_accounting(bcfg)
        del bws, g
        return {"workload": WORKLOAD_NAMES.get(bcfg.name, bcfg.name), "ms_per_call": ms_b, "tokens_per_s": b_ * t_ / (ms_b / 1e3),
                "algorithmic_bytes": bbytes, "GB/s": bbytes / (ms_b / 1e3) / 1e9,
                "hbm_frac": bbytes / (ms_b / 1e3) / 1e9 / HBM_PEAK_GBS}

    if bwd_ok:
        # one backward (ssd_chunk_scan_bwd) of the same workload; its states per
        # 64-token tile (2 x 134 MB at the 1.3B shape) already exceed the cache
        sections["backward"] = time_backward(cfg, sets[0], chunk, args.backward_steps)
        sections["backward"]["kernels"] = ("k_state_passes (both state passes, one launch), k_bwd_tile, k_bwd_fin, "
                                      "k_bwd_heads, k_bwd_sum_bc (+ k_prepare; k_bwd_dx where the n axis is split)")
        if not args.no_shapes and args.workload != "long16k_bf16":
            # the 16K-token workload's backward (N 256: the tile kernel takes the n axis in 2 slices)
            c3 = si.CONFIGS["long16k_bf16"]
            s3 = shape_sets["long16k_bf16"]
            sections["backward"]["long16k_bf16"] = time_backward(c3, s3[0], c3.chunk, max(5, args.backward_steps // 4))

    # the other two forward shapes
    if shape_names:
        # the other two forward workloads, timed the same way with fewer steps
        sections["shapes"] = {}
        for name in shape_names:
            c2 = si.CONFIGS[name]
            s2 = shape_sets[name]
            tm2 = time_forward(s2, max(10, K // 4), 20, args.repeats)
            _, summ = shape_summary(c2, c2.chunk, tm2)
            summ["workload"] = WORKLOAD_NAMES[name]
            summ["config"] = {"batch": c2.batch, "seqlen": c2.seqlen, "nheads": c2.nheads, "headdim": c2.headdim,
                              "dstate": c2.dstate, "ngroups": c2.ngroups, "chunk": c2.chunk}
            sections["shapes"][name] = summ

    # the decode steps straight before the forward: 180 ms of back-to-back GPU work
    if not args.no_decode:
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
        sections["decode"] = {"workload": "ssd_step batch 256, 64 heads, P 64, N 128, fp32 state",
                         "steps": args.decode_steps, "us_per_step": us, "GB/s": gbs,
                         "hbm_frac": gbs / HBM_PEAK_GBS, "bytes_per_step": dacc["bytes"],
                         "kernel": "k_step"}
        del state, dsets

    tm = time_forward(sets, K, args.warmup, args.repeats)
    ms_step, prep_ms, walk_ms, wall_s = tm["ms_step"], tm["ms_prepare"], tm["ms_walk"], tm["wall_s"]

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
        "config": {"workload": WORKLOAD_NAMES[args.workload],
                   "batch": Bz, "seqlen": T, "nheads": H,
                   "headdim": P, "dstate": N, "ngroups": G, "chunk": chunk, "storage": cfg.dtype,
                   "rotating_sets": len(sets)},
        "roofline": {"bound": "hbm", "kernel": WALK_KERNEL, "achieved": walk_gbs,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": walk_gbs / HBM_PEAK_GBS,
                     "traffic": traffic, "algorithmic_bytes_per_launch": acc["walk_bytes"],
                     "avg_launch_ms": walk_ms},
        "forward": {"ms_prepare": prep_ms, "ms_walk": walk_ms, "wall_s": wall_s,
                    "median_ms_per_step": tm["median_ms_step"], "repeats": len(tm["ms_step_blocks"]),
                    "ms_per_step_min": min(tm["ms_step_blocks"]), "ms_per_step_max": max(tm["ms_step_blocks"]),
                    "tflops": tflops, "mfma_frac": mfma_frac, "hbm_gbs": hbm_gbs, "hbm_frac": hbm_frac,
                    "roof_frac": roof_time / t_s, "algorithmic_flops": acc["flops"],
                    "algorithmic_bytes": acc["bytes"]},
        "device": device_info(torch),
    }
    out.update(sections)
    if "fused" in out:
        out["fused"]["vs_plain_forward"] = out["fused"]["ms_per_call"] / ms_step

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(first_inp, cfg)
        out["cpu_baseline"]["single_thread"] = cpu_single_thread(args.workload)
    else:
        out["cpu_baseline"] = None

    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
