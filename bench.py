#!/usr/bin/env python3
"""Throughput of causal GQA attention forward + backward on one MI355X.

A step is one pass of the whole path on one batch of synthetic input:
attn_fwd (O, LSE), then the backward's two phases, attn_bwd_dq (D =
rowsum(dO o O), dQ) and attn_bwd_dkdv (dK, dV) -- together exactly attn_bwd --
all on torch's current stream, inputs resident in HBM.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload gpt2_gqa] [--out-dtype f32|bf16]
    python bench.py --all-configs [--oracle]     # per-workload report, see below
    python bench.py --decode                     # few-query attention over a K/V cache
    python bench.py --naive                      # tiled forward against the naive materialised-score one
    python bench.py --rope                       # rotary q/k on fused-QKV views against the plain path

Prints one JSON line. `value` is fwd+bwd TFLOP/s counted with the causal
N^2/2 convention (forward 4d flops per visible pair, backward 2.5x that).
The roofline object describes the dominant kernel (the longest of the
three): the contraction flops that kernel performs per launch -- per visible
(query, key) pair 4d for the forward, 6d for the dQ pass (S, dP, dQ) and 8d
for the dK/dV pass (S, dP, dV, dK) -- divided by its mean duration, measured
with HIP events recorded on the launch stream around each launch in the timed
region (the other two kernels' means come from an untimed pass with events
around every kernel, so that the timed steps carry only the two event records
the roofline needs). cpu_baseline times the float64 oracle on this host on the
same workload (fwd + bwd).

--all-configs prints one JSON line per workload instead (tiny fp32 to the
wide d=128 stress shape): median, p10 and p90 over R repetitions (after 10
warm-up ones) of the forward, the backward and their sum, each repetition
bracketed by HIP events on the launch stream, with TFLOP/s at the median
against the published 2.5 PFLOP/s and against the dense bf16 matrix-core
rate this GPU sustains in a register-only MFMA loop (measured first, as is
the shader clock before and after). --oracle adds the float64 oracle's fwd and
bwd wall times on this host for each workload (median of 3; once for the
largest).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import tiled_causal_attention_amd as tca  # noqa: E402
import workloads  # noqa: E402

PEAK_MFMA_BF16_TFLOPS = 2500.0   # MI355X published dense bf16/fp16 matrix peak
OUT_DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16}
METRIC = "causal attn fwd+bwd TFLOP/s + % bf16 MFMA peak, B8 Hq12/Hkv4 N1024 d64"


def metric_for(s) -> str:
    """The same metric named for another workload's shape (the headline keeps METRIC verbatim)."""
    kind = "causal" if s.causal else "non-causal"
    return f"{kind} attn fwd+bwd TFLOP/s + % bf16 MFMA peak, B{s.B} Hq{s.Hq}/Hkv{s.Hkv} N{s.N} d{s.d}"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default=workloads.HEADLINE, choices=sorted(workloads.CONFIGS))
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-check", action="store_true")
    p.add_argument("--all-configs", action="store_true",
                   help="per-workload report (median/p10/p90) instead of the one-line benchmark")
    p.add_argument("--oracle", action="store_true", help="with --all-configs: time the oracle per workload")
    p.add_argument("--rope", action="store_true",
                   help="one JSON line: fwd+bwd with rotary q/k on views of one fused QKV buffer, "
                        "against the plain path on contiguous tensors")
    p.add_argument("--naive", action="store_true",
                   help="one JSON line: the forward of the workload, tiled against the naive materialised-score one")
    p.add_argument("--decode", action="store_true",
                   help="one JSON line per decode workload (few queries over a K/V cache) instead")
    p.add_argument("--ceiling", action="store_true",
                   help="one JSON line per instruction mix: the per-block mixes of the three kernels "
                        "run register/LDS-only at 1-4 waves per SIMD (what the mix itself can reach)")
    p.add_argument("--out-dtype", default="f32", choices=["f32", "bf16"],
                   help="element type of o, dq, dk, dv (lse is always float32)")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="run one plain 256 MiB device-to-device copy before the steps, so a "
                        "rocprofv3 --pmc run records FETCH_SIZE/WRITE_SIZE for a known byte count")
    return p.parse_args()


# Kernel sources whose HBM traffic was counted; a changed source voids the record.
KERNEL_SOURCES = {
    "attn_fwd": ["attn_fwd_mfma.hip", "tca_device.h"],
    "attn_bwd_dq": ["attn_bwd_mfma.hip", "tca_device.h"],
    "attn_bwd_dkdv": ["attn_bwd_mfma.hip", "tca_device.h"],
}


def source_digest(kernel: str) -> str:
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "tiled_causal_attention_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def counted_traffic(kernel: str, workload: str, out_dtype: str = "f32"):
    """HBM bytes per launch from the committed PMC record, if it matches the current source
    (records of the float32-output runs are keyed by the workload alone)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    key = workload if out_dtype == "f32" else f"{workload}/{out_dtype}_out"
    ent = rec.get(key, {}).get(kernel)
    if not ent or ent.get("source_digest") != source_digest(kernel):
        return None
    return ent["hbm_bytes_per_launch"]


def host_cpu() -> dict:
    """The host CPU: model name, physical cores and logical CPUs of the machine, and
    the logical CPUs this process may run on."""
    model, cores, logical = None, set(), 0
    phys = core = None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                key, _, val = line.partition(":")
                key, val = key.strip(), val.strip()
                if key == "processor":
                    logical += 1
                elif key == "model name" and model is None:
                    model = val
                elif key == "physical id":
                    phys = val
                elif key == "core id":
                    core = val
                    cores.add((phys, core))
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = os.cpu_count()
    return {"cpu_model": model, "physical_cores": len(cores) or None, "logical_cpus": logical or os.cpu_count(),
            "usable_cpus": usable}


def cpu_baseline(s: workloads.Shape, inputs):
    """The float64 oracle, as it stands, on this host's cores."""
    import oracle
    q, k, v, do = inputs
    units = s.B * s.Hkv
    # bounded sample: whole (b, kv-head) units, as many as keep it to ~10-30 s of CPU work
    work_per_unit = s.flops_fwd() * 3.5 / units        # fwd + bwd flops of one unit
    max_units = max(1, int(30e9 * 8 / work_per_unit))  # ~1 GFLOP/s/thread, 8 threads' worth
    nb = max(1, min(s.B, max_units // s.Hkv)) if max_units >= s.Hkv else 1
    nh = s.Hkv if max_units >= s.Hkv else max(1, min(s.Hkv, max_units))
    g = s.group
    qs, dos = q[:nb, :nh * g], do[:nb, :nh * g]
    ks, vs = k[:nb, :nh], v[:nb, :nh]
    t0 = time.perf_counter()
    oracle.attn_fwd(qs, ks, vs, s.causal, s.scale)
    t1 = time.perf_counter()
    oracle.attn_bwd(qs, ks, vs, dos, s.causal, s.scale)
    t2 = time.perf_counter()
    frac = (nb * nh) / units
    flops = (s.flops_fwd() + s.flops_bwd()) * frac
    return {
        "value": flops / (t2 - t0) / 1e12,
        "unit": "TFLOP/s",
        "cores": min(oracle.threads(), nb * nh),   # OpenMP threads that had a (b, kv-head) unit to run
        "kind": "oracle",
        **host_cpu(),
        "sample": f"{nb} of {s.B} batch rows x {nh} of {s.Hkv} KV heads (all {g} query heads each) "
                  f"= {frac:.3f} of the workload; fwd {t1 - t0:.2f} s + bwd {t2 - t1:.2f} s, float64",
    }


def sampled_check(s, inputs, out):
    """Largest error on sampled outputs of one (b, kv-head) unit against the oracle."""
    import numpy as np
    import oracle
    q, k, v, do = inputs
    o, lse, dq, dk, dv = (t.cpu().double().numpy() for t in out)
    b, hkv = s.B - 1, s.Hkv - 1
    rows = [(g, i) for g in range(s.group) for i in (0, s.N // 3, s.N // 2, s.N - 1)]
    keys = [0, s.N // 4, s.N - 1]
    ref = oracle.attn_sampled(q, k, v, do, b, hkv, rows, keys, s.causal, s.scale)
    hq = [hkv * s.group + g for g, _ in rows]
    ii = [i for _, i in rows]
    err = {
        "o": np.abs(o[b, hq, ii] - ref["o"]).max(),
        "lse": np.abs(lse[b, hq, ii] - ref["lse"]).max(),
        "dq": np.abs(dq[b, hq, ii] - ref["dq"]).max(),
        "dk": np.abs(dk[b, hkv, keys] - ref["dk"]).max(),
        "dv": np.abs(dv[b, hkv, keys] - ref["dv"]).max(),
    }
    return {f"max_abs_{kk}": float(vv) for kk, vv in err.items()}


def shader_clocks():
    """rocm-smi's current clocks (a child process), or None where it is unavailable."""
    import subprocess
    try:
        r = subprocess.run(["rocm-smi", "--showclocks", "--json"], capture_output=True, text=True, timeout=60)
        card = next(iter(json.loads(r.stdout).values()))
        return {k: v for k, v in card.items() if "sclk" in k.lower() or "mclk" in k.lower()}
    except Exception as e:  # noqa: BLE001 -- the report goes on without clocks
        return {"error": str(e)[:200]}


def measured_mfma_peak():
    """Dense bf16 matrix-core TFLOP/s of a register-only MFMA loop on this GPU."""
    import ctypes
    from tiled_causal_attention_amd import build as tca_build
    L = ctypes.CDLL(tca_build.MEASURE_LIB)
    L.tca_mfma_peak_launch.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    L.tca_mfma_peak_launch.restype = ctypes.c_int
    L.tca_mfma_peak_flops.argtypes = [ctypes.c_int, ctypes.c_int]
    L.tca_mfma_peak_flops.restype = ctypes.c_double
    blocks, iters = 256 * 8, 4096
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def launch():
        rc = L.tca_mfma_peak_launch(ctypes.c_void_p(out.data_ptr()), blocks, iters, st)
        if rc != 0:
            raise RuntimeError(f"mfma peak launch failed: {rc}")

    for _ in range(3):
        launch()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        launch()
    e1.record()
    torch.cuda.synchronize()
    return L.tca_mfma_peak_flops(blocks, iters) / (e0.elapsed_time(e1) / 10 * 1e-3) / 1e12


MIX_NAMES = ["mfma_only", "exp_only", "fma_only", "cvt_only", "fwd", "fwd_reg", "fwd_staged", "dq", "dkdv",
             "fwd_w8", "fwd_pingpong", "fwd_2q"]
MIX_VALU_PER_BLOCK = {"exp_only": 16, "fma_only": 16, "cvt_only": 8}


def ceiling_report(args):
    """Per instruction mix and waves per SIMD: SIMD cycles per 32x32 block (each wave loops
    over one block per iteration, no global memory traffic), the matrix-core busy fraction
    that implies (32 cycles per 32x32x16 product), and the rate the mix would sustain at the
    measured shader clock, in its own products' TFLOP/s."""
    import ctypes

    import numpy as np
    from tiled_causal_attention_amd import build as tca_build
    L = ctypes.CDLL(tca_build.MEASURE_LIB)
    L.tca_mix_launch.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                 ctypes.c_void_p]
    L.tca_mix_launch.restype = ctypes.c_int
    L.tca_mix_mfma_per_block.argtypes = [ctypes.c_int]
    L.tca_mix_mfma_per_block.restype = ctypes.c_int
    L.tca_mix_max_blocks_per_cu.argtypes = [ctypes.c_int]
    L.tca_mix_max_blocks_per_cu.restype = ctypes.c_int
    L.tca_mix_waves_per_block.argtypes = [ctypes.c_int]
    L.tca_mix_waves_per_block.restype = ctypes.c_int
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    iters = 4096
    peak = measured_mfma_peak()
    for mid, name in enumerate(MIX_NAMES):
        fit = L.tca_mix_max_blocks_per_cu(mid)
        wpb = L.tca_mix_waves_per_block(mid)
        for w in (1, 2, 3, 4):
            if w * wpb // 4 > 4 or w > fit:
                continue
            blocks = n_cu * w
            out = torch.empty(blocks * 512, dtype=torch.float32, device="cuda")
            cyc = torch.zeros(blocks * 16, dtype=torch.int64, device="cuda")
            for _ in range(2):
                rc = L.tca_mix_launch(mid, ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(cyc.data_ptr()),
                                      blocks, iters, st)
                if rc != 0:
                    raise RuntimeError(f"mix {name} launch failed: {rc}")
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            L.tca_mix_launch(mid, ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(cyc.data_ptr()), blocks, iters, st)
            e1.record()
            torch.cuda.synchronize()
            wall_s = e0.elapsed_time(e1) * 1e-3
            c = cyc.cpu().numpy().astype(np.float64).reshape(blocks, 8, 2)[:, :wpb].reshape(-1, 2)
            wps = w * wpb // 4                                 # waves per SIMD
            ns_wave = float(np.median(c[:, 1])) * 10.0 / iters  # 100 MHz counter: ns per block, per wave
            ns_simd = ns_wave / wps                            # per SIMD (wps waves share it)
            tick_ghz = float(np.median(c[:, 0] / c[:, 1])) * 0.1   # s_memtime rate
            nm = L.tca_mix_mfma_per_block(mid)
            row = {"mix": name, "waves_per_simd": wps, "ns_per_block_per_simd": round(ns_simd, 2),
                   "memtime_ghz": round(tick_ghz, 3), "wall_us": round(wall_s * 1e6, 1), "mfma_per_block": nm}
            if nm > 0:
                # every SIMD of the chip at this rate (the steady state of one resident set)
                flops = 4 * n_cu * nm * 32768.0 / (ns_simd * 1e-9)
                row["tflops"] = round(flops / 1e12, 1)
                row["pct_of_2500"] = round(100 * flops / 1e12 / PEAK_MFMA_BF16_TFLOPS, 1)
            if name in MIX_VALU_PER_BLOCK:
                row["ns_per_instruction_per_simd"] = round(ns_simd / MIX_VALU_PER_BLOCK[name], 3)
            row["measured_mfma_peak_tflops"] = round(peak, 1)
            print(json.dumps(row), flush=True)


def all_configs(args):
    import numpy as np
    out_dt = OUT_DTYPES[args.out_dtype]
    report = {"report": "per-workload fwd/bwd timing", "out_dtype": args.out_dtype,
              "clocks_before": shader_clocks()}
    peak = measured_mfma_peak()
    report["measured_mfma_bf16_tflops"] = peak
    print(json.dumps(report), flush=True)
    for name, s in workloads.CONFIGS.items():
        inputs = workloads.make_inputs(s)
        q, k, v, do = (t.cuda() for t in inputs)
        o = torch.empty((s.B, s.Hq, s.N, s.d), dtype=out_dt, device=q.device)
        lse = torch.empty((s.B, s.Hq, s.N), dtype=torch.float32, device=q.device)
        dq, dk, dv = (torch.empty(t.shape, dtype=out_dt, device=q.device) for t in (q, k, v))
        ws = tca.bwd_workspace(q, k)
        causal, scale = bool(s.causal), s.scale
        reps = 20 if s.N >= 8192 else 100

        def one(ev):
            ev[0].record()
            tca.attn_fwd(q, k, v, causal, scale, out=(o, lse))
            ev[1].record()
            tca.attn_bwd_dq(q, k, v, o, lse, do, dq, dk, dv, ws, causal, scale)
            tca.attn_bwd_dkdv(q, k, v, o, lse, do, dq, dk, dv, ws, causal, scale)
            ev[2].record()

        for _ in range(10):
            one([torch.cuda.Event(enable_timing=True) for _ in range(3)])
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(reps)]
        torch.cuda.synchronize()
        for ev in evs:
            one(ev)
        torch.cuda.synchronize()
        fwd = np.array([e[0].elapsed_time(e[1]) for e in evs])
        bwd = np.array([e[1].elapsed_time(e[2]) for e in evs])
        tot = fwd + bwd
        stats = lambda a: {"median_ms": float(np.median(a)), "p10_ms": float(np.percentile(a, 10)),
                           "p90_ms": float(np.percentile(a, 90))}
        ff, fb = s.flops_fwd(), s.flops_bwd()
        rec = {"workload": name, "B": s.B, "Hq": s.Hq, "Hkv": s.Hkv, "N": s.N, "d": s.d, "dtype": s.dtype,
               "out_dtype": args.out_dtype, "reps": reps, "fwd": stats(fwd), "bwd": stats(bwd), "fwd_bwd": stats(tot)}
        for key, fl, arr in (("fwd", ff, fwd), ("bwd", fb, bwd), ("fwd_bwd", ff + fb, tot)):
            tf = fl / (float(np.median(arr)) * 1e-3) / 1e12
            rec[key].update({"tflops": tf, "pct_published_peak": 100 * tf / PEAK_MFMA_BF16_TFLOPS,
                             "pct_measured_peak": 100 * tf / peak})
        if args.oracle:
            import oracle
            runs = 1 if s.N >= 8192 else 3
            tf_, tb_ = [], []
            for i in range(runs):
                print(f"oracle {name} run {i + 1}/{runs}", file=sys.stderr, flush=True)
                t0 = time.perf_counter()
                oracle.attn_fwd(*inputs[:3], s.causal, s.scale)
                t1 = time.perf_counter()
                oracle.attn_bwd(*inputs, s.causal, s.scale)
                t2 = time.perf_counter()
                tf_.append(t1 - t0)
                tb_.append(t2 - t1)
            rec["oracle"] = {"fwd_s": float(np.median(tf_)), "bwd_s": float(np.median(tb_)), "runs": runs,
                             "threads": oracle.threads(),
                             "gflops": (ff + fb) / (float(np.median(tf_)) + float(np.median(tb_))) / 1e9}
        print(json.dumps(rec), flush=True)
        del q, k, v, do, o, lse, dq, dk, dv, ws
        torch.cuda.empty_cache()
    print(json.dumps({"clocks_after": shader_clocks()}), flush=True)


def naive_report(args):
    """Forward of one workload (default the headline), the tiled kernel against the
    unoptimised materialised-score path (S = QK^T in HBM, softmax, PV), both timed by
    HIP events on the launch stream, median of 50 calls after 5 warm-up calls."""
    import numpy as np
    s = workloads.CONFIGS[args.workload]
    q, k, v, _ = (t.cuda() for t in workloads.make_inputs(s))
    o = torch.empty((s.B, s.Hq, s.N, s.d), device=q.device)
    lse = torch.empty((s.B, s.Hq, s.N), device=q.device)
    ws = torch.empty(int(tca.lib().attn_fwd_naive_workspace_bytes(s.B, s.Hq, s.N)), dtype=torch.uint8,
                     device=q.device)
    causal, scale = bool(s.causal), s.scale
    calls = {"tiled": lambda: tca.attn_fwd(q, k, v, causal, scale, out=(o, lse)),
             "naive": lambda: tca.attn_fwd_naive(q, k, v, causal, scale, out=(o, lse), workspace=ws)}
    med = {}
    for name, fn in calls.items():
        for _ in range(5):
            fn()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(50)]
        torch.cuda.synchronize()
        for e0, e1 in evs:
            e0.record()
            fn()
            e1.record()
        torch.cuda.synchronize()
        med[name] = float(np.median([e0.elapsed_time(e1) for e0, e1 in evs]))
    ff = s.flops_fwd()
    print(json.dumps({"workload": s.name, "B": s.B, "Hq": s.Hq, "Hkv": s.Hkv, "N": s.N, "d": s.d,
                      "tiled_fwd_ms": med["tiled"], "naive_fwd_ms": med["naive"],
                      "tiled_tflops": ff / (med["tiled"] * 1e-3) / 1e12,
                      "naive_tflops": ff / (med["naive"] * 1e-3) / 1e12,
                      "speedup": med["naive"] / med["tiled"], "score_matrix_bytes": ws.numel()}), flush=True)


def rope_report(args):
    """fwd+bwd of one workload (default the headline) with rotary q/k read from views of
    one fused [B, N, Hq + 2 Hkv, d] projection buffer and gradients written back into
    one such buffer, against the plain path on contiguous tensors; HIP events on the
    launch stream around each fwd+bwd, median over three interleaved rounds of 50 steps
    (10 warm-up steps before each). The rotary step keeps the forward's rotated keys
    (k_rot) for the backward, as a training step does; the variant in which each call
    rotates k itself is reported beside it."""
    import numpy as np
    s = workloads.CONFIGS[args.workload]
    q, k, v, do = (t.cuda() for t in workloads.make_inputs(s))
    cos, sin = (t.cuda() for t in workloads.rope_tables(s.N, s.d))
    buf = torch.empty((s.B, s.N, s.Hq + 2 * s.Hkv, s.d), dtype=q.dtype, device=q.device)
    gbuf = torch.empty((s.B, s.N, s.Hq + 2 * s.Hkv, s.d), device=q.device)
    views = lambda b: (b[:, :, :s.Hq].permute(0, 2, 1, 3), b[:, :, s.Hq:s.Hq + s.Hkv].permute(0, 2, 1, 3),
                       b[:, :, s.Hq + s.Hkv:].permute(0, 2, 1, 3))
    qv, kv, vv = views(buf)
    qv.copy_(q), kv.copy_(k), vv.copy_(v)
    gq, gk, gv = views(gbuf)
    o = torch.empty((s.B, s.Hq, s.N, s.d), device=q.device)
    lse = torch.empty((s.B, s.Hq, s.N), device=q.device)
    dq, dk, dv = (torch.empty(t.shape, device=q.device) for t in (q, k, v))
    L = tca.lib()
    wsf = torch.empty(int(L.attn_fwd_rope_workspace_bytes(tca.ATTN_BF16, tca.ATTN_F32, s.B, s.Hq, s.Hkv, s.N, s.d)),
                      dtype=torch.uint8, device=q.device)
    wsb = torch.empty(int(L.attn_bwd_rope_workspace_bytes(tca.ATTN_BF16, tca.ATTN_F32, s.B, s.Hq, s.Hkv, s.N, s.d)),
                      dtype=torch.uint8, device=q.device)
    ws = tca.bwd_workspace(q, k)
    causal, scale = bool(s.causal), s.scale

    kr = torch.empty((s.B, s.Hkv, s.N, s.d), dtype=q.dtype, device=q.device)

    def rope_step():   # training pattern: the forward's rotated keys kept for the backward
        tca.attn_fwd_rope(qv, kv, vv, cos, sin, causal, scale, out=(o, lse), workspace=wsf, k_rot=kr)
        tca.attn_bwd_rope(qv, kv, vv, o, lse, do, cos, sin, causal, scale, out=(gq, gk, gv), workspace=wsb,
                          k_rot=kr)

    def rope_rotate_twice_step():   # each call rotates k itself
        tca.attn_fwd_rope(qv, kv, vv, cos, sin, causal, scale, out=(o, lse), workspace=wsf)
        tca.attn_bwd_rope(qv, kv, vv, o, lse, do, cos, sin, causal, scale, out=(gq, gk, gv), workspace=wsb)

    def plain_step():
        tca.attn_fwd(q, k, v, causal, scale, out=(o, lse))
        tca.attn_bwd(q, k, v, o, lse, do, causal, scale, out=(dq, dk, dv), workspace=ws)

    # three rounds, the variants interleaved within each, 50 timed steps per variant and round
    times = {"plain": [], "rope_fused_qkv": [], "rope_rotate_k_twice": []}
    steps = (("plain", plain_step), ("rope_fused_qkv", rope_step), ("rope_rotate_k_twice", rope_rotate_twice_step))
    for _ in range(3):
        for name, fn in steps:
            for _ in range(10):
                fn()
            evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(50)]
            torch.cuda.synchronize()
            for e0, e1 in evs:
                e0.record()
                fn()
                e1.record()
            torch.cuda.synchronize()
            times[name] += [e0.elapsed_time(e1) for e0, e1 in evs]
    med = {name: float(np.median(t)) for name, t in times.items()}
    # the host's own time per step (argument checks and launches, no waiting), and each
    # step captured in a HIP graph and replayed (events around every replay), which
    # removes the host's share: labelled figures beside the eager ones
    host, graph = {}, {}
    for name, fn in steps:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(20):
            fn()
        host[name] = (time.perf_counter() - t0) / 20 * 1e6
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side):
                fn()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        for _ in range(10):
            g.replay()
        reps = []
        for _ in range(3):
            evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(50)]
            torch.cuda.synchronize()
            for e0, e1 in evs:
                e0.record()
                g.replay()
                e1.record()
            torch.cuda.synchronize()
            reps += [e0.elapsed_time(e1) for e0, e1 in evs]
        graph[name] = float(np.median(reps))
    fl = s.flops_fwd() + s.flops_bwd()
    print(json.dumps({"workload": s.name, "plain_fwd_bwd_ms": med["plain"], "rope_fwd_bwd_ms": med["rope_fused_qkv"],
                      "plain_tflops": fl / (med["plain"] * 1e-3) / 1e12,
                      "rope_tflops": fl / (med["rope_fused_qkv"] * 1e-3) / 1e12,
                      "rope_overhead": med["rope_fused_qkv"] / med["plain"] - 1.0,
                      "rope_rotate_k_twice_ms": med["rope_rotate_k_twice"],
                      "rope_rotate_k_twice_overhead": med["rope_rotate_k_twice"] / med["plain"] - 1.0,
                      "host_us_per_step": host, "graph_replay_ms": graph,
                      "graph_replay_rope_overhead": graph["rope_fused_qkv"] / graph["plain"] - 1.0}), flush=True)


def decode_report(args):
    """Few-query attention over a K/V cache: HBM-bound, so reported as GB/s of the
    minimum traffic (K and V once, Q, O, LSE) against the 8 TB/s HBM peak. Each
    repetition (both kernels of a call: key splits, then their merge) is bracketed
    by HIP events on the launch stream; median over the repetitions."""
    import numpy as np
    import oracle
    out_dt = OUT_DTYPES[args.out_dtype]
    if args.calibrate_copy:   # a plain 256 MiB device copy, the reference for --pmc byte counters
        src = torch.ones(64 << 20, dtype=torch.float32, device="cuda")
        torch.empty_like(src).copy_(src)
        torch.cuda.synchronize()
        del src
    for name, s in workloads.DECODE_CONFIGS.items():
        inputs = workloads.make_decode_inputs(s)
        q, k, v = (t.cuda() for t in inputs)
        o = torch.empty((s.B, s.Hq, s.Nq, s.d), dtype=out_dt, device=q.device)
        lse = torch.empty((s.B, s.Hq, s.Nq), dtype=torch.float32, device=q.device)
        nws = int(tca.lib().attn_decode_workspace_bytes(tca.ATTN_BF16 if s.dtype == "bf16" else tca.ATTN_F32,
                                                        s.B, s.Hq, s.Hkv, s.Nq, s.Nk, s.d))
        ws = tca.decode_workspace(nws, q.device)
        causal, scale = bool(s.causal), s.scale
        for _ in range(20):
            tca.attn_decode(q, k, v, causal, scale, out=(o, lse), workspace=ws)
        reps = 200
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        torch.cuda.synchronize()
        for e0, e1 in evs:
            e0.record()
            tca.attn_decode(q, k, v, causal, scale, out=(o, lse), workspace=ws)
            e1.record()
        torch.cuda.synchronize()
        t = np.array([e0.elapsed_time(e1) for e0, e1 in evs])
        med = float(np.median(t))
        nbytes = s.min_bytes(2 if args.out_dtype == "bf16" else 4)
        # second, labelled number: 20 calls captured in a HIP graph and replayed, so that no
        # host work sits between the launches; every replay's output is checked against
        # the eager result (bitwise: same kernels, same inputs)
        graph_us = None
        try:
            o_ref, l_ref = o.clone(), lse.clone()
            g = torch.cuda.CUDAGraph()
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                with torch.cuda.graph(g, stream=side):
                    for _ in range(20):
                        tca.attn_decode(q, k, v, causal, scale, out=(o, lse), workspace=ws)
            torch.cuda.current_stream().wait_stream(side)
            torch.cuda.synchronize()
            gt = []
            for _ in range(10):
                o.zero_()
                g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                g0.record()
                g.replay()
                g1.record()
                torch.cuda.synchronize()
                if not (torch.equal(o, o_ref) and torch.equal(lse, l_ref)):
                    raise RuntimeError("graph replay differs from the eager result")
                gt.append(g0.elapsed_time(g1) / 20)
            graph_us = float(np.median(gt)) * 1e3
            del g
        except Exception as e:  # noqa: BLE001 -- reported, the eager number stands
            print(f"graph replay not measured: {e}", file=sys.stderr)
        ro, rl = oracle.attn_decode(*inputs, s.causal, s.scale)
        t0 = time.perf_counter()
        oracle.attn_decode(*inputs, s.causal, s.scale)
        t_or = time.perf_counter() - t0
        rec = {"workload": name, "B": s.B, "Hq": s.Hq, "Hkv": s.Hkv, "Nq": s.Nq, "Nk": s.Nk, "d": s.d,
               "dtype": s.dtype, "out_dtype": args.out_dtype, "causal": s.causal, "reps": reps,
               "median_ms": med, "p10_ms": float(np.percentile(t, 10)), "p90_ms": float(np.percentile(t, 90)),
               "min_hbm_bytes": nbytes, "gb_per_s": nbytes / (med * 1e-3) / 1e9,
               "frac_hbm_peak": nbytes / (med * 1e-3) / 8e12,
               "graph_replay_us_per_call": graph_us,
               "graph_replay_gb_per_s": (nbytes / (graph_us * 1e-6) / 1e9) if graph_us else None,
               "max_abs_o": float(np.abs(o.float().cpu().double().numpy() - ro).max()),
               "max_abs_lse": float(np.abs(lse.cpu().double().numpy() - rl).max()),
               "oracle": {"seconds": t_or, "threads": oracle.threads(),
                          "gb_per_s": nbytes / t_or / 1e9}}
        print(json.dumps(rec), flush=True)
        del q, k, v, o, lse, ws
        torch.cuda.empty_cache()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this attention path runs on a single MI355X "
              "(sharding over batch and KV-head groups needs no communication and is not "
              "built here). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    tca.lib()  # fail loudly if the HIP library is missing
    if args.all_configs:
        all_configs(args)
        return
    if args.decode:
        decode_report(args)
        return
    if args.ceiling:
        ceiling_report(args)
        return
    if args.naive:
        naive_report(args)
        return
    if args.rope:
        rope_report(args)
        return

    s = workloads.CONFIGS[args.workload]
    inputs = workloads.make_inputs(s)
    q, k, v, do = (t.cuda() for t in inputs)
    dev = q.device
    out_dt = OUT_DTYPES[args.out_dtype]
    o = torch.empty((s.B, s.Hq, s.N, s.d), dtype=out_dt, device=dev)
    lse = torch.empty((s.B, s.Hq, s.N), dtype=torch.float32, device=dev)
    dq = torch.empty(q.shape, dtype=out_dt, device=dev)
    dk = torch.empty(k.shape, dtype=out_dt, device=dev)
    dv = torch.empty(v.shape, dtype=out_dt, device=dev)
    ws = tca.bwd_workspace(q, k)
    causal, scale = bool(s.causal), s.scale
    if args.calibrate_copy:
        src = torch.empty(64 << 20, dtype=torch.float32, device=dev)   # 256 MiB
        dst = torch.empty_like(src)
        src.fill_(1.0)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    names = ("attn_fwd", "attn_bwd_dq", "attn_bwd_dkdv")
    calls = {
        "attn_fwd": lambda: tca.attn_fwd(q, k, v, causal, scale, out=(o, lse)),
        "attn_bwd_dq": lambda: tca.attn_bwd_dq(q, k, v, o, lse, do, dq, dk, dv, ws, causal, scale),
        "attn_bwd_dkdv": lambda: tca.attn_bwd_dkdv(q, k, v, o, lse, do, dq, dk, dv, ws, causal, scale),
    }

    def step(ev=None, which=names):
        # ev: a pair of events recorded around each kernel named in `which`
        for n in names:
            timed = ev is not None and n in which
            if timed:
                ev[n][0].record()
            calls[n]()
            if timed:
                ev[n][1].record()

    def new_events(which):
        return {n: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for n in which}

    def mean_ms(evs, n):
        return sum(e[n][0].elapsed_time(e[n][1]) for e in evs) / len(evs)

    for _ in range(args.warmup):
        step()
    # untimed calibration pass: every kernel bracketed by events, to find the
    # dominant kernel and report the mean duration of the other two
    cal = [new_events(names) for _ in range(min(args.steps, 50))]
    torch.cuda.synchronize()
    for ev in cal:
        step(ev)
    torch.cuda.synchronize()
    kernels = {n: mean_ms(cal, n) for n in names}
    dom = max(kernels, key=kernels.get)
    # timed region: K steps, events only around the dominant kernel (each event
    # record between kernels costs step time a user does not pay)
    events = [new_events((dom,)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i], (dom,))
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    kernels[dom] = mean_ms(events, dom)

    flops_fwd, flops_bwd = s.flops_fwd(), s.flops_bwd()
    tflops = (flops_fwd + flops_bwd) / (ms_per_step * 1e-3) / 1e12
    t_fwd, t_dq, t_kv = kernels["attn_fwd"], kernels["attn_bwd_dq"], kernels["attn_bwd_dkdv"]
    kernel_flops = {"attn_fwd": flops_fwd, "attn_bwd_dq": 1.5 * flops_fwd, "attn_bwd_dkdv": 2.0 * flops_fwd}
    achieved = kernel_flops[dom] / (kernels[dom] * 1e-3) / 1e12
    roof = {"bound": "mfma", "achieved": achieved, "peak": PEAK_MFMA_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": achieved / PEAK_MFMA_BF16_TFLOPS, "traffic": counted_traffic(dom, s.name, args.out_dtype),
            "kernel": dom, "flops_per_launch": kernel_flops[dom]}

    result = {
        "metric": METRIC if s.name == workloads.HEADLINE else metric_for(s),
        "value": tflops,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if s.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": f"{s.name}: causal GQA attention fwd+bwd, B={s.B} Hq={s.Hq} "
                               f"Hkv={s.Hkv} N={s.N} d={s.d} {s.dtype} in, {args.out_dtype} out",
                   "global_batch": s.B, "seq_len": s.N, "parallelism": "single-gpu"},
        "pct_peak": 100.0 * tflops / PEAK_MFMA_BF16_TFLOPS,
        "fwd_tflops": flops_fwd / (t_fwd * 1e-3) / 1e12,
        "bwd_tflops": flops_bwd / ((t_dq + t_kv) * 1e-3) / 1e12,
        "kernel_ms": kernels,
        "kernel_ms_note": f"{dom}: HIP events in the timed region; the others: an untimed pass of {len(cal)} "
                          "steps with events around every kernel",
        "roofline": roof,
    }
    if not args.no_check:
        result["check"] = sampled_check(s, inputs, (o, lse, dq, dk, dv))
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(s, inputs)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
