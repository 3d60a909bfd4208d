#!/usr/bin/env python3
"""Throughput of the stabilised BF16 attention hot path on one MI355X.

A step is one pass of the whole path over the GPT-2-small attention layer
(B=8, H=12, N=1024, D=64, causal, bf16, synthetic seeded inputs with
duplicate-max rows): attn_fwd (duplicate-max shift on, with the rule's
outputs: per-row duplicate count and the P_bar == 1 flag) followed by attn_bwd
(attn_bwd_dq then attn_bwd_dkdv).  The optional per-row count of formed bf16
ones is a diagnostic; its cost is reported beside the step.  Inputs are
resident in HBM before the timed region.  The reported value is algorithmic
fwd+bwd TFLOPS (4 D + 10 D flops per visible query-key pair).

Printed: ONE JSON line with the metric, per-kernel HIP-event timings, the
roofline of the dominant kernel, a cold-cache variant, the other workload
shapes, and the FP64 oracle timed on the host (the cpu_baseline leg, which also
yields the signed-bias diagnostic against FP64).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "causal attn fwd+bwd TFLOPS (bf16) at GPT-2 shape; % of MFMA peak; O/dP signed bias"
PEAK_BF16_TFLOPS = 2516.6      # 256 CU x 4096 flop/clk/CU x 2.4 GHz, dense bf16 MFMA
PEAK_HBM_GBS = 8000.0
KERNEL_SOURCE_DIR = os.path.join(ROOT, "numerics_safe_softmax_amd", "csrc")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_gpt2_small.md")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    # the GPU needs tens of milliseconds of load to reach its working clock:
    # 300 warm-up steps (~35 ms) before 500 timed ones (~55 ms)
    p.add_argument("--steps", type=int, default=500)
    p.add_argument("--warmup", type=int, default=300)
    p.add_argument("--workload", default="gpt2_small")
    p.add_argument("--mode", type=int, default=1, choices=(1, 2),
                   help="stabilised forward: 1 = online shift, 2 = exact final shift (two passes)")
    p.add_argument("--no-cpu-baseline", action="store_true",
                   help="skip the host oracle leg (profiling runs)")
    p.add_argument("--no-other-workloads", action="store_true",
                   help="skip the timings of the other workload shapes and the cold-cache variant")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a plain 1 GiB device copy (reference for the HBM byte counters)")
    return p.parse_args()


def copy_calibration():
    """One plain device-to-device copy of 1 GiB: reads 2^30 bytes, writes 2^30
    bytes.  Profiled with the same FETCH_SIZE / WRITE_SIZE counters as the
    attention kernels, it gives the factor from counter units to bytes."""
    import torch
    n = (1 << 30) // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda:0")
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n * 4, "copy_bytes_written": n * 4}), flush=True)


def settle_clock(dev, seconds: float = 0.1) -> dict:
    """Untimed GPU load before the warm-up steps: an idle MI355X needs tens
    of milliseconds of load to reach its working clock (a loop of this step
    from idle ran its first ~20 ms about 10 % slow), longer than a few warm-up
    steps of ~0.1 ms take.  The load is bf16 GEMMs of unrelated data (torch),
    not steps of the workload: nothing they compute reaches the timed steps."""
    import torch
    a = torch.randn(4096, 4096, device=dev, dtype=torch.bfloat16)
    a = (a @ a) * (1.0 / 64.0)  # the GEMM library's own set-up, outside the settle time
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    n = 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(4):
            a = (a @ a) * (1.0 / 64.0)
        torch.cuda.synchronize()
        n += 4
    return {"seconds": round(time.perf_counter() - t0, 3), "gemms": n,
            "what": "untimed bf16 4096^3 GEMMs of unrelated data before the warm-up steps"}


def kernel_hash() -> str:
    """sha256 (first 16 hex digits) over the files of the kernel source
    directory in name order, each as its file name followed by its bytes: the
    kernels, the launchers and the schedule helpers."""
    h = hashlib.sha256()
    for name in sorted(os.listdir(KERNEL_SOURCE_DIR)):
        h.update(name.encode())
        h.update(open(os.path.join(KERNEL_SOURCE_DIR, name), "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary, or None when it is missing or the kernel source changed since."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    text = open(TRAFFIC_FILE).read()
    m = re.search(r"csrc_sha256_16:\s*([0-9a-f]+)", text)
    if not m or m.group(1) != kernel_hash():
        return None
    m = re.search(r"^%s_bytes_per_launch:\s*([0-9.eE+]+)" % re.escape(kernel), text, re.M)
    return float(m.group(1)) if m else None


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (attention heads "
              "would shard across GPUs with no exchange, each GPU running these kernels on its "
              "share). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import numerics_safe_softmax_amd as nss
    from numerics_safe_softmax_amd import inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    w = inputs.WORKLOADS[args.workload]
    B, H, N, D = w.B, w.H, w.N, w.D
    d = inputs.generate(w)
    t = {k: inputs.to_torch(v, dev) for k, v in d.items()}
    q, k, v, g = t["q"], t["k"], t["v"], t["dO"]
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    ties, pone, formed = (torch.empty((B, H, N), dtype=torch.int32, device=dev) for _ in range(3))
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    delta = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    kw = dict(scale=w.scale, causal=w.causal)

    def fwd(stabilise=args.mode, count_formed=False):
        nss.attn_fwd(q, k, v, o, lse, ties, pone, formed if count_formed else None, stabilise=stabilise,
                     beta=w.beta, stream=stream, **kw)

    def bwd_dq():
        nss.attn_bwd_dq(q, k, v, o, g, lse, dq, delta, stream=stream, **kw)

    def bwd_dkdv():
        nss.attn_bwd_dkdv(q, k, v, g, lse, delta, dk, dv, stream=stream, **kw)

    def step():
        fwd()
        bwd_dq()
        bwd_dkdv()

    settled = settle_clock(dev)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # whole-step wall clock over exactly K steps
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps

    # per-kernel average launch duration: K back-to-back launches of one kernel
    # between two HIP events on the launch stream (an event between every
    # launch would add its own overhead to each)
    us = {}
    for name, fn in (("fwd", fwd), ("bwd_dq", bwd_dq), ("bwd_dkdv", bwd_dkdv)):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        us[name] = e0.elapsed_time(e1) * 1e3 / args.steps

    # every forward mode, for comparison (plain, online shift, exact final shift)
    fwd_modes_us = {}
    for name, mode, cf in (("plain", 0, False), ("online_shift", 1, False), ("exact_shift", 2, False),
                           ("online_shift_with_formed_ones_count", 1, True)):
        for _ in range(3):
            fwd(stabilise=mode, count_formed=cf)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            fwd(stabilise=mode, count_formed=cf)
        e1.record(stream)
        torch.cuda.synchronize()
        fwd_modes_us[name] = e0.elapsed_time(e1) * 1e3 / args.steps

    fwd_flops, bwd_flops = w.fwd_flops(), w.bwd_flops()
    pairs = w.visible_pairs()
    tflops = (fwd_flops + bwd_flops) / (ms_per_step * 1e-3) / 1e12

    # algorithmic work of each kernel per launch (flops, compulsory HBM bytes)
    tb = B * H * N * D * 2
    rb = B * H * N * 4
    kinfo = {
        # S = QK^T and P_bar V: 4 D flops per visible pair; reads Q, K, V, writes O, LSE, 2 int rows
        "fwd": (4.0 * D * pairs, 4 * tb + 3 * rb),
        # dQ = scale dS K: 2 D per pair (its S / dP recompute is overhead of the split);
        # reads Q, K, V, O, dO, LSE, writes dQ, delta
        "bwd_dq": (2.0 * D * pairs, 6 * tb + 2 * rb),
        # S recompute, dP, dV, dK: 8 D per pair; reads Q, K, V, dO, LSE, delta, writes dK, dV
        "bwd_dkdv": (8.0 * D * pairs, 6 * tb + 2 * rb),
    }
    dom = max(us, key=lambda x: us[x])
    flops_dom, bytes_dom = kinfo[dom]
    achieved = flops_dom / (us[dom] * 1e-6) / 1e12
    traffic = measured_traffic(dom)
    roofline = {"kernel": dom, "bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS, "traffic": traffic,
                "algorithmic_bytes": bytes_dom, "avg_launch_us": us[dom]}

    # every kernel against both ceilings: its algorithmic flops against the
    # bf16 MFMA peak and its compulsory bytes against the 8 TB/s HBM peak
    per_kernel = {}
    for name, (fl, by) in kinfo.items():
        t_s = us[name] * 1e-6
        per_kernel[name] = {"avg_launch_us": us[name], "tflops": fl / t_s / 1e12,
                            "frac_mfma": fl / t_s / 1e12 / PEAK_BF16_TFLOPS,
                            "algorithmic_GBps": by / t_s / 1e9, "frac_hbm": by / t_s / 1e9 / PEAK_HBM_GBS,
                            "traffic": measured_traffic(name)}

    out = {
        "metric": METRIC,
        "value": tflops,
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": B, "H": H, "N": N, "D": D, "causal": w.causal,
                   "stabilise": {1: "online shift", 2: "exact final shift"}[args.mode], "beta": w.beta,
                   "global_batch": B, "seq_len": N,
                   "parallelism": "none (1 GPU)"},
        "pct_of_bf16_peak": 100.0 * tflops / PEAK_BF16_TFLOPS,
        "clock_settle": settled,
        "peak_assumption": "2516.6 TFLOPS dense bf16 = 256 CU x 4096 flop/clk x 2.4 GHz",
        "kernels_us": us,
        "fwd_us": us["fwd"],
        "bwd_us": us["bwd_dq"] + us["bwd_dkdv"],
        "fwd_tflops": fwd_flops / (us["fwd"] * 1e-6) / 1e12,
        "bwd_tflops": bwd_flops / ((us["bwd_dq"] + us["bwd_dkdv"]) * 1e-6) / 1e12,
        "fwd_modes_us": fwd_modes_us,
        "roofline": roofline,
        "kernels_roofline": per_kernel,
        "cpu_baseline": None,
    }

    if not args.no_other_workloads:
        out["cold_cache"] = cold_cache(t, w, nss, stream, args)
        out["other_workloads"] = other_workloads(w.name, nss, stream, args.mode)
    if not args.no_cpu_baseline:
        out["cpu_baseline"], out["bias"] = cpu_leg(w, d, nss, t, stream)
        out["cpu_baseline"]["gpu_over_cpu"] = tflops / out["cpu_baseline"]["value"]
    print(json.dumps(out), flush=True)


def time_path(t, w, nss, stream, mode, reps, sets=None):
    """Mean microseconds per step (attn_fwd, attn_bwd_dq, attn_bwd_dkdv; two HIP
    events around `reps` steps) and per kernel (`reps` back-to-back launches of
    one kernel between two events), rotating over the input sets given
    (default: one)."""
    import torch
    sets = sets or [t]
    B, H, N, D = w.B, w.H, w.N, w.D
    dev = t["q"].device
    bufs = []
    for x in sets:
        bufs.append({"o": torch.empty_like(x["q"]), "lse": torch.empty((B, H, N), dtype=torch.float32, device=dev),
                     "ties": torch.empty((B, H, N), dtype=torch.int32, device=dev),
                     "pone": torch.empty((B, H, N), dtype=torch.int32, device=dev),
                     "dq": torch.empty_like(x["q"]), "dk": torch.empty_like(x["q"]), "dv": torch.empty_like(x["q"]),
                     "delta": torch.empty((B, H, N), dtype=torch.float32, device=dev)})
    kw = dict(scale=w.scale, causal=w.causal, stream=stream)

    def fwd(i):
        x, b = sets[i % len(sets)], bufs[i % len(sets)]
        nss.attn_fwd(x["q"], x["k"], x["v"], b["o"], b["lse"], b["ties"], b["pone"], None, stabilise=mode,
                     beta=w.beta, **kw)

    def bwd_dq(i):
        x, b = sets[i % len(sets)], bufs[i % len(sets)]
        nss.attn_bwd_dq(x["q"], x["k"], x["v"], b["o"], x["dO"], b["lse"], b["dq"], b["delta"], **kw)

    def bwd_dkdv(i):
        x, b = sets[i % len(sets)], bufs[i % len(sets)]
        nss.attn_bwd_dkdv(x["q"], x["k"], x["v"], x["dO"], b["lse"], b["delta"], b["dk"], b["dv"], **kw)

    def step(i):
        fwd(i)
        bwd_dq(i)
        bwd_dkdv(i)

    def timed(fn):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(reps):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps

    for i in range(3 * len(sets)):
        step(i)
    torch.cuda.synchronize()
    # an idle GPU needs tens of milliseconds of load to reach its working
    # clock: warm up for about 50 ms, and time at least about 25 ms per figure
    t0 = time.perf_counter()
    i = 0
    while time.perf_counter() - t0 < 0.05:
        step(i)
        i += 1
        if i % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    per_step = (time.perf_counter() - t0) / i
    reps = max(reps, int(0.025 / per_step) + 1)
    step_us = timed(step)
    us = {"fwd": timed(fwd), "bwd_dq": timed(bwd_dq), "bwd_dkdv": timed(bwd_dkdv)}
    fwd_us, bwd_us = us["fwd"], us["bwd_dq"] + us["bwd_dkdv"]
    return {"step_us": step_us, "kernels_us": us, "fwd_us": fwd_us, "bwd_us": bwd_us,
            "fwd_tflops": w.fwd_flops() / (fwd_us * 1e-6) / 1e12,
            "bwd_tflops": w.bwd_flops() / (bwd_us * 1e-6) / 1e12,
            "fwd_bwd_tflops": (w.fwd_flops() + w.bwd_flops()) / (step_us * 1e-6) / 1e12}


def cold_cache(t, w, nss, stream, args):
    """The headline step rotating over 6 copies of the inputs (and outputs):
    about 6 x 100 MB, more than the 256 MB last-level cache holds, so each
    step starts with its operands in HBM only."""
    sets = [{k2: x.clone() for k2, x in t.items()} for _ in range(6)]
    r = time_path(t, w, nss, stream, args.mode, max(12, args.steps // 2), sets=sets)
    r["input_sets"] = len(sets)
    return r


def other_workloads(skip, nss, stream, mode):
    """fwd / bwd timings of the other synthetic workload shapes (parity-test
    configurations; reported beside the headline, not part of its value)."""
    import torch
    from numerics_safe_softmax_amd import inputs
    res = {}
    for name in ("gpt2_medium", "long_context", "sink"):
        if name == skip:
            continue
        w = inputs.WORKLOADS[name]
        d = inputs.generate(w)
        t = {k2: inputs.to_torch(x, torch.device("cuda:0")) for k2, x in d.items()}
        r = time_path(t, w, nss, stream, mode, 10 if name == "long_context" else 20)
        r["shape"] = "B%d H%d N%d D%d %s" % (w.B, w.H, w.N, w.D, "causal" if w.causal else "non-causal")
        r["pct_of_bf16_peak"] = 100.0 * r["fwd_bwd_tflops"] / PEAK_BF16_TFLOPS
        res[name] = r
        del t
    return res


def cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo), or "unknown"."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_leg(w, d, nss, t, stream):
    """The FP64 oracle on the host, on the whole workload (fwd + bwd), timed;
    its result also gives the signed-bias diagnostic of both GPU modes."""
    import numpy as np
    import torch

    import oracle
    from oracle import bias

    t0 = time.perf_counter()
    ref = oracle.forward(d["q"], d["k"], d["v"], scale=w.scale, causal=w.causal, stabilise=True,
                         beta=w.beta, want=["O", "tol_O", "lse", "tol_lse", "ties"])
    t1 = time.perf_counter()
    rb = oracle.backward(d["q"], d["k"], d["v"], d["dO"], ref, scale=w.scale, causal=w.causal)
    t2 = time.perf_counter()
    cores = oracle.threads()
    flops = w.fwd_flops() + w.bwd_flops()
    cpu = {"value": flops / (t2 - t0) / 1e12, "unit": "TFLOPS", "cores": cores, "kind": "oracle",
           "sample": "the whole %s workload (B=%d H=%d N=%d D=%d), FP64 forward + backward, "
                     "%.2f s + %.2f s" % (w.name, w.B, w.H, w.N, w.D, t1 - t0, t2 - t1),
           "seconds": t2 - t0, "fwd_seconds": t1 - t0, "bwd_seconds": t2 - t1,
           "nproc": os.cpu_count(), "cpu_model": cpu_model()}

    gO = inputs_f64(d["dO"])
    res = {}
    names = {0: "unstabilised", 1: "stabilised", 2: "stabilised_exact"}
    for stabilise in (0, 1, 2):
        f = nss.forward(t["q"], t["k"], t["v"], scale=w.scale, causal=w.causal, stabilise=stabilise,
                        beta=w.beta, stream=stream)
        b = nss.backward(t["q"], t["k"], t["v"], f["o"], t["dO"], f["lse"], scale=w.scale,
                         causal=w.causal, stabilise=stabilise, beta=w.beta, stream=stream)
        torch.cuda.synchronize()
        O = f["o"].float().cpu().numpy().astype(np.float64)
        dl = b["delta"].cpu().numpy().astype(np.float64)
        O_round = inputs_f64(oracle.bf16_from_double(ref["O"], "rne"))
        rep = bias.report(O, ref["O"], dl, rb["delta"], gO, ref["ties"],
                          np.ones(ref["ties"].shape, dtype=bool), w.v_skew_dims, O_ref_rounded=O_round)
        rep["max_err_over_tol"] = {
            "O": float(np.max(np.abs(O - ref["O"]) / ref["tol_O"])),
            "delta": float(np.max(np.abs(dl - rb["delta"]) / rb["tol_delta"]))}
        rep["pbar_one_events_on_tie_rows"] = int(f["pbar_one"].cpu().numpy()[ref["ties"] > 1].sum())
        rep["formed_ones_on_tie_rows"] = int(f["formed_ones"].cpu().numpy()[ref["ties"] > 1].sum())
        res[names[stabilise]] = rep
    res["bf16_accumulation_emulation"] = emulation_curves()
    res["O_mode_difference_z"] = bias.mode_difference(
        res["stabilised_exact"]["vs_rounded_reference"]["O_tie_rows_skewed_dims"],
        res["unstabilised"]["vs_rounded_reference"]["O_tie_rows_skewed_dims"])
    res["tie_rows"] = int((ref["ties"] > 1).sum())
    return cpu, res


def emulation_curves():
    """The pages' mechanism on the CPU (oracle.emulate_bf16_pv): P_bar V with
    every product and addition rounded to bf16, nearest-even vs ties-away,
    plain vs shifted; signed O error (bf16 ulps of the exact O, skewed V dims)
    grouped by the row's count of P_bar entries equal to 1.  Bounded sample:
    the tiny workload (all rows) and two heads of gpt2_small."""
    import numpy as np

    import oracle
    from oracle import bias
    from numerics_safe_softmax_amd import inputs
    out = {}
    t0 = time.perf_counter()
    for wname, heads in (("tiny", [0]), ("gpt2_small", [0, 1])):
        w = inputs.WORKLOADS[wname]
        d = inputs.generate(w)
        rows = oracle.head_rows(heads, w.N)
        ref = oracle.forward(d["q"], d["k"], d["v"], scale=w.scale, causal=w.causal, rows=rows, want=["O"])
        mask = ~np.isnan(ref["O"][..., 0])
        for stab in (False, True):
            for mode in ("rne", "rna"):
                r = oracle.emulate_bf16_pv(d["q"], d["k"], d["v"], scale=w.scale, causal=w.causal, stabilise=stab,
                                           beta=w.beta, accumulate=mode, rows=rows)
                out["%s/%s/%s" % (wname, "shift" if stab else "plain", mode)] = bias.event_curve(
                    r["O"], ref["O"], r["events"], mask, w.v_skew_dims)
    out["seconds"] = time.perf_counter() - t0
    return out


def inputs_f64(bits):
    from numerics_safe_softmax_amd import inputs
    return inputs.bits_to_float(bits).astype("float64")


if __name__ == "__main__":
    main()
