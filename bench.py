#!/usr/bin/env python3
"""Benchmark of the fused VQ dequant-matmul on one MI355X.

One step = the whole hot path over one batch of the dense MLP trio workload
(gate/up [17408][5120], down [5120][17408], d=2, K=256, fp16 scale per 64
weights = 4.25 bits per weight):
  decode : gate and up (which share their input) as one vq_moe_gemv launch
           over the two-expert stack of them, ids {0, 1}; vq_gemv on down;
           T = 1 token
  prefill: vq_gemm on the same gate+up stack (one launch, y [T][2][rows]) and
           on down, at T = 2048 tokens
Inputs are seeded synthetic tensors (codes uniform, codebook N(0, 0.02), scales
U[0.5, 1.5], x N(0, 1)) already resident in HBM.  The weights are replicated
so the per-step rotation touches >= 1 GiB and every call streams from HBM, not
from the 256 MB Infinity Cache.

The K timed steps run as two back-to-back blocks, K decode passes then K
prefill passes, each bracketed by HIP events on the launch stream.  Decode
passes are captured as HIP graphs of one pass per weight replica (as a model's
decode graph holds its layers), so graph-launch and event boundaries, which
cost 5-15 us of idle GPU each, fall once per 8 passes rather than inside every
pass; a short device-side spin before the first event hides the host's
submission of the first graph.  Prefill passes are one graph each.

Prints one JSON line.  `value` is the decode throughput (algorithmic bytes of
codes + scales + codebook + x + y over the decode block's time); prefill
TFLOP/s and both kernels' roofline fractions ride along.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
MFMA_F16_PEAK_TFLOPS = 2500.0   # MI355X dense fp16 MFMA

WORKLOAD = "dense_mlp_5120x17408_d2k256"
DECODE_T = 1
PREFILL_T = 2048
REPLICAS = 8


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=24)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-rows", type=int, default=1024,
                    help="rows of the gate matrix the CPU oracle sample covers")
    ap.add_argument("--profile-gate", action="store_true",
                    help="run only a few gate GEMV and gate+up stacked GEMM launches (for rocprofv3 --pmc passes)")
    ap.add_argument("--profile-sweep", choices=["A", "B"], default=None,
                    help="run only a few config-4 launches of matrix A (17408x5120) or B (5120x17408), d=4 K=256: "
                         "GEMV at T=1 and GEMM at T=4096 (for rocprofv3 --pmc passes)")
    ap.add_argument("--no-sweep", action="store_true", help="skip the config-4 sweep rooflines")
    ap.add_argument("--copy-probe", action="store_true",
                    help="run only a plain device copy of known size (counter calibration)")
    ap.add_argument("--configs", nargs="?", const="", default=None, metavar="FILTER",
                    help="print a per-workload report (every config, both kernels, median/p10/p90) "
                         "as markdown instead of the JSON line; FILTER keeps workloads whose name "
                         "contains it")
    return ap.parse_args()


COPY_PROBE_ELEMS = 1 << 28          # fp16 -> fp32 copy: reads 512 MiB, writes 1 GiB
COPY_READ_BYTES = 2 * COPY_PROBE_ELEMS
COPY_WRITE_BYTES = 4 * COPY_PROBE_ELEMS
PROFILES = os.path.join(ROOT, "profiles")
GATE_TAG = "dense_mlp_gate_17408x5120"           # profiles/pmc_*_<tag>.txt of the gate kernels
COPY_TAG = "torch_copy_2p28_fp16_to_fp32"        # profiles/pmc_*_<tag>.txt of the copy probe


def copy_probe():
    """A plain converting copy of known size (fp16 -> fp32, 2^28 elements),
    four times: what FETCH_SIZE and WRITE_SIZE read for it calibrates them
    against known traffic."""
    import torch
    src = torch.ones(COPY_PROBE_ELEMS, dtype=torch.float16, device="cuda")
    dst = torch.empty(COPY_PROBE_ELEMS, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    for _ in range(4):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_read_bytes": COPY_READ_BYTES, "copy_write_bytes": COPY_WRITE_BYTES,
                      "launches": 4}), flush=True)


def _pmc_value(fname, counter, kernel_prefix, grid=None):
    """Average per-dispatch value of `counter` for the first kernel whose
    name starts with kernel_prefix -- a plain prefix, or a compiled regular
    expression matched at the start of the line -- (and whose grid is `grid`,
    when given), from a profsum pmc summary."""
    path = os.path.join(PROFILES, fname)
    if not os.path.exists(path):
        return None, None
    digest = None
    with open(path) as fh:
        for line in fh:
            if line.startswith("kernel source digest:"):
                digest = line.split(":", 1)[1].strip()
            hit = (kernel_prefix.match(line) is not None) if hasattr(kernel_prefix, "match") \
                else line.startswith(kernel_prefix)
            if hit and (grid is None or f" grid={grid} " in line):
                for part in line.split():
                    if part.startswith(counter + "="):
                        return float(part.split("=", 1)[1]), digest
    return None, digest


def measured_traffic(kernel_prefix, tag, grid=None):
    """HBM bytes per launch of the named kernel from the committed FETCH_SIZE
    and WRITE_SIZE passes, each scaled by the same counter's reading for the
    1 GiB copy; None when a pass is missing or the kernels changed since."""
    from vq_dequant_matmul_gemv_amd.profsum import source_digest
    f, fd = _pmc_value(f"pmc_fetch_size_{tag}.txt", "FETCH_SIZE", kernel_prefix, grid)
    w, wd = _pmc_value(f"pmc_write_size_{tag}.txt", "WRITE_SIZE", kernel_prefix, grid)
    cf, _ = _pmc_value(f"pmc_fetch_size_{COPY_TAG}.txt", "FETCH_SIZE", "torch copy")
    cw, _ = _pmc_value(f"pmc_write_size_{COPY_TAG}.txt", "WRITE_SIZE", "torch copy")
    if None in (f, w, cf, cw) or fd != source_digest() or wd != source_digest():
        return None
    fetch_scale = (COPY_READ_BYTES / 1024) / cf     # true KiB per counted KiB
    write_scale = (COPY_WRITE_BYTES / 1024) / cw
    return round((f * fetch_scale + w * write_scale) * 1024)


SWEEP = "sweep_17408x5120_d4k256"
SWEEP_TAG = "sweep_d4k256_17408x5120_and_5120x17408"   # profiles/pmc_*_<tag>.txt of the sweep kernels
SWEEP_REPLICAS = 16                                   # 16 x 25 MB per matrix: every call streams from HBM


def sweep_rooflines(profile_only=None):
    """Config-4 kernels on one GPU: W_A [17408][5120] and W_B [5120][17408],
    d=4 K=256 g=64, vq_gemv at T = 1, 4 and 16 (HBM-bound; 4 and 16 on the
    matrix-core GEMV) and the GEMM at T = 256 and 4096 (MFMA-bound).  Per-launch durations from bursts of back-to-back launches
    in one graph (16 GEMVs / 4 GEMMs, rotating over weight replicas), timed
    with events on the launch stream, median of 5 bursts."""
    import re
    import torch
    from vq_dequant_matmul_gemv_amd import binding, synth
    dev = torch.device("cuda", 0)
    wl = synth.WORKLOADS[SWEEP]
    out = {}
    for name in ((profile_only,) if profile_only else ("A", "B")):
        spec = wl["tensors"][name]
        base = binding.VQTensor.from_host(synth.tensor(spec, SWEEP, name), spec, device=dev)
        reps = [base] + [binding.VQTensor(base.codes.clone(), base.codebook.clone(), base.scales.clone(), spec.rows,
                                          spec.cols, spec.d, spec.log2_k, spec.group)
                         for _ in range(SWEEP_REPLICAS - 1)]
        x1 = torch.from_numpy(synth.activations((1, spec.cols), SWEEP, name, "x", 1)).to(dev)
        x4 = torch.from_numpy(synth.activations((4, spec.cols), SWEEP, name, "x", 4)).to(dev)
        y4 = torch.empty((4, spec.rows), dtype=torch.float32, device=dev)
        x16 = torch.from_numpy(synth.activations((16, spec.cols), SWEEP, name, "x", 16)).to(dev)
        y16 = torch.empty((16, spec.rows), dtype=torch.float32, device=dev)
        x256 = torch.from_numpy(synth.activations((256, spec.cols), SWEEP, name, "x", 256)).to(dev)
        y256 = torch.empty((256, spec.rows), dtype=torch.float32, device=dev)
        xT = torch.from_numpy(synth.activations((4096, spec.cols), SWEEP, name, "x", 4096)).to(dev)
        y1 = torch.empty((1, spec.rows), dtype=torch.float32, device=dev)
        yT = torch.empty((4096, spec.rows), dtype=torch.float32, device=dev)
        gemv = [lambda w=reps[i % SWEEP_REPLICAS]: binding.gemv(w, x1, y1) for i in range(16)]
        gemv4 = [lambda w=reps[i % SWEEP_REPLICAS]: binding.gemv(w, x4, y4) for i in range(16)]
        gemv16 = [lambda w=reps[i % SWEEP_REPLICAS]: binding.gemv(w, x16, y16) for i in range(16)]
        gemm256 = [lambda w=reps[i % SWEEP_REPLICAS]: binding.gemm(w, x256, y256) for i in range(8)]
        gemm = [lambda w=reps[i % SWEEP_REPLICAS]: binding.gemm(w, xT, yT) for i in range(4)]
        if profile_only:
            for c in gemv[:4] + gemv4[:4] + gemm[:2]:
                c()
            torch.cuda.synchronize()
            continue
        for c in gemv + gemv4 + gemv16 + gemm256 + gemm:   # warm
            c()
        torch.cuda.synchronize()
        res = {}
        for key, calls in (("gemv_T1", gemv), ("gemv_T4", gemv4), ("gemv_T16", gemv16), ("gemm_T256", gemm256),
                           ("gemm_T4096", gemm)):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for c in calls:
                    c()
            times = []
            for _ in range(5):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                torch.cuda._sleep(1_000_000)
                a.record()
                g.replay()
                b.record()
                torch.cuda.synchronize()
                times.append(a.elapsed_time(b) * 1e-3 / len(calls))
            res[key] = sorted(times)[2]
            del g
        nb = tensor_bytes(spec, 1)
        nb4 = tensor_bytes(spec, 4)
        nb16 = tensor_bytes(spec, 16)
        gbps16 = nb16 / res["gemv_T16"] / 1e9
        tflops256 = 2.0 * 256 * spec.rows * spec.cols / res["gemm_T256"] / 1e12
        flops = 2.0 * 4096 * spec.rows * spec.cols
        gbps = nb / res["gemv_T1"] / 1e9
        gbps4 = nb4 / res["gemv_T4"] / 1e9
        tflops = flops / res["gemm_T4096"] / 1e12
        out[f"{name}_{spec.rows}x{spec.cols}"] = {
            "gemv_T1": {"bound": "hbm", "us": round(res["gemv_T1"] * 1e6, 2), "achieved": round(gbps, 2),
                        "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBPS, 4),
                        "algorithmic_bytes": nb,
                        "traffic": measured_traffic(re.compile(r"vq_gemv_kernel<4, 8, 64, \d+, \d+, false, 1, false>"),
                                                    SWEEP_TAG + "_" + name)},
            "gemv_T4": {"bound": "hbm", "us": round(res["gemv_T4"] * 1e6, 2), "achieved": round(gbps4, 2),
                        "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(gbps4 / HBM_PEAK_GBPS, 4),
                        "algorithmic_bytes": nb4,
                        "traffic": measured_traffic(re.compile(r"vq_gemv_kernel<4, 8, 64, \d+, \d+, false, 4, true>"),
                                                    SWEEP_TAG + "_" + name)},
            "gemv_T16": {"bound": "hbm", "us": round(res["gemv_T16"] * 1e6, 2), "achieved": round(gbps16, 2),
                         "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(gbps16 / HBM_PEAK_GBPS, 4),
                         "algorithmic_bytes": nb16},
            "gemm_T256": {"bound": "mfma", "us": round(res["gemm_T256"] * 1e6, 2), "achieved": round(tflops256, 2),
                          "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                          "frac": round(tflops256 / MFMA_F16_PEAK_TFLOPS, 4),
                          "algorithmic_bytes": tensor_bytes(spec, 256)},
            "gemm_T4096": {"bound": "mfma", "us": round(res["gemm_T4096"] * 1e6, 2), "achieved": round(tflops, 2),
                           "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                           "frac": round(tflops / MFMA_F16_PEAK_TFLOPS, 4),
                           "algorithmic_bytes": tensor_bytes(spec, 4096),
                           "traffic": measured_traffic("vq_gemm_kernel<4, 8, 64, GemmShape<8, 2, 4>",
                                                       SWEEP_TAG + "_" + name)}}
        del reps, base, xT, yT, x4, y4, x16, y16, x256, y256
        torch.cuda.empty_cache()
    if profile_only:
        print(f"profile-sweep {profile_only}: 4 GEMVs (T=1), 4 GEMVs (T=4) and 2 GEMMs (T=4096)", flush=True)
    return out


def tensor_bytes(spec, T):
    """Algorithmic bytes of one dense call: packed codes + fp16 scales + fp16
    codebook (once) + fp16 x + fp32 y.  Dequantized weights are never counted."""
    return (spec.rows * spec.words * 4 + spec.rows * (spec.cols // spec.group) * 2
            + spec.k * spec.d * 2 + T * spec.cols * 2 + T * spec.rows * 4)


def cpu_baseline(arrs, spec, rows):
    """The oracle as it stands, timed on the host on a bounded sample: the
    first `rows` rows of the gate matrix at T = 1 (unpack, dequant, float64
    matmul).  Reported in GB/s of the same algorithmic bytes."""
    import numpy as np
    from oracle import vq_oracle as O
    from vq_dequant_matmul_gemv_amd import synth
    x = synth.activations((1, spec.cols), "bench-cpu")
    words = np.ascontiguousarray(arrs["codes"][0, :rows])
    scales = np.ascontiguousarray(arrs["scales"][0, :rows])
    t0 = time.perf_counter()
    reps = 0
    while True:
        O.gemv_ref(words, arrs["codebook"], scales, x, spec.cols, spec.d, spec.log2_k, spec.group)
        reps += 1
        if time.perf_counter() - t0 > 10.0 or reps >= 50:
            break
    dt = (time.perf_counter() - t0) / reps
    sub = synth.Spec(rows, spec.cols, spec.d, spec.log2_k, spec.group)
    gbps = tensor_bytes(sub, 1) / dt / 1e9
    cores = len(os.sched_getaffinity(0))
    return {"value": round(gbps, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"gate matrix rows 0..{rows - 1} of 17408 (cols 5120, d=2 K=256 g=64), T=1: "
                      f"unpack + fp16 dequant + float64 matmul, {reps} reps, {dt * 1e3:.1f} ms each"}


REPORT_CMD = "python3 bench.py --configs"  # the full report (no filter)


def configs_report(only=""):
    """Every workload of the benchmark set, both kernels, timed as back-to-back
    calls in one HIP graph rotating over weight replicas (>= 1.1 GB touched
    per replay where the tensors allow, so calls stream from HBM, not the
    256 MB Infinity Cache); median, p10 and p90 over 30 replays of the per-call
    average.  Algorithmic counting: bytes = codes + scales + codebook + x + y
    (+ ids), routed calls counting only the distinct experts they hit;
    flops = 2 T rows cols (x top_k when routed).  Context: a plain read and
    torch's fp16 GEMM on uncompressed weights of the same shapes."""
    import numpy as np
    import torch
    from vq_dequant_matmul_gemv_amd import binding, synth

    dev = torch.device("cuda", 0)
    from vq_dequant_matmul_gemv_amd.profsum import source_digest
    out = [f"command: {REPORT_CMD}", f"kernel source digest: {source_digest()}",
           f"encoder source digest: {source_digest('encoder')}", "",
           "vq_gemv hands token counts above its measured crossover to the MFMA kernel (the rows with",
           "larger T under vq_gemv time that kernel); vq_gemm always runs the MFMA kernel.", "",
           "| workload | tensor | call | T | per call us (median, p10, p90) | GB/s | % of 8 TB/s | TFLOP/s | % of 2.5 PF |",
           "|---|---|---|---|---|---|---|---|---|"]

    def timed(calls, reps=30):
        torch.cuda.synchronize()
        for c in calls:
            c()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for c in calls:
                c()
        for _ in range(3):
            g.replay()
        torch.cuda.synchronize()
        per = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda._sleep(1_000_000)   # the GPU is busy while the graph is submitted
            a.record()
            g.replay()
            b.record()
            torch.cuda.synchronize()
            per.append(a.elapsed_time(b) * 1e3 / len(calls))
        del g
        return np.percentile(per, [50, 10, 90])

    def row(wl, name, call, T, us, nbytes, flops):
        med = us[0]
        gbs = nbytes / med / 1e3
        tf = flops / med / 1e6
        out.append(f"| {wl} | {name} | {call} | {T} | {us[0]:.2f} ({us[1]:.2f}, {us[2]:.2f}) | {gbs:.0f} | "
                   f"{100 * gbs / HBM_PEAK_GBPS:.1f} | {tf:.1f} | {100 * tf / MFMA_F16_PEAK_TFLOPS:.1f} |")
        print(out[-1], file=sys.stderr, flush=True)

    def replicas(spec, host, nbytes, cap=2048):
        base = binding.VQTensor.from_host(host, spec, device=dev)
        n = int(min(cap, max(1, -(-1.1e9 // nbytes))))
        reps = [base]
        for _ in range(n - 1):
            reps.append(binding.VQTensor(base.codes.clone(), base.codebook.clone(), base.scales.clone(),
                                         spec.rows, spec.cols, spec.d, spec.log2_k, spec.group,
                                         spec.experts))
        return reps

    def dense(wl, name, spec, gemv_T, gemm_T, key):
        host = synth.tensor(spec, *key)
        reps = replicas(spec, host, tensor_bytes(spec, 1))
        for fn, Ts in (("gemv", gemv_T), ("gemm", gemm_T)):
            for T in Ts:
                x = torch.from_numpy(synth.activations((T, spec.cols), *key, "x", T)).to(dev)
                y = torch.empty((T, spec.rows), dtype=torch.float32, device=dev)
                n = max(16, len(reps)) if T * spec.rows * 4 < 64e6 else max(4, min(len(reps), 8))
                calls = [(lambda w=reps[i % len(reps)]: getattr(binding, fn)(w, x, y)) for i in range(n)]
                us = timed(calls)
                row(wl, name, "vq_" + fn, T, us, tensor_bytes(spec, T), 2.0 * T * spec.rows * spec.cols)
        del reps
        torch.cuda.empty_cache()

    def dequant_row(wl, name, spec, key):
        """vq_dequant of the whole matrix: bytes = codes + scales + codebook
        read + the fp16 weights written."""
        host = synth.tensor(spec, *key)
        nbytes = spec.rows * spec.words * 4 + spec.rows * (spec.cols // spec.group) * 2 + spec.k * spec.d * 2 \
            + spec.rows * spec.cols * 2
        reps = replicas(spec, host, nbytes)
        out_w = torch.empty((spec.rows, spec.cols), dtype=torch.float16, device=dev)
        calls = [(lambda w=reps[i % len(reps)]: binding.dequant(w, out=out_w)) for i in range(max(8, len(reps)))]
        us = timed(calls)
        row(wl, name, "vq_dequant", "-", us, nbytes, 0.0)
        del reps
        torch.cuda.empty_cache()

    def stacked_pair(wl, name, spec, keys, gemv_Ts=(), gemm_Ts=()):
        """Two tensors sharing x (gate and up), stacked as two experts with
        per-expert codebooks: at T = 1 one vq_moe_gemv launch with ids {0, 1},
        at each of gemv_Ts / gemm_Ts one vq_gemv / vq_gemm launch over the
        stack."""
        t = [binding.VQTensor.from_host(synth.tensor(spec, *k), spec, device=dev) for k in keys]
        base = binding.VQTensor(torch.stack([t[0].codes, t[1].codes]), torch.stack([t[0].codebook, t[1].codebook]),
                                torch.stack([t[0].scales, t[1].scales]), spec.rows, spec.cols, spec.d,
                                spec.log2_k, spec.group, 2, True)
        del t
        nbytes = 2 * tensor_bytes(spec, 1)
        reps = [base] + [binding.VQTensor(base.codes.clone(), base.codebook.clone(), base.scales.clone(),
                                          spec.rows, spec.cols, spec.d, spec.log2_k, spec.group, 2, True)
                         for _ in range(int(max(0, -(-1.1e9 // nbytes) - 1)))]
        x = torch.from_numpy(synth.activations((1, spec.cols), *keys[0], "x", 1)).to(dev)
        ids = torch.tensor([[0, 1]], dtype=torch.int32, device=dev)
        y = torch.empty((1, 2, spec.rows), dtype=torch.float32, device=dev)
        calls = [(lambda w=reps[i % len(reps)]: binding.moe_gemv(w, x, ids, y=y)) for i in range(16)]
        us = timed(calls)
        row(wl, name, "vq_moe_gemv", 1, us, nbytes, 2.0 * 2 * spec.rows * spec.cols)
        for fn, Ts, label, n in (("gemv", gemv_Ts, "one GEMV", 16), ("gemm", gemm_Ts, "one GEMM", 4)):
            for T in Ts:
                xg = torch.from_numpy(synth.activations((T, spec.cols), *keys[0], "x", T)).to(dev)
                yg = torch.empty((T, 2, spec.rows), dtype=torch.float32, device=dev)
                calls = [(lambda w=reps[i % len(reps)]: getattr(binding, fn)(w, xg, yg)) for i in range(n)]
                us = timed(calls)
                tb = 2 * tensor_bytes(spec, T) - T * spec.cols * 2   # x read once
                row(wl, name.replace("ids {0,1}", label), "vq_" + fn, T, us, tb, 2.0 * 2 * T * spec.rows * spec.cols)
                del xg, yg
        del reps
        torch.cuda.empty_cache()

    def routed_gate_up(wl, spec, top_k, Ts, key_g, key_u):
        """Routed gate and up in one call: experts 2e / 2e + 1 of one stack
        (per-expert codebooks), ids 2e, 2e + 1 per slot (top_k doubled);
        vq_moe_gemv at the first token count, vq_moe_gemm at the second.
        Bytes and flops as for the two separate calls."""
        tg = binding.VQTensor.from_host(synth.tensor(spec, *key_g), spec, device=dev)
        tu = binding.VQTensor.from_host(synth.tensor(spec, *key_u), spec, device=dev)
        E = spec.experts
        base = binding.VQTensor(torch.stack([tg.codes, tu.codes], 1).reshape(2 * E, spec.rows, -1).contiguous(),
                                torch.stack([tg.codebook, tu.codebook]).repeat(E, 1, 1).contiguous(),
                                torch.stack([tg.scales, tu.scales], 1).reshape(2 * E, spec.rows, -1).contiguous(),
                                spec.rows, spec.cols, spec.d, spec.log2_k, spec.group, 2 * E, True)
        del tg, tu
        per_expert = spec.rows * spec.words * 4 + spec.rows * (spec.cols // spec.group) * 2
        reps = [base] + [binding.VQTensor(base.codes.clone(), base.codebook.clone(), base.scales.clone(),
                                          spec.rows, spec.cols, spec.d, spec.log2_k, spec.group, 2 * E, True)
                         for _ in range(int(max(0, min(7, -(-1.1e9 // (per_expert * 2 * E)) - 1))))]
        for fn, T in zip(("moe_gemv", "moe_gemm"), Ts):
            draws = [synth.zipf_routing(T, E, top_k, *key_g, "ids", T, r) for r in range(16)]
            ids = [torch.from_numpy(np.stack([2 * d, 2 * d + 1], -1).reshape(T, 2 * top_k).astype(np.int32))
                   .to(dev) for d in draws]
            x = torch.from_numpy(synth.activations((T, spec.cols), *key_g, "x", T)).to(dev)
            y = torch.empty((T, 2 * top_k, spec.rows), dtype=torch.float32, device=dev)
            ws = torch.empty(max(16, binding.workspace_bytes(T, 2 * top_k, 2 * E)), dtype=torch.uint8, device=dev)
            calls, nbytes = [], 0
            for i in range(16):
                w = reps[i % len(reps)]
                if fn == "moe_gemv":
                    calls.append(lambda w=w, d=ids[i]: binding.moe_gemv(w, x, d, y=y))
                else:
                    calls.append(lambda w=w, d=ids[i]: binding.moe_gemm(w, x, d, y=y, workspace=ws))
                hit = len(np.unique(draws[i]))
                nbytes += 2 * (hit * per_expert + spec.k * spec.d * 2 + x.numel() * 2 + T * top_k * spec.rows * 4
                               + T * top_k * 4)
            us = timed(calls)
            row(wl, "gate+up (experts 2e / 2e+1 of one stack, top-16)", "vq_" + fn, T, us, nbytes / 16,
                2.0 * 2 * T * top_k * spec.rows * spec.cols)
        del reps
        torch.cuda.empty_cache()

    def routed(wl, name, spec, top_k, Ts, x_per_slot, key):
        host = synth.tensor(spec, *key)
        per_expert = spec.rows * spec.words * 4 + spec.rows * (spec.cols // spec.group) * 2
        reps = replicas(spec, host, per_expert * spec.experts, cap=8)
        for fn, T in zip(("moe_gemv", "moe_gemm"), Ts):
            draws = [synth.zipf_routing(T, spec.experts, top_k, *key, "ids", T, r) for r in range(16)]
            ids = [torch.from_numpy(d.astype(np.int32)).to(dev) for d in draws]
            shape = (T, top_k, spec.cols) if x_per_slot else (T, spec.cols)
            x = torch.from_numpy(synth.activations(shape, *key, "x", T)).to(dev)
            y = torch.empty((T, top_k, spec.rows), dtype=torch.float32, device=dev)
            ws = torch.empty(max(16, binding.workspace_bytes(T, top_k, spec.experts)), dtype=torch.uint8, device=dev)
            calls, nbytes = [], 0
            for i in range(16):
                w = reps[i % len(reps)]
                if fn == "moe_gemv":
                    calls.append(lambda w=w, d=ids[i]: binding.moe_gemv(w, x, d, x_per_slot=x_per_slot, y=y))
                else:
                    calls.append(lambda w=w, d=ids[i]: binding.moe_gemm(w, x, d, x_per_slot=x_per_slot, y=y,
                                                                        workspace=ws))
                hit = len(np.unique(draws[i]))
                nbytes += (hit * per_expert + spec.k * spec.d * 2 + x.numel() * 2 + y.numel() * 4
                           + T * top_k * 4)
            us = timed(calls)
            row(wl, name, "vq_" + fn, T, us, nbytes / 16, 2.0 * T * top_k * spec.rows * spec.cols)
        del reps
        torch.cuda.empty_cache()

    W = synth.WORKLOADS
    keep = lambda wl: only in wl
    if keep("gemv_1024"):
        dense("gemv_1024", "w", W["gemv_1024"]["tensors"]["w"], [1], [], ("gemv_1024", "w"))
    wl = "dense_mlp_5120x17408_d2k256"
    for n in ("gate", "up", "down") if keep(wl) else ():
        # T = 2: a two-token verify step, T = 4 a four-token one; both kernels
        # timed for the crossover
        dense(wl, n, W[wl]["tensors"][n], [1, 2, 4], [2, 4, 2048], (wl, n))
    if keep(wl):
        stacked_pair(wl, "gate+up (two-expert stack, ids {0,1})", W[wl]["tensors"]["gate"],
                     ((wl, "gate"), (wl, "up")), gemv_Ts=(2, 4, 16), gemm_Ts=(2048,))
        dequant_row(wl, "gate", W[wl]["tensors"]["gate"], (wl, "gate"))
    wl = "moe_e256_4096x1024_d4k256"
    for n in ("gate", "down") if keep(wl) else ():
        routed(wl, n, W[wl]["tensors"][n], W[wl]["top_k"], (1, 1024), n == "down", (wl, n))
    if keep(wl):
        routed_gate_up(wl, W[wl]["tensors"]["gate"], W[wl]["top_k"], (1, 1024), (wl, "gate"), (wl, "up"))
    wl = "moe_mixed_tier_e256_2048x512"
    for tier in ("T1", "T2", "T3") if keep(wl) else ():
        for idx, n in ((0, "gate"), (2, "down")):
            routed(wl, f"{tier} {n}", synth.mixed_tier_spec(idx, tier), W[wl]["top_k"], (1, 512), idx == 2,
                   (wl, tier, idx))
    wl = "sweep_17408x5120_d4k256"
    for n in ("A", "B") if keep(wl) else ():
        Ts = sorted(set(W[wl]["tokens"]) | {2, 3})
        dense(wl, n, W[wl]["tensors"][n], Ts, Ts, (wl, n))
    if keep(wl):
        dequant_row(wl, "A", W[wl]["tensors"]["A"], (wl, "A"))

    # ---- the next rows: fused MLP epilogues, the bf16 profile, other code
    # widths, the encoder ----------------------------------------------------
    def mlp_chain(wl_name, gu_spec, dn_spec, T, routed_top_k=None):
        """gate/up stored as one tensor of interleaved rows with the SwiGLU
        epilogue (fp16 h), then down taking h; routed: down with the
        router-weighted combine.  Bytes: both tensors (distinct experts hit)
        + x + h + y; flops: both products."""
        key = ("next", wl_name)
        hg = synth.tensor(gu_spec, *key, "gu")
        hd = synth.tensor(dn_spec, *key, "dn")
        wgu = binding.VQTensor.from_host(hg, gu_spec, device=dev)
        wdn = binding.VQTensor.from_host(hd, dn_spec, device=dev)
        per_gu = gu_spec.rows * gu_spec.words * 4 + gu_spec.rows * (gu_spec.cols // gu_spec.group) * 2
        per_dn = dn_spec.rows * dn_spec.words * 4 + dn_spec.rows * (dn_spec.cols // dn_spec.group) * 2
        nrep = 1 if routed_top_k else int(max(1, -(-1.1e9 // (per_gu + per_dn))))
        reps = [(wgu, wdn)] + [(binding.VQTensor(wgu.codes.clone(), wgu.codebook.clone(), wgu.scales.clone(),
                                                 gu_spec.rows, gu_spec.cols, gu_spec.d, gu_spec.log2_k, gu_spec.group,
                                                 gu_spec.experts),
                                binding.VQTensor(wdn.codes.clone(), wdn.codebook.clone(), wdn.scales.clone(),
                                                 dn_spec.rows, dn_spec.cols, dn_spec.d, dn_spec.log2_k, dn_spec.group,
                                                 dn_spec.experts)) for _ in range(nrep - 1)]
        x = torch.from_numpy(synth.activations((T, gu_spec.cols), *key, "x", T)).to(dev)
        I = gu_spec.rows // 2
        calls, nbytes = [], 0
        if routed_top_k:
            k = routed_top_k
            draws = [synth.zipf_routing(T, gu_spec.experts, k, *key, "ids", T, r) for r in range(8)]
            ids = [torch.from_numpy(d.astype(np.int32)).to(dev) for d in draws]
            rw = torch.from_numpy(synth.router_weights(T, k, *key, "rw")).to(dev)
            h = torch.empty((T, k, I), dtype=torch.float16, device=dev)
            y = torch.empty((T, dn_spec.rows), dtype=torch.float32, device=dev)
            fn = binding.moe_gemv if T == 1 else binding.moe_gemm
            ws = torch.empty(max(16, binding.workspace_bytes(T, k, gu_spec.experts)), dtype=torch.uint8, device=dev)
            extra = {} if T == 1 else {"workspace": ws}
            for i in range(8):
                def c(d=ids[i]):
                    fn(wgu, x, d, y=h, epilogue="swiglu", **extra)
                    fn(wdn, h, d, x_per_slot=True, y=y, epilogue="combine", route_weights=rw, **extra)
                calls.append(c)
                hit = len(np.unique(draws[i]))
                nbytes += hit * (per_gu + per_dn) + x.numel() * 2 + 2 * h.numel() * 2 + y.numel() * 4
            flops = 2.0 * T * k * (gu_spec.rows * gu_spec.cols + dn_spec.rows * dn_spec.cols)
            nbytes /= 8
        else:
            h = torch.empty((T, I), dtype=torch.float16, device=dev)
            y = torch.empty((T, dn_spec.rows), dtype=torch.float32, device=dev)
            fn = binding.gemv if T == 1 else binding.gemm
            for i in range(max(8, nrep)):
                def c(p=reps[i % len(reps)]):
                    fn(p[0], x, y=h, epilogue="swiglu")
                    fn(p[1], h, y=y)
                calls.append(c)
            nbytes = per_gu + per_dn + x.numel() * 2 + 2 * h.numel() * 2 + y.numel() * 4
            flops = 2.0 * T * (gu_spec.rows * gu_spec.cols + dn_spec.rows * dn_spec.cols)
        us = timed(calls)
        call = ("vq_moe_gemv" if T == 1 else "vq_moe_gemm") if routed_top_k else ("vq_gemv" if T == 1 else "vq_gemm")
        row(wl_name, "MLP: gate/up SwiGLU (interleaved rows, fp16 h) -> down" +
            (" with router-weighted combine" if routed_top_k else ""), call + " x2", T, us, nbytes, flops)
        del reps, wgu, wdn
        torch.cuda.empty_cache()

    def bf16_rows(wl_name, spec, key):
        """The bf16 profile: bf16 x in, bf16 y out, against fp16 x / fp32 y."""
        host = synth.tensor(spec, *key)
        reps = replicas(spec, host, tensor_bytes(spec, 1), cap=24)
        for T, fn in ((1, "gemv"), (2048, "gemm")):
            xb = synth.activations_bf16((T, spec.cols), *key, "xb", T)
            x = torch.from_numpy(xb.view(np.int16)).to(dev).view(torch.bfloat16)
            y = torch.empty((T, spec.rows), dtype=torch.bfloat16, device=dev)
            n = 16 if T == 1 else 8
            calls = [(lambda w=reps[i % len(reps)]: getattr(binding, fn)(w, x, y)) for i in range(n)]
            us = timed(calls)
            row(wl_name, f"{spec.rows}x{spec.cols} bf16 x, bf16 y", "vq_" + fn, T, us,
                tensor_bytes(spec, T) - T * spec.rows * 2, 2.0 * T * spec.rows * spec.cols)
        del reps
        torch.cuda.empty_cache()

    def encode_row(rows, cols, d, b, g, n_s, iters):
        """vq_encode of one tensor (per call; the k-means++ seeding runs in
        one workgroup, the Lloyd iterations grid-wide); flops counted are the
        assignment's 3 d operations per (subvector, centroid) per pass."""
        w = torch.from_numpy(synth.weights(rows, cols, "bench-enc")).to(dev)
        idx, u = synth.fit_draws(rows * cols // d, n_s, 1 << b, "bench-enc")
        idx, u = torch.from_numpy(idx).to(dev), torch.from_numpy(u).to(dev)
        wsz = binding.LIB.vq_encode_workspace_bytes(rows, cols, d, b, n_s)
        ws = torch.empty(wsz, dtype=torch.uint8, device=dev)
        us = timed([lambda: binding.encode(w, d, b, g, idx, u, iters, workspace=ws)], reps=5)
        n = rows * cols // d
        ops = 3.0 * d * n * (1 << b) * (iters + 1)
        row("encoder", f"fit {rows}x{cols} d{d}/K{1 << b}/g{g}, sample {n_s}, {iters} Lloyd iterations",
            "vq_encode", "-", us, rows * cols * 4, ops)

    nx = "next_rows"
    if keep(nx):
        S = synth.Spec
        mlp_chain(nx, S(2 * 17408, 5120, 2, 8, 64), S(5120, 17408, 2, 8, 64), 1)
        mlp_chain(nx, S(2 * 17408, 5120, 2, 8, 64), S(5120, 17408, 2, 8, 64), 2048)
        mlp_chain(nx, S(2 * 1024, 4096, 4, 8, 64, experts=256), S(4096, 1024, 4, 8, 64, experts=256), 1, 8)
        mlp_chain(nx, S(2 * 1024, 4096, 4, 8, 64, experts=256), S(4096, 1024, 4, 8, 64, experts=256), 1024, 8)
        bf16_rows(nx, S(17408, 5120, 2, 8, 64), (nx, "bf16"))
        for (d, b) in ((2, 9), (4, 11), (4, 14), (8, 14)):
            spec = S(17408, 5120, d, b, 64)
            dense(nx, f"17408x5120 d{d}/K{1 << b}", spec, [1], [2048], (nx, d, b))
    if keep("encoder"):
        encode_row(1024, 4096, 4, 8, 64, 16384, 10)
    if only:
        print("\n".join(out), flush=True)
        return

    # context: a plain read and torch's fp16 GEMM on uncompressed weights
    out += ["", "context (same GPU, same run):", ""]
    src = torch.empty(1 << 29, dtype=torch.float16, device=dev).normal_()
    dst = torch.empty_like(src)
    us = timed([lambda: dst.copy_(src)] * 8)
    out.append(f"- plain stream (torch copy of 1 GiB fp16: 1 GiB read + 1 GiB written): {us[0]:.1f} us median = "
               f"{(2 << 30) / us[0] / 1e3:.0f} GB/s")
    del src, dst
    for (M, K, N) in ((17408, 5120, 2048), (17408, 5120, 4096), (5120, 17408, 4096)):
        a = torch.randn(M, K, device=dev, dtype=torch.float16)
        b = torch.randn(K, N, device=dev, dtype=torch.float16)
        us = timed([lambda: a @ b] * 8)
        out.append(f"- torch fp16 matmul (hipBLASLt), W {M}x{K} uncompressed, {N} tokens: {us[0]:.1f} us = "
                   f"{2.0 * M * K * N / us[0] / 1e6:.1f} TFLOP/s")
        del a, b
    print("\n".join(out), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: --gpus {args.gpus} is not supported "
              f"(this build runs on a single MI355X; multi-GPU sharding is design-only)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from vq_dequant_matmul_gemv_amd import binding, synth

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    if args.copy_probe:
        copy_probe()
        return
    if args.profile_sweep:
        sweep_rooflines(profile_only=args.profile_sweep)
        return
    if args.configs is not None:
        configs_report(args.configs)
        return

    wl = synth.WORKLOADS[WORKLOAD]
    names = ["gate", "up", "down"]
    specs = {n: wl["tensors"][n] for n in names}
    host = {n: synth.tensor(specs[n], WORKLOAD, n) for n in names}
    sg, sd = specs["gate"], specs["down"]

    # Gate and up share their input, so they are stored as one two-expert
    # stack (per-expert codebooks) and decoded by one routed launch with ids
    # {0, 1}, and run by one vq_gemm launch over the stack in prefill; the
    # single-tensor figures take per-expert views of the same stack.
    def stack_gate_up(src_gate, src_up):
        t = [binding.VQTensor.from_host(h, sg) for h in (src_gate, src_up)]
        return binding.VQTensor(torch.stack([t[0].codes, t[1].codes]), torch.stack([t[0].codebook, t[1].codebook]),
                                torch.stack([t[0].scales, t[1].scales]), sg.rows, sg.cols, sg.d, sg.log2_k,
                                sg.group, 2, True)

    def expert_view(st, e):
        return binding.VQTensor(st.codes[e], st.codebook[e], st.scales[e], st.rows, st.cols, st.d, st.log2_k,
                                st.group)

    base_gu = stack_gate_up(host["gate"], host["up"])
    base_down = binding.VQTensor.from_host(host["down"], sd)
    reps = []
    for r in range(REPLICAS):
        gu = base_gu if r == 0 else binding.VQTensor(base_gu.codes.clone(), base_gu.codebook.clone(),
                                                     base_gu.scales.clone(), sg.rows, sg.cols, sg.d, sg.log2_k,
                                                     sg.group, 2, True)
        down = base_down if r == 0 else binding.VQTensor(base_down.codes.clone(), base_down.codebook.clone(),
                                                         base_down.scales.clone(), sd.rows, sd.cols, sd.d,
                                                         sd.log2_k, sd.group)
        reps.append({"gate_up": gu, "gate": expert_view(gu, 0), "up": expert_view(gu, 1), "down": down})
    xd_gu = torch.from_numpy(synth.activations((DECODE_T, sg.cols), WORKLOAD, "xd", "gate_up")).to(dev)
    xd_dn = torch.from_numpy(synth.activations((DECODE_T, sd.cols), WORKLOAD, "xd", "down")).to(dev)
    xp_gu = torch.from_numpy(synth.activations((PREFILL_T, sg.cols), WORKLOAD, "xp", "gate_up")).to(dev)
    xp_dn = torch.from_numpy(synth.activations((PREFILL_T, sd.cols), WORKLOAD, "xp", "down")).to(dev)
    ids_gu = torch.tensor([[0, 1]] * DECODE_T, dtype=torch.int32, device=dev)
    yd_gu = torch.empty((DECODE_T, 2, sg.rows), dtype=torch.float32, device=dev)
    yd_g = torch.empty((DECODE_T, sg.rows), dtype=torch.float32, device=dev)
    yd_dn = torch.empty((DECODE_T, sd.rows), dtype=torch.float32, device=dev)
    yp = {n: torch.empty((PREFILL_T, specs[n].rows), dtype=torch.float32, device=dev) for n in names}
    yp_gu = torch.empty((PREFILL_T, 2, sg.rows), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    def dec_gate_up(i):
        binding.moe_gemv(reps[i]["gate_up"], xd_gu, ids_gu, y=yd_gu)

    def dec_pass(i):
        dec_gate_up(i)
        binding.gemv(reps[i]["down"], xd_dn, yd_dn)

    def dec_gate(i):
        binding.gemv(reps[i]["gate"], xd_gu, yd_g)

    def pre_gate(i):
        binding.gemm(reps[i]["gate"], xp_gu, yp["gate"])

    def pre_gate_up(i):
        binding.gemm(reps[i]["gate_up"], xp_gu, yp_gu)

    def pre_pass(i):
        pre_gate_up(i)
        binding.gemm(reps[i]["down"], xp_dn, yp["down"])

    if args.profile_gate:
        for i in range(4):
            dec_gate_up(i % REPLICAS)
        for i in range(4):
            dec_gate(i % REPLICAS)
        for i in range(2):
            pre_gate_up(i % REPLICAS)
        torch.cuda.synchronize()
        print("profile-gate: 4 gate+up routed GEMVs (T=1), 4 gate GEMVs (T=1), 2 gate+up stacked GEMMs "
              "(T=2048)", flush=True)
        return

    dec_bytes = {n: tensor_bytes(specs[n], DECODE_T) for n in names}
    pre_flops = {n: 2.0 * PREFILL_T * specs[n].rows * specs[n].cols for n in names}

    def ev():
        return torch.cuda.Event(enable_timing=True)

    # Decode: one graph per replica (for a remainder of steps) and one graph
    # of a pass over every replica in turn.  Prefill: one graph per replica.
    # Burst graphs of back-to-back launches rotating over the replicas give
    # the per-launch kernel durations for the rooflines.
    BURST = 2 * REPLICAS

    def capture(calls):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for fn, i in calls:
                fn(i)
        return g

    for i in range(REPLICAS):              # warm every code path eagerly first
        dec_pass(i)
        dec_gate(i)
        pre_pass(i)
        pre_gate(i)
    torch.cuda.synchronize()
    g_dec = [capture([(dec_pass, i)]) for i in range(REPLICAS)]
    g_dec_all = capture([(dec_pass, i) for i in range(REPLICAS)])
    g_pre = [capture([(pre_pass, i)]) for i in range(REPLICAS)]
    g_burst = {"gate_up": (capture([(dec_gate_up, i % REPLICAS) for i in range(BURST)]), BURST),
               "gate": (capture([(dec_gate, i % REPLICAS) for i in range(BURST)]), BURST),
               "gemm": (capture([(pre_gate_up, i) for i in range(REPLICAS)]), REPLICAS),
               "gemm_gate": (capture([(pre_gate, i) for i in range(REPLICAS)]), REPLICAS)}
    torch.cuda.synchronize()

    def decode_passes(n):
        full, rest = divmod(n, REPLICAS)
        for _ in range(full):
            g_dec_all.replay()
        for i in range(rest):
            g_dec[i].replay()

    def prefill_passes(n):
        for i in range(n):
            g_pre[i % REPLICAS].replay()

    decode_passes(args.warmup)
    prefill_passes(args.warmup)
    torch.cuda.synchronize()

    marks = [ev() for _ in range(4)]
    t0 = time.perf_counter()
    # A device-side spin (~0.4 ms) ahead of the first event keeps the GPU busy
    # while the host submits the first decode graph, so the decode block's
    # events time the kernels, not that submission (it is in the wall time).
    torch.cuda._sleep(1_000_000)
    marks[0].record()
    decode_passes(args.steps)
    marks[1].record()
    marks[2].record()
    prefill_passes(args.steps)
    marks[3].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # per-launch durations of the dominant kernels (inside the timed process,
    # same stream, back-to-back launches as in the steps): median of 5 burst
    # replays
    bursts = {}
    for key, (g, count) in g_burst.items():
        times = []
        for _ in range(5):
            a, b = ev(), ev()
            torch.cuda._sleep(1_000_000)   # the GPU is busy while the graph is submitted
            a.record()
            g.replay()
            b.record()
            torch.cuda.synchronize()
            times.append(a.elapsed_time(b) * 1e-3 / count)
        bursts[key] = sorted(times)[2]

    dec_time = marks[0].elapsed_time(marks[1]) * 1e-3
    pre_time = marks[2].elapsed_time(marks[3]) * 1e-3
    dec_gbps = sum(dec_bytes.values()) * args.steps / dec_time / 1e9
    pre_tflops = sum(pre_flops.values()) * args.steps / pre_time / 1e12

    gu_bytes = dec_bytes["gate"] + dec_bytes["up"]
    gu_gbps = gu_bytes / bursts["gate_up"] / 1e9
    gate_gbps = dec_bytes["gate"] / bursts["gate"] / 1e9
    gu_tflops = (pre_flops["gate"] + pre_flops["up"]) / bursts["gemm"] / 1e12
    # the stacked launch reads x once and writes both outputs
    gu_pre_bytes = 2 * tensor_bytes(sg, PREFILL_T) - PREFILL_T * sg.cols * 2

    out = {
        "metric": "VQ-GEMV effective HBM GB/s (% of peak) at batch 1; prefill VQ-GEMM TFLOP/s",
        "value": round(dec_gbps, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic",
        "config": {"workload": WORKLOAD, "decode_tokens": DECODE_T, "prefill_tokens": PREFILL_T,
                   "tensors": "gate,up [17408x5120]; down [5120x17408]; d=2 K=256 group=64 (4.25 bpw)",
                   "decode_calls": "gate+up: one routed GEMV over the two-expert stack, ids {0,1}; down: GEMV",
                   "prefill_calls": "gate+up: one GEMM over the two-expert stack; down: GEMM",
                   "weight_replicas": REPLICAS, "parallelism": "single GPU"},
        "pct_of_hbm_peak": round(100 * dec_gbps / HBM_PEAK_GBPS, 2),
        "decode_ms_per_step": round(dec_time / args.steps * 1e3, 4),
        "prefill": {"value": round(pre_tflops, 2), "unit": "TFLOP/s",
                    "pct_of_fp16_mfma_peak": round(100 * pre_tflops / MFMA_F16_PEAK_TFLOPS, 2),
                    "ms_per_step": round(pre_time / args.steps * 1e3, 4)},
        "kernel_us": {"gemv_gate_up_T1": round(bursts["gate_up"] * 1e6, 2),
                      "gemv_gate_T1": round(bursts["gate"] * 1e6, 2),
                      "gemm_gate_up_T2048": round(bursts["gemm"] * 1e6, 2),
                      "gemm_gate_T2048": round(bursts["gemm_gate"] * 1e6, 2)},
        "roofline": {"bound": "hbm", "kernel": "vq_moe_gemv over the gate+up stack (T=1, ids {0,1})",
                     "achieved": round(gu_gbps, 2), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(gu_gbps / HBM_PEAK_GBPS, 4),
                     "traffic": measured_traffic("vq_gemv_kernel<2, 8, 64, 5, 2, true,", GATE_TAG),
                     "algorithmic_bytes": gu_bytes},
        "roofline_single_tensor": {"bound": "hbm", "kernel": "vq_gemv (gate, T=1)",
                                   "achieved": round(gate_gbps, 2), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                                   "frac": round(gate_gbps / HBM_PEAK_GBPS, 4),
                                   "traffic": measured_traffic("vq_gemv_kernel<2, 8, 64, 5, 2, false,", GATE_TAG),
                                   "algorithmic_bytes": dec_bytes["gate"]},
        "roofline_prefill": {"bound": "mfma", "kernel": "vq_gemm over the gate+up stack (T=2048)",
                             "achieved": round(gu_tflops, 2), "peak": MFMA_F16_PEAK_TFLOPS,
                             "unit": "TFLOP/s", "frac": round(gu_tflops / MFMA_F16_PEAK_TFLOPS, 4),
                             "traffic": measured_traffic("vq_gemm_kernel<2, 8, 64", GATE_TAG),
                             "algorithmic_bytes": gu_pre_bytes},
    }
    if not args.no_sweep:
        # config 4 (the 17408x5120 / 5120x17408 d=4 K=256 sweep): its barred
        # points, GEMV at T = 1 and GEMM at T = 4096, on the same GPU
        del reps, g_dec, g_dec_all, g_pre, g_burst
        torch.cuda.empty_cache()
        out["roofline_sweep_config"] = sweep_rooflines()
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(host["gate"], specs["gate"], args.cpu_rows)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
