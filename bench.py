#!/usr/bin/env python3
"""Benchmark of the fused GEMM -> residual -> RMSNorm -> GEMM chain on one MI355X.

One step = the fused forward (coda_fwd) and the fused backward (coda_bwd, on the
forward's saved h, g, y, r) at the Llama-3-8B layer shape: M = 8192 tokens,
K0 = D = 4096, N = 28672 (ffn 14336, gate/up interleaved), bf16 storage, fp32
accumulation, eps = 1e-5. Inputs are seeded synthetic tensors with the value
distributions of the parity tests, already resident in HBM when timing starts.

Prints ONE JSON line on stdout (everything else goes to stderr):
  value     = algorithmic TFLOP per step / seconds per step (forward 2MK0D + 2MDN,
              backward 4MDN; epilogue arithmetic is not counted),
  roofline  = the longest kernel of the step against the bf16 dense MFMA peak,
              its duration from HIP events recorded around it on its stream in a
              second, instrumented pass of the same K steps (the headline steps
              carry events only at the two ends of the timed region),
  cpu_baseline = the fp64 oracle timed on a bounded sample of the same workload,
  unfused, configs = each fused pass against its unfused baseline (and the tiny,
              Llama-3 1B and 70B forwards), the two timed in alternating blocks so
              that both run at the same power-limited clock.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # 256 CU x 2.4 GHz x 4096 dense bf16 flop/clk/CU (MI355X)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
METRIC = "fused GEMM-Res-RMSNorm-GEMM TFLOP/s & % bf16 MFMA peak, Llama-3-8B shape"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def stage_work(M, K0, D, N):
    """Per-launch algorithmic work: ('flop', F) for MFMA kernels, ('byte', B) for HBM-bound ones. With at
    least 16 of the dW1 GEMM's 256-row tiles (D > 3840) s comes from that GEMM's side work, as partials
    [2 ceil(N / 256), M] that the s stage adds up; otherwise the s stage is a row kernel over dY and y."""
    ceil = lambda a, b: -(-a // b)
    rowdot = ceil(D, 256) >= 16
    return {
        "gemm0_residual_ssq": ("flop", 2 * M * K0 * D),
        "rms_combine": ("byte", M * ceil(D, 256) * 4 + M * 4),
        "gemm1_rowscale": ("flop", 2 * M * D * N),
        "gr_transpose": ("byte", M * D * 2 + M * 4 + D * ceil(M, 64) * 64 * 2),
        "wgrad_rowdot": ("flop", 2 * M * D * N),
        "s_combine": ("byte", (2 * ceil(N, 256) * M * 4 if rowdot else 2 * M * N * 2) + M * 4),
        "dgrad_rmsnorm_bwd": ("flop", 2 * M * N * D),
        "dgamma_combine": ("byte", ceil(M, 128) * D * 4 + D * 4),
    }


def _code_only(src: str) -> str:
    """C/C++ source without its comments and with runs of whitespace collapsed (string and character
    literals kept as they are), so that editing a comment does not change the digest."""
    out, i, n = [], 0, len(src)
    while i < n:
        c = src[i]
        if c in "\"'":
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        elif src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def kernel_source_digest(d=None) -> str:
    """sha256 over the code (comments and whitespace aside) of the sources the device code is built from;
    it identifies a counter measurement. The host-only validation in coda_host.cpp is left out."""
    import hashlib
    d = d or os.path.join(ROOT, "transformer_gemm_epilogue_res_amd", "csrc")
    h = hashlib.sha256()
    for name in sorted(os.listdir(d)):
        if name.endswith((".hip", ".hpp", ".h")):
            h.update(name.encode())
            h.update(_code_only(open(os.path.join(d, name), encoding="utf-8").read()).encode())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str):
    """HBM bytes per launch of `kernel` from profiles/hbm_traffic_llama3_8b.md (FETCH_SIZE and WRITE_SIZE
    passes, each scaled by the same counter's reading for a plain copy of known size), or None when that
    measurement was taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic_llama3_8b.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    try:
        blob = json.loads(text.split("```json", 1)[1].split("```", 1)[0])
    except (IndexError, ValueError):
        return None
    if blob.get("source_digest") != kernel_source_digest():
        return None
    k = blob.get("kernels", {}).get(kernel)
    return None if k is None else k["bytes_per_launch"]


def _quantiles(v, qs):
    import numpy as np
    return np.quantile(np.asarray(v, dtype=np.float64), qs)


def measured_sclk(kernel: str):
    """Shader clock (GHz) of `kernel` from profiles/sclk_llama3_8b.md (GRBM_GUI_ACTIVE over the 8 XCDs /
    dispatch duration), or None when that measurement was taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", "sclk_llama3_8b.md")
    if not os.path.exists(path):
        return None
    try:
        blob = json.loads(open(path).read().split("```json", 1)[1].split("```", 1)[0])
    except (IndexError, ValueError):
        return None
    if blob.get("source_digest") != kernel_source_digest():
        return None
    return blob.get("kernels", {}).get(kernel)


def measured_mfma_busy(kernel: str):
    """Fraction of the kernel's active cycles in which the SIMDs' matrix units are busy, from
    profiles/mfma_busy_llama3_8b.md (SQ_VALU_MFMA_BUSY_CYCLES over GRBM_GUI_ACTIVE x 1024 SIMDs), or None
    when that measurement was taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", "mfma_busy_llama3_8b.md")
    if not os.path.exists(path):
        return None
    try:
        blob = json.loads(open(path).read().split("```json", 1)[1].split("```", 1)[0])
    except (IndexError, ValueError):
        return None
    if blob.get("source_digest") != kernel_source_digest():
        return None
    k = blob.get("kernels", {}).get(kernel)
    return None if k is None else k["mfma_busy"]


def cpu_baseline(host, rows, ncols, total_rows, seed=0):
    """Time the fp64 oracle (as it is) on a sub-batch of sampled rows of the workload."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_info

    from oracle import coda_oracle as orc
    from transformer_gemm_epilogue_res_amd import inputs

    M, K0 = host["x"].shape
    D, N = host["W1"].shape
    R = len(rows)
    eps = inputs.EPS
    t0 = time.perf_counter()
    f = orc.forward(host["x"], host["W0"], host["z"], host["gamma"], host["W1"], eps)
    t1 = time.perf_counter()
    # the sub-batch's saved set in its storage types (outside the timing)
    gam = orc.f64(host["gamma"])
    h_s = torch.from_numpy(f["h"]).to(torch.bfloat16)
    g_s = torch.from_numpy(f["h"] * gam[None, :]).to(torch.bfloat16)
    y_s = torch.from_numpy(f["y"]).to(torch.bfloat16)
    r_s = torch.from_numpy(f["r"]).to(torch.float32)
    jc = None if ncols <= 0 else inputs.sample(D, ncols, seed, "dgamma_cols").numpy()
    nc = None if ncols <= 0 else inputs.sample(N, ncols, seed, "dw1_cols").numpy()
    cj, cn = (D, N) if ncols <= 0 else (ncols, ncols)
    t2 = time.perf_counter()
    orc.backward(host["dY"], y_s, h_s, g_s, r_s, host["gamma"], host["W1"], dgamma_cols=jc, dw1_cols=nc)
    t3 = time.perf_counter()
    # priced at the step's algorithmic work on this sub-batch (forward 2RK0D + 2RDN, backward 4RDN, the
    # same count as the GPU value), not at the oracle's own arithmetic (it recomputes G for dgamma)
    executed = 2 * R * (K0 * D + D * N) + 2 * R * N * D + 2 * R * N + 2 * R * N * cj + 2 * R * D * cn
    flops = 2 * R * (K0 * D + D * N) + 4 * R * D * N if ncols <= 0 else executed
    secs = (t1 - t0) + (t3 - t2)
    threads = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [1])
    what = "all" if ncols <= 0 else f"{ncols} sampled"
    return {"value": flops / secs / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": (f"fp64 numpy oracle on {R} of the 8B workload's {total_rows} rows: forward of those rows, then "
                       f"the backward of that {R}-row batch (s, G, da for every row; dgamma and dW1 on "
                       f"{what} columns); {flops / 1e9:.1f} GFLOP of the step's algorithmic work "
                       f"({executed / 1e9:.1f} GFLOP executed) in {secs:.2f} s"),
            "seconds": secs, "algorithmic_gflop": flops / 1e9, "executed_gflop": executed / 1e9,
            "cpu": platform.processor() or platform.machine(), "nproc": os.cpu_count()}


def oracle_configs(gpu, rows_per_cfg=256):
    """The oracle's forward timed on each configuration's seeded row sample (every row of the tiny one): rows/s
    and the extrapolated full-M time (rows are independent), and the GPU forward's error on those rows (its fp32
    y against the oracle's y: max|d| / rms; r: max relative)."""
    import numpy as np
    import torch

    from oracle import coda_oracle as orc
    from transformer_gemm_epilogue_res_amd import inputs

    out = {}
    for name, g in gpu.items():
        host, rows, M = g["host"], g["rows"], g["M"]
        t0 = time.perf_counter()
        f = orc.forward(host["x"], host["W0"], host["z"], host["gamma"], host["W1"], inputs.EPS)
        secs = time.perf_counter() - t0
        y = g["y32"].double().numpy()
        e_y = float(np.abs(y - f["y"]).max() / np.sqrt((f["y"] ** 2).mean()))
        e_r = float(np.abs(g["r"].double().numpy() / f["r"] - 1).max())
        R = len(rows)
        out[name] = {"rows": R, "seconds": round(secs, 4), "rows_per_s": round(R / secs, 1),
                     "extrapolated_full_s": round(secs * M / R, 3), "y_err_max_over_rms": e_y, "r_err_max_rel": e_r}
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-rows", type=int, default=8192, help="rows in the oracle's timed sample (0 = skip)")
    ap.add_argument("--cpu-cols", type=int, default=0,
                    help="dgamma / dW1 columns in the oracle's timed sample (0 = all)")
    ap.add_argument("--no-unfused", action="store_true", help="skip timing the unfused baseline")
    ap.add_argument("--no-swiglu", action="store_true", help="skip timing the SwiGLU block")
    ap.add_argument("--no-ce", action="store_true", help="skip timing the cross-entropy LM head")
    ap.add_argument("--no-cold", action="store_true", help="skip the cold-cache variant of the step")
    ap.add_argument("--no-shard", action="store_true", help="skip the data-parallel shard (M / 8) step")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the tiny, Llama-3 1B and Llama-3 70B forward configurations")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="before timing, run 3 plain device copies of this many bytes (a reference kernel of "
                         "known traffic for scaling hardware byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}): the chain's kernels run on a single "
              "device; there is no multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    import torch

    from transformer_gemm_epilogue_res_amd import _lib as L
    from transformer_gemm_epilogue_res_amd import inputs

    c = inputs.CONFIGS["llama3_8b"]
    M, K0, D, N = c["M"], c["K0"], c["D"], c["N"]
    dev = "cuda:0"
    torch.cuda.set_device(0)
    bf = torch.bfloat16
    log(f"[bench] llama3_8b M={M} K0={K0} D={D} N={N}: generating inputs on {dev}")
    gen = torch.Generator(device=dev)
    gen.manual_seed(0)

    def rnd(*shape, scale=1.0, shift=0.0):
        return (torch.randn(*shape, generator=gen, device=dev) * scale + shift).to(bf)

    x, W0 = rnd(M, K0), rnd(K0, D, scale=K0 ** -0.5)
    z, gamma = rnd(M, D), rnd(D, scale=0.1, shift=1.0)
    W1, dY = rnd(D, N, scale=D ** -0.5), rnd(M, N)
    fo = {"h": torch.empty(M, D, dtype=bf, device=dev), "g": torch.empty(M, D, dtype=bf, device=dev),
          "r": torch.empty(M, dtype=torch.float32, device=dev), "y": torch.empty(M, N, dtype=bf, device=dev)}
    bo = {"da": torch.empty(M, D, dtype=bf, device=dev), "dgamma": torch.empty(D, dtype=torch.float32, device=dev),
          "dW1": torch.empty(D, N, dtype=bf, device=dev), "s": torch.empty(M, dtype=torch.float32, device=dev)}
    fws = L.workspace(L.CODA_OP_FWD, M, D, N, dev)
    bws = L.workspace(L.CODA_OP_BWD, M, D, N, dev)
    F = L.bind_fwd(x, W0, z, gamma, W1, inputs.EPS, fo, fws)
    B = L.bind_bwd(dY, fo["y"], fo["h"], fo["g"], fo["r"], gamma, W1, bo, bws)
    stream = torch.cuda.current_stream(dev)
    sp = L.current_stream(dev)
    names = list(L.FWD_STAGE_NAMES) + list(L.BWD_STAGE_NAMES)

    def paired_ms(a, b, calls, rounds=5):
        """Mean ms per call of a() and of b(), timed in alternating blocks of calls / rounds calls each
        (events at the block ends only), so that both run in the same power and thermal state: under
        the socket power cap the clock a kernel gets depends on what ran before it, and timing one
        chain after another section of the bench would compare two different clocks."""
        reps = max(1, -(-calls // rounds))
        for f in (a, b, a, b):
            f()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(rounds)]
        for e in ev:
            e[0].record(stream)
            for _ in range(reps):
                a()
            e[1].record(stream)
            for _ in range(reps):
                b()
            e[2].record(stream)
        torch.cuda.synchronize()
        return (sum(e[0].elapsed_time(e[1]) for e in ev) / (rounds * reps),
                sum(e[1].elapsed_time(e[2]) for e in ev) / (rounds * reps))

    if args.copy_bytes > 0:
        src = torch.empty(args.copy_bytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] reference copy: 3 x {args.copy_bytes} bytes read + written")
        del src, dst

    log(f"[bench] warmup {args.warmup} steps")
    for _ in range(args.warmup):
        F.run(sp)
        B.run(sp)
    torch.cuda.synchronize()

    # The timed region: K whole steps back to back, HIP events only at its two ends (no
    # marker between the step's kernels; under the profiler each one delays the next dispatch).
    log(f"[bench] timing {args.steps} steps")
    t_a, t_b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    t_a.record(stream)
    for _ in range(args.steps):
        F.run(sp)
        B.run(sp)
    t_b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms_step = t_a.elapsed_time(t_b) / args.steps    # whole timed region / steps

    # The same K steps again, instrumented: an event after every stage gives the per-stage
    # (per-kernel) durations, the dominant kernel's roofline figures and the per-step spread.
    log(f"[bench] per-stage timing: {args.steps} more steps with an event after each stage")
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for k in range(args.steps):
        e = ev[k]
        e[0].record(stream)
        for i in range(F.nstages):
            F.stage(i, sp)
            e[1 + i].record(stream)
        for i in range(B.nstages):
            B.stage(i, sp)
            e[1 + F.nstages + i].record(stream)
    torch.cuda.synchronize()
    per = {n: 0.0 for n in names}
    step_ms = []
    for e in ev:
        for i, n in enumerate(names):
            per[n] += e[i].elapsed_time(e[i + 1])
        step_ms.append(e[0].elapsed_time(e[-1]))
    per = {n: v / args.steps for n, v in per.items()}          # ms per launch
    ms_instrumented = ev[0][0].elapsed_time(ev[-1][-1]) / args.steps

    # The forward and the backward each alone (events at block ends only), each paired with the unfused
    # baseline of the same pass: the unfused forward writes the same h, r, y (no g) and the unfused
    # backward reads the fused forward's saved set.
    unfused = None
    if args.no_unfused:
        fwd_ms = paired_ms(lambda: F.run(sp), lambda: None, args.steps)[0]
        bwd_ms = paired_ms(lambda: B.run(sp), lambda: None, args.steps)[0]
    else:
        log("[bench] timing the fused forward and backward, each alternating with the unfused baseline")
        uF = L.bind_fwd(x, W0, z, gamma, W1, inputs.EPS, dict(fo, g=None),
                        L.workspace(L.CODA_OP_UNFUSED_FWD, M, D, N, dev))
        uB = L.bind_bwd(dY, fo["y"], fo["h"], fo["g"], fo["r"], gamma, W1, bo,
                        L.workspace(L.CODA_OP_UNFUSED_BWD, M, D, N, dev))
        fwd_ms, ufwd_ms = paired_ms(lambda: F.run(sp), lambda: uF.run(sp, unfused=True), args.steps)
        bwd_ms, ubwd_ms = paired_ms(lambda: B.run(sp), lambda: uB.run(sp, unfused=True), args.steps)
        unfused = {"fwd_ms": round(ufwd_ms, 4), "bwd_ms": round(ubwd_ms, 4),
                   "fused_fwd_speedup": round(ufwd_ms / fwd_ms, 3), "fused_bwd_speedup": round(ubwd_ms / bwd_ms, 3)}
        log(f"[bench] unfused fwd {ufwd_ms:.3f} ms, bwd {ubwd_ms:.3f} ms")
        del uF, uB
    fwd_flop = 2 * M * K0 * D + 2 * M * D * N
    bwd_flop = 4 * M * D * N
    value = (fwd_flop + bwd_flop) / (ms_step * 1e-3) / 1e12
    work = stage_work(M, K0, D, N)
    kernels = {}
    for n in names:
        kind, amount = work[n]
        rate = amount / (per[n] * 1e-3)
        kernels[n] = {"us": round(per[n] * 1e3, 2),
                      ("tflops" if kind == "flop" else "gbps"): round(rate / (1e12 if kind == "flop" else 1e9), 1)}
    dom = max(names, key=lambda n: per[n])
    dk, damount = work[dom]
    if dk == "flop":
        ach = damount / (per[dom] * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(ach / PEAK_BF16_TFLOPS, 4), "traffic": measured_traffic(dom), "kernel": dom,
                "per_launch": f"{damount / 1e12:.4f} TFLOP", "avg_us": round(per[dom] * 1e3, 1)}
        clk = measured_sclk(dom)   # the power-limited clock the kernel runs at (2.4 GHz is the peak's)
        roof["sclk_ghz"] = clk
        roof["frac_at_sclk"] = None if clk is None else round(ach / (PEAK_BF16_TFLOPS * clk / 2.4), 4)
        roof["mfma_busy"] = measured_mfma_busy(dom)
    else:
        ach = damount / (per[dom] * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": measured_traffic(dom), "kernel": dom,
                "per_launch": f"{damount / 1e9:.3f} GB", "avg_us": round(per[dom] * 1e3, 1)}
    log(f"[bench] step {ms_step:.3f} ms (wall {wall / args.steps * 1e3:.3f} ms), {value:.1f} TFLOP/s; "
        f"fwd {fwd_ms:.3f} ms, bwd {bwd_ms:.3f} ms")
    for n in names:
        log(f"[bench]   {n:20s} {kernels[n]}")

    # Cold-cache variant: before each step a 512 MB scratch write evicts the 256 MB Infinity
    # Cache (outside the timed region; events bracket the step only).
    cold = None
    if not args.no_cold:
        scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        cms = []
        for _ in range(args.steps):
            scratch.fill_(1)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            F.run(sp)
            B.run(sp)
            b.record(stream)
            torch.cuda.synchronize()
            cms.append(a.elapsed_time(b))
        del scratch
        med = float(_quantiles(cms, (0.5,))[0])
        cold = {"ms_per_step_median": round(med, 4), "tflops": round((fwd_flop + bwd_flop) / med / 1e9, 1)}
        log(f"[bench] cold-cache step (median) {med:.3f} ms, {cold['tflops']} TFLOP/s")

    # One GPU's share of the batch under 8-way data parallelism (M / 8 rows): the same step at
    # the shard's shape, where GEMM0 and dgrad split their contraction.
    shard = None
    if not args.no_shard:
        Ms = M // 8
        xs, zs, dYs = x[:Ms].contiguous(), z[:Ms].contiguous(), dY[:Ms].contiguous()
        sfo = {k: v[:Ms].contiguous() for k, v in fo.items()}
        sbo = {"da": bo["da"][:Ms].contiguous(), "dgamma": bo["dgamma"], "dW1": bo["dW1"], "s": bo["s"][:Ms].contiguous()}
        SF = L.bind_fwd(xs, W0, zs, gamma, W1, inputs.EPS, sfo, L.workspace(L.CODA_OP_FWD, Ms, D, N, dev))
        SBk = L.bind_bwd(dYs, sfo["y"], sfo["h"], sfo["g"], sfo["r"], gamma, W1, sbo,
                         L.workspace(L.CODA_OP_BWD, Ms, D, N, dev))
        for _ in range(2):
            SF.run(sp)
            SBk.run(sp)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(args.steps):
            SF.run(sp)
            SBk.run(sp)
        b.record(stream)
        torch.cuda.synchronize()
        sms = a.elapsed_time(b) / args.steps
        sfl = 2 * Ms * K0 * D + 6 * Ms * D * N
        shard = {"M": Ms, "ms_per_step": round(sms, 4), "tflops": round(sfl / sms / 1e9, 1),
                 "pct_peak": round(100 * sfl / sms / 1e9 / PEAK_BF16_TFLOPS, 2)}
        log(f"[bench] data-parallel shard (M = {Ms}): step {sms:.3f} ms, {shard['tflops']} TFLOP/s")
        del xs, zs, dYs, sfo, sbo, SF, SBk

    # The backward through the first GEMM (dx, dW0 from the step's bf16 da): not part
    # of the headline step (the chain's metric stops at da), reported beside it.
    g0o = {"dx": torch.empty(M, K0, dtype=bf, device=dev), "dW0": torch.empty(K0, D, dtype=bf, device=dev)}
    G0 = L.BoundGemm0(bo["da"], x, W0, g0o)
    for _ in range(2):
        G0.run(sp)
    a0, b0 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a0.record(stream)
    for _ in range(args.steps):
        G0.run(sp)
    b0.record(stream)
    torch.cuda.synchronize()
    g0_ms = a0.elapsed_time(b0) / args.steps
    g0_flop = 2 * 2 * M * K0 * D
    bwd_gemm0 = {"ms": round(g0_ms, 4), "tflops": round(g0_flop / g0_ms / 1e9, 1),
                 "pct_peak": round(100 * g0_flop / g0_ms / 1e9 / PEAK_BF16_TFLOPS, 2)}
    log(f"[bench] backward through GEMM0 (dx, dW0): {g0_ms:.3f} ms, {bwd_gemm0['tflops']} TFLOP/s")

    # The SwiGLU block on the chain (coda_fwd_swiglu / coda_bwd_swiglu with the
    # output projection W2 [N/2, D]): reported beside the headline step.
    swiglu = None
    if not args.no_swiglu:
        Fh, E = N // 2, D
        W2, dOut = rnd(Fh, E, scale=Fh ** -0.5), rnd(M, E)
        so = dict(fo, o=torch.empty(M, Fh, dtype=bf, device=dev))
        sbo = dict(bo, dY=torch.empty(M, N, dtype=bf, device=dev), dW2=torch.empty(Fh, E, dtype=bf, device=dev))
        SF = L.bind_fwd_swiglu(x, W0, z, gamma, W1, inputs.EPS, so, fws)
        SB = L.bind_bwd_swiglu(dOut, W2, so["o"], so["y"], so["h"], so["g"], so["r"], gamma, W1, sbo,
                               L.workspace(L.CODA_OP_BWD_SWIGLU, M, D, N, dev))
        USB = L.bind_bwd_swiglu(dOut, W2, so["o"], so["y"], so["h"], so["g"], so["r"], gamma, W1, sbo,
                                L.workspace(L.CODA_OP_UNFUSED_BWD_SWIGLU, M, D, N, dev))
        t = {}
        t["fwd"], t["ufwd"] = paired_ms(lambda: SF.run(sp), lambda: SF.run(sp, unfused=True), args.steps)
        t["bwd"], t["ubwd"] = paired_ms(lambda: SB.run(sp), lambda: USB.run(sp, unfused=True), args.steps)
        s_bwd_flop = bwd_flop + 2 * 2 * M * Fh * E   # + dO = dOut W2^T and dW2 = o^T dOut
        swiglu = {"E": E, "fwd_ms": round(t["fwd"], 4), "bwd_ms": round(t["bwd"], 4),
                  "fwd_tflops": round(fwd_flop / t["fwd"] / 1e9, 1),
                  "bwd_tflops": round(s_bwd_flop / t["bwd"] / 1e9, 1),
                  "tflops": round((fwd_flop + s_bwd_flop) / (t["fwd"] + t["bwd"]) / 1e9, 1)}
        swiglu["pct_peak"] = round(100 * swiglu["tflops"] / PEAK_BF16_TFLOPS, 2)
        # the baseline unfuses only the activation step (the chain under it is the fused one)
        swiglu["activation_unfused"] = {"fwd_ms": round(t["ufwd"], 4), "bwd_ms": round(t["ubwd"], 4),
                                        "fused_fwd_speedup": round(t["ufwd"] / t["fwd"], 3),
                                        "fused_bwd_speedup": round(t["ubwd"] / t["bwd"], 3)}
        log(f"[bench] SwiGLU block: fwd {t['fwd']:.3f} ms, bwd {t['bwd']:.3f} ms, {swiglu['tflops']} TFLOP/s; "
            f"with the activation step unfused: fwd {t['ufwd']:.3f} ms, bwd {t['ubwd']:.3f} ms")
        del W2, dOut, so, sbo, SF, SB, USB

    # Cross-entropy on the Llama-3-8B LM head (coda_ce_fwd / coda_ce_bwd, V = 128256):
    # reported beside the headline step.
    ce = None
    if not args.no_ce:
        V = inputs.LM_VOCAB
        hl, Wl = rnd(M, D), rnd(V, D, scale=2.0 / D ** 0.5)
        tg = torch.randint(0, V, (M,), generator=gen, device=dev)
        dloss = torch.randn(M, generator=gen, device=dev)
        cfo = {"lse": torch.empty(M, dtype=torch.float32, device=dev),
               "loss": torch.empty(M, dtype=torch.float32, device=dev)}
        cbo = {"dlogits": torch.empty(M, V, dtype=bf, device=dev), "dh": torch.empty(M, D, dtype=bf, device=dev),
               "dW": torch.empty(V, D, dtype=bf, device=dev)}
        CF = L.bind_ce_fwd(hl, Wl, tg, cfo, L.workspace(L.CODA_OP_CE_FWD, M, D, V, dev))
        CB = L.bind_ce_bwd(hl, Wl, tg, cfo["lse"], dloss, cbo)
        # the forward storing its fp32 logits [M, V] and the backward reading them
        lg = torch.empty(M, V, dtype=torch.float32, device=dev)
        cso = {k: torch.empty_like(v) for k, v in cfo.items()}
        CFS = L.bind_ce_fwd(hl, Wl, tg, cso, L.workspace(L.CODA_OP_CE_FWD, M, D, V, dev), logits=lg)
        CBS = L.bind_ce_bwd(hl, Wl, tg, cso["lse"], dloss, cbo, logits=lg)
        # the unfused baseline stores the fp32 logits [M, V] in its workspace
        uws = None if args.no_unfused else L.workspace(L.CODA_OP_UNFUSED_CE_FWD, M, D, V, dev)
        t = {}
        # each variant alternating with the fused (recomputing) pass: fwd / bwd pair with stored logits,
        # then with the unfused baseline; the fused times are the mean of their pairings
        t["fwd"], t["sfwd"] = paired_ms(lambda: CF.run(sp), lambda: CFS.run(sp), args.steps)
        t["bwd"], t["sbwd"] = paired_ms(lambda: CB.run(sp), lambda: CBS.run(sp), args.steps)
        if uws is not None:
            f2, t["ufwd"] = paired_ms(lambda: CF.run(sp), lambda: CF.run(sp, unfused_ws=uws), args.steps)
            b2, t["ubwd"] = paired_ms(lambda: CB.run(sp), lambda: CB.run(sp, unfused_ws=uws), args.steps)
            t["fwd"], t["bwd"] = (t["fwd"] + f2) / 2, (t["bwd"] + b2) / 2
        ce_f, ce_b = 2 * M * D * V, 3 * 2 * M * D * V   # logits; recomputed logits, dh, dW
        ce = {"V": V, "fwd_ms": round(t["fwd"], 4), "bwd_ms": round(t["bwd"], 4),
              "fwd_tflops": round(ce_f / t["fwd"] / 1e9, 1), "bwd_tflops": round(ce_b / t["bwd"] / 1e9, 1),
              "tflops": round((ce_f + ce_b) / (t["fwd"] + t["bwd"]) / 1e9, 1)}
        ce["pct_peak"] = round(100 * ce["tflops"] / PEAK_BF16_TFLOPS, 2)
        log(f"[bench] cross-entropy LM head: fwd {t['fwd']:.3f} ms, bwd {t['bwd']:.3f} ms, {ce['tflops']} TFLOP/s")
        ce["stored_logits"] = {"fwd_ms": round(t["sfwd"], 4), "bwd_ms": round(t["sbwd"], 4),
                               "logits_gb": round(M * V * 4 / 1e9, 2),
                               "speedup_vs_recompute": round((t["fwd"] + t["bwd"]) / (t["sfwd"] + t["sbwd"]), 3)}
        log(f"[bench] cross-entropy with stored fp32 logits ({M * V * 4 / 1e9:.1f} GB): fwd {t['sfwd']:.3f} ms, "
            f"bwd {t['sbwd']:.3f} ms")
        if uws is not None:
            ce["unfused"] = {"fwd_ms": round(t["ufwd"], 4), "bwd_ms": round(t["ubwd"], 4),
                             "fused_fwd_speedup": round(t["ufwd"] / t["fwd"], 3),
                             "fused_bwd_speedup": round(t["ubwd"] / t["bwd"], 3)}
            log(f"[bench] unfused cross-entropy (stored fp32 logits): fwd {t['ufwd']:.3f} ms, "
                f"bwd {t['ubwd']:.3f} ms")
        del hl, Wl, tg, dloss, cfo, cbo, CF, CB, uws, lg, cso, CFS, CBS

    # The other forward configurations (tiny, Llama-3 1B, Llama-3 70B), fused against the unfused baseline,
    # reported beside the headline; one fp32-y forward per configuration gives its error on sampled rows.
    configs, cfg_gpu = None, {}
    if not args.no_configs:
        configs = {}
        for name in ("tiny", "llama3_1b", "llama3_70b"):
            cc = inputs.CONFIGS[name]
            Mc, K0c, Dc, Nc = cc["M"], cc["K0"], cc["D"], cc["N"]
            gc = torch.Generator(device=dev)
            gc.manual_seed(1)

            def rndc(*shape, scale=1.0, shift=0.0):
                return (torch.randn(*shape, generator=gc, device=dev) * scale + shift).to(bf)

            xc, W0c, zc = rndc(Mc, K0c), rndc(K0c, Dc, scale=K0c ** -0.5), rndc(Mc, Dc)
            gmc, W1c = rndc(Dc, scale=0.1, shift=1.0), rndc(Dc, Nc, scale=Dc ** -0.5)
            foc = {"h": torch.empty(Mc, Dc, dtype=bf, device=dev), "g": torch.empty(Mc, Dc, dtype=bf, device=dev),
                   "r": torch.empty(Mc, dtype=torch.float32, device=dev), "y": torch.empty(Mc, Nc, dtype=bf, device=dev)}
            FC = L.bind_fwd(xc, W0c, zc, gmc, W1c, inputs.EPS, foc, L.workspace(L.CODA_OP_FWD, Mc, Dc, Nc, dev))
            UC = L.bind_fwd(xc, W0c, zc, gmc, W1c, inputs.EPS, dict(foc, g=None),
                            L.workspace(L.CODA_OP_UNFUSED_FWD, Mc, Dc, Nc, dev))
            reps = args.steps if Mc * Nc * Dc > 1 << 30 else 200   # the tiny one: enough calls to time
            tc = {}
            tc["fused"], tc["unfused"] = paired_ms(lambda: FC.run(sp), lambda: UC.run(sp, unfused=True), reps)
            flc = 2 * Mc * K0c * Dc + 2 * Mc * Dc * Nc
            configs[name] = {"M": Mc, "K0": K0c, "D": Dc, "N": Nc, "gflop": round(flc / 1e9, 3),
                             "fused_ms": round(tc["fused"], 5), "unfused_ms": round(tc["unfused"], 5),
                             "fused_tflops": round(flc / tc["fused"] / 1e9, 1),
                             "pct_peak": round(100 * flc / tc["fused"] / 1e9 / PEAK_BF16_TFLOPS, 2),
                             "unfused_tflops": round(flc / tc["unfused"] / 1e9, 1),
                             "fused_vs_unfused": round(tc["unfused"] / tc["fused"], 3)}
            log(f"[bench] {name} forward: fused {tc['fused'] * 1e3:.1f} us ({configs[name]['fused_tflops']} TFLOP/s), "
                f"unfused {tc['unfused'] * 1e3:.1f} us")
            if args.cpu_rows > 0:   # one fp32-y forward for the error on the oracle's rows (cpu_baseline leg)
                rows = torch.arange(Mc) if Mc <= 256 else inputs.sample(Mc, 256, 0, "rows")
                y32 = L.fwd(xc, W0c, zc, gmc, W1c, inputs.EPS, torch.float32)
                ri = rows.to(dev)
                cfg_gpu[name] = {"M": Mc, "rows": rows.numpy(), "y32": y32["y"].index_select(0, ri).cpu(),
                                 "r": y32["r"].index_select(0, ri).cpu(),
                                 "host": {"x": xc.index_select(0, ri).cpu(), "z": zc.index_select(0, ri).cpu(),
                                          "W0": W0c.cpu(), "gamma": gmc.cpu(), "W1": W1c.cpu()}}
                del y32
            del xc, W0c, zc, gmc, W1c, foc, FC, UC
            torch.cuda.empty_cache()

    cpu = None
    if args.cpu_rows > 0 and configs is not None:
        log("[bench] oracle forward on each configuration's row sample")
        for name, o in oracle_configs(cfg_gpu).items():
            configs[name]["oracle"] = o
            log(f"[bench]   {name}: {o}")
    if args.cpu_rows > 0:
        log(f"[bench] cpu baseline: oracle on {args.cpu_rows} rows")
        rows = inputs.sample(M, args.cpu_rows, 0, "rows").to(dev)
        host = {"x": x.index_select(0, rows).cpu(), "z": z.index_select(0, rows).cpu(), "W0": W0.cpu(),
                "gamma": gamma.cpu(), "W1": W1.cpu(), "dY": dY.index_select(0, rows).cpu()}
        cpu = cpu_baseline(host, rows.cpu().numpy(), args.cpu_cols, M)
        log(f"[bench] cpu baseline {cpu['value'] * 1e3:.2f} GFLOP/s on {cpu['cores']} threads")

    rec = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "llama3_8b fused forward + backward", "M": M, "K0": K0, "D": D, "N": N,
                   "eps": inputs.EPS, "parallelism": "single GPU"},
        "pct_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "step_ms_p10_p50_p90": [round(float(q), 4) for q in _quantiles(step_ms, (0.1, 0.5, 0.9))],
        "ms_per_step_instrumented": round(ms_instrumented, 4),
        "cold_cache": cold, "dp8_shard": shard,
        "fwd": {"ms": round(fwd_ms, 4), "tflops": round(fwd_flop / fwd_ms / 1e9, 1),
                "pct_peak": round(100 * fwd_flop / fwd_ms / 1e9 / PEAK_BF16_TFLOPS, 2)},
        "bwd": {"ms": round(bwd_ms, 4), "tflops": round(bwd_flop / bwd_ms / 1e9, 1),
                "pct_peak": round(100 * bwd_flop / bwd_ms / 1e9 / PEAK_BF16_TFLOPS, 2),
                "s_combine_ms": round(per["s_combine"], 4)},
        "configs": configs, "bwd_gemm0": bwd_gemm0, "swiglu": swiglu, "cross_entropy": ce,
        "kernels": kernels, "roofline": roof, "unfused": unfused, "cpu_baseline": cpu,
        "kernel_source_digest": kernel_source_digest(),
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
