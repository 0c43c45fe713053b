"""Benchmark of the fused Matryoshka contrastive loss (fwd + bwd) on one MI355X.

One step = one call of the C ABI (every kernel of the forward, the statistics,
both backward passes and the loss reduction) on inputs already resident in
HBM.  Prints one JSON line.

Metric: fwd+bwd TFLOP/s with the algorithmic count 8 R N D per step (forward
2RND, logit recompute 2RND, dQ 2RND, dK 2RND; prefixes share one sweep), plus
pair-scores/s = R N P per step and the fraction of the BF16 dense MFMA peak.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6  # 256 CU x 2.4 GHz x 4096 FLOP/clk/CU, dense
PEAK_HBM_GBS = 8000.0
KERNEL_SOURCE = os.path.join(ROOT, "contrastive_embedding_loss_amd", "csrc", "kernels.hip")


def measured_traffic(workload: str):
    """HBM bytes per backward launch from the committed counter summary, or None.

    The summary's record names the sha256 of the kernel source it was measured
    on; a record for other source (the kernels changed since) is not used.
    """
    import hashlib

    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{workload}.md")
    if not os.path.exists(path):
        return None
    sha = hashlib.sha256(open(KERNEL_SOURCE, "rb").read()).hexdigest()[:16]
    for line in open(path):
        if line.startswith("traffic-record "):
            kv = dict(f.split("=", 1) for f in line.split()[1:])
            if kv.get("kernel") in ("k_bwd", "k_bwd_gen") and kv.get("source_sha256_16") == sha:
                return int(kv["read_bytes"]) + int(kv["write_bytes"])
    return None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="infonce_32768")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample", type=int, default=0,
                    help="time the oracle on a sample of this many rows of the same recipe instead of the "
                         "workload's own arrays (0: the workload's own arrays)")
    ap.add_argument("--no-gemm-ceiling", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB three times (a known-size kernel "
                         "against which the HBM byte counters are scaled) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU; --gpus {args.gpus} is not supported (the loss's multi-GPU "
              "sharding is a design only; the library runs on one GPU)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from contrastive_embedding_loss_amd import binding
    from contrastive_embedding_loss_amd.inputs import (ONESET_SIGLIP, WORKLOADS, bf16_bits_to_f32, make_inputs,
                                                       workload_inputs, workload_positives)

    dev = torch.device("cuda:0")
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": n, "bytes_written": n, "launches": 3}), flush=True)
        return

    w = WORKLOADS[args.workload]
    t0 = time.time()
    qb, kb = workload_inputs(w)
    oneset = w.kind == ONESET_SIGLIP
    k = torch.from_numpy(bf16_bits_to_f32(kb)).to(dev).to(torch.bfloat16)
    if oneset:  # the one-set form scores the set's own rows: q is a view of k
        q = k[w.row_offset:w.row_offset + w.R]
    else:
        q = torch.from_numpy(bf16_bits_to_f32(qb)).to(dev).to(torch.bfloat16)
    print(f"[bench] inputs {w.name} R={w.R} N={w.N} D={w.D} ready in {time.time() - t0:.1f}s", file=sys.stderr,
          flush=True)
    R, N, D, P = w.R, w.N, w.D, len(w.prefixes)
    f32 = dict(dtype=torch.float32, device=dev)
    loss = torch.empty(1, **f32)
    dq = torch.empty(R, D, **f32)
    dk = None if oneset else torch.empty(N, D, **f32)

    positives = workload_positives(w)  # entries with several positives: host CSR lists, staged each step

    def step(profile=False):
        return binding.fwd_bwd(q, k, w.prefixes, w.scale, w.bias, w.kind, weights=w.weights,
                               row_offset=w.row_offset, dq=dq, dk=dk, want_dk=not oneset, profile=profile,
                               positives=positives)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    binding.profile()  # clear
    print(f"[bench] warmup done ({args.warmup} steps)", file=sys.stderr, flush=True)

    # timed region: K steps, each step and each kernel bracketed by events on the launch stream
    stream = torch.cuda.current_stream(dev)
    marks = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for a_ev, b_ev in marks:
        a_ev.record(stream)
        step(profile=True)
        b_ev.record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    kern = binding.profile()
    ms_per_step = 1e3 * elapsed / args.steps
    step_ms = sorted(a_ev.elapsed_time(b_ev) for a_ev, b_ev in marks)

    # two-set kinds: forward 2RND + one logit recompute 2RND + dQ 2RND + dK 2RND; the one-set form
    # has the share's logits 2RND and dX 2RND, in one backward pass
    flops = (4.0 if oneset else 8.0) * R * N * D
    tflops = flops / (ms_per_step * 1e-3) / 1e12
    pair_scores = float(R) * N * P / (ms_per_step * 1e-3)
    # for comparison with implementations counted without the logit recompute: two-set 6RND
    # (forward, dQ, dK), one-set 4RND (logits, dX); and cells (pairs scored once) per second
    tflops_no_recompute = (4.0 if oneset else 6.0) * R * N * D / (ms_per_step * 1e-3) / 1e12
    cells = float(R) * N / (ms_per_step * 1e-3)
    kern_per_step = {n: t / args.steps for n, t in kern.items()}
    print(f"[bench] {ms_per_step:.3f} ms/step, {tflops:.1f} TFLOP/s; kernels (ms/step): "
          + ", ".join(f"{n}={t:.3f}" for n, t in sorted(kern_per_step.items(), key=lambda x: -x[1])),
          file=sys.stderr, flush=True)

    # dominant kernel: the backward pass kernel (launched twice per step: rows, columns).
    # Algorithmic MFMA work credited to one launch: 3 R N D = its gradient contraction 2 R N D
    # plus half of the single logit recompute 2 R N D that the step's count includes (each
    # launch actually executes a full recompute, 4 R N D in all; the extra is not credited).
    # (the compiled backward k_bwd, or the generic one for ladders without a compiled kernel and rows
    # wider than 1024)
    launches = 1 if oneset else 2
    bwd_name = "k_bwd" if "k_bwd" in kern_per_step else "k_bwd_gen"
    bwd_ms = kern_per_step.get(bwd_name, float("nan")) / launches
    bwd_tflops = (4.0 if oneset else 3.0) * R * N * D / (bwd_ms * 1e-3) / 1e12
    roofline = {"kernel": bwd_name, "bound": "mfma", "achieved": round(bwd_tflops, 1),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(bwd_tflops / PEAK_BF16_TFLOPS, 4),
                "traffic": measured_traffic(w.name), "avg_launch_ms": round(bwd_ms, 4),
                "executed_tflops": round(4.0 * R * N * D / (bwd_ms * 1e-3) / 1e12, 1)}

    # HBM-bound stages: algorithmic bytes (rows read once, tables and partials as laid out) per launch
    n_jt, n_it = -(-N // 128), -(-R // 128)
    stage_bytes = {
        # rows read once, the tables, and the sig-scaled FP16 copies of both row sets (with the two zero
        # blocks past each last row) that k_prep writes for the backward
        "k_prep": (R + N) * D * 2 + 4 * ((R + N) * (3 * P + 2) + R * P)
                  + ((-(-R // 16) + 2) * 16 + (-(-N // 16) + 2) * 16) * D * 2,
        "k_rowstats": 4 * R * P * (n_jt + 9),
        "k_colstats": 4 * N * P * (n_it + 9),
    }
    hbm_stages = {}
    for name, nbytes in stage_bytes.items():
        if name in kern_per_step:
            t = kern_per_step[name]
            hbm_stages[name] = {"ms": round(t, 4), "bytes": nbytes, "GB_per_s": round(nbytes / (t * 1e-3) / 1e9, 1),
                                "frac_of_8TBps": round(nbytes / (t * 1e-3) / 8e12, 3)}

    # ceiling of a plain library GEMM of the forward's contraction shape on this chip, timed in this
    # run: hipBLASLt through torch.matmul, BF16 in and out, R x D times D x N
    gemm = None
    if not args.no_gemm_ceiling:
        qg = q.contiguous()
        kt = k.t().contiguous()  # D x N, contiguous: a plain GEMM
        c = torch.matmul(qg, kt)
        for _ in range(2):
            torch.matmul(qg, kt, out=c)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(5)]
        torch.cuda.synchronize()
        for a_ev, b_ev in ev:
            a_ev.record(stream)
            torch.matmul(qg, kt, out=c)
            b_ev.record(stream)
        torch.cuda.synchronize()
        g_ms = sorted(a_ev.elapsed_time(b_ev) for a_ev, b_ev in ev)[len(ev) // 2]
        g_tf = 2.0 * R * N * D / (g_ms * 1e-3) / 1e12
        gemm = {"lib": "hipBLASLt (torch.matmul, bf16 in/out)", "shape": [R, D, N], "ms": round(g_ms, 4),
                "tflops": round(g_tf, 1), "pct_bf16_peak": round(100.0 * g_tf / PEAK_BF16_TFLOPS, 2)}
        del c, kt, qg
        torch.cuda.empty_cache()
        print(f"[bench] GEMM ceiling {R}x{D}x{N}: {g_ms:.3f} ms = {g_tf:.1f} TFLOP/s", file=sys.stderr, flush=True)

    cpu = None
    if not args.no_cpu_baseline:
        from oracle import bf16_bits_to_f64, contrastive_fwd_bwd

        cores = len(os.sched_getaffinity(0))
        kind = w.kind
        if args.cpu_sample:  # a sample of the same recipe (to bound the oracle's time)
            n_s = min(args.cpu_sample, R)
            pos_s = None
            if w.recipe == "band":  # entries of the same recipe, about n_s keys in all
                from contrastive_embedding_loss_amd.inputs import make_band_inputs
                e = w.extra
                qs, ks, rp_s, col_s = make_band_inputs(max(1, n_s * R // N), D, e["extra_pos"], e["hard_neg"],
                                                       w.noise, e["hard_noise"], w.seed)
                pos_s = (rp_s, col_s)
            else:
                qs, ks = make_inputs(n_s, n_s, D, w.recipe, w.noise, w.seed, w.extra.get("centroids", 256))
            if oneset:
                qs = ks  # the one-set sample scores its whole set
            off_s = 0
            what = "a sample of the same recipe and prefixes"
        else:  # the workload's own BF16 arrays, the very inputs the GPU steps ran on
            qs, ks, pos_s, off_s = qb, kb, positives, w.row_offset
            what = f"the {w.name} workload's own BF16 inputs (the arrays the timed GPU steps used)"
        r_s, c_s = qs.shape[0], ks.shape[0]
        print(f"[bench] oracle on {r_s}x{c_s} ({'sample' if args.cpu_sample else 'the workload itself'}) "
              f"on {cores} cores", file=sys.stderr, flush=True)
        t1 = time.perf_counter()
        contrastive_fwd_bwd(bf16_bits_to_f64(qs), bf16_bits_to_f64(ks), w.prefixes, w.scale, w.bias, kind,
                            weights=w.weights, row_offset=off_s, threads=cores, positives=pos_s)
        tc = time.perf_counter() - t1
        fl = 4.0 if oneset else 8.0
        cpu = {"value": round(fl * r_s * c_s * D / tc / 1e12, 5), "unit": "TFLOP/s", "cores": cores,
               "kind": "oracle",
               "sample": f"FP64 oracle fwd+bwd on {what}: {r_s}x{c_s}, D={D}, {P} prefixes, "
                         f"{tc:.1f} s; rate = {fl:.0f}*R*N*D/t"}
        print(f"[bench] oracle {tc:.1f} s", file=sys.stderr, flush=True)

    out = {
        "metric": "fwd+bwd TFLOP/s & pair-scores/s at N=32768, 5 prefixes; % BF16 MFMA peak",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "ms_per_step_median": round(step_ms[len(step_ms) // 2], 4),
        "ms_per_step_min": round(step_ms[0], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "R": R, "N": N, "D": D, "prefixes": list(w.prefixes),
                   "kind": ["infonce", "siglip", "infonce_rows", "oneset_siglip"][w.kind], "scale": w.scale,
                   "bias": w.bias,
                   "weights": list(w.weights) if w.weights else None, "recipe": w.recipe,
                   **({"extra_positives": int(positives[0][-1])} if positives is not None else {})},
        "pair_scores_per_s": pair_scores,
        "cells_per_s": cells,
        "tflops_no_recompute": round(tflops_no_recompute, 2),
        "pct_bf16_peak": round(100.0 * tflops / PEAK_BF16_TFLOPS, 2),
        "pct_of_gemm_ceiling": round(100.0 * tflops / gemm["tflops"], 2) if gemm else None,
        "gemm_ceiling": gemm,
        "kernel_ms_per_step": {n: round(t, 4) for n, t in kern_per_step.items()},
        "roofline": roofline,
        "hbm_stages": hbm_stages,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
