"""Benchmark of the prefill MMQ hot path on one MI355X.

A step is one pass of the whole hot path over one batch: quantise f32 activations to q8_1
(a1) and run the MMQ contraction with raw q4_0 weights (a3-a6). The weight repack (a2) is
one-time and untimed, as on the pages (metainfer section 3.2). Workload: q4_0 weights
N=4096 x K=4096 from N(0,0.02), activations M=2048 x K=4096 from N(0,1) with 0.1% outliers
x20, f32 output - the q4_0 prefill shape of the MMQ pages' 7B-class models, synthetic and
seeded (gen.CONFIGS["cfg2a_q4_0"]).

Prints ONE JSON line on stdout:
  value         whole-step throughput, TOPS = 2*M*N*K / step time (inputs resident in HBM)
  roofline      the MMQ kernel alone: algorithmic ops per launch / its mean launch time
                (HIP events on the launch stream, over the timed steps) against the int8
                MFMA dense peak (5.0 POP/s); traffic = HBM bytes per launch from rocprofv3
                counters when measured for this exact kernel, else null
  cpu_baseline  the CPU oracle (quantiser + per-block integer GEMM in C, OpenMP) timed on
                this host's cores on the same workload
Diagnostics go to stderr.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

INT8_PEAK_TOPS = 5000.0          # MI355X dense int8 MFMA, 5.0 POP/s
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, 8 TB/s

# HBM bytes per MMQ launch measured with rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE for the kernel
# version this file ships with (see profiles/); None until measured.
MEASURED_TRAFFIC_BYTES = None


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def cpu_baseline(raw, x, fmt, M, N, K, runs=3):
    """The oracle as it stands, timed on the host: q8_1 quantisation + per-block GEMM."""
    import oracle
    oracle.build()
    times = []
    for _ in range(runs):
        t0 = time.perf_counter()
        xq, xs, xsum = oracle.quantize_q8_1(x)
        oracle.gemm_c(fmt, raw, N, K, xq, xs, xsum)
        times.append(time.perf_counter() - t0)
    t = float(np.median(times))
    return {"value": 2.0 * M * N * K / t / 1e12, "unit": "TOPS", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"full workload (all {M} rows), median of {runs} runs of quantize_q8_1 + "
                      f"per-block C GEMM; {t:.2f} s per run"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline leg")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              f"(the path is single-GPU; sharding is design-only)", file=sys.stderr)
        sys.exit(2)

    import torch
    import block_quantized_int8_amd as mmq
    import gen

    cfg = gen.CONFIGS["cfg2a_q4_0"]
    fmt, M, N, K = cfg["fmt"], cfg["M"], cfg["N"], cfg["K"]
    dev = torch.device("cuda:0")
    raw = gen.weights(fmt, N, K, seed=0, cfg=cfg["cfg"])
    x = gen.act_f32(M, K, seed=0, cfg=cfg["cfg"], outlier_rate=cfg["outlier_rate"])
    log(f"[bench] workload {fmt} M={M} N={N} K={K}")

    xd = torch.from_numpy(x).to(dev)
    packed = mmq.repack_weights(fmt, torch.from_numpy(raw).to(dev), N, K)   # untimed, one-time
    act = torch.empty(mmq.act_bytes("q8_1", M, K), dtype=torch.uint8, device=dev)
    out = torch.empty((M, N), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        mmq.quantize_act(xd, out=act)
        if ev is not None:
            ev[1].record()
        mmq.gemm(fmt, packed, act, M, N, K, "f32", out=out)
        if ev is not None:
            ev[2].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: exactly `steps` steps, synchronised on both sides
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    step_s = (t1 - t0) / args.steps

    # per-kernel durations from HIP events on the launch stream (same steps, recorded apart so
    # the event records do not perturb the wall-clock figure above)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    q_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    g_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    g_ms_med = float(np.median([e[1].elapsed_time(e[2]) for e in evs]))

    ops = 2.0 * M * N * K
    tops = ops / step_s / 1e12
    gemm_tops = ops / (g_ms * 1e-3) / 1e12
    # algorithmic bytes of one MMQ launch: raw q4_0 weights + q8_1 activations + f32 output
    alg_bytes = N * K // 32 * 18 + M * K + M * (K // 32) * 4 + M * N * 4
    log(f"[bench] step {step_s * 1e6:.1f} us ({tops:.1f} TOPS); quantize {q_ms * 1e3:.1f} us; "
        f"mmq mean {g_ms * 1e3:.1f} us / median {g_ms_med * 1e3:.1f} us ({gemm_tops:.1f} TOPS, "
        f"{100 * gemm_tops / INT8_PEAK_TOPS:.1f}% int8 peak)")
    q_bytes = M * K * 4 + mmq.act_bytes("q8_1", M, K)
    log(f"[bench] quantize {q_bytes / (q_ms * 1e-3) / 1e9:.0f} GB/s "
        f"({100 * q_bytes / (q_ms * 1e-3) / 1e9 / HBM_PEAK_GBS:.1f}% HBM)")

    rec = {
        "metric": "MMQ prefill GEMM TOPS (2MNK/s) at M=2048,K=4096,N=4096 q4_0; % int8 MFMA peak",
        "value": round(tops, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_s * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8",
        "data": "synthetic",
        "config": {"workload": "q4_0 MMQ prefill: raw q4_0 weights N=4096 K=4096, q8_1 activations "
                               "M=2048 (quantised in-step), f32 out",
                   "M": M, "N": N, "K": K, "weights": "q4_0", "activations": "q8_1",
                   "step": "quantize_act + gemm (repack untimed)"},
        "pct_int8_peak": round(100 * tops / INT8_PEAK_TOPS, 2),
        "mmq_kernel_us": round(g_ms * 1e3, 2),
        "quantize_kernel_us": round(q_ms * 1e3, 2),
        "roofline": {"bound": "mfma", "achieved": round(gemm_tops, 2), "peak": INT8_PEAK_TOPS,
                     "unit": "TFLOP/s", "frac": round(gemm_tops / INT8_PEAK_TOPS, 4),
                     "traffic": MEASURED_TRAFFIC_BYTES,
                     "algorithmic_bytes": alg_bytes},
    }
    if not args.no_cpu:
        log("[bench] cpu baseline (oracle) ...")
        rec["cpu_baseline"] = cpu_baseline(raw, x, fmt, M, N, K)
        log(f"[bench] cpu baseline {rec['cpu_baseline']['value']:.4f} TOPS on {rec['cpu_baseline']['cores']} threads")
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
