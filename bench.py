"""Benchmark of the MMQ hot path on one MI355X.

A step is one pass of the whole hot path over one batch: quantise the f32 activations to q8_1
(a1) and run the MMQ contraction with the raw block weights (a3-a6; for MoE the device-side
expert grouping a7 as well). The weight repack (a2) is one-time and untimed, as on the pages
(metainfer section 3.2). Inputs are synthetic and seeded (gen.CONFIGS), resident in HBM before
the timed region starts.

Default workload: q4_0 weights N=4096 x K=4096 from N(0,0.02), activations M=2048 x K=4096
from N(0,1) with 0.1% outliers x20, f32 output - the q4_0 prefill shape of the MMQ pages'
7B-class models. `--workload` selects another of gen.CONFIGS for reference measurements (the
W8A8 workload's activations are int8 already, so its step is the GEMM alone; the dec*
workloads are decode batches of 1-16 tokens on the same weight shapes).

Timing (the pages' protocol: warm-up, then 30 samples of 100 back-to-back launches (or a
hipGraph replay) timed with hipEvents, median and min/max spread; P2 section 3.3):
  step time     all --steps steps are captured in one hipGraph; each timed replay is bracketed
                by HIP events recorded on the launch stream, so the per-step figure does not
                depend on --steps (no host launch or synchronisation cost inside it); value =
                2*M*N*K / median step time over --rounds replays.
  kernel times  per kernel, a hipGraph of 100 back-to-back launches, each replay bracketed by
                HIP events on the launch stream: 30 samples of the average launch duration
                (mean, median, min, max reported).
  interleaving  the step replays and the kernel samples alternate in --rounds rounds (minfer R1
                section 4: alternate A and B so that a change of machine load shows up as spread,
                not as a difference); the per-round step times are reported.
  cold MALL     --rotate R cycles R copies of the packed weights through the launches so every
                launch reads its weights from HBM rather than the 256 MB last-level cache
                (default for the decode workloads: enough copies for >= 1 GB).

Prints ONE JSON line on stdout:
  value         whole-step throughput, TOPS = 2*M*N*K / step time (2*T*top_k*N*K for MoE)
  roofline      the dominant kernel alone: algorithmic ops (or bytes) per launch / its mean
                event-timed launch time against the MI355X dense int8 MFMA peak (5.0 POP/s)
                or the HBM peak (8 TB/s, decode and MoE); traffic = HBM bytes per launch from
                rocprofv3 FETCH_SIZE + WRITE_SIZE counters scaled by the copy-kernel
                calibration, when measured for this exact kernel and workload, else null
  cpu_baseline  the CPU oracle (quantiser + per-block integer GEMM in C, OpenMP) timed on this
                host's cores, repeated over the workload for a bounded ~10 s, plus one short
                single-thread pass
Diagnostics go to stderr.
"""
from __future__ import annotations

import argparse
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

INT8_PEAK_TOPS = 5000.0          # MI355X dense int8 MFMA, 5.0 POP/s
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, 8 TB/s
VALU_PEAK_LANE_OPS = 256 * 4 * 16 * 2.4e9   # non-packed f32 vector lane-ops per second
HEADLINE = "q4_0_m2048_n4096_k4096"
METRIC = "MMQ prefill GEMM TOPS (2MNK/s) at M=2048,K=4096,N=4096 q4_0; % int8 MFMA peak"
DECODE_BATCH = 16                # the decode kernel's token batch
DECODE_MAX_BATCHES = 8           # mmq_gemm: up to this many batches ...
DECODE_MAX_ROUNDS = 8            # ... while batches x 16-row groups <= this many rounds of the CUs


def decode_path(M, N, cus):
    """Whether mmq_gemm runs an M x N product on the decode kernel (the library's own rule)."""
    if M <= DECODE_BATCH:
        return True
    nb = -(-M // DECODE_BATCH)
    return nb <= DECODE_MAX_BATCHES and nb * -(-N // 16) <= DECODE_MAX_ROUNDS * cus
COLD_BYTES = 1 << 30             # rotated weight copies for a cold-MALL run: at least this much

# HBM bytes per launch of the dominant kernel (for MUL_MAT_ID: route + gather launch), measured
# with rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE and scaled by the copy-kernel factors
# (profiles/ holds the summaries), with the hash of the kernel sources they were measured on:
# reported only while the sources still hash the same, else null.
MEASURED_TRAFFIC = {
    "q4_0_m2048_n4096_k4096": (94_416_986, "abb5fdd9cfc5cfd2"),
    "moe_iq1c_e64_t512_top8_n2048_k4096": (284_343_218 + 40_680, "99acccf9ff652c0d"),
    "moe_iq1t_e64_t512_top8_n2048_k4096": (370_881_786 + 40_679, "99acccf9ff652c0d"),
    "w8a8_m3072_n1536_k4096": (61_465_709, "b2f75c48e899bf66"),
    "q4_K_m512_n14336_k4096": (94_717_268, "abb5fdd9cfc5cfd2"),
    "q6_K_m2048_n4096_k11008": (306_039_285, "abb5fdd9cfc5cfd2"),
    "dec_q4_0_m8_n4096_k4096": (11_100_648, "e982aaa89fc10ad1"),
    "dec_q4_K_m8_n14336_k4096": (45_176_926, "e982aaa89fc10ad1"),
}
KERNEL_SOURCES = {
    "block": ["gemm_block.hip", "gemm_common.h"],
    "gather": ["gemm_block.hip", "gemm_id.hip", "gemm_common.h"],
    "w8a8": ["gemm_w8a8.hip", "gemm_common.h"],
    "mmvq": ["gemm_mmvq.hip", "gemm_id.hip", "gemm_common.h"],
}


def kernel_source_hash(kind):
    """First 16 hex digits of the SHA-256 of the kernel's source files, in order."""
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kind]:
        with open(os.path.join(ROOT, "block_quantized_int8_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(name, kind):
    rec = MEASURED_TRAFFIC.get(name)
    if rec is None or rec[1] != kernel_source_hash(kind):
        return None
    return rec[0]


RAW_BYTES_PER_32 = {"q8_0": 34, "q4_0": 18, "q4_K": 144 / 8, "iq1t": 76 / 8, "iq1c": 56 / 8, "iq1s": 50 / 8,
                    "q6_K": 210 / 8,
                    "i8_row": 32}
# vector ops per element-block of the scale step: exact conversion + FMA, twice for q6_K (one
# per 16-value half)
VALU_OPS_PER_EB = {"q6_K": 4}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def sclk_mhz():
    """Current shader clock of cuda:0 read from sysfs (the DPM level marked '*'), or None. A
    file read: this process has initialised the GPU, so it starts no other program for it. The
    card is matched by PCI bus when torch reports one, else the first card with the file."""
    import glob
    try:
        import torch
        bus = getattr(torch.cuda.get_device_properties(0), "pci_bus_id", None)
    except Exception:
        bus = None
    files = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
    if bus is not None:
        tag = f":{int(bus):02x}:"
        files = [f for f in files if tag in os.path.realpath(os.path.dirname(f))] or files
    try:
        for f in files:
            with open(f) as fh:
                for line in fh:
                    if "*" in line:
                        m = re.search(r"(\d+)\s*mhz", line, flags=re.I)
                        if m:
                            return int(m.group(1))
    except OSError:
        pass
    return None


def _oracle_env():
    return {"os_cpu_count": os.cpu_count(), "OMP_NUM_THREADS": os.environ.get("OMP_NUM_THREADS")}


def cpu_baseline(fmt, raw, x, M, N, K, grid=None, budget_s=10.0, min_runs=3, max_runs=50):
    """The oracle as it stands, timed on the host: q8_1 quantisation + per-block C GEMM over
    the whole workload, repeated until about `budget_s` seconds of CPU work (median reported),
    then one single-thread pass over the first rows."""
    import oracle
    oracle.build()

    def run(rows):
        if fmt == "i8_row":
            a, sa, w, sw = x
            oracle.gemm_w8a8(a[:rows], sa[:rows], w, sw)
        else:
            xq, xs, xsum = oracle.quantize_q8_1(x[:rows])
            oracle.gemm_c(fmt, raw, N, K, xq, xs, xsum, grid=grid)

    times = []
    t_start = time.perf_counter()
    while len(times) < min_runs or (time.perf_counter() - t_start < budget_s and len(times) < max_runs):
        t0 = time.perf_counter()
        run(M)
        times.append(time.perf_counter() - t0)
    t = float(np.median(times))
    cores = oracle.num_threads()
    # single-thread pass on a row sample sized to about a second at the multi-thread rate
    rows1 = int(max(1, min(M, round(M * 1.0 / max(t * cores, 1e-9)))))
    oracle.set_threads(1)
    t0 = time.perf_counter()
    run(rows1)
    t1 = time.perf_counter() - t0
    oracle.set_threads(cores)
    what = "W8A8 int GEMM + bf16 epilogue" if fmt == "i8_row" else "quantize_q8_1 + per-block C GEMM"
    return {"value": 2.0 * M * N * K / t / 1e12, "unit": "TOPS", "cores": cores, "kind": "oracle",
            "sample": f"full workload (M={M}, N={N}, K={K}) repeated {len(times)}x "
                      f"({sum(times):.1f} s of CPU work), median {t:.3f} s per run of {what}",
            "single_thread": {"value": 2.0 * rows1 * N * K / t1 / 1e12, "unit": "TOPS",
                              "sample": f"first {rows1} rows, one run, {t1:.2f} s"},
            **_oracle_env()}


def cpu_baseline_moe(fmt, raw_e, x, ids, E, N, K, grid=None, budget_s=10.0):
    """MoE oracle leg on a bounded sample: the dense per-block C GEMM of the tokens routed to
    each expert (in expert order) until ~budget_s seconds, scaled to pair-rows per s; a small
    workload is passed over again until the budget is used."""
    import oracle
    oracle.build()
    xq, xs, xsum = oracle.quantize_q8_1(x)
    rows_done, t_used, experts, passes = 0, 0.0, 0, 0
    wall0 = time.perf_counter()
    while t_used < budget_s and time.perf_counter() - wall0 < 6 * budget_s:
        for e in range(E):
            tt = np.nonzero((ids == e).any(axis=1))[0]
            if len(tt) == 0:
                continue
            t0 = time.perf_counter()
            oracle.gemm_c(fmt, raw_e[e], N, K, xq[tt], xs[tt], xsum[tt], grid=grid)
            t_used += time.perf_counter() - t0
            rows_done += len(tt)
            experts += 1
            if t_used >= budget_s:
                break
        passes += 1
        log(f"[bench] cpu baseline pass {passes}: {experts} expert products, {t_used:.1f} s")
    ops = 2.0 * rows_done * N * K
    return {"value": ops / t_used / 1e12, "unit": "TOPS", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"{experts} expert products over {passes} pass(es) ({rows_done} routed token rows) "
                      f"through the per-block C GEMM, {t_used:.1f} s", **_oracle_env()}


def cpu_leg(name):
    """The oracle timed on this host's cores over the named workload's own seeded inputs (the
    same draws the GPU leg uploads)."""
    import gen
    cfg = gen.CONFIGS[name]
    fmt, M, N, K = cfg["fmt"], cfg["M"], cfg["N"], cfg["K"]
    grid = gen.IQ1C_GRID if fmt in ("iq1c", "iq1s") else None
    log("[bench] cpu baseline (oracle) ...")
    if fmt == "i8_row":
        a, sa = gen.i8_rows(M, K, seed=0, cfg=cfg["cfg"], tensor=gen.T_ACT)
        w, sw = gen.i8_rows(N, K, seed=0, cfg=cfg["cfg"], tensor=gen.T_WEIGHT)
        r = cpu_baseline("i8_row", None, (a, sa, w, sw), M, N, K)
    elif "E" in cfg:
        E, top_k = cfg["E"], cfg["top_k"]
        raw_e = gen.moe_weights(fmt, E, N, K, seed=0, cfg=cfg["cfg"])
        x = gen.act_f32(M, K, seed=0, cfg=cfg["cfg"])
        ids = gen.moe_ids(M, top_k, E, seed=0, cfg=cfg["cfg"])
        r = cpu_baseline_moe(fmt, raw_e, x, ids, E, N, K, grid)
    else:
        raw = gen.weights(fmt, N, K, seed=0, cfg=cfg["cfg"])
        x = gen.act_f32(M, K, seed=0, cfg=cfg["cfg"], outlier_rate=cfg.get("outlier_rate", 0.0))
        r = cpu_baseline(fmt, raw, x, M, N, K, grid)
    log(f"[bench] cpu baseline {r['value']:.4f} TOPS on {r['cores']} threads: {r['sample']}")
    return r


def _graph(fns, n):
    """A hipGraph of n calls cycling through fns (each launches on the current stream)."""
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):                         # warm the capture stream outside capture
        for f in fns:
            f()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(n):
            fns[i % len(fns)]()
    return g


def timed(kernels, n_rot, steps, warmup, samples=30, per_sample=100, rounds=5):
    """kernels: [(name, fn(r))] launched in this order make one step on weight copy r.

    Step time: all `steps` steps captured in one hipGraph; each timed replay is bracketed by
    HIP events recorded on the launch stream (so host launch and synchronisation costs stay out
    of the figure, whatever `steps` is), with a synchronisation on both sides.
    Kernel times: per kernel, a hipGraph of `per_sample` back-to-back launches, each replay
    bracketed by HIP events: one sample of the average launch duration.
    The phases are interleaved (minfer R1 section 4: alternate the variants so that a change of
    load on the machine shows up as spread, not as a difference): `rounds` rounds, each one
    step replay and samples/rounds samples of every kernel. Returns (step seconds per round,
    {name: kernel samples [s]})."""
    import torch
    stream = torch.cuda.current_stream()
    def step(r):
        for _, f in kernels:
            f(r)
    for i in range(warmup):
        step(i % n_rot)
    torch.cuda.synchronize()
    g_step = _graph([lambda r=r: step(r) for r in range(n_rot)], steps)
    g_k = {name: _graph([lambda r=r, f=f: f(r) for r in range(n_rot)], per_sample) for name, f in kernels}
    g_step.replay()
    for g in g_k.values():
        g.replay()
    torch.cuda.synchronize()

    def event_time(g):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        g.replay()
        e1.record(stream)
        e1.synchronize()
        return e0.elapsed_time(e1) * 1e-3

    per_round = max(1, samples // rounds)
    step_s = []
    kt = {name: [] for name, _ in kernels}
    for _ in range(rounds):
        torch.cuda.synchronize()
        step_s.append(event_time(g_step) / steps)
        torch.cuda.synchronize()
        for name, _ in kernels:
            for _ in range(per_round):
                kt[name].append(event_time(g_k[name]) / per_sample)
    del g_step, g_k
    return np.array(step_s), {k: np.array(v) for k, v in kt.items()}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default=HEADLINE, help="one of gen.CONFIGS")
    ap.add_argument("--rotate", type=int, default=-1,
                    help="weight copies cycled through the steps (cold MALL); default: 1, or enough "
                         "for >= 1 GB on the decode workloads")
    ap.add_argument("--samples", type=int, default=30, help="kernel-timing samples")
    ap.add_argument("--rounds", type=int, default=5,
                    help="interleaved rounds of (one timed step replay, samples/rounds kernel samples)")
    ap.add_argument("--per-sample", type=int, default=100, help="graph-replayed launches per sample")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline leg")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run a plain 256 MiB device copy 5x (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              f"(the path is single-GPU; how it would shard is design-only)", file=sys.stderr)
        sys.exit(2)

    import gen

    # The CPU-oracle leg runs first, before this process touches the GPU: in a process whose
    # HIP runtime is live, the MoE leg's several hundred short OpenMP regions stalled for minutes
    # on the GPU host (the same leg alone there takes ~3 s).
    cpu_rec = None if args.no_cpu else cpu_leg(args.workload)

    import torch
    import block_quantized_int8_amd as mmq

    name = args.workload
    cfg = gen.CONFIGS[name]
    fmt, M, N, K = cfg["fmt"], cfg["M"], cfg["N"], cfg["K"]
    moe = "E" in cfg
    # decode kernel: dense batches as mmq_gemm dispatches them; MoE decode batches (T <= 10)
    decode = decode_path(M, N, torch.cuda.get_device_properties(0).multi_processor_count)
    dev = torch.device("cuda:0")
    log(f"[bench] workload {name}: {fmt} M={M} N={N} K={K}")
    ops = 2.0 * M * N * K
    extra = {}
    # the iq1c codebook: an input of the repack (and of the oracle leg)
    grid_np = gen.IQ1C_GRID if fmt in ("iq1c", "iq1s") else None
    grid_d = torch.from_numpy(grid_np.view(np.int16)).to(dev) if grid_np is not None else None

    def copies_of(t):
        if args.rotate > 0:
            n = args.rotate
        elif args.rotate == 0 or not decode:
            n = 1
        else:
            n = max(3, -(-COLD_BYTES // t.numel()))
        return [t] + [t.clone() for _ in range(n - 1)]

    if fmt == "i8_row":
        a, sa = gen.i8_rows(M, K, seed=0, cfg=cfg["cfg"], tensor=gen.T_ACT)
        w, sw = gen.i8_rows(N, K, seed=0, cfg=cfg["cfg"], tensor=gen.T_WEIGHT)
        packed = copies_of(mmq.repack_weights("i8_row", torch.from_numpy(w).to(dev), N, K,
                                              row_scale=torch.from_numpy(sw).to(dev)))
        act = torch.from_numpy(mmq.act_i8_pack_host(a, sa)).to(dev)
        out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)

        kernels = [("mmvq (decode)" if decode else "w8a8_gemm",
                    lambda r: mmq.gemm("i8_row", packed[r], act, M, N, K, "bf16", out=out))]
        dom = 0
        alg_bytes = N * K + 4 * N + M * K + 4 * M + 2 * M * N
    elif moe:
        E, top_k = cfg["E"], cfg["top_k"]
        T = M
        raw_e = gen.moe_weights(fmt, E, N, K, seed=0, cfg=cfg["cfg"])
        x = gen.act_f32(T, K, seed=0, cfg=cfg["cfg"])
        ids = gen.moe_ids(T, top_k, E, seed=0, cfg=cfg["cfg"])
        pb = mmq.packed_bytes(fmt, N, K)
        p0 = torch.empty(E * pb, dtype=torch.uint8, device=dev)
        for e in range(E):
            mmq.repack_weights(fmt, torch.from_numpy(np.ascontiguousarray(raw_e[e])).to(dev), N, K,
                               out=p0[e * pb:(e + 1) * pb], grid=grid_d)
        packed = copies_of(p0)
        xd = torch.from_numpy(x).to(dev)
        ids_d = torch.from_numpy(ids).to(dev)
        act = torch.empty(mmq.act_bytes("q8_1", T, K), dtype=torch.uint8, device=dev)
        out = torch.empty((T, top_k, N), dtype=torch.float32, device=dev)
        ws = torch.empty(mmq.gemm_id_workspace_bytes(E, T, top_k), dtype=torch.uint8, device=dev)

        kernels = [("quantize_q8_1", lambda r: mmq.quantize_act(xd, out=act)),
                   ("gemm_id (decode kernel, in-kernel grouping)" if T <= 10 and T * top_k <= 256
                    else "gemm_id (route + gather MMQ)",
                    lambda r: mmq.gemm_id(fmt, packed[r], E, act, ids_d, T, top_k, N, K, out=out, workspace=ws))]
        dom = 1
        ops = 2.0 * T * top_k * N * K
        used = len(np.unique(ids))
        alg_bytes = int(used * N * K / 32 * RAW_BYTES_PER_32[fmt]) + T * K + T * (K // 32) * 8 + \
            T * top_k * N * 4 + T * top_k * 4
        extra = {"E": E, "top_k": top_k, "experts_used": used}
    else:
        raw = gen.weights(fmt, N, K, seed=0, cfg=cfg["cfg"])
        x = gen.act_f32(M, K, seed=0, cfg=cfg["cfg"], outlier_rate=cfg.get("outlier_rate", 0.0))
        xd = torch.from_numpy(x).to(dev)
        packed = copies_of(mmq.repack_weights(fmt, torch.from_numpy(raw).to(dev), N, K, grid=grid_d))
        act = torch.empty(mmq.act_bytes("q8_1", M, K), dtype=torch.uint8, device=dev)
        out = torch.empty((M, N), dtype=torch.float32, device=dev)

        kernels = [("quantize_q8_1", lambda r: mmq.quantize_act(xd, out=act)),
                   ("mmvq (decode)" if decode else "mmq_block",
                    lambda r: mmq.gemm(fmt, packed[r], act, M, N, K, "f32", out=out))]
        dom = 1
        # raw weights + q8_1 activations (int8 values, f32 scale, int32 sum) + f32 output
        alg_bytes = int(N * K / 32 * RAW_BYTES_PER_32[fmt]) + M * K + M * (K // 32) * 8 + M * N * 4
    n_rot = len(packed)
    bound = "hbm" if (moe or decode) else "mfma"
    if n_rot > 1:
        extra["weight_copies_rotated"] = n_rot
        extra["weight_bytes_rotated"] = int(n_rot * packed[0].numel())

    torch.cuda.synchronize()
    step_rounds, kt = timed(kernels, n_rot, args.steps, args.warmup, args.samples, args.per_sample, args.rounds)
    step_s = float(np.median(step_rounds))
    sclk = sclk_mhz()
    tops = ops / step_s / 1e12
    log(f"[bench] step per round (us): " + ", ".join(f"{v * 1e6:.2f}" for v in step_rounds))
    kstats = []
    for kn, _ in kernels:
        c = kt[kn]
        kstats.append({"mean": float(c.mean()), "median": float(np.median(c)), "min": float(c.min()),
                       "max": float(c.max())})
        log(f"[bench] {kn}: per launch mean {c.mean() * 1e6:.3f} us, median {np.median(c) * 1e6:.3f} us, "
            f"min {c.min() * 1e6:.3f}, max {c.max() * 1e6:.3f} ({args.samples} samples x {args.per_sample} launches)")
    k_s = kstats[dom]["mean"]
    k_tops = ops / k_s / 1e12
    k_gbs = alg_bytes / k_s / 1e9
    log(f"[bench] step {step_s * 1e6:.2f} us ({tops:.1f} TOPS, {100 * tops / INT8_PEAK_TOPS:.1f}% int8 peak); "
        f"dominant kernel {k_s * 1e6:.2f} us = {k_tops:.1f} TOPS ({100 * k_tops / INT8_PEAK_TOPS:.1f}% int8), "
        f"{k_gbs:.0f} GB/s algorithmic ({100 * k_gbs / HBM_PEAK_GBS:.1f}% HBM); sclk {sclk} MHz")
    if len(kernels) == 2:
        q_bytes = M * K * 4 + mmq.act_bytes("q8_1", M, K)
        q_s = kstats[0]["mean"]
        log(f"[bench] quantize {q_bytes / q_s / 1e9:.0f} GB/s ({100 * q_bytes / q_s / 1e9 / HBM_PEAK_GBS:.1f}% HBM)")
        extra["quantize_kernel_us"] = round(q_s * 1e6, 3)

    if bound == "mfma":
        roof = {"bound": "mfma", "achieved": round(k_tops, 2), "peak": INT8_PEAK_TOPS, "unit": "TFLOP/s",
                "frac": round(k_tops / INT8_PEAK_TOPS, 4)}
    else:
        roof = {"bound": "hbm", "achieved": round(k_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(k_gbs / HBM_PEAK_GBS, 4)}
    if fmt != "i8_row" and not decode:
        # the per-block scale application: >= 2 vector ops (exact conversion + FMA) per
        # element-block E = rows * N * K/32, against 256 CU x 4 SIMD x 16 lanes x 2.4 GHz
        rows = M * cfg.get("top_k", 1)
        E = rows * N * (K // 32)
        nops = VALU_OPS_PER_EB.get(fmt, 2)
        roof["valu_ceiling"] = {"ops_per_element_block": nops, "peak_lane_ops": VALU_PEAK_LANE_OPS,
                                "frac": round(nops * E / k_s / VALU_PEAK_LANE_OPS, 4)}
    kind = "w8a8" if fmt == "i8_row" and not decode else "mmvq" if decode else "gather" if moe else "block"
    roof["traffic"] = measured_traffic(name, kind) if n_rot == 1 or name.startswith("dec") else None
    roof["kernel_source_hash"] = kernel_source_hash(kind)
    roof["kernel"] = kernels[dom][0]
    roof["kernel_us"] = {k: round(v * 1e6, 3) for k, v in kstats[dom].items()}
    roof["algorithmic_bytes"] = alg_bytes
    roof["algorithmic_ops"] = ops

    if args.calib_copy:
        src = torch.empty(1 << 28, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("[bench] calibration copy: 5 x 256 MiB device-to-device")

    desc = {"q4_0_m2048_n4096_k4096": "q4_0 MMQ prefill: raw q4_0 weights N=4096 K=4096, q8_1 activations M=2048 "
                          "(quantised in-step), f32 out"}
    rec = {
        "metric": METRIC if name == HEADLINE else f"MMQ TOPS (2MNK/s) on {name}",
        "value": round(tops, 3),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_s * 1e3, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8",
        "data": "synthetic",
        "config": {"workload": desc.get(name, name), "M": M, "N": N, "K": K, "weights": fmt,
                   "activations": "i8_token" if fmt == "i8_row" else "q8_1",
                   "step": "gemm (int8 activations given)" if fmt == "i8_row" else
                           "quantize_act + gemm" + ("_id" if moe else "") + " (repack untimed)",
                   "timing": f"one hipGraph of all {args.steps} steps, HIP events on the launch stream, median "
                             f"of {args.rounds} replays interleaved with the kernel samples "
                             f"({args.samples} samples x {args.per_sample} graph-replayed launches per kernel)",
                   "step_us_rounds": [round(v * 1e6, 3) for v in step_rounds],
                   **extra},
        "pct_int8_peak": round(100 * tops / INT8_PEAK_TOPS, 3),
        "sclk_mhz_after_run": sclk,
        "roofline": roof,
    }
    if cpu_rec is not None:
        rec["cpu_baseline"] = cpu_rec
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
