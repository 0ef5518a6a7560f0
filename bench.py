#!/usr/bin/env python3
"""Benchmark of the exact long-accumulator GEMM on one MI355X.

One step = one det_gemm call (decode, exact products, limb placement, digit
accumulation and the fused rounding to fp32) on the f32 4096x4096x4096
wide-range workload: entries sign*m*2^e with m uniform in [1,2), e uniform in
[-70, 70], 1% subnormal, seed 2.  Inputs are resident in HBM before timing
starts.  Timing uses HIP events on the stream the kernels run on (torch's
current stream), bracketed by device synchronisation.

Besides the headline line this prints nothing on stdout.  The JSON line also
carries:
  roofline      the GEMM kernel against the VALU lane-op peak (bound "alu")
  cpu_baseline  the plain C oracle timed on the host cores over a bounded
                block of output rows of the same workload
  parity        sampled outputs compared bit for bit with the oracle
  aux           det_gemm_partial, det_combine and det_finalize on the same
                workload (the other rows of the hot path), with HBM rates
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

# VALU lane-op peak: 256 CUs x 64 lanes x 2.4 GHz (one full-rate wave64
# instruction per CU per clock)
VALU_PEAK_LANE_OPS = 256 * 64 * 2.4e9
# algorithmic VALU lane-ops per MAC: product, exponent sum,
# digit index, shift, limb split, sign, and one add per limb
OPS_PER_MAC = {"f32": 10, "bf16": 8}
HBM_PEAK = 8.0e12
KERNEL_SOURCE = os.path.join(ROOT, "bitwise_deterministic_exact_amd", "csrc", "detgemm.hip")
TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "k_gemm_f32_4096_wide.md")


def recorded_traffic():
    """HBM bytes per launch of the GEMM kernel from the committed rocprofv3
    summary (FETCH_SIZE and WRITE_SIZE, scaled by the copy calibration), or
    None when the kernel source has changed since the counters were taken."""
    import hashlib
    try:
        with open(TRAFFIC_RECORD) as f:
            line = next(l for l in f if l.startswith("traffic-record:"))
        rec = json.loads(line.split(":", 1)[1])
        with open(KERNEL_SOURCE, "rb") as f:
            if hashlib.sha256(f.read()).hexdigest() != rec["source_sha256"]:
                return None
        return int((rec["fetch_kib"] * rec["fetch_scale"] + rec["write_kib"] * rec["write_scale"]) * 1024)
    except (OSError, StopIteration, KeyError, ValueError):
        return None


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def cpu_baseline(xb: np.ndarray, wb: np.ndarray, target_s: float = 15.0) -> dict:
    """Time the plain C oracle on a block of whole output rows (all N columns,
    full K) sized for roughly ``target_s`` seconds of host work."""
    from oracle import c_oracle
    threads = min(os.cpu_count() or 1, 16)
    K = xb.shape[1]
    N = wb.shape[0]
    cal_rows = 2 * threads
    t0 = time.perf_counter()
    c_oracle.partial(xb[:cal_rows], wb, nthreads=threads)
    rate = cal_rows * N * K / max(time.perf_counter() - t0, 1e-6)
    rows = int(max(threads, min(xb.shape[0], target_s * rate / (N * K))))
    rows = (rows // threads) * threads or threads
    t0 = time.perf_counter()
    c_oracle.partial(xb[:rows], wb, nthreads=threads)
    dt = time.perf_counter() - t0
    macs = rows * N * K
    return {"value": round(macs / dt / 1e9, 4), "unit": "GMAC/s", "cores": threads,
            "kind": "oracle",
            "sample": f"plain C oracle (exact_oracle.c), raw digits of the first {rows} output rows "
                      f"x all {N} columns at full K={K} ({macs:.3g} MAC, {dt:.1f} s)"}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--size", type=int, default=4096, help="M = N = K of the workload")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-aux", action="store_true")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain 256 MiB device copy (calibrates HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the exact GEMM here has no multi-GPU path "
              "(each GPU would run its own K- or output-shard; see DESIGN.md).", file=sys.stderr)
        return 2

    import torch
    import bitwise_deterministic_exact_amd as det
    from oracle import c_oracle
    from workloads import c3_wide_f32, f32_bits

    n = args.size
    log(f"generating the wide-range f32 workload {n}^3 (seed 2)")
    t0 = time.perf_counter()
    wl = c3_wide_f32(seed=2, n=n)
    xb, wb = wl.bits()
    log(f"generated in {time.perf_counter() - t0:.1f} s")
    dev = torch.device("cuda:0")
    x = torch.from_numpy(wl.x).to(dev)
    w = torch.from_numpy(wl.w).to(dev)
    y = torch.empty((n, n), dtype=torch.float32, device=dev)
    M = N = K = n
    macs = M * N * K

    def step():
        det.det_gemm(x, w, check_finite=False, out=y)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(args.steps):
        step()
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    gmacs = macs / (ms * 1e-3) / 1e9
    log(f"det_gemm {n}^3: {ms:.3f} ms/step, {gmacs:.1f} GMAC/s")

    # parity on sampled outputs (bit for bit against the C oracle)
    rng = np.random.default_rng(1234)
    rows = rng.integers(0, M, 256)
    cols = rng.integers(0, N, 256)
    got = y.cpu().numpy().view(np.uint32)[rows, cols]
    want = c_oracle.gemm_pairs(xb, wb, rows, cols, nthreads=min(os.cpu_count() or 1, 16))
    parity_ok = bool(np.array_equal(got, want))
    log(f"parity on 256 sampled outputs: {'bit-exact' if parity_ok else 'MISMATCH'}")

    achieved = OPS_PER_MAC["f32"] * macs / (ms * 1e-3)
    result = {
        "metric": "exact-GEMM GMAC/s (f32 4096^3) + % VALU peak; bit-exact vs oracle",
        "value": round(gmacs, 2),
        "unit": "GMAC/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int64",
        "data": "synthetic",
        "config": {"workload": f"det_gemm f32 M=N=K={n}, entries sign*m*2^e, m~U[1,2), "
                               f"e~U{{-70..70}}, 1% subnormal (e in [-149,-127]), seed 2",
                   "M": M, "N": N, "K": K, "inputs": "f32", "output": "f32"},
        "roofline": {"bound": "alu", "achieved": round(achieved / 1e12, 3),
                     "peak": round(VALU_PEAK_LANE_OPS / 1e12, 3), "unit": "Tlane-op/s",
                     "frac": round(achieved / VALU_PEAK_LANE_OPS, 4), "traffic": recorded_traffic(),
                     "ops_per_mac": OPS_PER_MAC["f32"], "kernel": "k_gemm<f32, fp32 out>"},
        "parity": {"sampled_outputs": 256, "bit_exact": parity_ok},
    }

    if not args.no_aux:
        aux = {}
        torch.cuda.synchronize()
        reps = 3

        def timed(fn):
            fn()
            torch.cuda.synchronize()
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record()
            for _ in range(reps):
                out = fn()
            e.record()
            torch.cuda.synchronize()
            return s.elapsed_time(e) / reps, out

        h = K // 2
        t_part, pa = timed(lambda: det.det_gemm_partial(x[:, :h], w[:, :h], check_finite=False))
        pb = det.det_gemm_partial(x[:, h:], w[:, h:], check_finite=False)
        t_comb, acc = timed(lambda: det.det_combine([pa, pb]))
        t_fin, yf = timed(lambda: det.det_finalize(acc))
        same = bool(torch.equal(yf.view(torch.int32), y.view(torch.int32)))
        acc_bytes = M * N * 18 * 8
        aux["partial_half_k"] = {"ms": round(t_part, 3),
                                 "GMAC/s": round(M * N * h / (t_part * 1e-3) / 1e9, 2)}
        aux["combine_2"] = {"ms": round(t_comb, 3),
                            "GB/s": round(3 * acc_bytes / (t_comb * 1e-3) / 1e9, 1),
                            "hbm_frac": round(3 * acc_bytes / (t_comb * 1e-3) / HBM_PEAK, 4)}
        aux["finalize"] = {"ms": round(t_fin, 3),
                           "GB/s": round((acc_bytes + M * N * 4) / (t_fin * 1e-3) / 1e9, 1),
                           "hbm_frac": round((acc_bytes + M * N * 4) / (t_fin * 1e-3) / HBM_PEAK, 4)}
        aux["sharded_equals_unsharded"] = same
        result["aux"] = aux
        log(f"aux: {aux}")
        del pa, pb, acc, yf

    if args.copy_probe:
        # a plain copy of known size: 256 MiB read + 256 MiB written; its
        # FETCH_SIZE / WRITE_SIZE readings calibrate those counters
        src = torch.empty(64 << 20, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(2):
            dst.copy_(src)
        torch.cuda.synchronize()
        result["copy_probe_bytes"] = {"read": src.numel() * 4, "write": dst.numel() * 4}
        del src, dst

    if not args.no_cpu_baseline:
        log("timing the C oracle on the host")
        result["cpu_baseline"] = cpu_baseline(xb, wb)
        log(f"cpu_baseline: {result['cpu_baseline']}")

    print(json.dumps(result), flush=True)
    return 0 if parity_ok else 1


if __name__ == "__main__":
    sys.exit(main())
