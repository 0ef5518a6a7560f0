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
  roofline      the GEMM kernel against the unit that binds it, its LDS atomic
                adds (one per MAC): atomic lane-ops per launch over the
                launch's duration (HIP events the library records around the
                kernel, on its stream), against the atomic rate a probe
                kernel measures in the same run; the VALU shares beside it
  cpu_baseline  the plain C oracle timed on the host cores over a bounded
                block of output rows of the same workload
  parity        sampled outputs compared bit for bit with the oracle's

The oracle (oracle/, test infrastructure) runs only in this file's
cpu_baseline leg: it is timed there on bounded samples of each workload, and
the outputs it computes on them are the ones each line's parity compares the
GPU's with.  `--workload` selects the other configurations; each prints one
line with its own cpu_baseline.
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

# VALU lane-op peak: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz (one full-rate
# wave64 instruction per SIMD every 4 clocks)
VALU_PEAK_LANE_OPS = 256 * 64 * 2.4e9
HBM_PEAK = 8.0e12
INT8_MFMA_PEAK = 5.0e15             # dense int8 ops/s (2 per MAC)
INT8_OPS_PER_MFMA = 2 * 16 * 16 * 64  # v_mfma_i32_16x16x64_i8, per wave instruction
# the f32 det_gemm kernel's work per product (MAC): one 64-bit LDS atomic add
# into a cell, and five VALU instructions (exponent-word add with the x word
# broadcast, cell address, shift amount, 24x24-bit product with x's
# significand from an SGPR, 64-bit shift)
GEMM8_LDS_ATOMICS_PER_MAC = 1
GEMM8_VALU_OPS_PER_MAC = 5
KERNEL_SOURCE = os.path.join(ROOT, "bitwise_deterministic_exact_amd", "csrc", "detgemm.hip")
PROBE_LIB = os.path.join(ROOT, "bitwise_deterministic_exact_amd", "liblds_probe.so")
PROFILE_RECORD = os.path.join(ROOT, "profiles", "k_gemm8_f32_4096_wide.md")
MC_PROFILE_RECORD = os.path.join(ROOT, "profiles", "k_slice_mma_bf16_8192x4096x4096.md")


class KernelEvents:
    """HIP events that libdetgemm.so records around the GEMM kernel of each
    call (det_set_kernel_events): one start/stop pair per timed step, on the
    stream the kernel runs on, read after the timed region."""

    def __init__(self, lib, n: int):
        import ctypes
        self.ctypes = ctypes
        # the HIP runtime torch loaded, which libdetgemm.so shares (same soname)
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.lib = lib
        self.pairs = []
        for _ in range(n):
            a, b = ctypes.c_void_p(), ctypes.c_void_p()
            if self.hip.hipEventCreate(ctypes.byref(a)) or self.hip.hipEventCreate(ctypes.byref(b)):
                raise RuntimeError("hipEventCreate failed")
            self.pairs.append((a, b))

    def arm(self, i: int) -> None:
        self.lib.det_set_kernel_events(self.pairs[i][0], self.pairs[i][1])

    def disarm(self) -> None:
        self.lib.det_set_kernel_events(None, None)

    def mean_ms(self) -> float:
        """average start-to-stop time (call after the device has synchronised)"""
        tot = 0.0
        for a, b in self.pairs:
            ms = self.ctypes.c_float()
            if self.hip.hipEventElapsedTime(self.ctypes.byref(ms), a, b):
                raise RuntimeError("hipEventElapsedTime failed")
            tot += ms.value
        return tot / len(self.pairs)

    def close(self) -> None:
        self.disarm()
        for a, b in self.pairs:
            self.hip.hipEventDestroy(a)
            self.hip.hipEventDestroy(b)


def lds_atomic_peak(bits: int, stream) -> dict:
    """The measured rate of non-returning LDS atomic adds (64-bit for the f32
    cells, 32-bit for bf16's) over all CUs, from the probe library
    (csrc/lds_probe.hip): lane-atomics per second, and per CU per clock at
    the 2.4 GHz peak engine clock."""
    import ctypes
    lib = ctypes.CDLL(PROBE_LIB)
    lib.lds_probe_add_rate.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                       ctypes.POINTER(ctypes.c_float)]
    lib.lds_probe_lane_ops.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int]
    lib.lds_probe_lane_ops.restype = ctypes.c_double
    blocks, steps = 2048, 4096
    ms = ctypes.c_float()
    rc = lib.lds_probe_add_rate(bits, blocks, steps, ctypes.c_void_p(stream), ctypes.byref(ms))
    if rc != 0:
        raise RuntimeError(f"LDS probe failed ({rc})")
    rate = lib.lds_probe_lane_ops(bits, blocks, steps) / (ms.value * 1e-3)
    return {"rate": rate, "per_cu_clock": rate / 256 / 2.4e9, "ms": ms.value,
            "probe": f"k_lds_add_rate<{bits}-bit>: {blocks} workgroups x {steps} adds per lane"}


def profile_record(path: str = PROFILE_RECORD, kernel: str = None):
    """A kernel's per-launch counters from a committed rocprofv3 summary (its
    `profile-record:` line, the first one or the one naming `kernel`): VALU
    instructions, FETCH_SIZE and WRITE_SIZE with the copy calibration, and
    whether the kernel source is still the one they were taken on.  None if
    there is no record."""
    import hashlib
    try:
        with open(path) as f:
            recs = [json.loads(l.split(":", 1)[1]) for l in f if l.startswith("profile-record:")]
        rec = next(r for r in recs if kernel is None or r["kernel"] == kernel)
        with open(KERNEL_SOURCE, "rb") as f:
            rec["current"] = hashlib.sha256(f.read()).hexdigest() == rec["source_sha256"]
        return rec
    except (OSError, StopIteration, KeyError, ValueError):
        return None


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ---------------------------------------------------------------- the cpu_baseline leg
# The only code in this file that runs the oracle (oracle/, test
# infrastructure, never on the timed GPU path).  It times the oracle on the
# host over bounded samples of each workload; the outputs the oracle computes
# on those samples are the ones the GPU's outputs are compared with.

def host_threads() -> int:
    return min(os.cpu_count() or 1, 16)


def host_cpu() -> str:
    """The host's CPU model and logical CPU count (Linux /proc/cpuinfo)."""
    model = "unknown CPU"
    try:
        with open("/proc/cpuinfo") as f:
            model = next(l.split(":", 1)[1].strip() for l in f if l.startswith("model name"))
    except (OSError, StopIteration):
        pass
    return f"{model}, {os.cpu_count()} logical CPUs"


def baseline_entry(macs: float, seconds: float, threads: int, sample: str) -> dict:
    return {"value": round(macs / max(seconds, 1e-9) / 1e9, 4), "unit": "GMAC/s", "cores": threads,
            "kind": "oracle", "sample": f"{sample} ({macs:.3g} MAC, {seconds:.2f} s)", "host": host_cpu()}


def cpu_baseline(xb: np.ndarray, wb: np.ndarray, target_s: float = 15.0, threads: int = 0) -> dict:
    """Time the plain C oracle on a block of whole output rows (all N columns,
    full K) sized for roughly ``target_s`` seconds of host work."""
    from oracle import c_oracle
    threads = threads or host_threads()
    K = xb.shape[1]
    N = wb.shape[0]
    cal_rows = min(2 * threads, xb.shape[0])
    t0 = time.perf_counter()
    c_oracle.partial(xb[:cal_rows], wb, nthreads=threads)
    rate = cal_rows * N * K / max(time.perf_counter() - t0, 1e-6)
    rows = int(max(threads, min(xb.shape[0], target_s * rate / (N * K))))
    rows = min(xb.shape[0], (rows // threads) * threads or threads)
    t0 = time.perf_counter()
    c_oracle.partial(xb[:rows], wb, nthreads=threads)
    dt = time.perf_counter() - t0
    return baseline_entry(rows * N * K, dt, threads,
                          f"plain C oracle (exact_oracle.c), raw digits of the first {rows} output rows "
                          f"x all {N} columns at full K={K}")


def oracle_pairs(xb: np.ndarray, wb: np.ndarray, rows, cols) -> np.ndarray:
    """The oracle's fp32 bits of the outputs (rows[i], cols[i])."""
    from oracle import c_oracle
    return c_oracle.gemm_pairs(xb, wb, rows, cols, nthreads=host_threads())


def oracle_gemm(xb: np.ndarray, wb: np.ndarray):
    """The oracle's fp32 bits of every output, and the seconds it took."""
    from oracle import c_oracle
    t0 = time.perf_counter()
    y = c_oracle.gemm(xb, wb, nthreads=host_threads())
    return y, time.perf_counter() - t0


def oracle_digits(xb: np.ndarray, wb: np.ndarray, threads: int = 0):
    """The oracle's raw digits of every output, and the seconds they took."""
    from oracle import c_oracle
    t0 = time.perf_counter()
    d = c_oracle.partial(xb, wb, nthreads=threads or host_threads())
    return d, time.perf_counter() - t0


def oracle_python_digits(xb: np.ndarray, wb: np.ndarray, dtype: str):
    """The plain Python (big-integer) oracle's raw digits, and its seconds."""
    from oracle import exact
    t0 = time.perf_counter()
    d = exact.partial(xb, wb, dtype)
    return d, time.perf_counter() - t0


def oracle_combine_finalize(parts) -> np.ndarray:
    from oracle import c_oracle
    return c_oracle.finalize(c_oracle.combine(parts))


def oracle_mse_bits(yb: np.ndarray, tb: np.ndarray):
    """fp32 bits of RNE(sum (y - t)^2) / n from the oracle: the exact sum is
    sum y y + sum t t - 2 sum y t, each from the oracle's raw digits over
    K-slices within its 2^19 limit (raw digits add), rounded by the oracle,
    then one IEEE fp32 division by n.  Also the seconds it took."""
    from oracle import c_oracle
    n = yb.size
    t0 = time.perf_counter()

    def value(a, b):
        total = 0
        for lo in range(0, n, 400_000):
            d = c_oracle.partial(a[lo:lo + 400_000].reshape(1, -1), b[lo:lo + 400_000].reshape(1, -1))
            total += sum(int(v) << (32 * j) for j, v in enumerate(d.reshape(-1).tolist()))
        return total

    exact = value(yb, yb) + value(tb, tb) - 2 * value(yb, tb)
    digits = [(exact >> (32 * j)) & 0xFFFFFFFF for j in range(17)] + [exact >> (32 * 17)]
    s32 = np.array([c_oracle.finalize(np.array(digits, dtype=np.int64).reshape(1, 18))[0]],
                   dtype=np.uint32).view(np.float32)[0]
    bits = int(np.array([np.float32(s32) / np.float32(n)], dtype=np.float32).view(np.uint32)[0])
    return bits, time.perf_counter() - t0


# ---------------------------------------------------------------- the GPU measurements

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
    ap.add_argument("--workload", default="wide4096",
                    choices=["wide4096", "small", "bf16cancel", "ksharded", "detlinear", "matrixcore", "loss"],
                    help="wide4096 (default, the headline): f32 4096^3 wide range; the others time "
                         "the f32 64x64x256, the bf16 1024^3, the 16-shard K=2^19 and the DetLinear "
                         "configurations, "
                         "(matrixcore) det_gemm on the DetLinear forward shape and (loss) the exact "
                         "mean-squared-error reduction of a DetLinear output")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the exact GEMM here has no multi-GPU path "
              "(each GPU would run its own K- or output-shard of the GEMM, and the shards' raw "
              "digits would be added with det_combine).", file=sys.stderr)
        return 2

    import torch
    import bitwise_deterministic_exact_amd as det
    from workloads import c3_wide_f32

    if args.workload != "wide4096":
        return other_workload(args)

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
    stream = torch.cuda.current_stream(dev)
    kev = KernelEvents(det._lib.load(), args.steps)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(args.steps):
        kev.arm(i)
        step()
    end.record(stream)
    kev.disarm()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    kernel_ms = kev.mean_ms()
    kev.close()
    gmacs = macs / (ms * 1e-3) / 1e9
    log(f"det_gemm {n}^3: {ms:.3f} ms/step, {gmacs:.1f} GMAC/s; GEMM kernel {kernel_ms:.3f} ms per launch")
    peak = lds_atomic_peak(64, stream.cuda_stream)
    log(f"LDS 64-bit atomic peak: {peak['rate'] / 1e12:.3f} T lane-ops/s ({peak['per_cu_clock']:.2f} per CU per clock)")

    # parity on sampled outputs (bit for bit against the C oracle)
    rng = np.random.default_rng(1234)
    rows = rng.integers(0, M, 256)
    cols = rng.integers(0, N, 256)
    got = y.cpu().numpy().view(np.uint32)[rows, cols]
    want = oracle_pairs(xb, wb, rows, cols)
    parity_ok = bool(np.array_equal(got, want))
    log(f"parity on 256 sampled outputs: {'bit-exact' if parity_ok else 'MISMATCH'}")

    # roofline: the GEMM kernel is held to its LDS atomics (one 64-bit add per
    # MAC) and its VALU (six instructions per MAC); the atomics bind.
    # achieved = atomic lane-ops per launch / the launch's duration measured
    # above with HIP events on its stream; peak = the atomic rate the probe
    # measured just now on this GPU.  traffic only while the committed profile
    # matches the kernel source.
    rec = profile_record()
    atomics = GEMM8_LDS_ATOMICS_PER_MAC * macs
    achieved = atomics / (kernel_ms * 1e-3)
    traffic = (int((rec["fetch_kib"] * rec["fetch_scale"] + rec["write_kib"] * rec["write_scale"]) * 1024)
               if rec and rec["current"] and rec["macs"] == macs else None)
    valu_issued = rec["valu_insts"] * 64 if rec and rec["current"] and rec["macs"] == macs else None
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
        "roofline": {"bound": "lds",
                     "achieved": round(achieved / 1e12, 4),
                     "peak": round(peak["rate"] / 1e12, 4), "unit": "T LDS-atomic lane-ops/s",
                     "frac": round(achieved / peak["rate"], 4),
                     "traffic": traffic,
                     "kernel": "k_gemm8<f32, 4-bit cells, 2 rows, 16 waves>",
                     "kernel_ms": round(kernel_ms, 4),
                     "per_mac": f"{GEMM8_LDS_ATOMICS_PER_MAC} ds_add_u64 lane-op + "
                                f"{GEMM8_VALU_OPS_PER_MAC} VALU lane-ops",
                     "peak_source": f"measured in this run: {peak['probe']}, "
                                    f"{peak['per_cu_clock']:.2f} lane-ops per CU per 2.4 GHz clock",
                     # the other unit the kernel is held to, at the same
                     # launch time: the VALU work per MAC over the VALU peak
                     "valu_frac": round(GEMM8_VALU_OPS_PER_MAC * macs / (kernel_ms * 1e-3) / VALU_PEAK_LANE_OPS, 4),
                     # VALU lane-ops issued per launch (rocprofv3
                     # SQ_INSTS_VALU x 64, committed profile) over the peak
                     "valu_issue_frac": (round(valu_issued / (kernel_ms * 1e-3) / VALU_PEAK_LANE_OPS, 4)
                                         if valu_issued else None),
                     "profile_current": bool(rec and rec["current"])},
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
        kev = KernelEvents(det._lib.load(), reps)
        for i in range(reps):
            kev.arm(i)
            pb = det.det_gemm_partial(x[:, h:], w[:, h:], check_finite=False)
        kev.disarm()
        torch.cuda.synchronize()
        part_kernel_ms = kev.mean_ms()
        kev.close()
        t_comb, acc = timed(lambda: det.det_combine([pa, pb]))
        t_fin, yf = timed(lambda: det.det_finalize(acc))
        same = bool(torch.equal(yf.view(torch.int32), y.view(torch.int32)))
        acc_bytes = M * N * 18 * 8
        # k_partial (f32): two 64-bit LDS atomic adds per product (four 16-bit
        # fields, two to a counter), against the same measured atomic peak
        part_atomics = 2 * M * N * (K - h)
        aux["partial_half_k"] = {"ms": round(t_part, 3),
                                 "GMAC/s": round(M * N * h / (t_part * 1e-3) / 1e9, 2),
                                 "kernel_ms": round(part_kernel_ms, 3),
                                 "roofline": {"bound": "lds", "per_mac": "2 ds_add_u64 lane-ops",
                                              "frac": round(part_atomics / (part_kernel_ms * 1e-3) / peak["rate"], 4)}}
        aux["combine_2"] = {"ms": round(t_comb, 3),
                            "GB/s": round(3 * acc_bytes / (t_comb * 1e-3) / 1e9, 1),
                            "hbm_frac": round(3 * acc_bytes / (t_comb * 1e-3) / HBM_PEAK, 4)}
        aux["finalize"] = {"ms": round(t_fin, 3),
                           "GB/s": round((acc_bytes + M * N * 4) / (t_fin * 1e-3) / 1e9, 1),
                           "hbm_frac": round((acc_bytes + M * N * 4) / (t_fin * 1e-3) / HBM_PEAK, 4)}
        aux["sharded_equals_unsharded"] = same
        del pa, pb, acc, yf
        aux["matrix_core_bf16"] = matrix_core_aux(det, dev, timed)
        result["aux"] = aux
        log(f"aux: {aux}")

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


def matrix_core_aux(det, dev, timed) -> dict:
    """det_gemm on the DetLinear forward shape (bf16 N(0,1), 8192 x 4096 x
    4096), where the call picks the matrix-core path: time, the path it took,
    the digit GEMMs' int8 rate against the dense int8 MFMA peak (the whole
    call's time, so a lower bound on the kernel's), and the same outputs
    compared bit for bit with the digit-accumulator path."""
    import torch
    import workloads as W
    wl = W.c5_detlinear_bf16()
    x = torch.from_numpy(wl.x.view(np.int16)).view(torch.bfloat16).to(dev)
    w = torch.from_numpy(wl.w.view(np.int16)).view(torch.bfloat16).to(dev)
    M, K = x.shape
    N = w.shape[0]
    t, y = timed(lambda: det.det_gemm(x, w, check_finite=False))
    plan = det.last_gemm_plan()
    # the kernel's own time, with the plan's S fixed: on the default path the
    # events would also span the launches of the paths the plan did not pick
    kev = KernelEvents(det._lib.load(), 3)
    with det.gemm_path("slices", plan["slices"]) if plan["slices"] > 0 else det.gemm_path("auto"):
        for i in range(3):
            kev.arm(i)
            det.det_gemm(x, w, check_finite=False)
        kev.disarm()
    torch.cuda.synchronize()
    kms = kev.mean_ms()
    kev.close()
    det.set_gemm_path("accumulator")
    try:
        y_acc = det.det_gemm(x, w, check_finite=False)
    finally:
        det.set_gemm_path("auto")
    S = plan["slices"]
    ops = 2.0 * S * S * M * N * K
    out = {"M": M, "N": N, "K": K, "ms": round(t, 3), "GMAC/s": round(M * N * K / (t * 1e-3) / 1e9, 1),
           "plan": plan, "equals_accumulator_path": bool(torch.equal(y.view(torch.int32),
                                                                     y_acc.view(torch.int32)))}
    if S:
        # executed MFMAs: rocprofv3 SQ_INSTS_MFMA per launch from the committed
        # profile (products with an all-zero lowest-plane fragment are skipped)
        rec = profile_record(MC_PROFILE_RECORD, f"k_slice_mma<{S}, 2>")
        executed = (rec["mfma_insts"] * INT8_OPS_PER_MFMA
                    if rec and rec["current"] and rec["int8_ops"] == ops else None)
        out["roofline"] = {"bound": "mfma", "kernel": f"k_slice_mma<{S}>", "kernel_ms": round(kms, 4),
                           "achieved": round(executed / (kms * 1e-3) / 1e12, 1) if executed else None,
                           "peak": INT8_MFMA_PEAK / 1e12, "unit": "TOP/s int8",
                           "frac": round(executed / (kms * 1e-3) / INT8_MFMA_PEAK, 4) if executed else None,
                           "ops": "executed v_mfma_i32_16x16x64_i8 x 32768 int8 ops per launch",
                           "dense_frac": round(ops / (kms * 1e-3) / INT8_MFMA_PEAK, 4),
                           "dense_ops": "2 S^2 M N K int8 ops (skipped products counted as done)",
                           "profile_current": bool(rec and rec["current"])}
    del x, w, y, y_acc
    return out


def loss_workload(det, dev, steps, warmup) -> dict:
    """exact_mse_loss of a DetLinear-sized f32 output (8192 x 4096, N(0,1))
    against an N(0,1) target: the time of the whole loss, the squared-
    difference kernel's share against the HBM roofline (its algorithmic bytes
    are the two operands, read once), and the loss's bits against the
    oracle's exact sum (sum y^2 + sum t^2 - 2 sum y t, formed from the
    oracle's digits of the three dot products, rounded by the oracle)."""
    import torch
    rng = np.random.default_rng(8)
    n = 8192 * 4096
    yb = rng.standard_normal(n, dtype=np.float32).view(np.uint32)
    tb = rng.standard_normal(n, dtype=np.float32).view(np.uint32)
    y = torch.from_numpy(yb.view(np.float32)).to(dev)
    t = torch.from_numpy(tb.view(np.float32)).to(dev)
    stream = torch.cuda.current_stream(dev)

    def timed(fn):
        for _ in range(max(1, warmup)):
            fn()
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record(stream)
        for _ in range(steps):
            fn()
        e.record(stream)
        torch.cuda.synchronize()
        return s.elapsed_time(e) / steps

    ms_loss = timed(lambda: det.exact_mse_loss(y, t))
    ms_digits = timed(lambda: det.exact_sqdiff_digits(y, t, check_finite=False))
    ms_dot = timed(lambda: det.exact_dot_digits(y, t, check_finite=False))
    loss = det.exact_mse_loss(y, t)
    got = int(loss.reshape(1).cpu().view(torch.int32).numpy().view(np.uint32)[0])
    want, t_oracle = oracle_mse_bits(yb, tb)
    nbytes = 2 * 4 * n
    rec = profile_record(os.path.join(ROOT, "profiles", "k_dot_f32_loss_8192x4096.md"),
                         "k_dot<f32, squared difference>")
    traffic = (int((rec["fetch_kib"] * rec["fetch_scale"] + rec["write_kib"] * rec["write_scale"]) * 1024)
               if rec and rec["current"] and rec["bytes"] == nbytes else None)
    return dict(metric="exact MSE loss, GB/s of operands (f32 8192x4096 prediction and target)",
                value=round(nbytes / (ms_loss * 1e-3) / 1e9, 1), unit="GB/s", ms_per_step=round(ms_loss, 4),
                dtype="int64",
                roofline={"bound": "hbm", "kernel": "k_dot<f32, squared difference> (+ the digit clear)",
                          "achieved": round(nbytes / (ms_digits * 1e-3) / 1e9, 1), "peak": HBM_PEAK / 1e9,
                          "unit": "GB/s", "frac": round(nbytes / (ms_digits * 1e-3) / HBM_PEAK, 4),
                          "traffic": traffic, "bytes": "8 n: both operands read once",
                          "profile_current": bool(rec and rec["current"])},
                dot={"kernel": "k_dot<f32, a*b>", "ms": round(ms_dot, 4),
                     "GB/s": round(nbytes / (ms_dot * 1e-3) / 1e9, 1),
                     "frac": round(nbytes / (ms_dot * 1e-3) / HBM_PEAK, 4)},
                parity={"loss_bits": got, "oracle_bits": want, "bit_exact": got == want},
                cpu_baseline=baseline_entry(3 * n, t_oracle, 1,
                                            "plain C oracle, the exact sum of the 3n products of the "
                                            "whole loss (one output: one thread)"),
                config={"workload": "exact_mse_loss of an 8192x4096 f32 output, N(0,1) prediction and "
                                    "target, seed 8", "n": n})


def small_workload(det, dev, steps, warmup) -> dict:
    """The f32 64x64x256 configuration (launch-bound): det_gemm and its
    two-shard composition at k = 100, every output and every digit against
    the oracle, and the oracle's time on the whole workload with one host
    thread, with all of them, and for the plain Python (big-integer) oracle."""
    import torch
    import workloads as W
    wl = W.c1_small_f32()
    xb, wb = wl.bits()
    x = torch.from_numpy(wl.x).to(dev)
    w = torch.from_numpy(wl.w).to(dev)
    y = torch.empty(64, 64, dtype=torch.float32, device=dev)
    ms = _timed(lambda: det.det_gemm(x, w, check_finite=False, out=y), steps, warmup)
    c = wl.cuts[0]
    parts = [det.det_gemm_partial(x[:, :c], w[:, :c], check_finite=False),
             det.det_gemm_partial(x[:, c:], w[:, c:], check_finite=False)]
    whole = det.det_gemm_partial(x, w, check_finite=False)
    y_s = det.det_finalize(det.det_combine(parts))
    digits, t_all = oracle_digits(xb, wb)
    digits_1, t_one = oracle_digits(xb, wb, threads=1)
    digits_py, t_py = oracle_python_digits(xb, wb, "f32")
    want = oracle_combine_finalize([digits])
    got = y.cpu().view(torch.int32).numpy().view(np.uint32)
    ok = (np.array_equal(got, want) and np.array_equal(whole.cpu().numpy(), digits)
          and torch.equal(y_s.view(torch.int32), y.view(torch.int32))
          and np.array_equal(digits_1, digits) and np.array_equal(digits_py, digits))
    macs = 64 * 64 * 256
    return dict(metric="exact-GEMM GMAC/s (f32 64x64x256, launch-bound)",
                value=round(macs / (ms * 1e-3) / 1e9, 3), unit="GMAC/s", ms_per_step=round(ms, 4),
                dtype="int64",
                parity={"outputs": "all 64^2, fp32 and raw digits", "shards_compose": True, "bit_exact": bool(ok)},
                cpu_baseline=baseline_entry(macs, t_all, host_threads(), "plain C oracle, every output"),
                cpu_baseline_1thread=baseline_entry(macs, t_one, 1, "plain C oracle, every output"),
                cpu_baseline_python=baseline_entry(macs, t_py, 1, "plain Python big-integer oracle, every output"),
                config={"workload": wl.name + ", seed 0, shards [0,100) and [100,256)", "M": 64, "N": 64,
                        "K": 256})


def _timed(fn, steps, warmup):
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(steps):
        fn()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / steps


def other_workload(args) -> int:
    """The other configurations: one JSON line each with their throughput, a
    parity check (full or sampled) against the oracle and the oracle's own
    rate on the host (cpu_baseline)."""
    import torch
    import bitwise_deterministic_exact_amd as det
    import workloads as W

    dev = torch.device("cuda:0")
    rng = np.random.default_rng(99)
    out = {"n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "data": "synthetic"}

    def to_dev(bits, dt):
        if dt == "f32":
            return torch.from_numpy(bits.view(np.float32)).to(dev)
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)

    def bits32(t):
        return t.cpu().contiguous().view(torch.int32).numpy().view(np.uint32)

    if args.workload == "matrixcore":
        steps, warmup = args.steps, args.warmup

        def timed(fn):
            for _ in range(max(1, warmup)):
                fn()
            torch.cuda.synchronize()
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record()
            for _ in range(steps):
                out_ = fn()
            e.record()
            torch.cuda.synchronize()
            return s.elapsed_time(e) / steps, out_

        mc = matrix_core_aux(det, dev, timed)
        wl = W.c5_detlinear_bf16()
        x, w = to_dev(wl.x, "bf16"), to_dev(wl.w, "bf16")
        y = det.det_gemm(x, w, check_finite=False)
        rows, cols = rng.integers(0, 8192, 64), rng.integers(0, 4096, 64)
        ok = bool(np.array_equal(bits32(y)[rows, cols], oracle_pairs(wl.x, wl.w, rows, cols)))
        ok = ok and mc["equals_accumulator_path"]
        out.update(metric="exact-GEMM GMAC/s (bf16 8192x4096x4096 N(0,1), det_gemm's own path choice)",
                   value=mc["GMAC/s"], unit="GMAC/s", ms_per_step=mc["ms"], dtype="int8",
                   plan=mc["plan"], roofline=mc.get("roofline"),
                   parity={"sampled_outputs": 64, "bit_exact": ok,
                           "equals_accumulator_path": mc["equals_accumulator_path"]},
                   cpu_baseline=cpu_baseline(wl.x, wl.w, target_s=3.0),
                   config={"workload": wl.name + ", seed 4 (the DetLinear forward GEMM)",
                           "M": 8192, "N": 4096, "K": 4096})
    elif args.workload == "loss":
        out.update(loss_workload(det, dev, args.steps, args.warmup))
    elif args.workload == "small":
        out.update(small_workload(det, dev, args.steps, args.warmup))
    elif args.workload == "bf16cancel":
        wl = W.c2_bf16_cancel()
        xb, wb = wl.bits()
        x, w = to_dev(xb, "bf16"), to_dev(wb, "bf16")
        y = torch.empty(1024, 1024, dtype=torch.float32, device=dev)
        ms = _timed(lambda: det.det_gemm(x, w, check_finite=False, out=y), args.steps, args.warmup)
        want, t_oracle = oracle_gemm(xb, wb)
        ok = bool(np.array_equal(bits32(y), want))
        macs = 1024 ** 3
        out.update(metric="exact-GEMM GMAC/s (bf16 1024^3, 10% negated w columns)",
                   value=round(macs / (ms * 1e-3) / 1e9, 2), unit="GMAC/s", ms_per_step=round(ms, 4),
                   dtype="int64", parity={"outputs": "all 1024^2", "bit_exact": ok},
                   cpu_baseline=baseline_entry(macs, t_oracle, host_threads(),
                                               "plain C oracle, every output of the workload"),
                   cpu_baseline_1thread=cpu_baseline(xb, wb, target_s=2.0, threads=1),
                   config={"workload": wl.name + ", seed 1", "M": 1024, "N": 1024, "K": 1024})
    elif args.workload == "ksharded":
        wl = W.c4_ksharded_f32()
        xb, wb = wl.bits()
        x, w = to_dev(xb, "f32"), to_dev(wb, "f32")
        K = x.shape[1]
        bounds = W.shard_bounds(K, wl.cuts)

        def sharded():
            parts = [det.det_gemm_partial(x[:, a:b], w[:, a:b], check_finite=False) for a, b in bounds]
            return det.det_finalize(W.apply_fold(parts, wl.fold, det.det_combine))

        y_s = sharded()
        y_u = det.det_gemm(x, w, check_finite=False)
        same = bool(torch.equal(y_s.view(torch.int32), y_u.view(torch.int32)))
        rows, cols = rng.integers(0, 2048, 16), rng.integers(0, 2048, 16)
        ok = same and bool(np.array_equal(bits32(y_u)[rows, cols], oracle_pairs(xb, wb, rows, cols)))
        steps = max(1, min(args.steps, 3))
        ms_s = _timed(sharded, steps, 0)
        ms_u = _timed(lambda: det.det_gemm(x, w, check_finite=False), steps, 0)
        macs = 2048 * 2048 * K
        out.update(metric="exact-GEMM GMAC/s (f32 2048^2 x K=2^19, 16 K-shards composed by a fold tree)",
                   value=round(macs / (ms_s * 1e-3) / 1e9, 2), unit="GMAC/s", ms_per_step=round(ms_s, 3),
                   steps=steps, warmup=0, dtype="int64",
                   unsharded={"ms": round(ms_u, 3), "GMAC/s": round(macs / (ms_u * 1e-3) / 1e9, 2)},
                   parity={"sharded_equals_unsharded": same, "sampled_outputs": 16, "bit_exact": ok},
                   cpu_baseline=cpu_baseline(xb, wb, target_s=3.0),
                   config={"workload": wl.name + ", seed 3", "M": 2048, "N": 2048, "K": K})
    else:
        wl = W.c5_detlinear_bf16()
        layer = det.DetLinear(4096, 4096, device=dev, dtype=torch.bfloat16)
        with torch.no_grad():
            layer.weight.copy_(to_dev(wl.w, "bf16"))
        x = to_dev(wl.x, "bf16").requires_grad_(True)

        def step():
            x.grad = None
            layer.weight.grad = None
            det.exact_mse_loss(layer(x)).backward()          # mean(y^2), its sum formed exactly

        ms = _timed(step, args.steps, args.warmup)
        y = layer(x).detach()
        rows, cols = rng.integers(0, 8192, 64), rng.integers(0, 4096, 64)
        ok = bool(np.array_equal(bits32(y)[rows, cols], oracle_pairs(wl.x, wl.w, rows, cols)))
        macs = 3 * 8192 * 4096 * 4096
        out.update(metric="DetLinear 4096->4096 bf16 fwd+bwd with the loss mean(y^2), 8192 tokens: "
                          "exact-GEMM GMAC/s",
                   value=round(macs / (ms * 1e-3) / 1e9, 2), unit="GMAC/s", ms_per_step=round(ms, 3),
                   tokens_per_s=round(8192 / (ms * 1e-3), 1), dtype="int64",
                   parity={"sampled_forward_outputs": 64, "bit_exact": ok},
                   cpu_baseline=cpu_baseline(wl.x, wl.w, target_s=3.0),
                   config={"workload": wl.name + ", seed 4", "tokens": 8192, "in": 4096, "out": 4096})
    print(json.dumps(out), flush=True)
    return 0 if out["parity"].get("bit_exact", False) else 1


if __name__ == "__main__":
    sys.exit(main())
