"""Write workload_digests.json: the SHA-256 of each generated configuration's
inputs (the operand bit patterns in row-major order, x then w, then the shard
plan where one applies).  Pinning the generators' bits this way means a change
of numpy, of the draw order or of a rounding step cannot change the workloads
silently.  Calls only the generators in workloads/ (no oracle, no GPU).

    python tests/golden/make_workload_digests.py
"""
import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "workload_digests.json")
GENERATORS = {"c1": W.c1_small_f32, "c2": W.c2_bf16_cancel, "c3": W.c3_wide_f32,
              "c4": W.c4_ksharded_f32, "c5": W.c5_detlinear_bf16}


def digest(wl) -> str:
    h = hashlib.sha256()
    xb, wb = wl.bits()
    for a in (xb, wb):
        h.update(memoryview(a.reshape(-1).view(a.dtype)))
    h.update(json.dumps({"cuts": wl.cuts, "fold": wl.fold}).encode())
    return h.hexdigest()


def main() -> None:
    out = {}
    for name, gen in GENERATORS.items():
        wl = gen()
        out[name] = {"workload": wl.name, "shape": list(wl.shape), "dtype": wl.dtype, "sha256": digest(wl)}
        print(name, out[name]["sha256"], flush=True)
        del wl
    with open(OUT, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")


if __name__ == "__main__":
    main()
