"""Build the HIP library libdetgemm.so in-tree for gfx950 with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SOURCES = [os.path.join(PKG, "csrc", "detgemm.hip")]
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libdetgemm.so")
# the benchmark's LDS-atomic peak probe: its own library, never loaded by the package
PROBE_SOURCES = [os.path.join(PKG, "csrc", "lds_probe.hip")]
PROBE_LIB = os.path.join(PKG, "liblds_probe.so")
ARCH = "gfx950"

# -packed-fp32-ops off: no v_pk_{add,mul,fma}_f32 in any generated code
HIPCC_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-shared", f"--offload-arch={ARCH}",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-Wall", "-Wno-unused-function", f"-I{INCLUDE}"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return "hipcc"


def _hipcc(sources, out: str, verbose: bool) -> str:
    cmd = [hipcc(), *HIPCC_FLAGS, "-o", out + ".tmp", *sources]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in res.stderr.splitlines()
                    if "packed-fp32-ops" not in l and l.strip())
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err:
        print(err, file=sys.stderr)
    os.replace(out + ".tmp", out)
    return out


def build(verbose: bool = False) -> str:
    """Build libdetgemm.so and the benchmark's probe library."""
    _hipcc(PROBE_SOURCES, PROBE_LIB, verbose)
    return _hipcc(SOURCES, LIB, verbose)


def device_asm(out_path: str) -> str:
    """Write the gfx950 assembly of the kernels (for inspection)."""
    cmd = [hipcc(), "-O3", "-std=c++17", f"--offload-arch={ARCH}", "--cuda-device-only", "-S",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", f"-I{INCLUDE}",
           "-o", out_path, *SOURCES]
    subprocess.run(cmd, check=True, capture_output=True)
    return out_path


if __name__ == "__main__":
    print(build(verbose=True))
