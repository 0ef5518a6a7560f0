"""The committed rocprofv3 summaries under profiles/ stay usable (CPU only).

Each summary states the commands that produced it and ends with
`profile-record:` lines that bench.py reads for the traffic and instruction
counts it reports.  These tests check, without a GPU:
- every command runs a committed Python file of this repository;
- every counter pass fits in one rocprofv3 run: rocprofv3 does not split
  counters over passes, and a pass that asks a block for more counters than
  it has fails on this hardware;
- no counter pass is combined with a system or runtime trace;
- every record parses and carries the fields bench.py reads.
"""
from __future__ import annotations

import glob
import json
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROFILES = sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md")))

# counters each block can collect in one pass (MI355X, ROCm 7.2), and the
# TCC slots that the derived FETCH_SIZE and WRITE_SIZE take
BLOCK_LIMIT = {"SQ": 8, "TCC": 4, "TCP": 4, "TA": 2, "TD": 2, "GRBM": 2}
DERIVED_TCC = {"FETCH_SIZE": 3, "WRITE_SIZE": 2}


def _commands(path: str) -> list[str]:
    with open(path) as f:
        return [l.strip() for l in f if l.startswith("    rocprofv3 ")]


def _records(path: str) -> list[dict]:
    with open(path) as f:
        return [json.loads(l.split(":", 1)[1]) for l in f if l.startswith("profile-record:")]


def test_profiles_exist():
    names = {os.path.basename(p) for p in PROFILES}
    assert {"k_gemm8_f32_4096_wide.md", "k_slice_mma_bf16_8192x4096x4096.md",
            "detlinear_step_bf16_8192x4096.md", "k_dot_f32_loss_8192x4096.md",
            "k_lds_add_rate_probe.md"} <= names


@pytest.mark.parametrize("path", PROFILES, ids=os.path.basename)
def test_commands_run_committed_files(path):
    cmds = _commands(path)
    assert cmds, "a summary gives the command that made it"
    for c in cmds:
        assert " -- " in c, c
        prog = c.split(" -- ", 1)[1].split()
        assert prog[0] in ("python3", "python"), c
        script = prog[1]
        assert not script.startswith("_work") and "/_work/" not in script, c
        assert os.path.isfile(os.path.join(ROOT, script)), c


@pytest.mark.parametrize("path", PROFILES, ids=os.path.basename)
def test_counter_passes_fit_one_run(path):
    for c in _commands(path):
        opts = c.split(" -- ", 1)[0].split()
        if "--pmc" not in opts:
            continue
        for banned in ("-s", "--sys-trace", "-r", "--runtime-trace", "--hip-trace", "--hsa-trace",
                       "--memory-copy-trace", "--scratch-memory-trace", "--marker-trace"):
            assert banned not in opts, c
        i = opts.index("--pmc") + 1
        counters = []
        while i < len(opts) and not opts[i].startswith("-"):
            counters.append(opts[i])
            i += 1
        assert counters, c
        used = dict.fromkeys(BLOCK_LIMIT, 0)
        seen = set()
        for name in counters:
            base = re.sub(r"_(sum|avr|min|max)$", "", name)
            if base in seen:
                continue
            seen.add(base)
            if base in DERIVED_TCC:
                used["TCC"] += DERIVED_TCC[base]
                continue
            block = base.split("_", 1)[0]
            assert block in used, f"unknown counter block in {name}: {c}"
            used[block] += 1
        for block, n in used.items():
            assert n <= BLOCK_LIMIT[block], f"{block}: {n} counters in one pass: {c}"


@pytest.mark.parametrize("path", PROFILES, ids=os.path.basename)
def test_records_parse(path):
    recs = _records(path)
    if os.path.basename(path) == "detlinear_step_bf16_8192x4096.md":
        return                                    # a step trace; bench.py reads no record from it
    assert recs, "a summary that bench.py can read ends with its record lines"
    with open(path) as f:
        text = f.read()
    m = re.search(r"source\s+`([^`]+)`", text)
    assert m and os.path.isfile(os.path.join(ROOT, m.group(1))), "the summary names its kernel source"
    for r in recs:
        assert isinstance(r["kernel"], str) and r["kernel"]
        assert re.fullmatch(r"[0-9a-f]{64}", r["source_sha256"])
        assert r["avg_us"] > 0


def test_bench_reads_its_records():
    import bench
    for path in (bench.PROFILE_RECORD, bench.MC_PROFILE_RECORD):
        rec = bench.profile_record(path)
        assert rec is not None and isinstance(rec["current"], bool)
        assert rec["fetch_kib"] > 0 and rec["fetch_scale"] > 0
