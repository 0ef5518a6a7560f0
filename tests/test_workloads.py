"""The generated inputs are pinned by SHA-256 (CPU only).

Every parity test and the benchmark draw their operands from the seeded
generators in workloads/; a numpy upgrade, a changed draw order or a changed
rounding step would change those operands without any test noticing.  Each
configuration's operand bits (row-major, x then w) and shard plan are hashed and
compared with tests/golden/workload_digests.json, written once by
tests/golden/make_workload_digests.py from the generators alone.

The K-sharded configuration (two 4 GiB operands, minutes to draw) is checked
only when DET_PIN_LARGE=1 is set; the others run in the default suite.
"""
import json
import os
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.join(HERE, "golden"))

import make_workload_digests as mk  # noqa: E402

with open(os.path.join(HERE, "golden", "workload_digests.json")) as f:
    PINNED = json.load(f)

LARGE = {"c4"}


@pytest.mark.parametrize("name", sorted(mk.GENERATORS))
def test_workload_bits_are_pinned(name):
    if name in LARGE and os.environ.get("DET_PIN_LARGE") != "1":
        pytest.skip("two 4 GiB operands: set DET_PIN_LARGE=1 to draw and hash them")
    wl = mk.GENERATORS[name]()
    pin = PINNED[name]
    assert wl.name == pin["workload"]
    assert list(wl.shape) == pin["shape"] and wl.dtype == pin["dtype"]
    assert mk.digest(wl) == pin["sha256"]


def test_digest_sees_a_one_bit_change():
    wl = mk.GENERATORS["c1"]()
    wl.x.view("u4")[17, 3] ^= 1
    assert mk.digest(wl) != PINNED["c1"]["sha256"]
