"""CPU checks of bench.py's contract pieces that need no GPU: the single-GPU
guard, the spread helper, the algorithmic byte counts behind the roofline
(against the packer's blob size) and the counter record it reads."""
import json
import os
import subprocess
import sys

import numpy as np
import pytest

from quantized_expert_ffn_topk_amd import abi
from quantized_expert_ffn_topk_amd.layer import make_desc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


@pytest.mark.parametrize("n", [2, 8])
def test_more_than_one_gpu_exits_with_a_message(n):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_percentiles_of_a_known_list():
    p = bench.percentiles(list(range(1, 101)))
    assert p["n"] == 100
    assert p["p50"] == pytest.approx(50.5)
    assert p["p10"] == pytest.approx(np.percentile(np.arange(1, 101), 10))
    assert p["p90"] == pytest.approx(np.percentile(np.arange(1, 101), 90))


@pytest.mark.parametrize("g", [32, 64])
def test_section_bytes_add_up_to_the_blob(g):
    # the roofline's per-expert bytes (gate/up and down sections) are the
    # packer's whole blob
    H, F = bench.H, bench.F
    d = make_desc(H, F, bench.E, bench.K_TOP, 1, g, bench.R_SCALE)
    assert bench.gu_section_bytes(H, F, g) + bench.dn_section_bytes(H, F, g) == abi.moe_blob_bytes(d)


def test_counter_record_parses():
    text = open(bench.TRAFFIC_RECORD).read()
    rec = json.loads(text.split("```json", 1)[1].split("```", 1)[0])
    assert rec["kernel"] == "gateup_bs1_kernel, down_bs1h_kernel"
    assert rec["traffic_bytes_per_launch"]["gateup"] > 0
    assert rec["traffic_bytes_per_launch"]["down"] > 0
    for path in rec["sources_sha256"]:
        assert os.path.exists(os.path.join(ROOT, path)), path
    t = bench.measured_traffic()
    # None once a listed source changed since the counters were taken
    assert t is None or t == rec["traffic_bytes_per_launch"]
