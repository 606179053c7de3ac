"""Host-side parts of bench.py's contract (no GPU needed): it measures one GPU
only and says so for --gpus above 1; the algorithmic work it reports follows
the stated formulas; its traffic record is tied to the grouped-GEMM sources."""
import json
import os
import subprocess
import sys

import bench
from mixture_experts_layer_topkrouter_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""  # no JSON line


def test_algorithmic_work_of_the_mixtral_slice():
    w = W.WORKLOADS["mixtral_top2_bf16"]
    work = bench.algorithmic(w, n_rows=8192, n_active=8)
    # 2 flops per MAC, three d x d_ff matrices (SwiGLU) per kept row
    assert work["expert_ffn"][1] == 8192 * 2 * 3 * 4096 * 14336
    # weights of the 8 experts + rows in and out + H written and read (bf16)
    assert work["expert_ffn"][2] == 8 * 3 * 4096 * 14336 * 2 + 8192 * 4096 * 2 * 2 + 8192 * 14336 * 2 * 2
    # permute: each token row read once, each kept row written once, 12 B of indices per assignment
    assert work["permute"][1] == 4096 * 4096 * 2 + 8192 * 4096 * 2 + 8192 * 12
    # combine: kept rows read, output written, 8 B per assignment
    assert work["unpermute"][1] == 8192 * 4096 * 2 + 4096 * 4096 * 2 + 8192 * 8


def test_traffic_records_are_keyed_to_the_stage_sources(monkeypatch):
    """A stage's counter record counts only while that stage's kernel sources
    hash to the value it was measured with; otherwise bench.py reports its
    traffic as null."""
    import glob
    paths = sorted(glob.glob(os.path.join(ROOT, "profiles", "*_hbm_traffic.json")))
    assert paths, "no HBM traffic records under profiles/"
    for path in paths:
        name = os.path.basename(path)[:-len("_hbm_traffic.json")]
        with open(path) as f:
            rec = json.load(f)
        assert rec["copy_probe"]["bytes"] > 0
        for stage, st in rec["stages"].items():
            assert st["read_bytes"] >= 0 and st["write_bytes"] >= 0 and len(st["sources_sha256"]) == 64
            fresh = st["sources_sha256"] == bench.stage_sources_sha256(stage)
            expect = int(st["read_bytes"] + st["write_bytes"]) if fresh else None
            assert bench.measured_traffic(name, stage) == expect
        monkeypatch.setattr(bench, "stage_sources_sha256", lambda stage: "0" * 64)
        assert all(bench.measured_traffic(name, stage) is None for stage in rec["stages"])
        monkeypatch.undo()
    assert bench.measured_traffic("no_such_workload") is None
