"""CPU checks of the parts of bench.py's contract that need no GPU: the
one-GPU refusal, the source hash that ties recorded counters to the kernel
sources, and the rule that counters are used only when that hash matches."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]


def test_source_hash_ignores_comments_not_code(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    src.write_text("// a comment\n__global__ void k(int* p) { p[0] = 1; }  /* note */\n")
    monkeypatch.setattr(bench, "CSRC", str(tmp_path))
    h0 = bench.kernel_source_hash()
    src.write_text("// another comment\n\n   __global__ void k(int* p) { p[0] = 1; }   \n\n")
    assert bench.kernel_source_hash() == h0          # comments, blank lines, indentation
    src.write_text("__global__ void k(int* p) { p[0] = 2; }\n")
    assert bench.kernel_source_hash() != h0          # the code changed
    (tmp_path / "more.h").write_text("#define X 1\n")
    assert bench.kernel_source_hash() != h0          # every csrc file counts


def test_traffic_used_only_on_matching_sources(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILE_DIR", str(tmp_path))
    rec = {"kernel_source_hash": bench.kernel_source_hash(), "traffic_bytes_per_launch": 1234}
    (tmp_path / "traffic_w.json").write_text(json.dumps(rec))
    assert bench.measured_traffic("w") == 1234
    rec["kernel_source_hash"] = "0" * 16
    (tmp_path / "traffic_w.json").write_text(json.dumps(rec))
    assert bench.measured_traffic("w") is None
    assert bench.measured_traffic("absent") is None


def test_committed_profiles_match_the_sources():
    """Every committed traffic record was taken on the kernel sources as
    they are: a kernel change must be followed by new counter runs."""
    recs = sorted(f for f in os.listdir(bench.PROFILE_DIR) if f.startswith("traffic_"))
    assert recs
    h = bench.kernel_source_hash()
    stale = [f for f in recs
             if json.load(open(os.path.join(bench.PROFILE_DIR, f))).get("kernel_source_hash") != h]
    assert not stale, f"recorded on other kernel sources: {stale}"
