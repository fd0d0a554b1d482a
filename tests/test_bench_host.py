"""Host-side checks of bench.py's contract that need no GPU: it refuses more
than one GPU with a message, refuses a batch override without a context,
and reports the stored HBM traffic only for the decode sources it was
measured on."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def run_bench(*args):
    return subprocess.run([sys.executable, BENCH, *args], cwd=ROOT,
                          capture_output=True, text=True, timeout=300)


def test_more_than_one_gpu_is_refused():
    r = run_bench("--gpus", "2")
    assert r.returncode != 0
    assert "one GPU" in r.stderr or "one GPU" in r.stdout
    assert not any(line.startswith("{") for line in r.stdout.splitlines())


def test_batch_override_needs_a_context():
    if not os.path.exists(os.path.join(ROOT, "mla_latent_kv_33_amd",
                                       "libmla.so")):
        pytest.skip("libmla.so not built")
    r = run_bench("--batch", "8")
    assert r.returncode != 0
    assert "--batch needs --context" in r.stderr


def test_stored_traffic_follows_the_source_hash(tmp_path, monkeypatch):
    sys.path.insert(0, ROOT)
    import bench
    s = json.load(open(bench.PMC_SUMMARY))
    # the committed counters are reported only while their hash matches
    expect = (s["hbm_bytes_per_launch"]
              if s["kernel_source_hash"] == bench.kernel_source_hash()
              else None)
    assert bench.stored_traffic(630267904.0) == expect
    # a summary taken on other sources is never reported
    other = dict(s, kernel_source_hash="0" * 16)
    p = tmp_path / "pmc.json"
    p.write_text(json.dumps(other))
    monkeypatch.setattr(bench, "PMC_SUMMARY", str(p))
    assert bench.stored_traffic(630267904.0) is None
    # read and write bytes add up to the reported total
    assert abs(s["hbm_read_bytes_per_launch"] + s["hbm_write_bytes_per_launch"]
               - s["hbm_bytes_per_launch"]) < 1.0
