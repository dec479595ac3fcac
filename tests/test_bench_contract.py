"""bench.py's contract on the host: one GPU only, the options that apply to
the multiscale workload only, and the HBM-traffic records keyed by the digest
of the kernel sources they were taken with."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True,
                          text=True, timeout=300)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_multiscale_options_are_refused_elsewhere():
    r = _run("--workload", "2", "--verify")
    assert r.returncode == 2 and "workload (5) only" in r.stderr


def test_ops_per_pair_counts_the_shifted_loop():
    assert bench.ops_per_pair(3) == 8 and bench.ops_per_pair(1) == 4


def test_traffic_records_match_their_kernel_and_sources(tmp_path, monkeypatch):
    # the committed records resolve for their own workload and kernel only
    assert bench.pmc_traffic("k_lse_valu<3,true>", 2) is not None
    assert bench.pmc_traffic("k_lse_mfma<52>", 3) is not None
    assert bench.pmc_traffic("k_lse_valu<3,true>", 4) is None
    assert bench.pmc_traffic("k_lse_valu<2,true>", 2) is None
    # a record whose digest no longer matches the sources is ignored
    prof = tmp_path / "profiles"
    prof.mkdir()
    name = bench.PMC_RECORDS[2][0]
    text = open(os.path.join(ROOT, "profiles", name)).read()
    digest = bench.kernel_source_digest(bench.PMC_RECORDS[2][1])
    (prof / name).write_text(text.replace(digest, "0" * 64))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_digest", lambda sources=None: digest)
    assert bench.pmc_traffic("k_lse_valu<3,true>", 2) is None
