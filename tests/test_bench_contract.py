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


def test_slots_per_pair_count_each_pair_form():
    # fp32 difference form: 8 VALU + exp2 at 4 slots; fp64: 7 fp64 VALU at 2,
    # the conversion at 2, the add and the exp2; tile-local: 4 VALU + exp2;
    # tile-local on the matrix cores: d K = 1 MFMA steps (2d flops at twice
    # the lane rate: d slots) + exp2 + 1 fma
    assert bench.slots_per_pair(3, "f32") == 12 and bench.slots_per_pair(1, "f32") == 8
    assert bench.slots_per_pair(3, "f64") == 21
    assert bench.slots_per_pair(3, "local") == 8 and bench.slots_per_pair(1, "local") == 6
    assert bench.slots_per_pair(3, "split") == 13
    assert bench.slots_per_pair(3, "local_mfma") == 8 and bench.slots_per_pair(2, "local_mfma") == 7


def test_traffic_records_match_their_kernel_and_sources(tmp_path, monkeypatch):
    # every committed record names its kernel and the digest of the sources it
    # was taken with; it resolves only for that kernel and only while the
    # sources still have that digest
    import re

    for w, (name, sources) in bench.PMC_RECORDS.items():
        text = open(os.path.join(ROOT, "profiles", name)).read()
        m = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)\s+kernel_sources_sha256:\s*([0-9a-f]+)"
                      r"\s+kernel:\s*(\S+)", text)
        assert m, name
        fresh = m.group(2) == bench.kernel_source_digest(sources)
        got = bench.pmc_traffic(m.group(3), w)
        assert got == (float(m.group(1)) if fresh else None)
        assert bench.pmc_traffic(m.group(3) + "x", w) is None
    assert bench.pmc_traffic("k_lse_valu<3,true>", 99) is None
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
