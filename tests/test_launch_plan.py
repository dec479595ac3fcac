"""Host-only checks of the pair kernels' launch-size arithmetic
(``csrc/launch_plan.h``), compiled with the host C++ compiler: a dispatch
holds at most 2^32 - 1 work-items, so the dense half-step's column split must
keep tiles * G workgroups of 512 work-items under that, up to the largest
clouds the library accepts, and refuse (not truncate) beyond."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(os.path.dirname(HERE), "log_domain_sinkhorn_amd", "csrc")
LIMIT = (1 << 32) - 1


@pytest.fixture(scope="module")
def planner(tmp_path_factory):
    cxx = shutil.which("g++") or shutil.which("c++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    exe = str(tmp_path_factory.mktemp("plan") / "launch_plan_check")
    subprocess.run([cxx, "-std=c++17", "-O1", "-I", CSRC, os.path.join(HERE, "launch_plan_check.cpp"),
                    "-o", exe], check=True)

    def run(cases):
        text = "".join(f"{n} {m} {s} {d}\n" for n, m, s, d in cases)
        out = subprocess.run([exe], input=text, capture_output=True, text=True, check=True).stdout
        lines = out.splitlines()
        assert lines[0] == f"max_blocks_512 {LIMIT // 512}"
        return [tuple(int(v) for v in ln.split()) for ln in lines[1:]]

    return run


SIZES = [1, 37, 1000, 20000, 10**6, 1 << 24, 1 << 27, 1 << 28, 1 << 30, (1 << 30) + 1, 1 << 31]


def test_dense_split_always_fits_one_dispatch(planner):
    cases = [(n, m, s, 3) for n in SIZES for m in SIZES for s in (256, 768)]
    for (n, m, s, d), (G, glog, cps, nchunks, tiles, ok) in zip(cases, planner(cases)):
        assert tiles == (n + 127) // 128 and nchunks == (m + 15) // 16
        assert G >= 1 and G & (G - 1) == 0 and 1 << glog == G and G <= 64
        assert cps * G >= nchunks  # every chunk belongs to a split
        if ok:
            assert tiles * G * 512 <= LIMIT, (n, m, G)
        else:
            assert tiles * 512 > LIMIT, (n, m)  # refused only when one split is already too many


def test_dense_split_at_the_limit(planner):
    # 2^27 rows: 2^20 tiles; 8 splits would be 2^32 work-items, one too many
    (G, _, _, _, tiles, ok), = planner([(1 << 27, 1 << 27, 768, 3)])
    assert ok and tiles == 1 << 20 and G == 4
    # 2^30 rows: 2^23 tiles of 512 work-items is exactly 2^32: refused
    (_, _, _, _, tiles, ok), = planner([(1 << 30, 1000, 768, 3)])
    assert tiles == 1 << 23 and not ok
    # the common sizes keep the split they had before the cap
    (G2, *_), (G4, *_) = planner([(20000, 20000, 768, 3), (10**6, 10**6, 768, 3)])
    assert G2 == 16 and G4 == 8
