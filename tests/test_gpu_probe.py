"""The issue-rate probes behind the bench's ceilings: every kind runs and
reports a positive rate, the pair kinds report pairs at the rate divided by
their counted instructions per pair, and bad arguments are refused."""
import math

import pytest

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

# counted (non-transcendental) lane-instructions per pair of each pair probe
PAIR_COUNTS = {"PAIR_F32": 8, "PAIR_F32_NOEXP": 8, "PAIR_F64": 9, "PAIR_TILE_F32": 4, "PAIR_SPLIT_F32": 9,
               "PAIR_TILE_MFMA": 1}
KINDS = ("FMA_F32", "EXP_F32", "FMA_F64", "PAIR_F32", "PAIR_F32_NOEXP", "PAIR_F64", "SUB_F32",
         "FMAC_F32", "ADD_F64", "CVT_F32_F64", "PAIR_TILE_F32", "PAIR_SPLIT_F32",
         "PAIR_TILE_MFMA")


@pytest.fixture(scope="module")
def sk():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import log_domain_sinkhorn_amd as sk

    return sk


@pytest.mark.parametrize("name", KINDS)
def test_probe_kind_reports_its_rate(sk, name):
    lanes, pairs, ms = sk.probe_issue_rate(getattr(sk, "PROBE_" + name), 2000)
    assert math.isfinite(lanes) and lanes > 0.0 and ms > 0.0
    if name in PAIR_COUNTS:
        assert pairs == pytest.approx(lanes / PAIR_COUNTS[name], rel=1e-9)
    else:
        assert not pairs


def test_probe_refuses_bad_arguments(sk):
    with pytest.raises(sk.SinkhornError) as ei:
        sk.probe_issue_rate(99, 10)
    assert ei.value.code == sk.ERR_INVALID_ARG
    with pytest.raises(sk.SinkhornError) as ei:
        sk.probe_issue_rate(sk.PROBE_FMA_F32, 0)
    assert ei.value.code == sk.ERR_INVALID_ARG
