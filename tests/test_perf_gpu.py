"""Performance regression check on MI355X with a control.

tests/perf/mi355x_baseline.json holds per-launch times of the decode layers
(Llama-3.1-8B bf16 asymmetric and Qwen3-4B fp16 symmetric, M = 1) and the
Llama prefill layers (M = 1920) recorded by `bench.py --perf-record`, beside
two control kernels timed in the same run (a 1 GiB streaming read and the
sustained MFMA loop).  This test measures the same points and controls now;
each point's time ratio is divided by the control's speed ratio (the box and
its clocks differ from run to run), and a point more than 25 % slower after
that normalisation fails.  Boxes differ by a few percent, and the band leaves
room for that."""
import json
import os

import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BASELINE = os.path.join(ROOT, "tests", "perf", "mi355x_baseline.json")


@pytest.mark.skipif(not torch.cuda.is_available(), reason="no GPU")
def test_no_regression_against_the_recorded_baseline():
    import sys
    sys.path.insert(0, ROOT)
    import bench
    from gpu_util import note
    with open(BASELINE) as f:
        base = json.load(f)
    note("[gpu] perf: measuring the regression points and controls")
    now = bench.perf_points(torch.device("cuda:0"), torch.cuda.Stream())
    res = bench.perf_compare(base, now)
    for r in res:
        note(f"[gpu] perf {r['point']}: {r['base_us']} -> {r['now_us']} us, control x{r['control_speedup']}, "
             f"normalised {r['normalized_ratio']}")
    bad = [r for r in res if r["regressed"]]
    assert not bad, f"regressions beyond 25 % after normalising by the control: {bad}"
