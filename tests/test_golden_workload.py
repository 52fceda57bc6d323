"""The Wan share workload and the bench protocol against the figures the pages print.

tests/golden/lightx2v_fast_ulysses_microbenchmark.json holds the values of the
LightX2V PR "Add fast-ulysses attention backend", Attention microbenchmark:
6820 rows per rank, 27280 rows in all, 40 heads of 128 at Ulysses degree 4,
bf16, 10 warm-up and 50 timed iterations reported as median, P90 and min, and
every backend's output equal to the others' (max abs diff 0).
"""
import json
import os
import sys

import pytest

from ulysses_sequence_attention_amd import inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLDEN = os.path.join(ROOT, "tests", "golden", "lightx2v_fast_ulysses_microbenchmark.json")


@pytest.fixture(scope="module")
def page():
    with open(GOLDEN) as fh:
        return json.load(fh)


def test_end_to_end_workload_is_the_pages_layer(page):
    w = inputs.E2E_P4
    assert w.s_local == page["local_sequence_length_per_rank"]
    assert w.degree == page["ulysses_degree"]
    assert w.rows == page["global_sequence_length"] == w.degree * w.s_local
    assert (w.hq, w.hkv, w.head_dim) == (page["heads"], page["heads"], page["head_dim"])


def test_wan_share_is_one_rank_of_the_pages_layer(page):
    for w in (inputs.WAN_SHARE, inputs.WAN_SHARE_G5):
        assert w.rows == page["global_sequence_length"]
        assert w.hq * page["ulysses_degree"] == page["heads"]
        assert w.head_dim == page["head_dim"]


def test_bench_defaults_follow_the_pages_protocol(page, monkeypatch):
    """bench.py's defaults: the pages' warm-up and iteration counts."""
    sys.path.insert(0, ROOT)
    import bench
    monkeypatch.setattr(sys, "argv", ["bench.py"])
    args = bench.parse()
    assert (args.warmup, args.steps, args.gpus) == (page["warmup"], page["iterations"], 1)


def test_bench_reports_the_pages_statistics(page):
    src = open(os.path.join(ROOT, "bench.py")).read()
    for stat in page["statistics"]:
        assert f'"{stat}"' in src


def test_pages_require_identical_outputs(page):
    """The pages accept a faster exchange only when its output equals the default path's exactly; the GPU
    tests hold head-group splits, the pipeline and the workspace-free call to byte equality."""
    assert page["backends_max_abs_diff"] == 0.0
