"""Host checks of bench.py's counter-traffic gating: a committed rocprofv3
traffic figure is reported only while the sources of its workload are the
ones it was measured on."""

import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_every_profiled_workload_names_its_sources():
    for w in bench.ONLY:
        assert w in bench.WORKLOAD_SRCS, w
        for path in bench.WORKLOAD_SRCS[w]:
            assert os.path.isfile(path), path


def test_traffic_reported_only_on_matching_sources(tmp_path, monkeypatch):
    f = tmp_path / "traffic.json"
    good = {"sources_hash": bench.sources_hash("m1_layer"), "traffic_bytes_per_call": 123}
    stale = {"sources_hash": "0" * 16, "traffic_bytes_per_call": 456}
    f.write_text(json.dumps({"m1_layer": good, "decode": stale}))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.committed_traffic("m1_layer") == 123
    assert bench.committed_traffic("decode") is None      # measured on other sources
    assert bench.committed_traffic("long_1m") is None     # never measured
    f.write_text("not json")
    assert bench.committed_traffic("m1_layer") is None


def test_hash_covers_the_launch_plan_and_the_abi():
    names = {os.path.basename(p) for p in bench.WORKLOAD_SRCS["m1_layer"]}
    assert {"prefill_heads.hip", "tiles.h", "internal.h", "lightning_api.cpp", "lightning.h"} <= names
