"""bench.py refuses more than one GPU before touching any (no GPU needed)."""
import json
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_several_gpus(capsys, monkeypatch):
    if ROOT not in sys.path:
        sys.path.insert(0, ROOT)
    import bench
    monkeypatch.setattr(sys, "argv", ["bench.py", "--gpus", "2"])
    with pytest.raises(SystemExit) as ex:
        bench.main()
    assert ex.value.code == 2
    line = capsys.readouterr().out.strip().splitlines()[-1]
    assert "one GPU" in json.loads(line)["error"]


def test_cpu_baseline_times_the_oracle_not_the_generator():
    if ROOT not in sys.path:
        sys.path.insert(0, ROOT)
    import bench
    import synth
    out = bench.cpu_baseline(synth.TINY, 0.05)
    assert out["kind"] == "oracle" and out["value"] > 0 and out["cores"] >= 1
    assert "outside the timer" in out["sample"]
