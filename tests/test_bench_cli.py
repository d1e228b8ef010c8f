"""bench.py command-line contract checks that need no GPU."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=120, cwd=ROOT)


@pytest.mark.parametrize("n", [2, 8])
def test_more_than_one_gpu_exits_with_a_message(n):
    r = _run("--gpus", str(n))
    assert r.returncode != 0
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == n and "one GPU" in line["error"]


def test_help_lists_the_measurement_options():
    r = _run("--help")
    assert r.returncode == 0
    for opt in ("--steps", "--warmup", "--config", "--epilogue", "--seeding", "--zipf-update", "--tune", "--probe"):
        assert opt in r.stdout, opt


def test_stream_overlap_from_a_hand_made_timeline():
    """The chunked-stream overlap figures from a timeline whose unions and
    intersections are worked out by hand: copy-in windows [0,2) [1,3) [5,6)
    (union 4 ms), compute windows [2,4) [2.5,3.5) [6,7) (union 3 ms), labels out [4,4.5) twice and
    [7,8); copy and compute overlap on [2,3) only (1 ms)."""
    import bench
    tl = [[0, 0, 0.0, 2.0, 2.0, 4.0, 4.0, 4.5],
          [0, 1, 1.0, 3.0, 2.5, 3.5, 4.0, 4.5],
          [0, 2, 5.0, 6.0, 6.0, 7.0, 7.0, 8.0]]
    o = bench.stream_overlap(tl, 3, h2d_bytes=4e9)
    assert o["chunks_recorded"] == 3 and o["chunks_issued"] == 3
    assert o["wall_ms"] == 8.0
    assert o["h2d_busy_ms"] == 4.0 and o["compute_busy_ms"] == 3.0 and o["d2h_busy_ms"] == 1.5
    assert o["both_busy_ms"] == 1.0
    assert o["h2d_busy_frac"] == 0.5
    assert abs(o["hidden_frac_of_shorter"] - 1.0 / 3.0) < 1e-12
    assert abs(o["h2d_gbs_while_copying"] - 1000.0) < 1e-9      # 4 GB in 4 ms
    assert bench.stream_overlap([], 5, 4e9) == {"chunks_recorded": 0, "chunks_issued": 5}


def test_assign_traffic_calibration_and_staleness(tmp_path, monkeypatch):
    """HBM bytes per assign launch from a counter summary: each counter is
    scaled by what it read for a plain copy of known size (here FETCH_SIZE
    read the 1 GiB copy as 512 MiB, so fetches count twice), and the figure is
    withdrawn (None) for another shape or another assign source."""
    import bench
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "traffic_cx.txt").write_text(
        "# header\nB=1\nN=1000\nD=128\nK=64\nassign_source_sha256=abc\ncopy_bytes=1073741824\n"
        "copy_fetch_kib=524288\ncopy_write_kib=1048576\nassign_fetch_kib=1000\nassign_write_kib=10\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "assign_source_sha", lambda: "abc")
    assert bench.assign_traffic("cx", 1, 1000, 128, 64) == 1000 * 1024 * 2.0 + 10 * 1024 * 1.0
    assert bench.assign_traffic("cx", 1, 1001, 128, 64) is None      # another shape
    assert bench.assign_traffic("cy", 1, 1000, 128, 64) is None      # no summary
    monkeypatch.setattr(bench, "assign_source_sha", lambda: "def")
    assert bench.assign_traffic("cx", 1, 1000, 128, 64) is None      # counters taken on another source
