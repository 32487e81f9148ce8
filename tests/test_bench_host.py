"""bench.py on the host: it measures one GPU and says so for any other
count, and its traffic figure is tied to the sources it was measured on."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def _run(args, env_extra=None):
    env = dict(os.environ, **(env_extra or {}))
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + args, cwd=ROOT,
                          env=env, capture_output=True, text=True, timeout=120)


def test_more_than_one_gpu_exits_with_a_message():
    for args, extra in ((["--gpus", "2"], None), (["--gpus", "8"], None), ([], {"WORLD_SIZE": "2"})):
        r = _run(args, extra)
        assert r.returncode == 2, (args, r.stdout, r.stderr)
        assert "measures one GPU" in r.stderr and r.stdout == ""


def test_source_digest_ignores_comments_and_tracks_code(tmp_path, monkeypatch):
    d = bench.source_digest()
    assert len(d) == 16 and int(d, 16) >= 0
    # the same sources in another directory, with comments and spacing
    # changed: same digest; one token changed: another digest
    for name in bench.HEADLINE_SOURCES:
        with open(os.path.join(bench.CSRC, name)) as f:
            text = f.read()
        (tmp_path / name).write_text("// a new comment\n" + text.replace("\n", "\n  ") + "\n/* x */\n")
    monkeypatch.setattr(bench, "CSRC", str(tmp_path))
    assert bench.source_digest() == d
    name = sorted(bench.HEADLINE_SOURCES)[-1]
    text = (tmp_path / name).read_text()
    (tmp_path / name).write_text(text.replace("return", "return ", 1).replace("0x", "0X", 1))
    assert bench.source_digest() != d


def test_traffic_is_reported_only_for_the_measured_sources():
    with open(bench.TRAFFIC_FILE) as f:
        t = json.load(f)
    assert bench.traffic_for(t["source_digest"]) == t["hbm_bytes_per_launch"]
    assert bench.traffic_for("0" * 16) is None
    # the stored figure is FETCH_SIZE x 2 + WRITE_SIZE x 1 (KiB per dispatch)
    want = t["fetch_size_kib"] * 1024 * t["fetch_factor_from_copy"] + \
        t["write_size_kib"] * 1024 * t["write_factor_from_copy"]
    assert abs(want - t["hbm_bytes_per_launch"]) < 4096
    assert 1.0 <= t["hbm_bytes_per_launch"] / t["algorithmic_bytes_per_launch"] < 1.01
