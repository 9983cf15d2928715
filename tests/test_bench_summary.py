"""Host logic of bench.py's profile summaries (CPU): the dominant kernel's HBM
traffic is its FETCH_SIZE per dispatch scaled by what the same counter reads
for the 2 GiB streaming read, and its WRITE_SIZE scaled by what that counter
reads for the bench's 64 MiB device copy; the counter summary averages each
counter per dispatch.  Synthetic rocprofv3-style databases."""
import json
import os
import sqlite3

import pytest

import bench

DOM = "void tqproj::proj_kernel<0, 2, 2, 6, 2, true, true, false, 1>(tqproj::ProjArgs)"
SUMS = "void tqproj::proj_kernel<0, 2, 2, 6, 2, true, true, true, 1>(tqproj::ProjArgs)"
ROWS4 = "void tqproj::proj_kernel<0, 2, 2, 6, 2, true, true, false, 4>(tqproj::ProjArgs)"
COPY = "__amd_rocclr_copyBuffer"
READ = "void (anonymous namespace)::stream_read_kernel(uint4 const*, unsigned long, unsigned int*)"


def _db(path, kernels=(), counters=()):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    c = sqlite3.connect(path)
    if kernels:
        c.execute("create table kernels (name text, duration integer)")
        c.executemany("insert into kernels values (?, ?)", kernels)
    if counters:
        c.execute("create table counters_collection (kernel_name text, counter_name text, "
                  "dispatch_id integer, value real)")
        c.executemany("insert into counters_collection values (?, ?, ?, ?)", counters)
    c.commit()
    c.close()


def test_profile_summary_scales_traffic_by_the_calibrations(tmp_path, monkeypatch, capsys):
    kt, fe, wr = (str(tmp_path / d) for d in ("kt", "fetch", "write"))
    _db(os.path.join(kt, "a", "kt.db"),
        kernels=[(DOM, 12000), (DOM, 13000), ("other_kernel", 5000), (SUMS, 99000), (ROWS4, 24000)])
    # per dispatch the counter arrives split over instances (summed per dispatch);
    # the streaming read of 2 GiB reports half its true bytes (scale 2), the
    # copy's writes are counted in full (scale 1)
    _db(os.path.join(fe, "f.db"),
        counters=[(READ, "FETCH_SIZE", 1, 524288), (READ, "FETCH_SIZE", 1, 524288),
                  (COPY, "FETCH_SIZE", 2, 1000),              # not a calibration
                  (DOM, "FETCH_SIZE", 3, 9000), (DOM, "FETCH_SIZE", 3, 10000),
                  (DOM, "FETCH_SIZE", 4, 21000), (ROWS4, "FETCH_SIZE", 5, 99000)])
    _db(os.path.join(wr, "w.db"),
        counters=[(COPY, "WRITE_SIZE", 1, 65536), (COPY, "WRITE_SIZE", 2, 20000),
                  (DOM, "WRITE_SIZE", 3, 300), (DOM, "WRITE_SIZE", 4, 500)])
    out = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(out))
    bench.profile_summary(kt, fe, wr)
    rec = json.loads(out.read_text())
    assert rec["kernel"] == DOM
    assert rec["fetch_scale"] == 2.0 and rec["write_scale"] == 1.0
    assert rec["fetch_bytes"] == 20000 * 1024 * 2      # mean of 19000 and 21000 KiB, x2
    assert rec["write_bytes"] == 400 * 1024            # mean of 300 and 500 KiB
    assert rec["hbm_bytes_per_launch"] == rec["fetch_bytes"] + rec["write_bytes"]
    assert rec["kernel_source_sha"] == bench.kernel_source_sha()
    text = capsys.readouterr().out
    assert "avg duration 12.500 us" in text
    assert rec["trace_avg_launch_us"] == 12.5 and rec["trace_launches"] == 2


def test_profile_summary_needs_the_calibrations(tmp_path, monkeypatch):
    kt, fe, wr = (str(tmp_path / d) for d in ("kt", "fetch", "write"))
    _db(os.path.join(kt, "kt.db"), kernels=[(DOM, 12000)])
    _db(os.path.join(fe, "f.db"), counters=[(DOM, "FETCH_SIZE", 1, 9000)])
    _db(os.path.join(wr, "w.db"), counters=[(DOM, "WRITE_SIZE", 1, 300)])
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "t.json"))
    with pytest.raises(SystemExit):
        bench.profile_summary(kt, fe, wr)
    assert not (tmp_path / "t.json").exists()


def test_counter_summary_averages_per_dispatch(tmp_path, capsys):
    d = str(tmp_path / "pmc")
    _db(os.path.join(d, "p.db"),
        counters=[(DOM, "SQ_INSTS_VALU", 1, 100), (DOM, "SQ_INSTS_VALU", 1, 50),
                  (DOM, "SQ_INSTS_VALU", 2, 250),
                  ("void (anonymous namespace)::gemm_kernel<0, false, 4>(...)", "SQ_INSTS_MFMA", 7, 64),
                  ("unrelated", "SQ_INSTS_VALU", 9, 1)])
    bench.counter_summary([d])
    text = capsys.readouterr().out.splitlines()
    assert text[0] == "gate/up"
    assert text[1].split() == ["SQ_INSTS_VALU", "200.0"]   # (150 + 250) / 2 dispatches
    assert text[2] == "prefill GEMM, 256-row tiles (down shape)"
    assert text[3].split() == ["SQ_INSTS_MFMA", "64.0"]
    assert len(text) == 4


def test_bench_refuses_more_than_one_gpu():
    """--gpus N > 1 exits with a message: the bench measures one GPU."""
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(os.path.dirname(bench.__file__), "bench.py"),
                        "--gpus", "2"], capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
