"""Host-side logic of bench.py (no GPU): the --gpus guard and the conversion
of rocprofv3 counter databases into the lm_head traffic record."""
import json
import os
import sqlite3
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=60)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def _db(path, counter, rows):
    c = sqlite3.connect(path)
    c.execute("create table counters_collection (kernel_name text, dispatch_id int, counter_name text, value real)")
    c.executemany("insert into counters_collection values (?, ?, ?, ?)",
                  [(k, d, counter, v) for k, d, v in rows])
    c.commit()
    c.close()


LM = "void gemvq::gemv_wave_kernel<1, 1, 1>(gemvq::GemvArgs)"
CAL = "void at::native::vectorized_elementwise_kernel<4, at::native::neg_kernel_cuda(...)>"
OTHER = "void gemvq::gemv_kernel<1, 0, true, 2, true>(gemvq::GemvArgs)"


def test_traffic_record(tmp_path, monkeypatch):
    known_kib = (bench.CALIB_MIB << 20) / 1024
    # the fetch counter reads half the true bytes, split over two instances per dispatch
    fetch_rows = [(CAL, d, known_kib / 4) for d in (1, 2) for _ in range(2)]
    fetch_rows += [(LM, d, 50_000.0) for d in (3, 4) for _ in range(2)]
    fetch_rows += [(OTHER, 5, 1.0)]     # not a recorded kernel in this database
    write_rows = [(CAL, 1, known_kib), (LM, 3, 10.0), (LM, 4, 30.0)]
    fdb, wdb = str(tmp_path / "f.db"), str(tmp_path / "w.db")
    _db(fdb, "FETCH_SIZE", fetch_rows)
    _db(wdb, "WRITE_SIZE", write_rows)
    out = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "PROFILE_TRAFFIC", str(out))
    bench.write_traffic(fdb, wdb, "cmd")
    t = json.loads(out.read_text())
    assert t["calibration"]["fetch_factor"] == pytest.approx(2.0)
    assert t["calibration"]["write_factor"] == pytest.approx(1.0)
    assert t["fetch_size_kib_per_dispatch"] == pytest.approx(100_000.0)
    assert t["hbm_fetch_bytes_per_launch"] == 2 * 100_000 * 1024
    assert t["hbm_write_bytes_per_launch"] == 20 * 1024
    assert t["bytes_per_launch"] == 2 * 100_000 * 1024 + 20 * 1024
    assert t["kernel_source_hash"] == bench.kernel_source_hash()
    assert bench.traffic_entry(0) == t["bytes_per_launch"]


def test_traffic_record_needs_one_lm_head_kernel(tmp_path, monkeypatch):
    fdb, wdb = str(tmp_path / "f.db"), str(tmp_path / "w.db")
    _db(fdb, "FETCH_SIZE", [(CAL, 1, 1.0)])
    _db(wdb, "WRITE_SIZE", [(CAL, 1, 1.0)])
    monkeypatch.setattr(bench, "PROFILE_TRAFFIC", str(tmp_path / "t.json"))
    with pytest.raises(SystemExit):
        bench.write_traffic(fdb, wdb, "cmd")


def test_stale_traffic_record_is_ignored(tmp_path, monkeypatch):
    p = tmp_path / "t.json"
    p.write_text(json.dumps({"kernel_source_hash": "not-this-source", "bytes_per_launch": 123}))
    monkeypatch.setattr(bench, "PROFILE_TRAFFIC", str(p))
    assert bench.traffic_entry(0) is None


def test_traffic_records_for_every_recorded_kernel(tmp_path, monkeypatch):
    """Each recorded kernel present in the databases gets its own record
    (bytes per launch against its algorithmic bytes)."""
    known_kib = (bench.CALIB_MIB << 20) / 1024
    sw = "void gemvq::gemv_kernel<3, 0, 2, true, true>(gemvq::GemvArgs)"
    c5 = "void gemvq::gemv_wave_kernel<2, 0, 2, true>(gemvq::GemvArgs)"
    fetch_rows = [(CAL, 1, known_kib / 2), (LM, 2, 100.0), (sw, 3, 500.0), (c5, 4, 700.0)]
    write_rows = [(CAL, 1, known_kib), (LM, 2, 1.0), (sw, 3, 2.0), (c5, 4, 3.0)]
    fdb, wdb = str(tmp_path / "f.db"), str(tmp_path / "w.db")
    _db(fdb, "FETCH_SIZE", fetch_rows)
    _db(wdb, "WRITE_SIZE", write_rows)
    kernels = [(tag, pat, alg, str(tmp_path / (tag + ".json"))) for tag, pat, alg, _ in bench.traffic_kernels()]
    monkeypatch.setattr(bench, "traffic_kernels", lambda: kernels)
    bench.write_traffic(fdb, wdb, "cmd")
    got = {p.name for p in tmp_path.glob("*.json")}
    assert got == {"lm_head_argmax.json", "swiglu_gemv_9728x2560.json", "c5_q4k_q8_gemv_from_f32_28672x8192.json"}
    t = json.loads((tmp_path / "swiglu_gemv_9728x2560.json").read_text())
    assert t["hbm_fetch_bytes_per_launch"] == 2 * 500 * 1024 and t["hbm_write_bytes_per_launch"] == 2 * 1024
    assert t["traffic_over_algorithmic"] == pytest.approx((1000 * 1024 + 2048) / t["algorithmic_bytes_per_launch"], abs=1e-4)


def test_shared_traffic_record_reaches_every_entry(tmp_path, monkeypatch):
    """A record whose tag joins several breakdown entries with '+' is
    attached to each of them; entries without a record are left alone."""
    rec = tmp_path / "pair.json"
    rec.write_text(json.dumps({"kernel_source_hash": bench.kernel_source_hash(), "bytes_per_launch": 1234}))
    monkeypatch.setattr(bench, "traffic_kernels",
                        lambda: [("lm_head_argmax", "x", 1, str(tmp_path / "none.json")),
                                 ("a_1x2+a_2x1", "y", 1000, str(rec))])
    kern = {"a_1x2": {"us": 1.0}, "a_2x1": {"us": 2.0}, "b": {"us": 3.0}}
    bench.attach_traffic(kern)
    assert kern["a_1x2"]["traffic"] == 1234 and kern["a_2x1"]["traffic"] == 1234
    assert "traffic" not in kern["b"]


def test_config_algorithmic_bytes():
    """Per-config bytes: the weights plus the vectors each config moves
    (x and y; config 4's h written and read back; config 5's Q8 codes and
    scales written once by its single launch)."""
    alg = bench.config_algorithmic_bytes()
    assert alg["c1"] == 589_824 + 4_096 + 4_096
    assert alg["c2"] == 33_914_880 + 124_928
    assert alg["c3"] == bench.lm_head_algorithmic_bytes() == 208_588_800 + 4_096 + 4
    assert alg["c4"] == 48_445_440 + 10_240 + 77_824 + 10_240
    assert alg["c5"] == 132_120_576 + 32_768 + 8_192 + 512 + 114_688
