"""The profile-summary tool on small SQLite databases shaped like rocprofv3's
(a `kernels` table and a `pmc_events` table): dispatch selection (last N, after
leaving out the last M), the copy-scaled HBM traffic and the SQ derived metrics,
each against values worked out by hand."""
import json
import sqlite3

import pytest

from kv_cache_int2_amd import rocprof_summary as R


def _db(path, dispatches, counters=()):
    """dispatches: (id, name, start, duration ns); counters: (id, counter, value)."""
    con = sqlite3.connect(path)
    con.execute("create table kernels (dispatch_id int, name text, start int, duration int)")
    con.execute("create table pmc_events (dispatch_id int, counter_name text, counter_value real)")
    con.executemany("insert into kernels values (?, ?, ?, ?)", dispatches)
    con.executemany("insert into pmc_events values (?, ?, ?)", counters)
    con.commit()
    con.close()
    return str(path)


def test_tail_leaves_out_the_last_dispatches(tmp_path):
    # 10 write launches of 1..10 us in start order, a decode launch between them
    rows = [(i, "quant_write_kernel<0, 4, 4, true>", 10 * i, 1000 * (i + 1)) for i in range(10)]
    rows.append((99, "decode_int2<4, 4, 1, 1, false>", 55, 375_000))
    db = _db(tmp_path / "t.db", rows)
    r = R.tail_stats(db, "quant_write", 3, 2)          # launches 6, 7, 8 us (the last two, 9 and 10, left out)
    assert r["calls"] == 3 and r["avg_us"] == pytest.approx(7.0)
    assert (r["min_us"], r["max_us"]) == (6.0, 8.0)
    r = R.tail_stats(db, "quant_write", 4)             # 7..10 us
    assert r["avg_us"] == pytest.approx(8.5) and r["total_ms"] == pytest.approx(0.034)
    assert R.tail_stats(db, "decode_int2", 5)["calls"] == 1


def test_trace_summary_names_the_left_out_dispatches(tmp_path, capsys):
    rows = [(i, "quant_write_kernel<0, 4, 4, true>", i, 2000) for i in range(6)]
    db = _db(tmp_path / "t.db", rows)
    R.main(["trace", db, "--command", "cmd", "--tail", "quant_write_kernel<0:3:2"])
    out = capsys.readouterr().out
    assert "Last 3 dispatches of quant_write_kernel<0 before its last 2:" in out
    assert "| quant_write_kernel<0 (last 3) | 3 | 2.00 |" in out


def test_pmc_traffic_is_scaled_by_the_copy_kernel(tmp_path, capsys):
    # the kernel's counter is summed over two hardware instances per dispatch;
    # the copy of 1 MiB each way reads 2048 KiB fetched and 1024 KiB written
    # (a fetch counter twice the true bytes, a write counter exact)
    ks = [(1, "decode_int2", 0, 1), (2, "decode_int2", 1, 1), (3, "decode_int2", 2, 1), (4, "copy_pages_kernel", 3, 1)]
    fetch = [(1, "FETCH_SIZE", 500.0), (1, "FETCH_SIZE", 500.0),     # 1000 KiB
             (2, "FETCH_SIZE", 1500.0), (2, "FETCH_SIZE", 1500.0),   # 3000 KiB
             (3, "FETCH_SIZE", 2500.0), (3, "FETCH_SIZE", 2500.0),   # 5000 KiB
             (4, "FETCH_SIZE", 2048.0)]
    write = [(1, "WRITE_SIZE", 10.0), (2, "WRITE_SIZE", 30.0), (3, "WRITE_SIZE", 50.0), (4, "WRITE_SIZE", 1024.0)]
    fdb = _db(tmp_path / "f.db", ks, fetch)
    wdb = _db(tmp_path / "w.db", ks, write)
    src = tmp_path / "k.hip"
    src.write_bytes(b"kernel source")
    R.main(["pmc", "--fetch", fdb, "--write", wdb, "--kernel", "decode_int2", "--copy", "copy_pages",
            "--copy-bytes", str(1 << 20), "--workload", "w", "--source", str(src), "--command", "c",
            "--algorithmic-bytes", str(2 << 20), "--tail", "2"])
    res = json.loads(capsys.readouterr().out)
    # last two dispatches: fetch (3000 + 5000) / 2 KiB at 1/2 true bytes per counted byte,
    # write (30 + 50) / 2 KiB at 1
    assert res["fetch_size"]["scale"] == pytest.approx(0.5)
    assert res["fetch_size"]["bytes_per_launch"] == pytest.approx(4000 * 1024 * 0.5)
    assert res["write_size"]["bytes_per_launch"] == pytest.approx(40 * 1024)
    assert res["hbm_bytes_per_launch"] == pytest.approx(2000 * 1024 + 40 * 1024)
    assert res["traffic_over_algorithmic"] == pytest.approx((2000 + 40) / 2048)
    import hashlib
    assert res["kernel_source_sha256"] == hashlib.sha256(b"kernel source").hexdigest()


def test_sq_metrics_follow_the_derived_formulas(tmp_path):
    ks = [(d, "decode_int2", d, 1) for d in (1, 2, 3)]
    vals = []
    for d, (busy, active, gui) in {1: (1024e3, 256e3, 2e3), 2: (512e3, 128e3, 1e3), 3: (9e9, 9e9, 1.0)}.items():
        # two hardware instances each for the summed SQ counters, GRBM taken as the maximum
        vals += [(d, "SQ_VALU_MFMA_BUSY_CYCLES", busy / 2), (d, "SQ_VALU_MFMA_BUSY_CYCLES", busy / 2),
                 (d, "SQ_ACTIVE_INST_VALU", active / 2), (d, "SQ_ACTIVE_INST_VALU", active / 2),
                 (d, "SQ_INSTS_VALU", 100.0 * d), (d, "SQ_INSTS_MFMA", 10.0 * d),
                 (d, "GRBM_GUI_ACTIVE", gui), (d, "GRBM_GUI_ACTIVE", gui / 2)]
    db = _db(tmp_path / "q.db", ks, vals)
    r = R.sq_stats(db, "decode_int2", cu_num=256, simd_num=1024, tail=2, skip_last=1)   # dispatches 1, 2
    # MfmaUtil = 100 busy / (gui 1024): 50 % for both; VALUBusy = 100 active / 256 / gui: 50 % for both
    assert r["dispatches"] == 2
    assert r["mfma_util_pct"] == pytest.approx(50.0)
    assert r["valu_busy_pct"] == pytest.approx(50.0)
    assert r["valu_insts"] == pytest.approx(150.0) and r["mfma_insts"] == pytest.approx(15.0)
