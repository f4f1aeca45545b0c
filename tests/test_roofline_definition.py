"""The bytes-per-token definition used by bench.py reproduces the roofline percentages the
roadmap page prints for its own decode measurements (golden file with citation)."""

import json
import os

from tile_scheduled_persistent_amd.configs import LLAMA_1B, QWEN3_06B, QWEN3_4B, WORKLOADS

HERE = os.path.dirname(os.path.abspath(__file__))


def test_pages_roofline_percentages_reproduced():
    g = json.load(open(os.path.join(HERE, "golden", "roadmap_decode_roofline.json")))
    models = {"qwen3-0.6b-shaped": QWEN3_06B, "qwen3-4b-shaped": QWEN3_4B}
    for case in g["cases"]:
        m = models[case["model"]]
        bytes_per_token = m.weight_bytes_per_token() - 2 * m.hidden + m.kv_bytes_per_position() * g["attended_positions"]
        roof = g["bandwidth_gb_s"] * 1e9 / bytes_per_token
        pct = 100.0 * case["tok_s"] / roof
        assert round(pct) == case["pct_of_roofline"], (case, pct)


def test_workload_bytes_per_token():
    # weights once (tied head once, one embedding row) + K/V of the attended positions (mean over
    # the 64 steps: 1023 + 32.5) + one K/V write
    wl = WORKLOADS["llama1b"]
    assert LLAMA_1B.weight_bytes_per_token() == 2_471_632_896
    assert LLAMA_1B.kv_bytes_per_position() == 32_768
    assert wl.bytes_per_token() == 2_471_632_896 + 32_768 * 1055.5 + 32_768
    assert WORKLOADS["qwen4b_32k"].bytes_per_token() == QWEN3_4B.weight_bytes_per_token() + 147_456 * (32767 + 16.5) + 147_456


def _fake_counter_db(path, counter, rows):
    import sqlite3

    con = sqlite3.connect(path)
    con.execute("create table counters_collection (kernel_name text, dispatch_id integer, counter_name text, value real)")
    con.executemany("insert into counters_collection values (?, ?, ?, ?)", [(k, d, counter, v) for k, d, v in rows])
    con.commit()
    con.close()


def test_counter_traffic_calibration(tmp_path):
    """The traffic summary scales FETCH_SIZE by the stream-read dispatches (known bytes, the decode
    kernel's load form) and WRITE_SIZE by the copy kernel; per-dispatch values of one counter are
    summed over the rows (instances) of that dispatch."""
    from tile_scheduled_persistent_amd import prof

    read_bytes, copy_bytes = 2 << 30, 1 << 30
    worker = "void tiles::tiles_worker<64, 4, false, false>(tiles::KernelArgs)"
    sr = "tiles::stream_read(unsigned char const*, long, unsigned int*)"
    copy = "__amd_rocclr_copyBuffer"
    # the counter reads half the bytes a kernel fetches; a dispatch's value arrives in two rows
    fetch = [(worker, 1, 40.0e6), (worker, 1, 40.0e6), (worker, 2, 80.0e6), (sr, 3, 2 ** 20 / 2), (sr, 3, 2 ** 20 / 2),
             (sr, 4, 2 ** 20), (copy, 5, copy_bytes / 2048)]
    write = [(worker, 1, 1000.0), (worker, 2, 1000.0), (copy, 5, copy_bytes / 1024)]
    _fake_counter_db(str(tmp_path / "f.db"), "FETCH_SIZE", fetch)
    _fake_counter_db(str(tmp_path / "w.db"), "WRITE_SIZE", write)
    d = prof.traffic(str(tmp_path / "f.db"), str(tmp_path / "w.db"), "tiles_worker", copy_bytes, read_bytes)
    assert d["FETCH_SIZE"]["kib_per_dispatch"] == [80.0e6, 80.0e6]
    assert d["FETCH_SIZE"]["stream_read_factor"] == 2.0
    assert d["FETCH_SIZE"]["copy_factor"] == 2.0
    assert d["WRITE_SIZE"]["factor"] == 1.0
    assert d["traffic_bytes_per_launch"] == 80.0e6 * 1024 * 2 + 1000.0 * 1024
