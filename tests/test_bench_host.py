"""Host-side checks of bench.py's contract (no GPU): more than one GPU is refused with a
message before any device work, and the command line parses."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=120, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    r = _bench("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr or "single MI355X" in r.stderr
    assert r.stdout == ""  # no JSON line


def test_command_line_parses():
    r = _bench("--help")
    assert r.returncode == 0
    for opt in ("--steps", "--warmup", "--workload", "--backward", "--ep-shards", "--tiled"):
        assert opt in r.stdout


# --------------------------------------------------------------- bench.py's host arithmetic

import json  # noqa: E402
import shutil  # noqa: E402

sys.path.insert(0, ROOT)
import bench  # noqa: E402
from sparse_mixture_experts_level_amd import workloads as wl  # noqa: E402


def test_tail_rows_follows_the_tail_rule():
    # the Mixtral-shaped layer's routed groups (seed 0, drawn on the GPU): five last tiles of
    # <= 128 rows (11, 54, 32, 30, 27); the 214-, 225- and 175-row ones stay in large tiles
    rows = [982, 1035, 993, 1078, 943, 1056, 1054, 1051]
    assert bench.tail_rows(rows, 4096) == 11 + 54 + 32 + 30 + 27
    # a tail launch of 8 groups x 16 column tiles would be too small to run: no tails
    assert bench.tail_rows(rows, 1024) == 0
    assert bench.tail_rows([256, 512, 0], 1 << 20) == 0  # whole tiles and empty groups leave none


def test_big_regime_rule():
    assert bench.big_regime(8192, 8, 4096)
    assert not bench.big_regime(8192, 64, 128)  # capacity 128: no group reaches a 256-row tile
    assert not bench.big_regime(100, 0, 100)


def test_stage_work_of_the_deepseek_shaped_layer():
    w = wl.get_workload("deepseek_v3_bf16")
    T, d, f, fs = w.num_tokens, w.d_model, w.d_ff, w.d_ff_shared
    R, E_t = 6651, 212
    work = bench.stage_work(w, R, E_t, [26] * 256, T, 2, 80, 20480)
    # streaming regime: touched experts' weights once, the kept rows read and written once
    assert work["gate_up"]["bytes"] == 2 * (E_t * 2 * f * d + R * d + R * f)
    assert work["down"]["bytes"] == 2 * (E_t * d * f + R * f + R * d)
    assert work["gate_up"]["flop"] == 4.0 * R * d * f and work["down"]["flop"] == 2.0 * R * d * f
    assert "stream" in work["gate_up"]["kernel"]
    # the shared expert: every token, one group on the large tiles (16384 rows: no tail)
    assert work["shared_gate_up"]["flop"] == 4.0 * T * d * fs
    assert work["shared_down"]["bytes"] == 2 * (d * fs + T * fs + T * d)
    assert "big" in work["shared_down"]["kernel"]


def test_roofline_picks_the_bound_by_the_ridge():
    # ridge = 2.5e15 / 8e12 = 312.5 FLOP/B
    hbm = bench.roofline_of({"flop": 100.0 * 8e9, "bytes": 8e9}, 1000.0, 2)  # 8 GB in 1 ms
    assert hbm["bound"] == "hbm" and hbm["unit"] == "GB/s"
    assert abs(hbm["achieved"] - 8000.0) < 1e-6 and abs(hbm["frac"] - 1.0) < 1e-9
    mfma = bench.roofline_of({"flop": 1.25e12, "bytes": 1e9}, 1000.0, 2)  # 1.25 TFLOP in 1 ms
    assert mfma["bound"] == "mfma" and mfma["unit"] == "TFLOP/s"
    assert abs(mfma["achieved"] - 1250.0) < 1e-6 and abs(mfma["frac"] - 0.5) < 1e-9
    f32 = bench.roofline_of({"flop": 1e12, "bytes": 1e6}, 1000.0, 4)  # fp32 layers: the fp32 peak
    assert f32["peak"] == bench.MFMA_F32_PEAK_TFLOPS


def test_counter_traffic_needs_the_sources_it_was_taken_on(tmp_path, monkeypatch):
    for p in bench.GEMM_SOURCES:
        (tmp_path / p).parent.mkdir(parents=True, exist_ok=True)
        shutil.copy(os.path.join(ROOT, p), tmp_path / p)
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    rec = {"source_hash": bench.source_hash(bench.GEMM_SOURCES), "hbm_bytes_per_launch": 123}
    (tmp_path / "profiles" / "traffic_gate_up_demo.json").write_text(json.dumps(rec))
    assert bench.counter_traffic("demo", "gate_up") == 123
    assert bench.counter_traffic("other", "gate_up") is None  # no record
    with open(tmp_path / bench.GEMM_SOURCES[0], "a") as fh:
        fh.write("// changed\n")
    assert bench.counter_traffic("demo", "gate_up") is None  # kernels changed since the counters


def test_committed_traffic_records_match_the_kernels():
    """The traffic records under profiles/ were taken on the grouped-GEMM sources as they are."""
    h = bench.source_hash(bench.GEMM_SOURCES)
    names = [n for n in os.listdir(os.path.join(ROOT, "profiles")) if n.startswith("traffic_")]
    assert names
    for n in names:
        with open(os.path.join(ROOT, "profiles", n)) as fh:
            assert json.load(fh)["source_hash"] == h, n
