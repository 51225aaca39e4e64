"""CPU tests of bench.py's host logic: the algorithmic byte counts its rooflines divide by, the conversion of
rocprofv3 counter CSVs into per-kernel HBM bytes and matrix-core cycles, and the one-GPU guard. No GPU work."""
import csv
import json
import os
import subprocess
import sys
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parent.parent
sys.path.insert(0, str(ROOT))
import bench  # noqa: E402
from kda_gated_delta_chunk_amd.source_hash import csrc_hash  # noqa: E402

FIELDS = ["Correlation_Id", "Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]


def _csv(path, counter, rows):
    """rows: (dispatch id, kernel name, value in KiB)."""
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=FIELDS)
        w.writeheader()
        for i, name, value in rows:
            w.writerow({"Correlation_Id": i, "Dispatch_Id": i, "Kernel_Name": name, "Counter_Name": counter,
                        "Counter_Value": value})


def test_prefill_algorithmic_bytes_of_the_4096_token_workload():
    # q, k, g, v, o at 256 B per token-head and beta at 2 B: 1,282 B per token-head, plus S_final (6.3 MB)
    total, per = bench.prefill_algorithmic_bytes(4096, 96, 128, 128, 1)
    assert total == 4096 * 96 * 1282 + 96 * 128 * 128 * 4 == 510_394_368
    assert per["prep"] == 4096 * 96 * 770 == 302_776_320
    assert per["state"] == 4096 * 96 * 512 + 96 * 128 * 128 * 4 == 207_618_048
    # fp32 I/O doubles the per-token bytes; an initial state adds its read
    t32, _ = bench.prefill_algorithmic_bytes(64, 2, 32, 32, 1, es=4, with_S0=True)
    assert t32 == 64 * 2 * (3 * 32 * 4 + 32 * 4 + 4 + 32 * 4) + 2 * 2 * 32 * 32 * 4


def _counter_runs(tmp_path):
    k_prep = "void kda::kda_chunk_prep<true, 128, false, false>(kda::PrepParams)"
    k_bwd = "void kda::(anonymous namespace)::kda_bwd_kernel<true, 128, false, false>(float const*)"
    copy = "__amd_rocclr_copyBuffer"
    gib = 1 << 20  # 1 GiB in KiB
    # dispatch order: a small copy, the 1 GiB calibration copy, the prep's first leg (3 dispatches), a later
    # leg of the prep with other bytes, a 2 GiB copy (not the calibration), the backward kernel
    fetch = [(1, copy, 64.0), (2, copy, gib / 2), (3, k_prep, 1000.0), (4, k_prep, 1000.0), (5, k_prep, 1000.0),
             (6, k_prep, 4000.0), (7, copy, gib), (8, k_bwd, 500.0)]
    write = [(1, copy, 64.0), (2, copy, gib), (3, k_prep, 2000.0), (4, k_prep, 2000.0), (5, k_prep, 2000.0),
             (6, k_prep, 2000.0), (7, copy, 2 * gib), (8, k_bwd, 100.0)]
    f, w = tmp_path / "fetch.csv", tmp_path / "write.csv"
    _csv(f, "FETCH_SIZE", fetch)
    _csv(w, "WRITE_SIZE", write)
    return f, w


def test_traffic_from_counters_calibrates_on_the_first_large_copy(tmp_path):
    f, w = _counter_runs(tmp_path)
    out = bench.traffic_from_counters(str(f), str(w), str(tmp_path / "traffic.json"))
    # FETCH_SIZE read half of the 1 GiB copy's bytes, WRITE_SIZE all of them (the 2 GiB copy is not used)
    assert out["fetch_scale"] == pytest.approx(2.0) and out["write_scale"] == pytest.approx(1.0)
    assert out["csrc_hash"] == csrc_hash()
    prep = out["kernels"]["kda::kda_chunk_prep<true, 128, false, false>"]
    # first leg = the first three dispatches; all legs = every dispatch
    assert prep["fetch_bytes"] == pytest.approx(1000 * 1024 * 2.0)
    assert prep["write_bytes"] == pytest.approx(2000 * 1024 * 1.0)
    assert prep["traffic_bytes"] == pytest.approx(prep["fetch_bytes"] + prep["write_bytes"])
    assert prep["traffic_bytes_all_legs"] == pytest.approx((1750 * 2.0 + 2000) * 1024)
    # kernels in an anonymous namespace keep their own names
    assert "kda::kda_bwd_kernel<true, 128, false, false>" in out["kernels"]
    assert json.loads((tmp_path / "traffic.json").read_text()) == out


def test_mfma_from_counters_adds_busy_cycles_of_the_first_leg(tmp_path):
    f, w = _counter_runs(tmp_path)
    path = tmp_path / "traffic.json"
    bench.traffic_from_counters(str(f), str(w), str(path))
    k = "void kda::kda_chunk_prep<true, 128, false, false>(kda::PrepParams)"
    sq = tmp_path / "sq.csv"
    _csv(sq, "SQ_VALU_MFMA_BUSY_CYCLES", [(3, k, 10.0), (4, k, 20.0), (5, k, 30.0), (6, k, 1000.0)])
    out = bench.mfma_from_counters(str(sq), str(path))
    assert out["kernels"]["kda::kda_chunk_prep<true, 128, false, false>"]["mfma_busy_cycles"] == pytest.approx(20.0)


def test_mfma_from_counters_refuses_a_summary_of_other_sources(tmp_path):
    path = tmp_path / "traffic.json"
    path.write_text(json.dumps({"csrc_hash": "0" * 16, "kernels": {}}))
    sq = tmp_path / "sq.csv"
    _csv(sq, "SQ_VALU_MFMA_BUSY_CYCLES", [])
    with pytest.raises(SystemExit):
        bench.mfma_from_counters(str(sq), str(path))


def test_bench_runs_on_one_gpu_only():
    env = dict(os.environ, CUDA_VISIBLE_DEVICES="")
    r = subprocess.run([sys.executable, str(ROOT / "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       env=env, cwd=str(ROOT), timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""
