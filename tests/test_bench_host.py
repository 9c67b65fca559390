"""Host-side pieces of bench.py, on the CPU.

The byte counts that every GB/s figure divides by are checked against the
per-token sizes the workload's tensor shapes fix (bf16 activations: AdaLN
reads and writes D values, the gated residual reads two and writes one row of
D, SwiGLU reads 2F and writes F, QK reads and writes q and k of H x Dh plus a
12-byte position).  The oracle-rate leg of the CPU baseline runs on the
32-token workload.
"""
import math

import pytest

import bench
import oracle
import synthetic_inputs as si


def test_more_than_one_gpu_is_refused_before_any_device_work(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err


@pytest.mark.parametrize("name", ["tiny", "full5s", "batch2"])
def test_chain_bytes_per_token(name):
    wl = si.WORKLOADS[name]
    b = bench.op_bytes(wl)
    R, B, N = wl.R, wl.B, wl.N
    per_token = {"adaln": 2 * 2 * wl.D, "residual": 3 * 2 * wl.D, "swiglu": 3 * 2 * wl.F,
                 "qk": 4 * 2 * wl.H * wl.Dh}
    if name != "tiny":
        # the 1344x768 workloads: 16,384 + 24,576 + 98,304 + 32,768 = 172,032 bytes per token
        assert per_token == {"adaln": 16384, "residual": 24576, "swiglu": 98304, "qk": 32768}
    # per-launch extras: the [B, D] modulation vectors, positions once per token of a sample, the two
    # RMSNorm weights
    assert b["adaln"] == R * per_token["adaln"] + 2 * B * wl.D * 2
    assert b["residual"] == R * per_token["residual"] + B * wl.D * 2
    assert b["swiglu"] == R * per_token["swiglu"]
    assert b["qk"] == R * per_token["qk"] + 12 * N + 2 * wl.Dh * 2
    assert b["positions"] == 12 * N


def test_next_row_bytes_full5s():
    wl = si.WORKLOADS["full5s"]
    b = bench.op_bytes(wl, next_rows=True)
    nb, keep = 1953, 489  # ceil(124,992 / 64) blocks; 1953 - floor(0.75 * 1953) kept
    assert bench.dit_keep(nb) == keep
    assert b["residual_adaln"] == 4 * wl.R * wl.D * 2 + 3 * wl.D * 2  # 8 bytes per element
    assert b["residual_adaln"] < b["adaln"] + b["residual"]  # the fusion saves the re-read of x_out
    assert b["qk_layout"] == b["qk"]
    assert b["scores"] == 2 * 32 * nb * 128 * 4 + 32 * nb * nb * 4
    assert b["topk"] == 32 * nb * nb * 4 + 32 * nb * keep * 4


def test_committed_traffic_is_gated_by_workload_and_close_to_algorithmic():
    assert bench.committed_traffic("swiglu", "tiny") is None  # no counter summary for that workload
    t = bench.committed_traffic("swiglu", "full5s")
    if t is not None:  # present while the kernel source matches the summary's hash
        assert abs(t / bench.op_bytes(si.WORKLOADS["full5s"])["swiglu"] - 1) < 0.02


def test_next_row_oracle_rates_on_the_tiny_workload():
    wl = si.WORKLOADS["tiny"]
    ins = si.make_inputs(wl, "cpu", names=["q", "k", "wq", "wk", "res_x", "res_y"])
    pos = oracle.packed_positions(*wl.grid, wl.n_extra)
    rates = bench.next_row_oracle_rates(wl, ins, pos, fused_tokens=32, fused_seconds=0.01, threads=1)
    assert set(rates) == {"fused_residual_adaln", "qk_layout", "residual_change", "subblock_pool",
                          "subblock_scores", "subblock_topk"}
    for row in rates.values():
        rate = row.get("tokens_per_s") or row.get("scores_per_s") or row.get("rows_per_s")
        assert rate is not None and rate > 0 and math.isfinite(rate)
        assert row["threads"] >= 1 and row["sample"]
    assert rates["subblock_scores"]["sample"].startswith("1 query blocks x 1 key blocks")  # 32 tokens: one block


def test_sq_summary_from_synthetic_counter_files(tmp_path):
    import csv

    topk = "void dit::(anonymous namespace)::subblock_topk_kernel<8>(float const*, int*, int, int, int, int)"
    trace, sq = tmp_path / "trace", tmp_path / "sq"
    trace.mkdir()
    sq.mkdir()
    with open(trace / "t_kernel_trace.csv", "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(["Kernel_Name", "Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z", "Start_Timestamp", "End_Timestamp"])
        w.writerow([topk, 64 * 1953, 32, 1, 1_000, 201_000])  # 200 us
        w.writerow([topk, 64 * 100, 32, 1, 0, 50_000])  # a smaller launch, left out
    waves = 62_496
    vals = {"SQ_WAVES": waves, "SQ_INSTS_VALU": waves * 1000, "SQ_INSTS_SALU": waves * 500, "SQ_INSTS_LDS": waves * 80,
            "SQ_INSTS_MFMA": 0, "SQ_INSTS_VMEM_RD": waves * 8, "SQ_WAIT_INST_LDS": 25, "SQ_WAVE_CYCLES": 100}
    with open(sq / "p_counter_collection.csv", "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"])
        for c, v in vals.items():
            w.writerow([7, topk, 64 * 1953 * 32, c, v])
    assert bench.summarize_sq(str(trace), str(sq), "full5s", out_dir=str(tmp_path)) == 0
    text = (tmp_path / "kernels_full5s_sq_counters.md").read_text()
    row = next(line for line in text.splitlines() if line.startswith("| topk |"))
    cells = [c.strip() for c in row.strip("|").split("|")]
    # waves, VALU / wave, SALU / wave, LDS / wave, MFMA / wave, VMEM / wave, LDS wait %, avg us
    assert cells[1:10] == ["1", "62496", "1000.0", "500.0", "80.0", "0.0", "8.0", "25.0", "200.00"]
    # 62.5 M wave instructions in 200 us against 256 x 4 x 2.4e9 / 4 per second
    assert float(cells[10]) == pytest.approx(100 * waves * 1000 / 200e-6 / (256 * 4 * 2.4e9 / 4), abs=0.06)


def test_value_is_withheld_when_parity_fails():
    good = {"value": 6500.0, "cpu_baseline": {"parity_ok": True}}
    assert bench.gate_on_parity(good, {"a": True}) and good["value"] == 6500.0
    assert good["parity_checked"] is True and good["parity_ok"] is True
    bad_oracle = {"value": 6500.0, "cpu_baseline": {"parity_ok": False}}
    assert not bench.gate_on_parity(bad_oracle, {"a": True})
    assert bad_oracle["value"] is None and bad_oracle["value_if_parity_held"] == 6500.0
    assert bad_oracle["parity_ok"] is False
    bad_consistency = {"value": 1.0, "cpu_baseline": {"parity_ok": True}}
    assert not bench.gate_on_parity(bad_consistency, {"a": True, "b": False}) and bad_consistency["value"] is None
    unchecked = {"value": 2.0}
    assert bench.gate_on_parity(unchecked, {"a": True})
    assert unchecked["parity_checked"] is False and unchecked["parity_ok"] is None and unchecked["value"] == 2.0


def test_ceilings_summary_from_synthetic_trace(tmp_path):
    wl = si.WORKLOADS["full5s"]
    nbytes = bench.op_bytes(wl, next_rows=True)
    stats = {"p_swiglu": {"name": "pattern_split_rows_kernel", "calls": 10, "avg_us": 1800.0},
             "swiglu": {"name": "swiglu_kernel<true>", "calls": 10, "avg_us": 1890.0},
             "p_head_major": {"name": "pattern_head_major_kernel", "calls": 20, "avg_us": 350.0},
             "qk_layout": {"name": "qk_rmsnorm_rope3d_head_major_kernel<16>", "calls": 10, "avg_us": 728.0}}
    bench.write_ceilings_summary(stats, nbytes, wl, "full5s", "cmd", str(tmp_path))
    text = (tmp_path / "ceilings_full5s.md").read_text()
    assert "| 1.050 |" in text  # 1890 / 1800
    assert "| 1.040 |" in text  # 728 / (2 x 350)
    assert nbytes["p_swiglu"] == nbytes["swiglu"]

