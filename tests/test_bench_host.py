"""Host-side pieces of bench.py: the single-GPU guard, the rocprofv3 counter summaries and the workgroup-timeline summary."""
import csv
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

HEADER = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id", "Grid_Size",
          "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size", "Scratch_Size", "VGPR_Count",
          "Accum_VGPR_Count", "SGPR_Count", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]


def _csv(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(HEADER)
        for i, (kernel, counter, value) in enumerate(rows):
            w.writerow([i, i, "Agent 1", 1, 1, 1, 256, 1, kernel, 256, 0, 0, 8, 0, 16, counter, value, 0, 1])


def test_multi_gpu_request_exits_with_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_pmc_summary_scales_by_copy_calibration(tmp_path, capsys):
    gib_kib = (1 << 30) / 1024
    k = "_ZN3pva12_GLOBAL__N_115fwd_bf16_kernelILi128EEEv"
    _csv(tmp_path / "f.csv", [("other", "FETCH_SIZE", 5.0), (k, "FETCH_SIZE", 1000.0), (k, "FETCH_SIZE", 3000.0)])
    _csv(tmp_path / "w.csv", [(k, "WRITE_SIZE", 4000.0)])
    _csv(tmp_path / "cf.csv", [("__amd_rocclr_copyBuffer", "FETCH_SIZE", gib_kib / 2)])
    _csv(tmp_path / "cw.csv", [("__amd_rocclr_copyBuffer", "WRITE_SIZE", gib_kib)])

    class A:
        workload = "tiny"
        pmc_summary = [str(tmp_path / n) for n in ("f.csv", "w.csv", "cf.csv", "cw.csv")]
    bench.pmc_summary(A)
    rec = dict(line.split(": ", 1) for line in capsys.readouterr().out.strip().splitlines())
    assert float(rec["copy_fetch_factor"]) == pytest.approx(0.5)
    # mean 2000 KiB fetched per dispatch at factor 0.5 -> 4000 KiB; 4000 KiB written at factor 1
    assert int(rec["fetch_bytes_per_launch"]) == 4000 * 1024
    assert int(rec["write_bytes_per_launch"]) == 4000 * 1024
    assert int(rec["traffic_bytes_per_launch"]) == 8000 * 1024


def test_stored_traffic_requires_current_sources(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    path = bench.traffic_file("bf16", "wl")
    with open(path, "w") as f:
        f.write(f"# comment: ignored\nsource_sha256_16: {bench.kernel_source_hash('bf16')}\n"
                "traffic_bytes_per_launch: 12345\n")
    assert bench.stored_traffic("bf16", "wl") == 12345
    with open(path, "w") as f:
        f.write("source_sha256_16: 0000000000000000\ntraffic_bytes_per_launch: 12345\n")
    assert bench.stored_traffic("bf16", "wl") is None
    assert bench.stored_traffic("fp8", "missing") is None


def test_algorithmic_bytes():
    import workloads
    w = workloads.WORKLOADS["mixed_res"]()
    assert bench.algorithmic_bytes(w) == 4 * 2 * 25072 * 32 * 128
    w8 = workloads.WORKLOADS["mixed_res_fp8"]()
    assert bench.algorithmic_bytes(w8) == 5 * 25072 * 32 * 128 + 12 * 8 * 32


def test_counter_summary_ratios(tmp_path, capsys):
    k = "_ZN3pva12_GLOBAL__N_115fwd_bf16_kernelILi128EEEv"
    cycles = 1000.0  # per XCD
    vals = {"GRBM_GUI_ACTIVE": 8 * cycles, "SQ_VALU_MFMA_BUSY_CYCLES": 0.5 * 1024 * cycles,
            "SQ_VALU_MFMA_COEXEC_CYCLES": 0.25 * 1024 * cycles, "SQ_INSTS_MFMA": 1024 * cycles / 64,
            "SQ_INSTS_VALU": 5 * 1024 * cycles / 64, "SQ_LDS_BANK_CONFLICT": 7.0, "SQ_ACTIVE_INST_LDS": 1.0,
            "SQ_ACTIVE_INST_VALU": 1.0, "SQ_BUSY_CYCLES": 1.0, "TCC_HIT_sum": 900.0, "TCC_MISS_sum": 100.0}
    _csv(tmp_path / "sq.csv", [("other", "SQ_INSTS_MFMA", 1e9)] + [(k, c, v) for c, v in vals.items()])
    _csv(tmp_path / "u.csv", [(k, "MfmaUtil", 49.0)])

    class A:
        workload = "tiny"
        counter_summary = [str(tmp_path / "sq.csv"), str(tmp_path / "u.csv")]
    bench.counter_summary(A)
    rec = dict(line.split(": ", 1) for line in capsys.readouterr().out.strip().splitlines())
    assert float(rec["mfma_busy_pct"]) == pytest.approx(50.0)
    assert float(rec["valu_coissue_pct_of_mfma_busy"]) == pytest.approx(50.0)
    assert float(rec["mfma_cycles_per_instruction"]) == pytest.approx(32.0)
    assert float(rec["valu_instructions_per_mfma"]) == pytest.approx(5.0)
    assert float(rec["l2_hit_pct"]) == pytest.approx(90.0)
    assert float(rec["lds_bank_conflict_cycles"]) == 7.0
    assert float(rec["mfma_util_derived_pct"]) == pytest.approx(49.0)


def _timed_csv(path, kernel, vals, ns):
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(HEADER)
        for i, (counter, value) in enumerate(vals.items()):
            w.writerow([i, 7, "Agent 1", 1, 1, 1, 256, 1, kernel, 256, 0, 0, 8, 0, 16, counter, value, 0, ns])


def test_stall_summary_decomposes_the_fraction_of_peak(tmp_path, capsys):
    import workloads
    k = "_ZN3pva12_GLOBAL__N_115fwd_bf16_kernelILi128EEEv"
    w = workloads.WORKLOADS["mixed_res"]()
    useful = 4 * w.head_dim * w.num_heads * sum(t * (t + 1) // 2 + i * (t + i)
                                                  for t, i in zip(w.text_len, w.image_len))
    cycles = 2.4e6  # shader cycles per XCD; 2 ms at 1.2 GHz
    busy = useful / 1024  # busy cycles whose every FLOP is useful
    wave = {"GRBM_GUI_ACTIVE": 8 * cycles, "SQ_WAVE_CYCLES": 2.5 * 1024 * cycles / 4,
            "SQ_WAIT_ANY": 0.25 * 2.5 * 1024 * cycles / 4, "SQ_WAIT_INST_ANY": 0.5 * 2.5 * 1024 * cycles / 4,
            "SQ_ACTIVE_INST_ANY": 0.25 * 2.5 * 1024 * cycles / 4, "SQ_LDS_DATA_FIFO_FULL": 0.0,
            "SQ_LDS_CMD_FIFO_FULL": 0.0}
    issue = {"GRBM_GUI_ACTIVE": 8 * cycles, "SQ_VALU_MFMA_BUSY_CYCLES": busy, "SQ_INSTS_MFMA": busy / 32,
             "SQ_INSTS_VALU": 5 * busy / 32, "SQ_ACTIVE_INST_VALU": 1.0, "SQ_ACTIVE_INST_LDS": 1.0,
             "SQ_WAIT_INST_LDS": 0.0}
    _timed_csv(tmp_path / "a.csv", k, wave, 2_000_000)
    _timed_csv(tmp_path / "b.csv", k, issue, 2_000_000)

    class A:
        workload = "mixed_res"
        stall_summary = [str(tmp_path / "a.csv"), str(tmp_path / "b.csv")]
    bench.stall_summary(A)
    rec = dict(line.split(": ", 1) for line in capsys.readouterr().out.strip().splitlines())
    assert float(rec["resident_waves_per_simd"]) == pytest.approx(2.5)
    assert float(rec["waiting_to_issue_pct_of_wave_cycles"]) == pytest.approx(50.0)
    assert float(rec["waiting_on_counters_or_barrier_pct_of_wave_cycles"]) == pytest.approx(25.0)
    assert float(rec["shader_clock_ghz_fastest_dispatch"]) == pytest.approx(1.2)
    assert float(rec["clock_share_of_2.4_ghz"]) == pytest.approx(0.5)
    assert float(rec["useful_share_of_mfma_busy_flops"]) == pytest.approx(1.0)
    assert float(rec["mfma_busy_cycles_per_instruction"]) == pytest.approx(32.0)
    busy_share = float(rec["mfma_busy_pct"]) / 100
    assert float(rec["frac_from_counters"]) == pytest.approx(busy_share * 0.5, abs=1e-3)
    # the same product is the useful FLOPs over the peak's FLOPs in the counted duration
    peak_flops = bench.PEAK_TFLOPS["bf16"] * 1e12 * 2e-3
    assert float(rec["frac_from_counters"]) == pytest.approx(useful / peak_flops, rel=2e-3)


def test_stored_counters_require_current_sources(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    path = bench.counters_file("fp8", "wl")
    body = ("mfma_busy_pct: 47.4\nvalu_coissue_pct_of_mfma_busy: 55.0\nvalu_instructions_per_mfma: 15.67\n"
            "lds_bank_conflict_cycles: 0\nl2_hit_pct: 92.1\nshader_clock_ghz_fastest_dispatch: 1.924\n")
    with open(path, "w") as f:
        f.write(f"# comment: ignored\nsource_sha256_16: {bench.kernel_source_hash('fp8')}\n" + body)
    assert bench.stored_counters("fp8", "wl")["mfma_busy_pct"] == 47.4
    with open(path, "w") as f:
        f.write("source_sha256_16: 0000000000000000\n" + body)
    assert bench.stored_counters("fp8", "wl") is None
    assert bench.stored_counters("bf16", "missing") is None


def test_source_hash_ignores_comments():
    code = 'int f(int x) { return x + 1; }  // one\n/* two */ const char* s = "a // b";\n'
    assert bench.code_tokens(code) == bench.code_tokens(code.replace("one", "uno").replace("two", "dos"))
    assert bench.code_tokens(code) != bench.code_tokens(code.replace("x + 1", "x + 2"))
    assert '"a // b"' in bench.code_tokens(code)


def test_padded_batch_matches_the_oracle_padding():
    """The padded comparator's inputs, built by the bench on host tensors:
    layout and (B, 1, Lmax, Lmax) mask equal the oracle's padded formulation
    exactly, and unpad() returns the packed rows."""
    import numpy as np
    import torch
    import oracle
    import workloads
    w = workloads.custom([37, 0, 200, 5, 1], [300, 64, 0, 0, 3], 2, 64, seed=12, name="padded_host")
    q, k, v = workloads.bf16_inputs(w)
    qp, kp, vp, mask, _, _ = bench.padded_batch(w, q, k, v)
    assert np.array_equal(mask.numpy(), oracle.padded_mask(w.text_len, w.image_len))
    for x, xp in ((q, qp), (k, kp), (v, vp)):
        assert np.array_equal(xp.float().numpy().astype(np.float64), oracle.padded_layout(x.float().numpy(), w.seq_len))
    assert torch.equal(bench.unpad(qp, w), q)


def test_next_row_arguments_parse(monkeypatch):
    """Every configuration the bench line's next_rows runs is a valid
    bench.py command line (a typo would only show as a failed row)."""
    import workloads
    for name, extra in bench.NEXT_ROWS.items():
        monkeypatch.setattr(sys, "argv", ["bench.py", *extra, "--steps", "5", "--warmup", "5", "--no-other-configs",
                                          "--no-cpu", "--no-padded", "--cold-iters", "0"])
        a = bench.parse()
        assert a.workload in workloads.WORKLOADS, name
        assert a.kernel_only or a.split_keys > 1, name


def test_timeline_summary_of_known_records():
    """Two CUs, three workgroups each (real-time ticks of 10 ns, a shader
    clock of 1.5 GHz): the summary's per-tile time, cycles, prologue,
    epilogue, refill gap, clocks and CU time shares follow from the records."""
    rows = []
    # (cu, start, prologue end, loop end, end) in ticks; 10 tiles per item
    plan = [(0, 0, 300, 10300, 10500), (0, 0, 300, 10300, 10500), (0, 10600, 10900, 20900, 21100),
            (1, 0, 300, 10300, 10500), (1, 0, 300, 10300, 10500), (1, 10600, 10900, 20900, 21100)]
    for i, (cu, a, b, c, d) in enumerate(plan):
        cyc = (c - b) * 10 * 1.5  # ns * GHz
        rows.append([a, b, c, d, 1000, 1000 + int(cyc), cu << 8, 0, 10, 10, i, 1])
    rows.append([0] * 12)  # an empty slot (not written)
    lines = dict(l.split(": ", 1) for l in bench.timeline_summary(np.array(rows, dtype=np.uint64), 6))
    assert lines["records"] == "6"
    assert lines["cus"] == "2"
    assert float(lines["span_us"]) == pytest.approx(211.0)
    assert float(lines["per_tile_ns_median"]) == pytest.approx(10000.0)
    assert float(lines["per_tile_shader_cycles_median"]) == pytest.approx(15000.0)
    assert float(lines["prologue_us_median"]) == pytest.approx(3.0)
    assert float(lines["epilogue_us_median"]) == pytest.approx(2.0)
    assert float(lines["refill_gap_us_median"]) == pytest.approx(1.0)
    assert float(lines["shader_clock_ghz_median"]) == pytest.approx(1.5)
    shares = dict(kv.split(":") for kv in lines["cu_time_pct_with_k_computing_workgroups"].split())
    # per CU: two loops over [3, 103) us, one over [109, 209) us, within 211 us
    assert float(shares["2"]) == pytest.approx(100 * 100 / 211, abs=0.1)
    assert float(shares["1"]) == pytest.approx(100 * 100 / 211, abs=0.1)
    assert float(shares["0"]) == pytest.approx(100 * 11 / 211, abs=0.1)
